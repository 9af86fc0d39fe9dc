// Internal interface between the C-ABI front end (fa_api.cpp) and the HIP
// launcher (fa_fwd.hip).  Not installed, not part of the public header.
#pragma once

#include <stdint.h>

namespace fa {

struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;  // may be null
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, D;
  float scale;
  int causal;
  int dtype;      // fa_dtype
  void* stream;   // hipStream_t
};

// Arguments are already validated.  Returns FA_OK or FA_ERR_HIP.
int launch_forward(const LaunchArgs& a);

// Query rows per workgroup of the forward kernel (the grid-size limit depends on it).
constexpr int kRowsPerBlock = 128;

}  // namespace fa

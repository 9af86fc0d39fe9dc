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
  int window;     // causal sliding window, 0 = none
  int dtype;      // fa_dtype
  void* stream;   // hipStream_t
};

// Arguments are already validated.  Returns FA_OK or FA_ERR_HIP.
int launch_forward(const LaunchArgs& a);

// Key-split forward: partials into `workspace` (layout below), then the merge
// into a.o / a.lse, both on a.stream.  Arguments are already validated.
int launch_forward_split(const LaunchArgs& a, int n_splits, void* workspace);

// The same, with the partials in the library's per-device scratch array
// (FA_SPLIT_SCRATCH_BYTES); the caller has checked that they fit.  Returns
// FA_OK or FA_ERR_HIP.
int launch_forward_split_noalloc(const LaunchArgs& a, int n_splits);

// Merge of n_parts normalised partials: part_o [n_parts][rows][D] fp32,
// part_lse [n_parts][rows] -> o [rows][D] (dtype), lse [rows].  Validated.
int launch_merge(const float* part_o, const float* part_lse, int n_parts, int64_t rows, int D,
                 void* o, float* lse, int dtype, void* stream);

// Workspace of the key-split forward: partial O, fp32 [splits][rows][D], then
// partial LSE, fp32 [splits][rows], starting at the next 256-byte boundary.
inline int64_t split_partial_o_bytes(int64_t rows, int64_t D, int64_t splits) {
  return (splits * rows * D * 4 + 255) / 256 * 256;
}
inline int64_t split_workspace_bytes(int64_t rows, int64_t D, int64_t splits) {
  return split_partial_o_bytes(rows, D, splits) + splits * rows * 4;
}

// Backward: gradients dq [B,Hq,Nq,D], dk and dv [B,Hkv,Nk,D] (16-bit types).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;  // may be null
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;   // backward_workspace_bytes(B*Hq*Nq) bytes, 16-byte aligned
  int B, Hq, Hkv, Nq, Nk, D;
  float scale;
  int causal;
  int window;        // causal sliding window, 0 = none
  int dtype;
  void* stream;
};

// Arguments are already validated.  Returns FA_OK or FA_ERR_HIP.
int launch_backward(const BwdArgs& a);
// Backward of the residual chain (n_layers 1 .. kMaxChainLayers, D = 64 or
// 128, no bias or window): a as for the last layer (a.dq, a.dk unused),
// q/k_layers the layers' inputs and dq/dk_layers their gradients, oldest
// first; a.dv receives dV.
int launch_backward_chain(const BwdArgs& a, const void* const* q_layers,
                          const void* const* k_layers, void* const* dq_layers,
                          void* const* dk_layers, int n_layers);

// Backward workspace: delta fp32 [rows], then lse2 fp32 [rows] from the next
// 256-byte boundary (rows = B*Hq*Nq).
inline int64_t backward_lse2_offset(int64_t rows) { return (rows + 63) / 64 * 64; }  // floats
inline int64_t backward_workspace_bytes(int64_t rows) {
  return (backward_lse2_offset(rows) + rows) * 4;
}

// Block Attention Residual chain: the logits are sum_l Q_l K_l^T * scale over
// n_layers (1 .. kMaxChainLayers) layers, oldest first; a.q and a.k are the
// last layer's (also q_layers[n-1], k_layers[n-1]), a.v its V.  16-bit types,
// no bias, no window.  Arguments are already validated.
constexpr int kMaxChainLayers = 4;
int launch_forward_chain(const LaunchArgs& a, const void* const* q_layers,
                         const void* const* k_layers, int n_layers);
// Largest key-split count accepted.
constexpr int kMaxSplits = 1024;

// Query rows per workgroup of the forward kernel (the grid-size limit depends on it).
constexpr int kRowsPerBlock = 128;

}  // namespace fa

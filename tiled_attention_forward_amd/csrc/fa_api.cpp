// C-ABI front end of libfa.so: argument validation and dispatch.
//
// fa_check_args is pure host arithmetic on the argument values (no HIP call, no
// pointer dereference), so it can be exercised on a machine without a GPU.

#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

int elem_bytes(int dtype) {
  switch (dtype) {
    case FA_DTYPE_BF16: return 2;
    case FA_DTYPE_FP16: return 2;
    case FA_DTYPE_FP32: return 4;
    default: return 0;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [p, p + n) overlap?
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

extern "C" int fa_check_args(const void* q, const void* k, const void* v, const void* bias,
                             const void* o, const float* lse, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, float scale,
                             int causal, int dtype) {
  (void)causal;
  const int esz = elem_bytes(dtype);
  if (esz == 0) return FA_ERR_DTYPE;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || D < 0) return FA_ERR_BAD_SIZE;
  if (Hq > 0 && Hkv < 1) return FA_ERR_BAD_SIZE;
  if (Hq > 0 && Hq % Hkv != 0) return FA_ERR_HEAD_GROUPS;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const bool empty = (B == 0 || Hq == 0 || Nq == 0);
  if (empty) return FA_OK;
  if (q == nullptr || o == nullptr || lse == nullptr) return FA_ERR_NULL_POINTER;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_NULL_POINTER;
  const int64_t lim = int64_t(1) << 30;
  if (Nq >= lim || Nk >= lim || B >= lim || Hq >= lim) return FA_ERR_TOO_LARGE;
  const int64_t tiles = (Nq + fa::kRowsPerBlock - 1) / fa::kRowsPerBlock;
  if (B * Hq > (int64_t(1) << 31) / tiles) return FA_ERR_TOO_LARGE;
  // Byte offsets inside one head's Q/K/V, and inside one block of bias rows,
  // are 32-bit in the kernel's buffer loads.
  const int64_t lim31 = int64_t(1) << 31;
  if (Nq * D * esz >= lim31 || Nk * D * esz >= lim31) return FA_ERR_TOO_LARGE;
  if (bias != nullptr && int64_t(fa::kRowsPerBlock) * Nk * esz >= lim31) return FA_ERR_TOO_LARGE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (bias != nullptr && !aligned(bias, 16)) || !aligned(lse, 4))
    return FA_ERR_ALIGNMENT;
  const uint64_t nq_b = uint64_t(B) * Hq * Nq * D * esz;
  const uint64_t nkv_b = uint64_t(B) * Hkv * Nk * D * esz;
  const uint64_t nb_b = bias ? uint64_t(B) * Hq * Nq * Nk * esz : 0;
  const uint64_t nl_b = uint64_t(B) * Hq * Nq * 4;
  if (overlap(o, nq_b, q, nq_b) || overlap(o, nq_b, k, nkv_b) || overlap(o, nq_b, v, nkv_b) ||
      overlap(o, nq_b, bias, nb_b) || overlap(o, nq_b, lse, nl_b) ||
      overlap(lse, nl_b, q, nq_b) || overlap(lse, nl_b, k, nkv_b) ||
      overlap(lse, nl_b, v, nkv_b) || overlap(lse, nl_b, bias, nb_b))
    return FA_ERR_OVERLAP;
  return FA_OK;
}

extern "C" int fa_forward(const void* q, const void* k, const void* v, const void* bias,
                          void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                          int64_t Nk, int64_t D, float scale, int causal, int dtype,
                          void* stream) {
  const int st = fa_check_args(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal,
                               dtype);
  if (st != FA_OK) return st;
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  fa::LaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.bias = bias;
  a.o = o;
  a.lse = lse;
  a.B = int(B);
  a.Hq = int(Hq);
  a.Hkv = int(Hkv);
  a.Nq = int(Nq);
  a.Nk = int(Nk);
  a.D = int(D);
  a.scale = scale;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = stream;
  return fa::launch_forward(a);
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SIZE: return "a size is negative, or Hkv < 1";
    case FA_ERR_HEAD_GROUPS: return "Hq is not a multiple of Hkv";
    case FA_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGNMENT: return "a tensor pointer is misaligned (16 bytes; lse 4 bytes)";
    case FA_ERR_OVERLAP: return "o or lse overlaps another buffer";
    case FA_ERR_TOO_LARGE: return "a size exceeds the kernel's index range";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    default: return "unknown status";
  }
}

extern "C" const char* fa_version(void) { return "fa 0.1.0 gfx950"; }

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
    case FA_DTYPE_FP8_E4M3: return 1;
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
  // 64 and 128; 80, 96 (kept in a 128-wide tile) and 256 for the 16-bit types
  const bool dim_ok = D == 64 || D == 128 || ((D == 80 || D == 96 || D == 256) && esz == 2);
  if (!dim_ok) return FA_ERR_HEAD_DIM;
  const bool fp8 = dtype == FA_DTYPE_FP8_E4M3;
  if (fp8 && bias != nullptr) return FA_ERR_DTYPE;  // FP8 takes no logit term
  const int oesz = fp8 ? 2 : esz;                    // FP8 inputs give a bf16 o
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
  const uint64_t no_b = uint64_t(B) * Hq * Nq * D * oesz;
  const uint64_t nkv_b = uint64_t(B) * Hkv * Nk * D * esz;
  const uint64_t nb_b = bias ? uint64_t(B) * Hq * Nq * Nk * esz : 0;
  const uint64_t nl_b = uint64_t(B) * Hq * Nq * 4;
  if (overlap(o, no_b, q, nq_b) || overlap(o, no_b, k, nkv_b) || overlap(o, no_b, v, nkv_b) ||
      overlap(o, no_b, bias, nb_b) || overlap(o, no_b, lse, nl_b) ||
      overlap(lse, nl_b, q, nq_b) || overlap(lse, nl_b, k, nkv_b) ||
      overlap(lse, nl_b, v, nkv_b) || overlap(lse, nl_b, bias, nb_b))
    return FA_ERR_OVERLAP;
  return FA_OK;
}

namespace {

int forward_common(const void* q, const void* k, const void* v, const void* bias, void* o,
                   float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                   int64_t D, float scale, int causal, int window, int dtype, void* stream) {
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
  a.window = window;
  a.dtype = dtype;
  a.stream = stream;
  return fa::launch_forward(a);
}

}  // namespace

extern "C" int fa_forward(const void* q, const void* k, const void* v, const void* bias,
                          void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                          int64_t Nk, int64_t D, float scale, int causal, int dtype,
                          void* stream) {
  return forward_common(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, 0, dtype,
                        stream);
}

extern "C" int fa_forward_window(const void* q, const void* k, const void* v, const void* bias,
                                 void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                                 int64_t Nq, int64_t Nk, int64_t D, float scale, int64_t window,
                                 int dtype, void* stream) {
  if (window < 1) return FA_ERR_BAD_SIZE;
  if (window >= (int64_t(1) << 30)) return FA_ERR_TOO_LARGE;
  return forward_common(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, 1, int(window),
                        dtype, stream);
}

extern "C" int fa_forward_chain(const void* const* q_layers, const void* const* k_layers,
                                int64_t num_layers, const void* v, void* o, float* lse,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                int64_t D, float scale, int causal, int dtype, void* stream) {
  if (q_layers == nullptr || k_layers == nullptr) return FA_ERR_NULL_POINTER;
  if (num_layers < 1 || num_layers > fa::kMaxChainLayers) return FA_ERR_BAD_SIZE;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return FA_ERR_DTYPE;
  if (D != 64 && D != 80 && D != 96 && D != 128) return FA_ERR_HEAD_DIM;
  // each layer's operands against v, o and lse (sizes, pointers, overlap)
  for (int64_t l = 0; l < num_layers; ++l) {
    const int st = fa_check_args(q_layers[l], k_layers[l], v, nullptr, o, lse, B, Hq, Hkv, Nq,
                                 Nk, D, scale, causal, dtype);
    if (st != FA_OK) return st;
  }
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  const int n = int(num_layers);
  fa::LaunchArgs a;
  a.q = q_layers[n - 1];
  a.k = k_layers[n - 1];
  a.v = v;
  a.bias = nullptr;
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
  a.window = 0;
  a.dtype = dtype;
  a.stream = stream;
  return fa::launch_forward_chain(a, q_layers, k_layers, n);
}

namespace {

// Sizes of the key-split path, after the common checks: index limits of the
// packed row space and of the grid.
int check_split_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t D, int esz,
                      int64_t num_splits) {
  if (num_splits < 1 || num_splits > fa::kMaxSplits) return FA_ERR_BAD_SIZE;
  const int64_t lim31 = int64_t(1) << 31;
  const __int128 rows = __int128(Hq / Hkv) * Nq;  // packed rows of one KV head
  if (rows * D * esz >= lim31) return FA_ERR_TOO_LARGE;
  const int64_t tiles = (int64_t(rows) + fa::kRowsPerBlock - 1) / fa::kRowsPerBlock;
  if (__int128(B) * Hkv * tiles * num_splits >= lim31) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

}  // namespace

extern "C" int fa_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D,
                                        int64_t num_splits, int64_t* bytes) {
  if (bytes == nullptr) return FA_ERR_NULL_POINTER;
  if (B < 0 || Hq < 0 || Nq < 0 || D < 0) return FA_ERR_BAD_SIZE;
  if (num_splits < 1 || num_splits > fa::kMaxSplits) return FA_ERR_BAD_SIZE;
  if (D != 64 && D != 80 && D != 96 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  const __int128 rows = __int128(B) * Hq * Nq;
  if (rows * D * 4 * num_splits >= (__int128(1) << 62)) return FA_ERR_TOO_LARGE;
  *bytes = fa::split_workspace_bytes(int64_t(rows), D, num_splits);
  return FA_OK;
}

extern "C" int fa_split_count(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                              int64_t D, int64_t* num_splits) {
  if (num_splits == nullptr) return FA_ERR_NULL_POINTER;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || D < 0) return FA_ERR_BAD_SIZE;
  if (Hq > 0 && Hkv < 1) return FA_ERR_BAD_SIZE;
  if (Hq > 0 && Hq % Hkv != 0) return FA_ERR_HEAD_GROUPS;
  if (D != 64 && D != 80 && D != 96 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  *num_splits = 1;
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  const int64_t lim = int64_t(1) << 30;
  if (B >= lim || Hq >= lim || Nq >= lim || Nk >= lim) return FA_ERR_TOO_LARGE;
  // About 512 workgroups: two per compute unit, as many as are resident at
  // once (register and LDS limits of the forward kernel), so the grid runs in
  // one round; each split keeps at least 4 key tiles so the partials stay a
  // small fraction of the traffic.
  constexpr int64_t kTargetBlocks = 512;
  const __int128 rows = __int128(Hq / Hkv) * Nq;
  const __int128 units = __int128(B) * Hkv * ((rows + fa::kRowsPerBlock - 1) / fa::kRowsPerBlock);
  if (units >= kTargetBlocks) return FA_OK;
  int64_t s = (kTargetBlocks + int64_t(units) - 1) / int64_t(units);
  const int64_t tiles = (Nk + 63) / 64;
  const int64_t cap = tiles / 4 > 1 ? tiles / 4 : 1;
  if (s > cap) s = cap;
  if (s > fa::kMaxSplits) s = fa::kMaxSplits;
  *num_splits = s;
  return FA_OK;
}

namespace {

// Checks shared by the two key-split entry points (everything except the
// partials' storage), and the launch arguments.  *need receives the bytes of
// the partials.
int split_common(const void* q, const void* k, const void* v, const void* bias, void* o,
                 float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                 int64_t D, float scale, int causal, int dtype, int64_t num_splits,
                 void* stream, fa::LaunchArgs* a, int64_t* need) {
  int st = fa_check_args(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype);
  if (st != FA_OK) return st;
  *need = 0;
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  st = check_split_sizes(B, Hq, Hkv, Nq, D, elem_bytes(dtype), num_splits);
  if (st != FA_OK) return st;
  *need = fa::split_workspace_bytes(B * Hq * Nq, D, num_splits);
  a->q = q;
  a->k = k;
  a->v = v;
  a->bias = bias;
  a->o = o;
  a->lse = lse;
  a->B = int(B);
  a->Hq = int(Hq);
  a->Hkv = int(Hkv);
  a->Nq = int(Nq);
  a->Nk = int(Nk);
  a->D = int(D);
  a->scale = scale;
  a->causal = causal != 0;
  a->window = 0;
  a->dtype = dtype;
  a->stream = stream;
  return FA_OK;
}

}  // namespace

extern "C" int fa_forward_split(const void* q, const void* k, const void* v, const void* bias,
                                void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                                int64_t Nq, int64_t Nk, int64_t D, float scale, int causal,
                                int dtype, int64_t num_splits, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  fa::LaunchArgs a;
  int64_t need = 0;
  const int st = split_common(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype,
                              num_splits, stream, &a, &need);
  if (st != FA_OK) return st;
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need)
    return FA_ERR_WORKSPACE;
  const int esz = elem_bytes(dtype);
  const int oesz = dtype == FA_DTYPE_FP8_E4M3 ? 2 : esz;  // FP8 inputs give a bf16 o
  const int64_t rows = B * Hq * Nq;
  const uint64_t nq_b = uint64_t(rows) * D * esz;
  const uint64_t no_b = uint64_t(rows) * D * oesz;
  const uint64_t nkv_b = uint64_t(B) * Hkv * Nk * D * esz;
  const uint64_t nb_b = bias ? uint64_t(rows) * Nk * esz : 0;
  const uint64_t nl_b = uint64_t(rows) * 4;
  if (overlap(workspace, need, q, nq_b) || overlap(workspace, need, k, nkv_b) ||
      overlap(workspace, need, v, nkv_b) || overlap(workspace, need, bias, nb_b) ||
      overlap(workspace, need, o, no_b) || overlap(workspace, need, lse, nl_b))
    return FA_ERR_OVERLAP;
  return fa::launch_forward_split(a, int(num_splits), workspace);
}

extern "C" int fa_forward_split_noalloc(const void* q, const void* k, const void* v,
                                        const void* bias, void* o, float* lse, int64_t B,
                                        int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                        int64_t D, float scale, int causal, int dtype,
                                        int64_t num_splits, void* stream) {
  fa::LaunchArgs a;
  int64_t need = 0;
  const int st = split_common(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype,
                              num_splits, stream, &a, &need);
  if (st != FA_OK) return st;
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  if (need > FA_SPLIT_SCRATCH_BYTES) return FA_ERR_SCRATCH_LIMIT;
  return fa::launch_forward_split_noalloc(a, int(num_splits));
}

extern "C" int fa_merge(const float* part_o, const float* part_lse, int64_t num_parts,
                        int64_t rows, int64_t D, void* o, float* lse, int dtype, void* stream) {
  const int esz = elem_bytes(dtype);
  if (esz == 0 || dtype == FA_DTYPE_FP8_E4M3) return FA_ERR_DTYPE;
  if (num_parts < 0 || rows < 0 || D < 0) return FA_ERR_BAD_SIZE;
  if (D < 4 || D > 65536 || D % 4 != 0) return FA_ERR_HEAD_DIM;
  if (rows == 0) return FA_OK;
  if (o == nullptr || lse == nullptr) return FA_ERR_NULL_POINTER;
  if (num_parts > 0 && (part_o == nullptr || part_lse == nullptr)) return FA_ERR_NULL_POINTER;
  if (num_parts >= (int64_t(1) << 31) || __int128(num_parts) * rows * D >= (__int128(1) << 60) ||
      __int128(rows) * D >= (__int128(1) << 60))
    return FA_ERR_TOO_LARGE;
  if (!aligned(part_o, 16) || !aligned(o, 16) || !aligned(part_lse, 4) || !aligned(lse, 4))
    return FA_ERR_ALIGNMENT;
  const uint64_t po_b = uint64_t(num_parts) * rows * D * 4, pl_b = uint64_t(num_parts) * rows * 4;
  const uint64_t o_b = uint64_t(rows) * D * esz, l_b = uint64_t(rows) * 4;
  if (overlap(o, o_b, part_o, po_b) || overlap(o, o_b, part_lse, pl_b) ||
      overlap(o, o_b, lse, l_b) || overlap(lse, l_b, part_o, po_b) ||
      overlap(lse, l_b, part_lse, pl_b))
    return FA_ERR_OVERLAP;
  return fa::launch_merge(part_o, part_lse, int(num_parts), rows, int(D), o, lse, dtype, stream);
}

extern "C" int fa_backward_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t* bytes) {
  if (bytes == nullptr) return FA_ERR_NULL_POINTER;
  if (B < 0 || Hq < 0 || Nq < 0) return FA_ERR_BAD_SIZE;
  const __int128 rows = __int128(B) * Hq * Nq;
  if (rows >= (__int128(1) << 60)) return FA_ERR_TOO_LARGE;
  *bytes = fa::backward_workspace_bytes(int64_t(rows));
  return FA_OK;
}

namespace {

// The backward's checks; fills *a for the launch, or sets *empty when there is
// nothing to compute.
int backward_prepare(const void* q, const void* k, const void* v, const void* bias,
                     const void* o, const float* lse, const void* dout, void* dq, void* dk,
                     void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                     int64_t D, float scale, int causal, int window, int dtype, void* workspace,
                     int64_t workspace_bytes, void* stream, fa::BwdArgs* a, bool* empty) {
  *empty = false;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_FP32)
    return FA_ERR_DTYPE;  // no FP8 backward
  int st = fa_check_args(q, k, v, bias, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (D != 64 && D != 80 && D != 96 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;  // the backward kernels' tiles
  if (D == 256 && bias != nullptr) return FA_ERR_HEAD_DIM;  // D = 256: no logit term
  if (dtype == FA_DTYPE_FP32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;  // as the fp32 forward
  const int esz = elem_bytes(dtype);
  const bool no_rows = (B == 0 || Hq == 0 || Nq == 0);
  const bool no_keys = (B == 0 || Hkv == 0 || Nk == 0);
  if (no_rows && no_keys) {
    *empty = true;
    return FA_OK;
  }
  // pointers fa_check_args does not cover, or skipped for an empty row space
  if (!no_rows && (dout == nullptr || dq == nullptr)) return FA_ERR_NULL_POINTER;
  if (!no_keys && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return FA_ERR_NULL_POINTER;
  if (no_rows && (!aligned(k, 16) || !aligned(v, 16))) return FA_ERR_ALIGNMENT;
  const int64_t lim = int64_t(1) << 30;
  if (B >= lim || Hq >= lim || Hkv >= lim || Nq >= lim || Nk >= lim) return FA_ERR_TOO_LARGE;
  const int64_t lim31 = int64_t(1) << 31;
  // dK/dV kernel: the packed query rows of one KV head, and its grid
  if (Hkv > 0 && __int128(Hq / Hkv) * Nq * D * esz >= lim31) return FA_ERR_TOO_LARGE;
  if (Nk * D * esz >= lim31) return FA_ERR_TOO_LARGE;
  if (__int128(B) * Hkv * ((Nk + 127) / 128) >= lim31) return FA_ERR_TOO_LARGE;
  if (__int128(B) * Hq * ((Nq + 127) / 128) >= lim31) return FA_ERR_TOO_LARGE;  // dQ grid
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FA_ERR_ALIGNMENT;
  const int64_t rows = B * Hq * Nq;
  const int64_t need = fa::backward_workspace_bytes(rows);
  if (rows > 0 && (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need))
    return FA_ERR_WORKSPACE;
  // outputs and workspace must not overlap the inputs or each other
  const uint64_t nq_b = uint64_t(rows) * D * esz;
  const uint64_t nkv_b = uint64_t(B) * Hkv * Nk * D * esz;
  const uint64_t nb_b = bias ? uint64_t(rows) * Nk * esz : 0;
  const uint64_t nl_b = uint64_t(rows) * 4;
  const uint64_t ws_b = rows > 0 ? uint64_t(need) : 0;
  struct Buf { const void* p; uint64_t n; };
  const Buf ins[] = {{q, nq_b}, {k, nkv_b}, {v, nkv_b}, {bias, nb_b}, {o, nq_b}, {lse, nl_b},
                     {dout, nq_b}};
  const Buf outs[] = {{dq, nq_b}, {dk, nkv_b}, {dv, nkv_b}, {workspace, ws_b}};
  for (const Buf& a : outs) {
    for (const Buf& b : ins)
      if (overlap(a.p, a.n, b.p, b.n)) return FA_ERR_OVERLAP;
    for (const Buf& b : outs)
      if (&a != &b && overlap(a.p, a.n, b.p, b.n)) return FA_ERR_OVERLAP;
  }
  a->q = q;
  a->k = k;
  a->v = v;
  a->bias = bias;
  a->o = o;
  a->dout = dout;
  a->lse = lse;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->workspace = workspace;
  a->B = int(B);
  a->Hq = int(Hq);
  a->Hkv = int(Hkv);
  a->Nq = int(Nq);
  a->Nk = int(Nk);
  a->D = int(D);
  a->scale = scale;
  a->causal = causal != 0;
  a->window = window;
  a->dtype = dtype;
  a->stream = stream;
  return FA_OK;
}

int backward_common(const void* q, const void* k, const void* v, const void* bias, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t B,
                    int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, float scale,
                    int causal, int window, int dtype, void* workspace, int64_t workspace_bytes,
                    void* stream) {
  fa::BwdArgs a;
  bool empty;
  const int st = backward_prepare(q, k, v, bias, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, D,
                                  scale, causal, window, dtype, workspace, workspace_bytes,
                                  stream, &a, &empty);
  if (st != FA_OK || empty) return st;
  return fa::launch_backward(a);
}

}  // namespace

extern "C" int fa_backward(const void* q, const void* k, const void* v, const void* bias,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                           int64_t D, float scale, int causal, int dtype, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  return backward_common(q, k, v, bias, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, D, scale,
                         causal, 0, dtype, workspace, workspace_bytes, stream);
}

extern "C" int fa_backward_window(const void* q, const void* k, const void* v, const void* bias,
                                  const void* o, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                                  int64_t Nq, int64_t Nk, int64_t D, float scale, int64_t window,
                                  int dtype, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  if (window < 1) return FA_ERR_BAD_SIZE;
  if (window >= (int64_t(1) << 30)) return FA_ERR_TOO_LARGE;
  return backward_common(q, k, v, bias, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, D, scale,
                         1, int(window), dtype, workspace, workspace_bytes, stream);
}

extern "C" int fa_backward_chain(const void* const* q_layers, const void* const* k_layers,
                                 int64_t num_layers, const void* v, const void* o,
                                 const float* lse, const void* dout, void* const* dq_layers,
                                 void* const* dk_layers, void* dv, int64_t B, int64_t Hq,
                                 int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, float scale,
                                 int causal, int dtype, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  if (q_layers == nullptr || k_layers == nullptr || dq_layers == nullptr || dk_layers == nullptr)
    return FA_ERR_NULL_POINTER;
  if (num_layers < 1 || num_layers > fa::kMaxChainLayers) return FA_ERR_BAD_SIZE;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return FA_ERR_DTYPE;  // as fa_forward_chain
  if (D != 64 && D != 80 && D != 96 && D != 128) return FA_ERR_HEAD_DIM;  // as fa_forward_chain
  const int n = int(num_layers);
  fa::BwdArgs a;
  bool empty = false;
  for (int l = 0; l < n; ++l) {
    const int st = backward_prepare(q_layers[l], k_layers[l], v, nullptr, o, lse, dout,
                                    dq_layers[l], dk_layers[l], dv, B, Hq, Hkv, Nq, Nk, D, scale,
                                    causal, 0, dtype, workspace, workspace_bytes, stream, &a,
                                    &empty);
    if (st != FA_OK) return st;
  }
  if (empty) return FA_OK;
  // across layers: no output may overlap any layer's input or another output
  const int esz = elem_bytes(dtype);
  const int64_t rows = B * Hq * Nq;
  const uint64_t nq_b = uint64_t(rows) * D * esz;
  const uint64_t nkv_b = uint64_t(B) * Hkv * Nk * D * esz;
  const uint64_t ws_b = rows > 0 ? uint64_t(fa::backward_workspace_bytes(rows)) : 0;
  struct Buf { const void* p; uint64_t n; };
  Buf ins[2 * fa::kMaxChainLayers + 4], outs[2 * fa::kMaxChainLayers + 2];
  int ni = 0, no = 0;
  for (int l = 0; l < n; ++l) {
    ins[ni++] = {q_layers[l], nq_b};
    ins[ni++] = {k_layers[l], nkv_b};
    outs[no++] = {dq_layers[l], nq_b};
    outs[no++] = {dk_layers[l], nkv_b};
  }
  ins[ni++] = {v, nkv_b};
  ins[ni++] = {o, nq_b};
  ins[ni++] = {lse, uint64_t(rows) * 4};
  ins[ni++] = {dout, nq_b};
  outs[no++] = {dv, nkv_b};
  outs[no++] = {workspace, ws_b};
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return FA_ERR_OVERLAP;
    for (int j = 0; j < no; ++j)
      if (i != j && overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FA_ERR_OVERLAP;
  }
  return fa::launch_backward_chain(a, q_layers, k_layers, dq_layers, dk_layers, n);
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SIZE: return "a size is negative, or Hkv < 1";
    case FA_ERR_HEAD_GROUPS: return "Hq is not a multiple of Hkv";
    case FA_ERR_HEAD_DIM:
      return "head dimension D must be 64 or 128 (80, 96 and 256: bf16/fp16 forward, window, "
             "key split and backward, 256 with no logit term in the backward; the residual "
             "chain takes 64, 80, 96 and 128)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGNMENT: return "a tensor pointer is misaligned (16 bytes; lse 4 bytes)";
    case FA_ERR_OVERLAP: return "o or lse overlaps another buffer";
    case FA_ERR_TOO_LARGE: return "a size exceeds the kernel's index range";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_WORKSPACE: return "the key-split workspace is NULL, too small or misaligned";
    case FA_ERR_SCRATCH_LIMIT:
      return "the key-split partials exceed the library's scratch array (FA_SPLIT_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

extern "C" const char* fa_version(void) { return "fa 0.3.0 gfx950"; }

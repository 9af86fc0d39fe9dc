// Attention backward for gfx950 (MI355X): gradients dQ, dK, dV of the fused
// forward from its saved output O and per-row LSE.
//
// Method: the forward keeps no S or P; the backward recomputes them from Q, K
// and the saved statistic and applies the chain rule ("FlashAttention
// principles and Triton practice", xnwp.cn/news/15505, §2.3 and §4.3; the
// kwkr.cn/news/592482 tutorial, §2.4).  With P = exp(S - LSE):
//     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
// The pages note that dQ collects contributions from every key block; here it
// gets a kernel of its own (one workgroup per query block, looping over key
// tiles), so no atomics are needed and the results are deterministic, at the
// price of computing S and dP twice.
//
// Kernels (16-bit types; D = 64, 128, and 80, 96 in 128-wide tiles, 256
// without a logit term), launched in this order:
//  * fa_bwd_dq_kernel: the forward's layout -- each wave owns 32 query rows,
//    one per lane; S^T = K Q^T and dP^T = V dO^T on 32x32x16 MFMAs with Q and
//    dO rows held in registers and K/V tiles streamed through LDS; then
//    dQ^T += K^T dS^T with K read transposed from LDS.  Its prologue forms
//    delta_i = sum_d dO_id O_id and lse2_i = LSE_i log2(e) (+inf for rows
//    with LSE = -inf, so that their P is exactly 0), fp32, and stores both;
//  * fa_bwd_dkdv_kernel: the roles swapped -- each wave owns 32 keys, one per
//    lane, and the query rows of the KV head's group (packed as the key-split
//    forward packs them) stream through LDS in 32- or 64-row tiles with their
//    delta and lse2: S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//    dK^T += Q^T dS with Q and dO read transposed from LDS.
// P and dS are rounded to the input type for the MFMAs (as P is in the
// forward); all sums are fp32.  fp32 inputs (D = 64, 128) take three plain
// vector-arithmetic kernels instead (fa_bwd32_dq_kernel, then
// fa_bwd32_kv_kernel for dV and for dK), described where they are defined.
//
// The Block Attention Residual chain (NL = 2-4 layers, the "Block Attention
// Residual" post): the logits are the sum of every layer's Q_l K_l^T * scale,
// so both kernels take every layer's Q and K, form S from all their products,
// and then dQ_l = scale dS K_l (dQ kernel) and dK_l = scale dS^T Q_l (dK/dV
// kernel) for a group of layers per launch.
//
// LDS tiles are row-major and unpadded, filled straight from HBM by buffer
// loads with the LDS flag; the 16-byte chunk c of tile row r is stored at
// chunk c ^ lds_swizzle<D>(r), which keeps both access patterns (16-byte row
// reads and transposed reads) free of bank conflicts.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 256;  // 4 waves
// Head sizes 80 and 96 keep the 128-wide LDS row layout of D = 128: the
// 16-byte chunks past the real row are loaded from an offset past every
// resource, which reads 0, so they add nothing to the products; the kernels
// run ceil(D/16) contraction steps and ceil(D/32) output column blocks and
// store only the real columns.
constexpr int lds_width(int D) { return (D == 80 || D == 96) ? 128 : D; }
// dK/dV kernel at D = 64 without a logit term: 3 workgroups per compute unit
// (168 VGPRs, a small spill) measured 11% faster than 2 (180 VGPRs) on the
// B2 H16 S4096 causal backward; with a logit term the spill grows, so 2.
#ifndef FA_DKDV_MINB64
#define FA_DKDV_MINB64 3
#endif
// Where the dK/dV kernel keeps its key block's K and V, and the height of the
// query tiles it streams:
//  * D = 64: K and V in registers, 64-row query tiles;
//  * D = 128 without a logit term: K in registers, V in LDS (32 KB) and 32-row
//    query tiles (two 16.3 KB stages), 66 KB in all: two workgroups per compute
//    unit at 256 VGPRs without spilling.  Before, the non-causal instance kept
//    V in registers too, with 64-row tiles, and spilled 140 bytes per lane
//    (147 MB of scratch writes per B8 H32 S2048 backward, their reloads
//    waited in the tile loop): that backward took 2.26 ms, 1.88 ms now; the
//    causal instances kept K and V in LDS, one workgroup per compute unit:
//    1.30 ms, 1.11 ms now;
//  * D = 128 with a logit term: K and V in LDS (64 KB) and 64-row tiles, one
//    workgroup per compute unit (the layout above spilled 188 bytes there).
#ifndef FA_DKDV128_VLDS
#define FA_DKDV128_VLDS 1
#endif
//  * D = 256: K in registers, V in LDS (64 KB), 32-row query tiles (two
//    32.3 KB stages), one workgroup per compute unit.  The dK and dV
//    accumulators together (256 registers) do not fit beside the rest, so
//    the kernel runs its query tiles twice: first for dV (S and P only), then
//    for dK (S, P, dP and dS), with one accumulator set.
// (D = 80 and 96 take the D = 128 layouts: their LDS rows are 128 wide)
constexpr bool dkdv_pair(int D, bool causal, bool bias) {  // two workgroups per CU at D = 128
  return D > 64 && D < 256 && !bias;
}
constexpr bool dkdv_k_in_lds(int D, bool causal, bool bias) {
  return D > 64 && D < 256 && !dkdv_pair(D, causal, bias);
}
constexpr bool dkdv_v_in_lds(int D, bool causal, bool bias) {
  return D == 256 || (D > 64 && (!dkdv_pair(D, causal, bias) || FA_DKDV128_VLDS));
}
// The instance that runs at 256 VGPRs takes its LDS offsets from two
// registers (OffsetsLean) rather than from 24: with the table it spilled.
constexpr bool dkdv_lean_offsets(int D, bool causal, bool bias) {
  return dkdv_pair(D, causal, bias) && FA_DKDV128_VLDS;
}
constexpr int dkdv_qtile(int D, bool causal, bool bias) {
  return (D == 256 || (dkdv_pair(D, causal, bias) && FA_DKDV128_VLDS)) ? 32 : 64;
}
// Keys per tile in the dQ kernel: 64, and 32 at D = 256, whose Q and dO
// fragments (128 VGPRs) and dQ accumulator (128) take one workgroup per
// compute unit already.
constexpr int dq_ktile(int D, int NL) { return (D == 256 || (D > 64 && NL > 1)) ? 32 : 64; }

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;  // [B*Hq*Nq]
  float* lse2;   // [B*Hq*Nq]
  void* dq;
  void* dk;
  void* dv;
  int Hq, Hkv, Nq, Nk;
  int BH, BHkv;
  int group;
  int n_qblk;    // 128-row query blocks per (b, hq)
  int n_kblk;    // 128-key blocks per (b, hk)
  float c;       // scale * log2(e)
  float scale;
  int bias_vec;  // bias rows allow 8-byte loads (Nk % 4 == 0)
  int window;    // causal sliding window (keys i-window+1 .. i), 0 = none
  int64_t rows;  // B * Hq * Nq
  // Block Attention Residual chain (NL > 1 instances): every layer's Q and K,
  // oldest first (the logits are the sum of their products), their dQ and dK,
  // and the first of the chain_targets(D, NL) layers whose dQ (dQ kernel) and
  // dK (dK/dV kernel) this launch forms; dV is formed with target 0 only.
  const void* chain_q[kMaxChainLayers];
  const void* chain_k[kMaxChainLayers];
  void* chain_dq[kMaxChainLayers];
  void* chain_dk[kMaxChainLayers];
  int target;
};

// Chain layers whose gradients one launch forms: all of them at D = 64 (four
// dQ or dK accumulators of 32 registers), two at D = 128 (64 each beside the
// layers' Q or K fragments, 128 registers).
constexpr int chain_targets(int D, int NL) { return D == 64 ? NL : (NL < 2 ? NL : 2); }

// Direct LDS loads of an R x D tile (16-bit, row-major in HBM at a buffer
// resource, first row at byte soff) into the swizzled LDS layout.  Load i of
// wave w fills LDS bytes [1 KB * (w*NI + i), +1 KB) of the tile, lane l the
// 16 bytes at l*16; off[i] is the lane's source offset within the tile.
template <int R, int D>
struct TileLoad {
  static constexpr int DL = lds_width(D);
  static constexpr int RB = D * 2;         // bytes per row in HBM
  static constexpr int CPR = DL * 2 / 16;  // 16-byte chunks per LDS row
  static constexpr int NI = R * CPR / kBwdThreads;
  static_assert(NI * kBwdThreads == R * CPR, "tile must split into whole wave loads");
  int off[NI];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = (wave * NI + i) * 64 + lane;
      const int row = q / CPR, pc = q % CPR;
      const int c = pc ^ lds_swizzle<DL>(row);  // the HBM chunk this LDS chunk holds
      off[i] = c < D / 8 ? row * RB + c * 16 : int(0x80000000u);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* lds, int wave,
                                        uint32_t soff) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (wave * NI + i) * 1024), 16,
                                               unsigned(off[i]), soff, 0, 0);
  }
};

// Per-lane LDS offsets for reading MFMA operands out of a swizzled tile with
// RB bytes per row.
//  row_off[st]: the lane's 16-byte chunk 2*st + g of row ln (A/B operand with
//    the contraction along the row: lane = row, 8 consecutive columns);
//  tr_off[t][db]: the lane's 8-byte piece for ds_read_b64_tr_b16 over the
//    16-row group at row 8*t + 4g + (lane>>2 & 3), column block db: the lane
//    receives 4 consecutive rows of column 32*db + lane % 32 (within a 16-lane
//    group, lane 4a+b receives element b of the chunks read by lanes a, a+4,
//    a+8, a+12); t = 0 and t = 1 give the two halves of one MFMA fragment.
template <int D>
struct Offsets {
  static constexpr int DL = lds_width(D);
  static constexpr int RB = DL * 2;  // bytes per LDS row
  static constexpr int NS = (D + 15) / 16;
  static constexpr int NDB = (D + 31) / 32;
  int row_off[NS];
  int tr_off[2][NDB];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, ln = lane & 31;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      row_off[st] = ln * RB + (((2 * st + g) ^ lds_swizzle<DL>(ln)) * 16);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int r = 8 * t + 4 * g + ((lane >> 2) & 3);
        const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        tr_off[t][db] = r * RB + ((c ^ lds_swizzle<DL>(r)) * 16) + 8 * (lane & 1);
      }
  }
  __device__ __forceinline__ int row(int st) const { return row_off[st]; }
  __device__ __forceinline__ int tr(int t, int db) const { return tr_off[t][db]; }
  __device__ __forceinline__ Offsets fresh() const { return *this; }
};

// The same offsets from two registers: chunk 2*st + g differs from chunk g in
// bits 1-3 only, which the swizzle's XOR leaves alone, so the row offset of
// step st is that of step 0 XOR 32*st; column block db likewise XORs 64*db
// into the transposed offset, and rows +8 flip bit 1 of the swizzle (XOR 32)
// and add 8 rows.  For kernels that run short of registers.
template <int D>
struct OffsetsLean {
  static constexpr int DL = lds_width(D);
  static constexpr int RB = DL * 2;  // bytes per LDS row
  int row0, tr0;
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, ln = lane & 31;
    row0 = ln * RB + ((g ^ lds_swizzle<DL>(ln)) * 16);
    const int r = 4 * g + ((lane >> 2) & 3);
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr0 = r * RB + ((c ^ lds_swizzle<DL>(r)) * 16) + 8 * (lane & 1);
  }
  __device__ __forceinline__ int row(int st) const { return row0 ^ (32 * st); }
  __device__ __forceinline__ int tr(int t, int db) const {
    return (tr0 ^ (64 * db + 32 * t)) + t * 8 * RB;
  }
  // A copy whose registers the compiler must treat as new values, so that the
  // XORs above are redone where they are used instead of being hoisted out of
  // the tile loop into registers of their own.
  __device__ __forceinline__ OffsetsLean fresh() const {
    OffsetsLean o = *this;
    asm volatile("" : "+v"(o.row0), "+v"(o.tr0));
    return o;
  }
};

template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag lds_frag(const char* p) {
  return __builtin_bit_cast(typename Elem<T>::Frag, *reinterpret_cast<const u32x4*>(p));
}

// Two transposed reads (rows +0..3 and +8..11 of a 16-row group, this lane's
// pieces at grp + off0 and grp + off1) -> one MFMA fragment.
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag lds_frag_tr(const char* grp, int off0, int off1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(grp + off0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(grp + off1));
  const u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(typename Elem<T>::Frag, u32x4{lw[0], lw[1], hw[0], hw[1]});
}

// Registers 8h..8h+7 of a 32x32 accumulator, rounded to T as one fragment.
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag pack_half(const f32x16& x, int h) {
  f32x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = x[8 * h + i];
  return Elem<T>::pack8(v);
}

// Store a transposed 32 x (32*NDB) accumulator (lane = output row, register r
// of block db = column 32*db + 8*(r/4) + 4*g + r%4) times `mul` as row `row`
// of a row-major [.., D] tensor: one v_permlane32_swap per word pair gives each
// lane 8 consecutive columns, written as one 16-byte store.
template <typename T, int NDB, int D>
__device__ __forceinline__ void store_rows(T* dst_row, const f32x16 (&acc)[NDB], float mul,
                                           int g, bool ok) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      f32x4 a4, b4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a4[e] = acc[db][8 * pr + e] * mul;
        b4[e] = acc[db][8 * pr + 4 + e] * mul;
      }
      const u32x2 aw = Elem<T>::narrow4(a4), bw = Elem<T>::narrow4(b4);
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(u32(aw[e]), u32(bw[e]), false, false);
        const u32 r0 = r[0], r1 = r[1];
        out[e] = r0;
        out[2 + e] = r1;
      }
      // (D = 80, 96: the last block's columns past D are not stored)
      if (ok && (D % 32 == 0 || db * 32 + 16 * pr + 8 * g < D))
        *reinterpret_cast<u32x4*>(dst_row + db * 32 + 16 * pr + 8 * g) = out;
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, hq, 128-row query block), 64-key tiles.  It also
// forms each row's delta = rowsum(dO o O) and lse2 = LSE log2(e) and leaves
// them in the workspace for the dK/dV kernel, which runs after it.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool BIAS, bool WINDOW, int NL = 1>
__global__ __launch_bounds__(kBwdThreads, (D == 256 || (D > 64 && NL > 1) || NL > 2) ? 1 : 2)
void fa_bwd_dq_kernel(BwdParams p) {
  using E = Elem<T>;
  using Frag = typename E::Frag;
  static_assert(NL == 1 || (!BIAS && !WINDOW && D <= 128), "chain instances");
  constexpr int BN = dq_ktile(D, NL);
  constexpr int NS = (D + 15) / 16, NDB = (D + 31) / 32, NKB = BN / 32;
  constexpr int RB = D * 2;                // bytes per row in HBM
  constexpr int LRB = lds_width(D) * 2;    // bytes per row in LDS
  constexpr int TILE = BN * LRB;  // bytes per K (or V) tile
  // per buffer: the K tiles of the NL layers, then the V tile
  __shared__ __attribute__((aligned(16))) char smem[2][(NL + 1) * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;

  // Causal: heaviest blocks first (as in the forward), the query heads of one
  // KV head at one rank dealt to one XCD.  Non-causal: head-major, the ids of
  // one XCD consecutive, so that a head's blocks share that XCD's L2 copy of
  // K and V.
  int bh, tile;
  if (CAUSAL) {
    const unsigned G = unsigned(p.group), units_per_rank = unsigned(p.BH) / G;
    const UnitMember um = xcd_group_units(blockIdx.x, gridDim.x, G);
    bh = int((um.unit % units_per_rank) * G + um.member);
    const int rank = int(um.unit / units_per_rank);
    const int half = (p.n_qblk + 1) / 2;
    tile = rank < half ? p.n_qblk - 1 - rank : rank - half;
  } else {
    const unsigned logical = xcd_contiguous(blockIdx.x, gridDim.x);
    bh = int(logical / unsigned(p.n_qblk));
    tile = int(logical % unsigned(p.n_qblk));
  }
  const int b = bh / p.Hq, hk = (bh - b * p.Hq) / p.group;
  const int64_t kv_head = int64_t(b) * p.Hkv + hk;
  const int64_t row_base = int64_t(bh) * p.Nq;
  const T* Gh = static_cast<const T*>(p.dout) + row_base * D;
  const T* Vh = static_cast<const T*>(p.v) + kv_head * p.Nk * D;
  const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(Gh, uint32_t(p.Nq) * RB);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(Vh, uint32_t(p.Nk) * RB);
  __amdgpu_buffer_rsrc_t q_rs[NL], k_rs[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const T* Ql = static_cast<const T*>(NL > 1 ? p.chain_q[l] : p.q) + row_base * D;
    const T* Kl = static_cast<const T*>(NL > 1 ? p.chain_k[l] : p.k) + kv_head * p.Nk * D;
    q_rs[l] = make_rsrc(Ql, uint32_t(p.Nq) * RB);
    k_rs[l] = make_rsrc(Kl, uint32_t(p.Nk) * RB);
  }

  const int q_blk = tile * 128;
  const int wq0 = q_blk + wave * 32;
  const int qi = wq0 + ln;
  const bool wave_has_rows = wq0 < p.Nq;
  const int wq_last = min(wq0 + 31, p.Nq - 1);
  const int blk_last = min(q_blk + 127, p.Nq - 1);

  // Q (every layer's) and dO rows of this lane: B operands of S^T = K Q^T
  // and dP^T = V dO^T
  Frag qf[NL][NS], gf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int off = qi * RB + (16 * st + 8 * g) * 2;
#pragma unroll
    for (int l = 0; l < NL; ++l)
      qf[l][st] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(q_rs[l], off, 0, 0));
    gf[st] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(g_rs, off, 0, 0));
  }
  const bool row_ok = qi < p.Nq;
  // delta of this lane's row: the lane holds half of the row's dO (chunks
  // 2*st + g), reads the same half of O and adds its partner's (lane ^ 32).
  // lse2 = +inf for rows with LSE = -inf (no visible key), so their P is 0.
  float dlt, lse2;
  {
    const T* Oh = static_cast<const T*>(p.o) + row_base * D;
    const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(Oh, uint32_t(p.Nq) * RB);
    float acc = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const u32x4 ow =
          __builtin_amdgcn_raw_buffer_load_b128(o_rs, qi * RB + (16 * st + 8 * g) * 2, 0, 0);
      const u32x4 gw = __builtin_bit_cast(u32x4, gf[st]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(E::widen(ow[w] & 0xffffu), E::widen(gw[w] & 0xffffu), acc);
        acc = fmaf(E::widen(ow[w] >> 16), E::widen(gw[w] >> 16), acc);
      }
    }
    acc += __shfl_xor(acc, 32, 64);
    const float l = row_ok ? p.lse[row_base + qi] : -INFINITY;
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    dlt = row_ok ? acc : 0.f;
    if (row_ok && g == 0) {
      p.delta[row_base + qi] = dlt;
      p.lse2[row_base + qi] = lse2;
    }
  }

  // bias rows of this block (resource over the block's rows)
  const T* bblk = BIAS ? static_cast<const T*>(p.bias) + (row_base + q_blk) * p.Nk
                       : static_cast<const T*>(p.q);
  const __amdgpu_buffer_rsrc_t b_rs =
      make_rsrc(bblk, BIAS ? uint32_t(blk_last - q_blk + 1) * uint32_t(p.Nk) * 2 : 0u);

  TileLoad<BN, D> tl;
  tl.init(wave, lane);
  Offsets<D> of;
  of.init(lane);

  // one accumulator set per target layer of this launch
  constexpr int NT = chain_targets(D, NL);
  f32x16 acc[NT][NDB];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[i][db] = f32x16{};

  int n_kv = (p.Nk + BN - 1) / BN;
  if (CAUSAL) n_kv = min(n_kv, blk_last / BN + 1);
  // sliding window (causal only): row i sees keys i-W+1 .. i
  const int W = (CAUSAL && WINDOW) ? p.window : 0;
  const int j_lo = W > 0 ? min(n_kv, max(0, q_blk - W + 1) / BN) : 0;
  const int wave_key_lo = W > 0 ? max(0, wq0 - W + 1) : 0;

  auto issue = [&](int j, int buf) {
#pragma unroll
    for (int l = 0; l < NL; ++l) tl.issue(k_rs[l], smem[buf] + l * TILE, wave, uint32_t(j) * BN * RB);
    tl.issue(v_rs, smem[buf] + NL * TILE, wave, uint32_t(j) * BN * RB);
  };

  // (the K tiles dQ is formed against: the target layers')
  const int tgt = NL > 1 ? p.target : 0;
  auto compute = [&](int j, int buf) {
    const char* sV = smem[buf] + NL * TILE;
    const int key0 = j * BN;
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int l = 0; l < NL; ++l)
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const Frag kf = lds_frag<T>(smem[buf] + l * TILE + kb * 32 * LRB + of.row_off[st]);
          s[kb] = E::mma(kf, qf[l][st], (l == 0 && st == 0) ? f32x16{} : s[kb]);
        }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const Frag vf = lds_frag<T>(sV + kb * 32 * LRB + of.row_off[st]);
        dp[kb] = E::mma(vf, gf[st], st == 0 ? f32x16{} : dp[kb]);
      }
    }
    // register r of block kb: key key0 + kb*32 + 8*(r/4) + 4*g + r%4 of row qi
    const bool need_mask = (key0 + BN > p.Nk) || (CAUSAL && key0 + BN - 1 > wq0) ||
                           (W > 0 && key0 <= wq0 + 31 - W);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float bvals[16];
      if constexpr (BIAS) {
        const int row_off = (qi - q_blk) * p.Nk + key0 + kb * 32 + 4 * g;
        if (p.bias_vec) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(b_rs, (row_off + 8 * q4) * 2, 0, 0);
            bvals[4 * q4 + 0] = E::widen(w[0] & 0xffffu);
            bvals[4 * q4 + 1] = E::widen(w[0] >> 16);
            bvals[4 * q4 + 2] = E::widen(w[1] & 0xffffu);
            bvals[4 * q4 + 3] = E::widen(w[1] >> 16);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            bvals[r] = E::widen(__builtin_amdgcn_raw_buffer_load_b16(
                b_rs, (row_off + 8 * (r >> 2) + (r & 3)) * 2, 0, 0));
        }
      }
      // logits, then one masking pass for the whole block (tested once,
      // not per register), then P and dS^T
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        t[r] = BIAS ? fmaf(s[kb][r], p.c, fmaf(bvals[r], kLog2e, -lse2))
                    : fmaf(s[kb][r], p.c, -lse2);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= p.Nk || (CAUSAL && key > qi) || (W > 0 && key <= qi - W)) t[r] = -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(t[r]);
        s[kb][r] = pr * (dp[kb][r] - dlt);  // dS^T
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Frag dsf = pack_half<T>(s[kb], h);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (NT > 1 && tgt + i >= NL) break;
          const char* sKt = smem[buf] + (tgt + i) * TILE;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const Frag kt = lds_frag_tr<T>(sKt + (kb * 32 + 16 * h) * LRB, of.tr_off[0][db], of.tr_off[1][db]);
            acc[i][db] = E::mma(kt, dsf, acc[i][db]);
          }
        }
      }
  };

  if (n_kv > j_lo) {
    issue(j_lo, 0);
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
  }
  for (int j = j_lo; j < n_kv; ++j) {
    const int cur = (j - j_lo) & 1;
    if (j + 1 < n_kv) issue(j + 1, cur ^ 1);
    const bool active = wave_has_rows &&
                        (!CAUSAL || (j * BN <= wq_last && j * BN + BN - 1 >= wave_key_lo));
    if (active) compute(j, cur);
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (NT > 1 && tgt + i >= NL) break;
    T* dst = static_cast<T*>(NL > 1 ? p.chain_dq[tgt + i] : p.dq) + (row_base + qi) * D;
    store_rows<T, NDB, D>(dst, acc[i], p.scale, g, row_ok);
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, hk, 128-key block), 64-row query tiles over
// the group's packed rows r = (hq - hk*group)*Nq + i (query position r % Nq).
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool BIAS, bool WINDOW, int NL = 1>
__global__ __launch_bounds__(kBwdThreads, (NL > 2 ? 1
                                          : D == 64 ? ((BIAS || NL > 1) ? 2 : FA_DKDV_MINB64)
                                                    : (dkdv_pair(D, CAUSAL, BIAS) && NL == 1) ? 2 : 1))
void fa_bwd_dkdv_kernel(BwdParams p) {
  using E = Elem<T>;
  using Frag = typename E::Frag;
  static_assert(NL == 1 || (!BIAS && !WINDOW && D <= 128), "chain instances");
  constexpr int BQ = dkdv_qtile(D, CAUSAL, BIAS);
  constexpr int NS = (D + 15) / 16, NDB = (D + 31) / 32, NQB = BQ / 32;
  constexpr int RB = D * 2;                   // bytes per row in HBM
  constexpr int LRB = lds_width(D) * 2;       // bytes per row in LDS
  constexpr int TILE = BQ * LRB;              // bytes per Q (or dO) tile (each layer's Q)
  constexpr bool K_LDS = dkdv_k_in_lds(D, CAUSAL, BIAS);  // the block's K in LDS, else registers
  constexpr bool V_LDS = dkdv_v_in_lds(D, CAUSAL, BIAS);  // the block's V in LDS, else registers
  constexpr int KB_BYTES = 128 * LRB;                       // bytes of the block's K (or V)
  // per stage: the Q tiles of the NL layers, dO tile, lse2[BQ], delta[BQ]
  constexpr int STAGE = (NL + 1) * TILE + 2 * BQ * 4;
  constexpr int KV_BYTES = (K_LDS ? KB_BYTES : 0) + (V_LDS ? KB_BYTES : 0);
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE + (KV_BYTES ? KV_BYTES : 16)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;

  // Causal: low key blocks see the most query rows; heavy blocks first, rank
  // major.  Non-causal: head-major with the ids of one XCD consecutive, so
  // that the key blocks of a KV head run together on one XCD and stream the
  // same Q and dO rows through its L2.
  int bhk, kt;
  if (CAUSAL) {
    bhk = int(blockIdx.x % unsigned(p.BHkv));
    const int rank = int(blockIdx.x / unsigned(p.BHkv));
    const int half = (p.n_kblk + 1) / 2;
    kt = rank < half ? rank : p.n_kblk - 1 - (rank - half);
  } else {
    const unsigned logical = xcd_contiguous(blockIdx.x, gridDim.x);
    bhk = int(logical / unsigned(p.n_kblk));
    kt = int(logical % unsigned(p.n_kblk));
  }
  const int b = bhk / p.Hkv, hk = bhk - b * p.Hkv;
  const int64_t kv_head = int64_t(b) * p.Hkv + hk;
  const int64_t row_base = (int64_t(b) * p.Hq + int64_t(hk) * p.group) * p.Nq;
  const int R = p.group * p.Nq;  // packed query rows of this KV head
  const T* Kh = static_cast<const T*>(p.k) + kv_head * p.Nk * D;
  const T* Vh = static_cast<const T*>(p.v) + kv_head * p.Nk * D;

  const T* Gg = static_cast<const T*>(p.dout) + row_base * D;
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(Kh, uint32_t(p.Nk) * RB);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(Vh, uint32_t(p.Nk) * RB);
  const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(Gg, uint32_t(R) * RB);
  __amdgpu_buffer_rsrc_t q_rs[NL], kl_rs[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const T* Ql = static_cast<const T*>(NL > 1 ? p.chain_q[l] : p.q) + row_base * D;
    const T* Kl = static_cast<const T*>(NL > 1 ? p.chain_k[l] : p.k) + kv_head * p.Nk * D;
    q_rs[l] = make_rsrc(Ql, uint32_t(R) * RB);
    kl_rs[l] = make_rsrc(Kl, uint32_t(p.Nk) * RB);
  }
  // the layer whose dK this launch forms; dV with the first launch only
  const int tgt = NL > 1 ? p.target : 0;
  const bool with_dv = NL == 1 || p.target == 0;
  const __amdgpu_buffer_rsrc_t l_rs = make_rsrc(p.lse2 + row_base, uint32_t(R) * 4);
  const __amdgpu_buffer_rsrc_t d_rs = make_rsrc(p.delta + row_base, uint32_t(R) * 4);

  const int k_blk = kt * 128;
  const int kw0 = k_blk + wave * 32;  // first key of this wave
  const int kj = kw0 + ln;            // the key this lane owns

  TileLoad<BQ, D> tl;
  tl.init(wave, lane);
  std::conditional_t<dkdv_lean_offsets(D, CAUSAL, BIAS), OffsetsLean<D>, Offsets<D>> of;
  of.init(lane);

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T,
  // held in registers or read from the block's copy in LDS
  Frag kf[NL][K_LDS ? 1 : NS], vf[V_LDS ? 1 : NS];
  char* sK = smem + 2 * STAGE;
  char* sV = sK + (K_LDS ? KB_BYTES : 0);
  if constexpr (K_LDS || V_LDS) {
    TileLoad<128, D> kl;
    kl.init(wave, lane);
    if constexpr (K_LDS) kl.issue(k_rs, sK, wave, uint32_t(k_blk) * RB);
    if constexpr (V_LDS) kl.issue(v_rs, sV, wave, uint32_t(k_blk) * RB);
  }
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int off = kj * RB + (16 * st + 8 * g) * 2;
    if constexpr (!K_LDS)
#pragma unroll
      for (int l = 0; l < NL; ++l)
        kf[l][st] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(kl_rs[l], off, 0, 0));
    if constexpr (!V_LDS)
      vf[st] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(v_rs, off, 0, 0));
  }

  // TWO (D = 256): a dV pass, then a dK pass, both accumulating into dva;
  // otherwise one pass with both accumulators
  constexpr bool TWO = D == 256;
  int pass = 0;
  constexpr int NTG = chain_targets(D, NL);  // target layers of this launch (dK)
  f32x16 dva[NDB], dka[NTG][TWO ? 1 : NDB];

  // Query tiles: BQ rows i0 .. i0+BQ-1 of one query head h of the group
  // (packed row r0 = h*Nq + i0), so a row's query position is i0 plus its
  // offset in the tile; rows at or past Nq belong to the next head (or lie
  // past the group's last row, where the loads return 0) and are masked.
  // Tiles ti = i0 / BQ in [ti_lo, ti_end) of every head matter to this
  // workgroup: causal, a tile whose last position precedes the block's first
  // key sees none of it; with a window, a tile whose first position comes W or
  // more after the block's last key sees none either.
  const int W = (CAUSAL && WINDOW) ? p.window : 0;
  const int NT = (p.Nq + BQ - 1) / BQ;  // tiles per head
  const int ti_lo = CAUSAL ? min(NT, k_blk / BQ) : 0;
  const int ti_end = W > 0 ? min(NT, (k_blk + 126 + W) / BQ + 1) : NT;
  const int n_vis = max(0, ti_end - ti_lo);  // visible tiles per head

  auto issue = [&](int r0, int buf) {
    char* st = smem + buf * STAGE;
    const uint32_t soff = uint32_t(r0) * RB;
#pragma unroll
    for (int l = 0; l < NL; ++l) tl.issue(q_rs[l], st + l * TILE, wave, soff);
    tl.issue(g_rs, st + NL * TILE, wave, soff);
    // lse2 and delta: BQ floats each, 16 bytes per lane of waves 0 and 1
    if (wave == 0) {
      if (lane < BQ / 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(l_rs, (lds_void*)(st + (NL + 1) * TILE), 16,
                                                 unsigned(lane * 16), uint32_t(r0) * 4, 0, 0);
    } else if (wave == 1) {
      if (lane < BQ / 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d_rs, (lds_void*)(st + (NL + 1) * TILE + BQ * 4), 16,
                                                 unsigned(lane * 16), uint32_t(r0) * 4, 0, 0);
    }
  };

  auto compute = [&](int r0, int i0, int buf) {
    const auto ofs = of.fresh();
    const char* sQ = smem + buf * STAGE;            // layer 0's Q tile
    const char* sQt = sQ + tgt * TILE;              // the target layer's
    const char* sG = sQ + NL * TILE;
    const float* sL = reinterpret_cast<const float*>(sQ + (NL + 1) * TILE);
    const float* sD = sL + BQ;
    // bias rows of this tile (reads past the group's rows or keys return 0)
    const T* btile = BIAS ? static_cast<const T*>(p.bias) + (row_base + r0) * p.Nk
                          : static_cast<const T*>(p.q);
    const __amdgpu_buffer_rsrc_t b_rs =
        make_rsrc(btile, BIAS ? uint32_t(min(BQ, R - r0)) * uint32_t(p.Nk) * 2 : 0u);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int ib0 = i0 + qb * 32;  // query position of this 32-row block's first row
      if (ib0 >= p.Nq) break;
      const int ib1 = min(ib0 + 31, p.Nq - 1);  // and of its last valid row
      if (CAUSAL && ib1 < kw0) continue;  // all masked
      if (W > 0 && ib0 > kw0 + 31 + W - 1) continue;
      const bool want_dv = (!TWO || pass == 0) && with_dv, want_dk = !TWO || pass == 1;
      f32x16 s, dp = f32x16{};
#pragma unroll
      for (int l = 0; l < NL; ++l)
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const Frag qa = lds_frag<T>(sQ + l * TILE + qb * 32 * LRB + ofs.row(st));
          const Frag kb = K_LDS ? lds_frag<T>(sK + wave * 32 * LRB + ofs.row(st)) : kf[l][st];
          s = E::mma(qa, kb, (l == 0 && st == 0) ? f32x16{} : s);
        }
      if (want_dk) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const Frag ga = lds_frag<T>(sG + qb * 32 * LRB + ofs.row(st));
          const Frag vb = V_LDS ? lds_frag<T>(sV + wave * 32 * LRB + ofs.row(st)) : vf[st];
          dp = E::mma(ga, vb, st == 0 ? f32x16{} : dp);
        }
      }
      // register r: query row qb*32 + 8*(r/4) + 4*g + r%4 of the tile, key kj
      const bool tail = ib0 + 32 > p.Nq;
      const bool need_mask =
          tail || (CAUSAL && ib0 < kw0 + 31) || (W > 0 && ib1 >= kw0 + W);
      // logits, then one masking pass for the whole block (tested once,
      // not per register), then P and dS
      // (the logits replace the scores in s)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int qr = qb * 32 + 8 * q4 + 4 * g;  // tile row of register 4*q4
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL + qr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          s[r] = fmaf(s[r], p.c, -l4[e]);
          if constexpr (BIAS) {
            // key kj's column of tile row qr + e (2-byte loads: the lanes of a
            // wave read 32 adjacent keys of one row)
            const u32 bw = __builtin_amdgcn_raw_buffer_load_b16(
                b_rs, ((qr + e) * p.Nk + min(kj, p.Nk)) * 2, 0, 0);
            s[r] = fmaf(E::widen(bw), kLog2e, s[r]);
          }
        }
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = i0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);  // register r's row
          if (pos >= p.Nq || (CAUSAL && kj > pos) || (W > 0 && kj <= pos - W)) s[r] = -INFINITY;
        }
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + qb * 32 + 8 * q4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          const float pr = __builtin_amdgcn_exp2f(s[r]);
          s[r] = pr;
          dp[r] = pr * (dp[r] - d4[e]);  // dS
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Frag pf = pack_half<T>(s, h);
        const Frag dsf = pack_half<T>(dp, h);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if (want_dv) {
            const Frag gt = lds_frag_tr<T>(sG + (qb * 32 + 16 * h) * LRB, ofs.tr(0, db), ofs.tr(1, db));
            dva[db] = E::mma(gt, pf, dva[db]);
          }
          if (want_dk) {
#pragma unroll
            for (int i = 0; i < NTG; ++i) {
              if (NTG > 1 && tgt + i >= NL) break;
              const Frag qt = lds_frag_tr<T>(sQt + i * TILE + (qb * 32 + 16 * h) * LRB,
                                             ofs.tr(0, db), ofs.tr(1, db));
              if constexpr (TWO) dva[db] = E::mma(qt, dsf, dva[db]);
              else dka[i][db] = E::mma(qt, dsf, dka[i][db]);
            }
          }
        }
      }
    }
  };

  const bool key_ok = kj < p.Nk;
  const int64_t krow = (kv_head * p.Nk + kj) * D;
  T* dk_row = static_cast<T*>(p.dk) + krow;
  T* dv_row = static_cast<T*>(p.dv) + (kv_head * p.Nk + kj) * D;
  // the visible tiles in order: head h, tile ti (i0 = ti * BQ)
  const int n_tiles = n_vis > 0 ? p.group * n_vis : 0;
  for (pass = 0; pass < (TWO ? 2 : 1); ++pass) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dva[db] = f32x16{};
#pragma unroll
      for (int i = 0; i < NTG; ++i)
        if constexpr (!TWO) dka[i][db] = f32x16{};
    }
    int h = 0, ti = ti_lo;
    if (n_tiles > 0) issue(ti * BQ, 0);
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
    int buf = 0;
    for (int u = 0; u < n_tiles; ++u) {
      int hn = h, tn = ti + 1;  // the next visible tile
      if (tn == ti_end) {
        tn = ti_lo;
        ++hn;
      }
      if (u + 1 < n_tiles) issue(hn * p.Nq + tn * BQ, buf ^ 1);
      compute(h * p.Nq + ti * BQ, ti * BQ, buf);
      __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      __syncthreads();
      h = hn;
      ti = tn;
      buf ^= 1;
    }
    if constexpr (TWO) {
      if (pass == 0) store_rows<T, NDB, D>(dv_row, dva, 1.f, g, key_ok);
      else store_rows<T, NDB, D>(dk_row, dva, p.scale, g, key_ok);
    } else {
#pragma unroll
      for (int i = 0; i < NTG; ++i) {
        if (NTG > 1 && tgt + i >= NL) break;
        T* row = NL > 1 ? static_cast<T*>(p.chain_dk[tgt + i]) + krow : dk_row;
        store_rows<T, NDB, D>(row, dka[i], p.scale, g, key_ok);
      }
      if (with_dv) store_rows<T, NDB, D>(dv_row, dva, 1.f, g, key_ok);
    }
  }
}

template <typename T, int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, bool bias, hipStream_t s, unsigned g_dq,
                        unsigned g_kv) {
  void* args[] = {const_cast<BwdParams*>(&p)};
  hipError_t e = hipSuccess;
  const void* dq;
  const void* kv;
  if constexpr (D == 256) {
    // (no logit term at D = 256: the API refuses one)
    if (causal && p.window > 0) {
      dq = reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, false, true>);
      kv = reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, false, true>);
    } else if (causal) {
      dq = reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, false, false>);
      kv = reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, false, false>);
    } else {
      dq = reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, false, false, false>);
      kv = reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, false, false, false>);
    }
  } else if (causal && p.window > 0) {
    dq = bias ? reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, true, true>)
              : reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, false, true>);
    kv = bias ? reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, true, true>)
              : reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, false, true>);
  } else if (causal) {
    dq = bias ? reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, true, false>)
              : reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, false, false>);
    kv = bias ? reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, true, false>)
              : reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, false, false>);
  } else {
    dq = bias ? reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, false, true, false>)
              : reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, false, false, false>);
    kv = bias ? reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, false, true, false>)
              : reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, false, false, false>);
  }
  if (g_dq) {
    e = hipLaunchKernel(dq, dim3(g_dq), dim3(kBwdThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (g_kv) e = hipLaunchKernel(kv, dim3(g_kv), dim3(kBwdThreads), args, 0, s);
  return e;
}


// ---- fp32 inputs ---------------------------------------------------------------
// The same chain rule in plain fp32 vector arithmetic: no rounding of P or dS
// and no reduced-precision products (the matrix cores' fp32 rate is a
// sixteenth of their 16-bit rate, and fp32 is the parity dtype, not the
// throughput one).  One lane per query row (dQ kernel) or per key (dV and dK
// kernels); the other side streams through LDS in 32-row tiles, and each lane
// reads the tile's rows from LDS as broadcasts.  Head sizes 64 and 128.
constexpr int kB32Threads = 128;  // rows (or keys) per workgroup
constexpr int kB32Tile = 32;      // streamed rows per LDS tile

struct Bwd32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* bias;  // [B, Hq, Nq, Nk] or null
  const float* o;
  const float* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;       // workspace: delta_i per row
  float* lse2;        // workspace: LSE_i log2(e) per row (+inf for LSE = -inf)
  int B, Hq, Hkv, Nq, Nk, window;
  int n_qblk, n_kblk;
  float scale;
  float c;            // scale * log2(e)
};

__device__ __forceinline__ bool b32_visible(int i, int j, int Nq, int Nk, bool causal, int window) {
  return i < Nq && j < Nk && (!causal || j <= i) && (window <= 0 || j > i - window);
}

// dQ and delta: lane = query row i of head (b, h)
template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kB32Threads) void fa_bwd32_dq_kernel(Bwd32Params p) {
  __shared__ float sK[kB32Tile][D];
  __shared__ float sV[kB32Tile][D];
  __shared__ float sB[kB32Threads][kB32Tile + 1];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / p.n_qblk;
  const int row0 = (blockIdx.x % p.n_qblk) * kB32Threads;
  const int i = row0 + tid;
  const int b = bh / p.Hq, h = bh % p.Hq, hk = h / (p.Hq / p.Hkv);
  const bool valid = i < p.Nq;
  const size_t qrow = (size_t(bh) * p.Nq + (valid ? i : 0)) * D;
  const size_t kv0 = size_t(b * p.Hkv + hk) * p.Nk * D;
  // D = 128: the dQ columns in two halves, each a pass over the keys (the
  // Q and dO rows and a full accumulator would not fit the registers)
  constexpr int NH = D > 64 ? 2 : 1, DH = D / NH;
  float q[D], dov[D], dq[DH];
  float delta = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? p.q[qrow + d] : 0.f;
    dov[d] = valid ? p.dout[qrow + d] : 0.f;
    delta = fmaf(dov[d], valid ? p.o[qrow + d] : 0.f, delta);
  }
  const float l = valid ? p.lse[size_t(bh) * p.Nq + i] : 0.f;
  const float lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;   // rows with no key: P = 0
  if (valid) {
    p.delta[size_t(bh) * p.Nq + i] = delta;
    p.lse2[size_t(bh) * p.Nq + i] = lse2;
  }
  // keys any row of the block can see
  const int last_row = min(p.Nq, row0 + kB32Threads) - 1;
  const int j_end = CAUSAL ? min(p.Nk, last_row + 1) : p.Nk;
  const int j_begin = p.window > 0 ? max(0, row0 - p.window + 1) : 0;
#pragma unroll 1
  for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
  for (int d = 0; d < DH; ++d) dq[d] = 0.f;
  for (int t0 = (j_begin / kB32Tile) * kB32Tile; t0 < j_end; t0 += kB32Tile) {
    __syncthreads();   // the previous tile's reads are done
    for (int e = tid; e < kB32Tile * D; e += kB32Threads) {
      const int r = e / D, d = e % D;
      const bool in = t0 + r < p.Nk;
      sK[r][d] = in ? p.k[kv0 + size_t(t0 + r) * D + d] : 0.f;
      sV[r][d] = in ? p.v[kv0 + size_t(t0 + r) * D + d] : 0.f;
    }
    if constexpr (BIAS) {
      for (int e = tid; e < kB32Threads * kB32Tile; e += kB32Threads) {
        const int r = e / kB32Tile, c = e % kB32Tile;
        const bool in = row0 + r < p.Nq && t0 + c < p.Nk;
        sB[r][c] = in ? p.bias[(size_t(bh) * p.Nq + row0 + r) * p.Nk + t0 + c] : 0.f;
      }
    }
    __syncthreads();
    for (int jj = 0; jj < kB32Tile; ++jj) {
      if (!b32_visible(i, t0 + jj, p.Nq, p.Nk, CAUSAL, p.window)) continue;
      float sdot = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        sdot = fmaf(q[d], sK[jj][d], sdot);
        dp = fmaf(dov[d], sV[jj][d], dp);
      }
      const float off = BIAS ? fmaf(sB[tid][jj], kLog2e, -lse2) : -lse2;
      const float pr = exp2f(fmaf(sdot, p.c, off));
      const float ds = pr * (dp - delta);
#pragma unroll
      for (int d = 0; d < DH; ++d) dq[d] = fmaf(ds, sK[jj][hf * DH + d], dq[d]);
    }
  }
  if (valid) {
#pragma unroll
    for (int d = 0; d < DH; ++d) p.dq[qrow + hf * DH + d] = dq[d] * p.scale;
  }
  }
}

// dV (PASS 0) or dK (PASS 1): lane = key j of KV head (b, hk); the query rows
// of every head of the group stream through LDS with their lse2 and delta
template <int D, bool CAUSAL, bool BIAS, int PASS>
__global__ __launch_bounds__(kB32Threads) void fa_bwd32_kv_kernel(Bwd32Params p) {
  __shared__ float sQ[kB32Tile][D];
  __shared__ float sO[kB32Tile][D];   // dO rows
  __shared__ float sL[kB32Tile];      // lse2
  __shared__ float sD[kB32Tile];      // delta
  const int tid = threadIdx.x;
  const int bhk = blockIdx.x / p.n_kblk;
  const int key0 = (blockIdx.x % p.n_kblk) * kB32Threads;
  const int j = key0 + tid;
  const int b = bhk / p.Hkv, hk = bhk % p.Hkv;
  const int grp = p.Hq / p.Hkv;
  const bool valid = j < p.Nk;
  const size_t krow = (size_t(bhk) * p.Nk + (valid ? j : 0)) * D;
  // dK at D = 128: the columns in two halves, each a pass over the rows
  constexpr int NH = (PASS == 1 && D > 64) ? 2 : 1, DH = D / NH;
  float kr[D], vr[PASS == 1 ? D : 1], acc[DH];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = valid ? p.k[krow + d] : 0.f;
    if constexpr (PASS == 1) vr[d] = valid ? p.v[krow + d] : 0.f;
  }
  // rows any key of the block is visible to
  const int last_key = min(p.Nk, key0 + kB32Threads) - 1;
  const int i_begin = CAUSAL ? key0 : 0;
  const int i_end = p.window > 0 ? min(p.Nq, last_key + p.window) : p.Nq;
#pragma unroll 1
  for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  for (int hh = 0; hh < grp; ++hh) {
    const int bh = b * p.Hq + hk * grp + hh;
    for (int t0 = (i_begin / kB32Tile) * kB32Tile; t0 < i_end; t0 += kB32Tile) {
      __syncthreads();
      for (int e = tid; e < kB32Tile * D; e += kB32Threads) {
        const int r = e / D, d = e % D;
        const bool in = t0 + r < p.Nq;
        const size_t g = (size_t(bh) * p.Nq + (in ? t0 + r : 0)) * D + d;
        sQ[r][d] = in ? p.q[g] : 0.f;
        sO[r][d] = in ? p.dout[g] : 0.f;
      }
      if (tid < kB32Tile) {
        const bool in = t0 + tid < p.Nq;
        sL[tid] = in ? p.lse2[size_t(bh) * p.Nq + t0 + tid] : INFINITY;
        sD[tid] = in ? p.delta[size_t(bh) * p.Nq + t0 + tid] : 0.f;
      }
      __syncthreads();
      for (int ii = 0; ii < kB32Tile; ++ii) {
        const int i = t0 + ii;
        if (!b32_visible(i, j, p.Nq, p.Nk, CAUSAL, p.window)) continue;
        float sdot = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          sdot = fmaf(sQ[ii][d], kr[d], sdot);
          if constexpr (PASS == 1) dp = fmaf(sO[ii][d], vr[d], dp);
        }
        const float bv = BIAS ? p.bias[(size_t(bh) * p.Nq + i) * p.Nk + j] : 0.f;
        const float off = BIAS ? fmaf(bv, kLog2e, -sL[ii]) : -sL[ii];
        const float pr = exp2f(fmaf(sdot, p.c, off));
        if constexpr (PASS == 0) {
#pragma unroll
          for (int d = 0; d < DH; ++d) acc[d] = fmaf(pr, sO[ii][d], acc[d]);
        } else {
          const float ds = pr * (dp - sD[ii]);
#pragma unroll
          for (int d = 0; d < DH; ++d) acc[d] = fmaf(ds, sQ[ii][hf * DH + d], acc[d]);
        }
      }
    }
  }
  if (valid) {
    float* out = PASS == 0 ? p.dv : p.dk;
    const float f = PASS == 0 ? 1.f : p.scale;
#pragma unroll
    for (int d = 0; d < DH; ++d) out[krow + hf * DH + d] = acc[d] * f;
  }
  }
}

template <int D, bool CAUSAL, bool BIAS>
hipError_t launch_bwd32_cb(const Bwd32Params& p, hipStream_t s) {
  const unsigned g_dq = unsigned(p.n_qblk) * unsigned(p.B * p.Hq);
  const unsigned g_kv = unsigned(p.n_kblk) * unsigned(p.B * p.Hkv);
  if (g_dq) fa_bwd32_dq_kernel<D, CAUSAL, BIAS><<<g_dq, kB32Threads, 0, s>>>(p);
  if (g_kv) {
    fa_bwd32_kv_kernel<D, CAUSAL, BIAS, 0><<<g_kv, kB32Threads, 0, s>>>(p);
    fa_bwd32_kv_kernel<D, CAUSAL, BIAS, 1><<<g_kv, kB32Threads, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd32_d(const Bwd32Params& p, bool causal, bool bias, hipStream_t s) {
  if (causal) return bias ? launch_bwd32_cb<D, true, true>(p, s) : launch_bwd32_cb<D, true, false>(p, s);
  return bias ? launch_bwd32_cb<D, false, true>(p, s) : launch_bwd32_cb<D, false, false>(p, s);
}

}  // namespace

// Chain: one dQ and one dK/dV launch per group of chain_targets(D, NL) layers
// (targets t .. t + NT - 1), in order on the stream; each dQ launch also
// rewrites the same row sums into the workspace, which the dK/dV launch after
// it reads.
template <typename T, int D, int NL>
hipError_t launch_bwd_chain_nl(BwdParams& p, bool causal, hipStream_t s, unsigned g_dq,
                               unsigned g_kv, void* const* dq_layers, void* const* dk_layers) {
  const void* dq = causal ? reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, true, false, false, NL>)
                          : reinterpret_cast<const void*>(&fa_bwd_dq_kernel<T, D, false, false, false, NL>);
  const void* kv = causal ? reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, true, false, false, NL>)
                          : reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<T, D, false, false, false, NL>);
  for (int l = 0; l < NL; ++l) {
    p.chain_dq[l] = dq_layers[l];
    p.chain_dk[l] = dk_layers[l];
  }
  for (int t = 0; t < NL; t += chain_targets(D, NL)) {
    p.target = t;
    void* args[] = {&p};  // (the arguments are copied at each launch)
    hipError_t e = hipSuccess;
    if (g_dq) e = hipLaunchKernel(dq, dim3(g_dq), dim3(kBwdThreads), args, 0, s);
    if (e == hipSuccess && g_kv) e = hipLaunchKernel(kv, dim3(g_kv), dim3(kBwdThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static BwdParams make_bwd_params(const BwdArgs& a);

// fp32 inputs (D = 64 or 128): delta and dQ, then dV, then dK, in order on the
// stream; the dV and dK kernels read delta from the workspace.
static int launch_backward_f32(const BwdArgs& a) {
  Bwd32Params p{};
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.bias = static_cast<const float*>(a.bias);
  p.o = static_cast<const float*>(a.o);
  p.dout = static_cast<const float*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<float*>(a.dq);
  p.dk = static_cast<float*>(a.dk);
  p.dv = static_cast<float*>(a.dv);
  p.delta = static_cast<float*>(a.workspace);
  p.lse2 = p.delta + backward_lse2_offset(int64_t(a.B) * a.Hq * a.Nq);
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.window = a.causal ? a.window : 0;
  p.n_qblk = (a.Nq + kB32Threads - 1) / kB32Threads;
  p.n_kblk = (a.Nk + kB32Threads - 1) / kB32Threads;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  const hipError_t e = a.D == 64 ? launch_bwd32_d<64>(p, a.causal, a.bias != nullptr, s)
                                 : launch_bwd32_d<128>(p, a.causal, a.bias != nullptr, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int launch_backward(const BwdArgs& a) {
  if (a.dtype == FA_DTYPE_FP32) return launch_backward_f32(a);
  BwdParams p = make_bwd_params(a);
  const unsigned g_dq = unsigned(p.n_qblk) * unsigned(p.BH);
  const unsigned g_kv = unsigned(p.n_kblk) * unsigned(p.BHkv);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  hipError_t e;
  auto launch = [&](auto tag) {
    using T = decltype(tag);
    switch (a.D) {
      case 64: return launch_bwd_d<T, 64>(p, a.causal, a.bias, s, g_dq, g_kv);
      case 80: return launch_bwd_d<T, 80>(p, a.causal, a.bias, s, g_dq, g_kv);
      case 96: return launch_bwd_d<T, 96>(p, a.causal, a.bias, s, g_dq, g_kv);
      case 256: return launch_bwd_d<T, 256>(p, a.causal, a.bias, s, g_dq, g_kv);
      default: return launch_bwd_d<T, 128>(p, a.causal, a.bias, s, g_dq, g_kv);
    }
  };
  if (a.dtype == FA_DTYPE_BF16) {
    e = launch(__bf16{});
  } else {
    e = launch(_Float16{});
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int launch_backward_chain(const BwdArgs& a, const void* const* q_layers,
                          const void* const* k_layers, void* const* dq_layers,
                          void* const* dk_layers, int n_layers) {
  if (n_layers == 1) return launch_backward(a);
  BwdParams p = make_bwd_params(a);
  for (int l = 0; l < kMaxChainLayers; ++l) {
    p.chain_q[l] = l < n_layers ? q_layers[l] : nullptr;
    p.chain_k[l] = l < n_layers ? k_layers[l] : nullptr;
  }
  const unsigned g_dq = unsigned(p.n_qblk) * unsigned(p.BH);
  const unsigned g_kv = unsigned(p.n_kblk) * unsigned(p.BHkv);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  auto launch_d = [&](auto tag, auto dtag) {
    using T = decltype(tag);
    constexpr int D = decltype(dtag)::value;
    switch (n_layers) {
      case 2: return launch_bwd_chain_nl<T, D, 2>(p, a.causal, s, g_dq, g_kv, dq_layers, dk_layers);
      case 3: return launch_bwd_chain_nl<T, D, 3>(p, a.causal, s, g_dq, g_kv, dq_layers, dk_layers);
      default: return launch_bwd_chain_nl<T, D, 4>(p, a.causal, s, g_dq, g_kv, dq_layers, dk_layers);
    }
  };
  auto launch = [&](auto tag) {
    switch (a.D) {
      case 64: return launch_d(tag, std::integral_constant<int, 64>{});
      case 80: return launch_d(tag, std::integral_constant<int, 80>{});
      case 96: return launch_d(tag, std::integral_constant<int, 96>{});
      default: return launch_d(tag, std::integral_constant<int, 128>{});
    }
  };
  const hipError_t e = a.dtype == FA_DTYPE_BF16 ? launch(__bf16{}) : launch(_Float16{});
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static BwdParams make_bwd_params(const BwdArgs& a) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.bias = a.bias;
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.delta = static_cast<float*>(a.workspace);
  p.rows = int64_t(a.B) * a.Hq * a.Nq;
  p.lse2 = p.delta + backward_lse2_offset(p.rows);
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.BH = a.B * a.Hq;
  p.BHkv = a.B * a.Hkv;
  p.group = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
  p.n_qblk = (a.Nq + 127) / 128;
  p.n_kblk = (a.Nk + 127) / 128;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.bias_vec = (a.Nk % 4) == 0;
  p.window = a.window;
  for (int l = 0; l < kMaxChainLayers; ++l) {
    p.chain_q[l] = p.chain_k[l] = nullptr;
    p.chain_dq[l] = p.chain_dk[l] = nullptr;
  }
  p.target = 0;
  return p;
}

}  // namespace fa

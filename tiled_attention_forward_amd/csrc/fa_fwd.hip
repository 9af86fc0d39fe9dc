// Fused tiled attention forward for gfx950 (MI355X): kernels and launcher.
//
// Method: "FlashAttention principles and Triton practice" (xnwp.cn/news/15505)
// §2.2 and §3.3, and the kwkr.cn/news/592482 tutorial §2.2-§2.3: one workgroup
// keeps a block of query rows resident, streams K/V column tiles through LDS
// and folds each tile into a running (max, sum, un-normalised output) with the
// online softmax update; S and P exist only in registers.  The divide by the
// row sum happens once at the end, and the row statistic is written as
// LSE = m + ln(l) (kwkr.cn §2.4).  The optional additive logit tile of the
// Block Attention Residual post (iqiancheng.github.io, "v1" and "v2") is read
// straight into the registers that hold the score tile, after the scaling and
// before the softmax.
//
// Work layout (all choices made for CDNA4, not taken from the pages):
//  * workgroup = 4 waves x 32 query rows = 128 rows of one (batch, query head);
//    the 1-D grid lists the heaviest causal row blocks first and deals the
//    blocks that read the same K/V rows to one XCD (see the id mapping);
//  * each wave computes the transposed score block S^T = K . Q^T with
//    32x32 MFMAs (bf16/fp16: v_mfma_f32_32x32x16, fp32: v_mfma_f32_32x32x2f32),
//    so one lane holds one query row and 16 of the 32 keys of a block: row max
//    and row sum are in-lane reductions plus one v_permlane32_swap;
//  * the output is accumulated transposed too, O^T += V^T . P^T, so the same
//    lane owns the same query row in S^T and in O^T: the online-softmax
//    rescale is a per-lane scalar and P feeds the MFMA B operand straight from
//    the S^T registers without any shuffle;
//  * bf16/fp16: K and V tiles go from HBM straight into LDS with buffer loads
//    that carry the LDS flag, row-major and unpadded, the 16-byte chunks of
//    each row XOR-swizzled so that both read patterns are free of bank
//    conflicts; the V operand of P.V is read with the transposing
//    ds_read_b64_tr_b16.  fp32: staged through registers, K padded, V stored
//    transposed;
//  * two LDS buffers: tile j+1 is requested while tile j is being computed;
//    one barrier per tile;
//  * exp is the hardware base-2 exponential with scale*log2(e) folded into one
//    FMA; the rescale of the running output is skipped until the row max has
//    grown by more than a threshold; masks are applied only on tiles that
//    cross the causal diagonal, the window edge or the end of the keys, and
//    tiles wholly outside every row's visible range are skipped.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "../../include/fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kThreads = kWaves * 64;
// Build-time tuning knobs.  The defaults are the measured best on MI355X; a
// variant is compiled with -D<knob>=<value> (build.build(extra_flags=...)).
// Keys per K/V tile and 32-row query blocks per wave of the fused instances:
#ifndef FA_BN64
#define FA_BN64 64  // D = 64
#endif
#ifndef FA_BN128
#define FA_BN128 64  // D = 80, 96, 128 (those the two lines further down do not set)
#endif
#ifndef FA_QB64
#define FA_QB64 1  // D = 64, 16-bit, no bias
#endif
#ifndef FA_QB128
#define FA_QB128 1  // D = 128 instances other than the non-causal bias-free one
#endif
// 16-bit fused non-causal instances at D = 128 without a bias: two 32-row
// query blocks per wave over 32-key tiles (256 VGPRs; the 24-byte spill is
// the prologue's and the epilogue's, none in the loop), which halves the LDS
// operand reads per MFMA.  The causal instance would spill inside its loop
// and keeps one block over 64-key tiles.
#ifndef FA_QB128N
#define FA_QB128N 2
#endif
#ifndef FA_BN128N
#define FA_BN128N 32
#endif
// Workgroups per compute unit asked of the compiler at D = 64
#ifndef FA_MINB64
#define FA_MINB64 2
#endif
// K fragment offsets kept opaque to the compiler (one add per read)
#ifndef FA_OPAQUE_KOFF
#define FA_OPAQUE_KOFF 1
#endif
// The wave index read as a scalar, so the direct-load destinations are scalar
#ifndef FA_SCALAR_WAVE
#define FA_SCALAR_WAVE 1
#endif
// Key-split instances over one row block (decode): K/V loads non-temporal
#ifndef FA_SPLIT_KV_STREAM
#define FA_SPLIT_KV_STREAM 1
#endif
constexpr int kPolicyNT = 2;  // buffer-load cache policy: non-temporal
// Key-split instances at D = 128 without a bias (decode-like shapes, bound by
// the K/V stream): 32-key tiles, 163-166 VGPRs, so three workgroups fit a
// compute unit (decode B8 20/4 heads, 32768 keys: 96.2 us against 100.5 with
// 64-key tiles; a third LDS buffer adds nothing, 96.8 us).
#ifndef FA_SPLIT_BN128
#define FA_SPLIT_BN128 32
#endif
// Logit tiles staged through LDS by direct loads (16-bit, 64-key tiles)
#ifndef FA_BIAS_LDS
#define FA_BIAS_LDS 1
#endif
// Key halves per workgroup of the causal D = 64 fused instances (1 or 2):
// 16-bit, and FP8
#ifndef FA_KH64
#define FA_KH64 1
#endif
#ifndef FA_KH64_F8
#define FA_KH64_F8 2
#endif

constexpr int kBN64 = FA_BN64;         // keys per K/V tile, D = 64
constexpr int kBN128 = FA_BN128;       // keys per K/V tile, D = 128
constexpr int kQB64 = FA_QB64;         // 32-row query blocks per wave, D = 64
constexpr int kQB128 = FA_QB128;       // 32-row query blocks per wave, D = 128
constexpr int kQB128N = FA_QB128N;
constexpr int kBN128N = FA_BN128N;
constexpr float kTau = 8.f;            // lazy-rescale threshold (log2 units)
static_assert(kWaves * 32 >= kRowsPerBlock,
              "grid-size validation assumes at least this block height");

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  void* o;
  float* lse;
  int Hq, Hkv, Nq, Nk;
  int BH;        // B * Hq
  int group;     // Hq / Hkv
  int n_qtiles;  // ceil(Nq / rows per workgroup)
  float c;       // |scale| * log2(e), never 0 (see the launcher)
  float scale_abs;  // c / log2(e): the bias path scales in natural-log units
  u32 q_sign;    // sign bits XORed into Q when scale < 0
  int bias_vec;  // bias rows allow 16-byte vector loads
  int window;         // causal sliding window (keys i-window+1 .. i), 0 = none
  // Block Attention Residual chain (NL > 1 instances): Q and K of every layer
  // of the chain, oldest first; the last pair is also in q and k
  const void* chain_q[kMaxChainLayers];
  const void* chain_k[kMaxChainLayers];
  // key-split path only: o and lse point at the fp32 partial outputs
  int n_splits;       // key ranges per row block
  int64_t part_rows;  // B * Hq * Nq, the row stride between splits
};

// Key position inside a V^T tile row.  Within each group of 16 keys the 4-key
// runs are stored in the order 0,2,1,3, so that the 8 keys one lane half feeds
// to a P.V MFMA (keys 0-3 and 8-11, or 4-7 and 12-15) are contiguous.
__device__ __forceinline__ int vt_pos_of_group(int kg) {  // kg = key / 4
  const int r = kg & 3;
  const int sigma = (r == 1) ? 2 : (r == 2) ? 1 : r;
  return (kg >> 2) * 16 + sigma * 4;
}

// One 16-byte-per-lane direct HBM->LDS load, issued from inline assembly (M0
// holds the wave's LDS destination).  The compiler then neither knows nor
// waits for it: the builtin's load draws a wait for every outstanding vector
// load before the first transposed V read of the tile, which also drains the
// bias loads of the next tile issued at the top of the loop.  The kernel's
// own vmcnt(0) before the tile barrier covers these loads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int POL>
__device__ __forceinline__ void dma16_asm(__amdgpu_buffer_rsrc_t rs, lds_void* dst,
                                          unsigned voff, unsigned soff) {
  const unsigned m = static_cast<unsigned>(reinterpret_cast<size_t>(dst));
  if constexpr (POL == kPolicyNT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(m), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// SPLIT = false: one workgroup per (batch, query head, 128-row block); O and
// LSE are final.
// SPLIT = true (key-split path): the query heads that share a KV head are
// taken as one row space of group * Nq rows (rows r = (hq - hk*group)*Nq + i,
// contiguous in Q, O, LSE and bias), one workgroup per (batch, KV head,
// 128-row block, key range); it writes the normalised partial O (fp32) and
// partial LSE of its key range, to be combined by fa_merge_kernel.
// WINDOW (with CAUSAL): sliding window of p.window keys per row.
// NL > 1 (Block Attention Residual chain): the logits are the sum over NL
// layers of Q_l K_l^T * scale, the K tiles of all layers sharing one LDS
// buffer with the V tile; 16-bit types, no bias, no key split, no window.
// KH = 2 (two key halves): 8 waves; waves w and w + 4 own the same 32 rows,
// the first four stream the first half of the row block's key tiles through
// their own pair of LDS buffers and the last four the second half; at the end
// the second half hands its (max, sum, output) state to the first through
// LDS, which merges the two with the online-softmax merge and writes O and
// LSE.  Halving the longest workgroup's loop lets the grid run in two rounds
// with the heaviest row blocks first (for causal grids the per-block work
// ranges from 1 to Nk/64 tiles).  16-bit and FP8 fused instances only.
template <typename T, int D, int BN, int QB, bool CAUSAL, bool BIAS, bool SPLIT, bool WINDOW,
          int NL, int KVPOL, int KH>
// (waves per SIMD asked of the compiler: fp32 at D = 128 with 64-key tiles
// holds 137 KB of LDS, so one workgroup per compute unit, and the D = 256
// bias and window instances keep their accumulators in AGPRs at one)
__global__ __launch_bounds__(kThreads * KH,
                             (D == 64                                                  ? FA_MINB64
                              : (D == 256 && (BIAS || WINDOW))                         ? 1
                              : (std::is_same<T, float>::value && D == 128 && BN == 64) ? 1
                                                                                        : 2))
void fa_fwd_kernel(Params p) {
  using E = Elem<T>;
  using Frag = typename E::Frag;
  constexpr bool F32 = std::is_same<T, float>::value;
  constexpr bool F8 = std::is_same<T, fp8e4m3>::value;
  // outputs: fp32 partials (key split); bf16 for FP8 inputs; else the input type
  using OutT = typename std::conditional<
      SPLIT, float, typename std::conditional<F8, __bf16, T>::type>::type;
  constexpr bool OUT_F32 = F32 || SPLIT;
  constexpr int KP = E::KP;
  constexpr int KS = 2 * KP;         // contraction length of one MFMA
  // Head dims 80 and 96 (16-bit types): the LDS tiles keep the 128-wide row
  // layout, the chunks past the real row are zero-filled by out-of-range loads,
  // and the products run over ceil(D/16) contraction steps and ceil(D/32)
  // output column blocks; only the real columns are stored.
  constexpr int DL = (D == 80 || D == 96) ? 128 : D;   // LDS row width, elements
  static_assert(D == 64 || D == 80 || D == 96 || D == 128 || D == 256, "head dim");
  static_assert(D == DL || !F32, "fp32 takes head dims 64 and 128");
  constexpr int NS = (D + KS - 1) / KS;  // MFMAs per 32x32 score block
  constexpr int ESZ = sizeof(T);
  constexpr int VEC = 16 / ESZ;      // elements per 16-byte vector
  // 16-bit types: K and V tiles go from HBM straight into LDS (buffer loads
  // with the LDS flag), row-major and unpadded, 16-byte chunks XOR-swizzled
  // per row against bank conflicts; the P.V operand is read from V with
  // ds_read_b64_tr_b16.  fp32: staged through registers, K padded, V stored
  // transposed (V^T).
  constexpr bool VTR = !F32;
  constexpr int KSTR = D + VEC;      // fp32: K tile row stride, elements
  constexpr int VSTR = BN + VEC;     // fp32: V^T tile row stride, elements
  constexpr int RB = DL * ESZ;       // 16-bit: bytes per K/V tile row
  constexpr int CPR = DL / VEC;      // 16-byte chunks per LDS tile row
  constexpr int CPRG = D * ESZ / 16; // 16-byte chunks per row in HBM
  constexpr int KT = VTR ? BN * DL : BN * KSTR;  // elements per K buffer
  constexpr int VT = VTR ? BN * DL : D * VSTR;   // elements per V buffer
  constexpr int DNI = VTR ? BN * CPR / (64 * kWaves) : 1;  // LDS loads per wave per matrix
  static_assert(!VTR || DNI * 64 * kWaves == BN * CPR, "tile must split into whole wave loads");
  constexpr int NKB = BN / 32;       // 32-key blocks per tile
  constexpr int NDB = (D + 31) / 32; // 32-wide column blocks of the output
  constexpr int QW = 32 * QB;        // query rows per wave
  constexpr int BM = kWaves * QW;    // query rows per workgroup
  constexpr int KCH = BN * D / VEC / kThreads;            // K vectors per thread
  constexpr int VTASKS = (BN / 4) * (D / VEC);            // 4-key x VEC-column tasks
  constexpr int VTPT = (VTASKS + kThreads - 1) / kThreads;
  static_assert(VTR || KCH * kThreads * VEC == BN * D, "K tile must split evenly");
  static_assert(NL >= 1 && NL <= kMaxChainLayers, "chain length");
  static_assert(NL == 1 || (VTR && !BIAS && !SPLIT && !WINDOW), "chain instances");
  static_assert(!F8 || (NL == 1 && !BIAS && D == DL && BN == 64), "FP8 instances");
  static_assert(KH == 1 || (KH == 2 && VTR && NL == 1 && !SPLIT && !BIAS), "key-half instances");
  // FP8: P is stored as e4m3 for the P.V product.  It is taken as
  // 2^(t - m_ref + 7) with the rescale threshold at 1, so every p lies in
  // (0, 2^8] (e4m3 reaches 448) and values down to 2^-13 of the row max stay
  // normal numbers (e4m3's smallest is 2^-6); l and O carry the same factor.
  constexpr float kTauT = F8 ? 1.f : kTau;
  constexpr float kPShift = F8 ? 7.f : 0.f;
  constexpr int NKO = F8 ? NS / 2 : NS;   // K fragment reads per 32-key block
  constexpr int KTL = NL * KT;       // elements of the K tiles of all layers
  constexpr int BUF = KTL + VT;      // elements per LDS buffer
  // KH = 2: floats per lane of the state the second key half hands over
  // (m, l, then the output accumulators), stored [row wave][value][lane]
  constexpr int XN = QB * (2 + 16 * NDB);
  constexpr int XBYTES = KH == 2 ? kWaves * XN * 64 * 4 : 0;
  // 16-bit logit tiles (64 keys, rows whose length allows 16-byte loads) go
  // HBM -> LDS by direct loads into a 4 KB region of each wave's own, 8 lanes
  // per 128-byte row so that each load covers whole rows, and are read back
  // in the score layout.  One tile per wave: D = 64 then takes 48 KB of LDS
  // and 148 VGPRs, three workgroups per compute unit (two tiles per wave
  // allowed only two: B2 H16 S4096 D64 causal + bias 160.3 vs 143.4 us).
  // (not the D = 128 window instance: it spilled 232 bytes that way)
  constexpr bool BLDS = BIAS && VTR && QB == 1 && BN == 64 && !(WINDOW && D == 128) && FA_BIAS_LDS;
  constexpr int BTILE = 32 * BN * 2;                  // bytes of one wave's logit tile
  constexpr int BLDS_BYTES = BLDS ? kWaves * BTILE : 0;
  constexpr int KV_ELEMS = (KH * 2 * BUF * ESZ >= XBYTES) ? KH * 2 * BUF
                                                          : (XBYTES + ESZ - 1) / ESZ;
  constexpr int SMEM_ELEMS = KV_ELEMS + BLDS_BYTES / ESZ;
  // two LDS buffers per key half: tile j+1 loads while tile j is computed
  __shared__ __attribute__((aligned(16))) T smem[SMEM_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave: the row wave (0-3); half: which half of the key tiles (KH = 2)
  const int wave = (tid >> 6) & (kWaves - 1);
  const int half = KH == 2 ? tid >> 8 : 0;
  const int g = lane >> 5, ln = lane & 31;

  // Workgroup id -> (head, query block).
  //  * causal: ids are rank-major and the first half of the ranks take the
  //    heavy query blocks in descending order, the second half the light ones
  //    ascending, so co-resident workgroups carry complementary amounts of
  //    work; the query heads of one KV head at one rank are dealt to one XCD
  //    (ids go round-robin to the 8 XCDs), where they share the L2 copy of K
  //    and V; with one query head per KV head and B*Hq a multiple of 8 all
  //    blocks of a head land on one XCD;
  //  * non-causal (all blocks equal): the ids one XCD receives are renumbered
  //    to be consecutive in head-major order, so the query blocks of a head
  //    run at the same time on one XCD and re-read K and V from its L2.
  //  * key-split: the same head-major renumbering over (batch, KV head,
  //    split, row block), so the row blocks that read one key range of a KV
  //    head run together on one XCD.
  int b, hk, tile, split = 0;
  int64_t row_base;  // global index (over B*Hq*Nq) of row 0 of this row space
  int n_rows;        // rows of this row space
  if constexpr (SPLIT) {
    const unsigned logical = xcd_contiguous(blockIdx.x, gridDim.x);
    tile = int(logical % unsigned(p.n_qtiles));
    const unsigned rest = logical / unsigned(p.n_qtiles);
    split = int(rest % unsigned(p.n_splits));
    const int bhk = int(rest / unsigned(p.n_splits));
    b = bhk / p.Hkv;
    hk = bhk - b * p.Hkv;
    row_base = (int64_t(b) * p.Hq + int64_t(hk) * p.group) * p.Nq;
    n_rows = p.group * p.Nq;
  } else {
    int bh;
    if (CAUSAL) {
      // unit = rank * (B*Hkv) + KV head: the `group` query heads of one KV
      // head at one rank, dealt to one XCD, where they stream the same K/V
      // rows through its L2
      const unsigned G = unsigned(p.group), units_per_rank = unsigned(p.BH) / G;
      const UnitMember um = xcd_group_units(blockIdx.x, gridDim.x, G);
      const unsigned unit = um.unit, member = um.member;
      bh = int((unit % units_per_rank) * G + member);
      const int rank = int(unit / units_per_rank);
      if constexpr (KH == 2) {
        // the grid runs in more than one round: heaviest row blocks first,
        // so the last to start are the shortest
        tile = p.n_qtiles - 1 - rank;
      } else {
        const int hr = (p.n_qtiles + 1) / 2;
        tile = rank < hr ? p.n_qtiles - 1 - rank : rank - hr;
      }
    } else {
      const unsigned logical = xcd_contiguous(blockIdx.x, gridDim.x);
      bh = int(logical / unsigned(p.n_qtiles));
      tile = int(logical % unsigned(p.n_qtiles));
    }
    b = bh / p.Hq;
    hk = (bh - b * p.Hq) / p.group;
    row_base = int64_t(bh) * p.Nq;
    n_rows = p.Nq;
  }
  const int64_t kv_head = int64_t(b) * p.Hkv + hk;
  const int64_t out_base = SPLIT ? row_base + int64_t(split) * p.part_rows : row_base;

  const T* Qh = static_cast<const T*>(p.q) + row_base * D;
  const T* Kh = static_cast<const T*>(p.k) + kv_head * p.Nk * D;
  // per layer of a chain (NL = 1: the one Q and K above)
  __amdgpu_buffer_rsrc_t ql_rs[NL], kl_rs[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const T* ql = NL == 1 ? Qh : static_cast<const T*>(p.chain_q[l]) + row_base * D;
    const T* kl = NL == 1 ? Kh : static_cast<const T*>(p.chain_k[l]) + kv_head * p.Nk * D;
    ql_rs[l] = make_rsrc(ql, uint32_t(n_rows) * D * ESZ);
    kl_rs[l] = make_rsrc(kl, uint32_t(p.Nk) * D * ESZ);
  }
  const T* Vh = static_cast<const T*>(p.v) + kv_head * p.Nk * D;
  OutT* Oh = static_cast<OutT*>(p.o) + out_base * D;
  float* Lh = p.lse + out_base;
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(Kh, uint32_t(p.Nk) * D * ESZ);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(Vh, uint32_t(p.Nk) * D * ESZ);
  const float c = p.c;
  // Exponent factor.  Without a bias the row max and the exponent act on the
  // raw scores s, p = 2^(s*c - m).  With one the logit t = s*|scale| + b is
  // formed first (one FMA) and p = 2^(t*log2(e) - m).
  const float scale_abs = p.scale_abs;
  const float ce = BIAS ? kLog2e : c;

  const int q_blk = tile * BM;
  const int wq0 = q_blk + wave * QW;      // first row of this wave
  const bool wave_has_rows = wq0 < n_rows;
  const int wq_last = min(wq0 + QW, n_rows) - 1;
  const int blk_last = min(q_blk + BM, n_rows) - 1;
  int qi[QB];                             // the row this lane owns in block qb
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qi[qb] = wq0 + 32 * qb + ln;

  // Causal query positions.  Without the key split a row is its position.
  // With it, row r sits at position r % Nq; a run of rows [r0, r1] inside one
  // head covers positions r0 % Nq .. r1 % Nq, and a run that crosses a head
  // boundary is taken to cover 0 .. Nq-1 (a safe over-estimate).
  auto pos_max = [&](int r0, int r1) {
    if constexpr (!SPLIT) return r1;
    return (r0 / p.Nq == r1 / p.Nq) ? r1 % p.Nq : p.Nq - 1;
  };
  auto pos_min = [&](int r0, int r1) {
    if constexpr (!SPLIT) return r0;
    return (r0 / p.Nq == r1 / p.Nq) ? r0 % p.Nq : 0;
  };
  int qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qpos[qb] = SPLIT ? qi[qb] % p.Nq : qi[qb];
  const int wave_pos_max = pos_max(wq0, wq_last);
  // Sliding window (causal only): the row at position i sees keys i-W+1 .. i.
  const int W = (CAUSAL && WINDOW) ? p.window : 0;
  const int wave_key_lo = W > 0 ? max(0, pos_min(wq0, wq_last) - W + 1) : 0;

  int n_kv = (p.Nk + BN - 1) / BN;
  if (CAUSAL) n_kv = min(n_kv, pos_max(q_blk, blk_last) / BN + 1);
  // tiles wholly left of every row's window are skipped
  const int j_lo = W > 0 ? min(n_kv, max(0, pos_min(q_blk, blk_last) - W + 1) / BN) : 0;
  // Key tiles [j_begin, j_end) of this workgroup: all visible tiles, or the
  // split's share of them (balanced, empty only when splits outnumber tiles).
  int j_begin = j_lo, j_end = n_kv;
  if constexpr (SPLIT) {
    const int nt = n_kv - j_lo;
    j_begin = j_lo + int(int64_t(split) * nt / p.n_splits);
    j_end = j_lo + int(int64_t(split + 1) * nt / p.n_splits);
  }

  // ---- Q fragments: B operand of S^T = K Q^T, loaded once ---------------------
  Frag qf[NL][QB][NS];
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int off = (qi[qb] * D + s * KS + g * KP) * ESZ;  // rows past Nq read 0
      if constexpr (F8) {
        if (s % 2 == 0) {  // steps s and s+1 from chunk s + g (see the K reads)
          u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(ql_rs[l], qi[qb] * D + (s + g) * 16, 0, 0);
          raw ^= p.q_sign;
          qf[l][qb][s] = __builtin_bit_cast(Frag, u32x2{raw[0], raw[1]});
          qf[l][qb][s + 1] = __builtin_bit_cast(Frag, u32x2{raw[2], raw[3]});
        }
      } else if constexpr (F32) {
        const u32 raw = __builtin_amdgcn_raw_buffer_load_b32(ql_rs[l], off, 0, 0);
        qf[l][qb][s] = __builtin_bit_cast(float, raw ^ p.q_sign);
      } else {
        u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(ql_rs[l], off, 0, 0);
        raw ^= p.q_sign;
        qf[l][qb][s] = __builtin_bit_cast(Frag, raw);
      }
    }

  // ---- bias: rows of this query block ----------------------------------------
  // Read once overall, but each 128-byte line is touched by several of a
  // wave's loads in a row, so the loads keep the default cache policy (a
  // non-temporal hint lets lines go before the next touch).
  using BiasVec = typename std::conditional<F32, u32x4, u32x2>::type;
  BiasVec bcur[QB][NKB][4], bnext[QB][NKB][4];
  // (without a bias the resource is built over an empty range and never read)
  const T* bblk = BIAS ? static_cast<const T*>(p.bias) + (row_base + q_blk) * p.Nk
                       : static_cast<const T*>(p.q);
  const __amdgpu_buffer_rsrc_t b_rs =
      make_rsrc(bblk, BIAS ? uint32_t(blk_last - q_blk + 1) * uint32_t(p.Nk) * ESZ : 0u);
  auto load_bias = [&](BiasVec (&dst)[QB][NKB][4], int j) {
    if constexpr (BIAS) {
      if (p.bias_vec) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const int row_off = (qi[qb] - q_blk) * p.Nk + j * BN + kb * 32;
            if constexpr (F32) {
              // 4 keys per load: keys 8*q4 + 4*g + 0..3, the score layout itself
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                dst[qb][kb][q4] = __builtin_amdgcn_raw_buffer_load_b128(
                    b_rs, (row_off + 8 * q4 + 4 * g) * ESZ, 0, 0);
            } else {
              // 8 keys per load: keys 16*h + 8*g + 0..7 land in slots 2h
              // (first 4) and 2h+1 (last 4); swap_bias_halves puts them where
              // the score registers expect them
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(
                    b_rs, (row_off + 16 * h + 8 * g) * ESZ, 0, 0);
                dst[qb][kb][2 * h] = u32x2{raw[0], raw[1]};
                dst[qb][kb][2 * h + 1] = u32x2{raw[2], raw[3]};
              }
            }
          }
      } else {
        // rows not aligned for vector loads: element loads (values past the
        // row end belong to masked keys; past the block they read 0)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int off = ((qi[qb] - q_blk) * p.Nk + j * BN + kb * 32 + 8 * q4 + 4 * g) * ESZ;
              if constexpr (F32) {
                BiasVec v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  v[e] = __builtin_amdgcn_raw_buffer_load_b32(b_rs, off + 4 * e, 0, 0);
                dst[qb][kb][q4] = v;
              } else {
                u32 w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  w[e] = __builtin_amdgcn_raw_buffer_load_b16(b_rs, off + 2 * e, 0, 0);
                dst[qb][kb][q4] = BiasVec{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
              }
            }
      }
    }
  };
  // After a 16-byte load, lane half 0 holds keys 16h+0..7 of its row and lane
  // half 1 keys 16h+8..15; the score layout wants keys 16h+0..3 and 16h+8..11
  // in half 0 and 16h+4..7 and 16h+12..15 in half 1.  One swap per word pair
  // exchanges the middle quarters.
  auto swap_bias_halves = [&]() {
    if constexpr (BIAS && !F32) {
      if (p.bias_vec) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const u32 x = bcur[qb][kb][2 * h][w], y = bcur[qb][kb][2 * h + 1][w];
                const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
                const u32 r0 = r[0], r1 = r[1];
                bcur[qb][kb][2 * h][w] = r0;
                bcur[qb][kb][2 * h + 1][w] = r1;
              }
      }
    }
  };
  auto bias_at = [&](int qb, int kb, int r) -> float {
    if constexpr (F32) {
      const u32 w = bcur[qb][kb][r >> 2][r & 3];
      return __builtin_bit_cast(float, w);
    } else if constexpr (F8) {
      return 0.f;  // FP8 instances take no bias
    } else {
      const u32 w = bcur[qb][kb][r >> 2][(r & 3) >> 1];
      return E::widen((r & 1) ? (w >> 16) : (w & 0xffffu));
    }
  };

  // ---- K/V staging through registers -------------------------------------------
  u32x4 kreg[VTR ? 1 : KCH];
  u32x4 vreg[VTR ? 1 : VTPT][4];   // fp32 V^T path: 4 keys x VEC columns per task

  // LDS chunk swizzles of this instance (K read by rows, V read transposed)
  auto swz_k = [](int r) {
    if constexpr (F8) return f8_swizzle_rows<D>(r);
    else return lds_swizzle_rows<DL>(r);
  };
  auto swz_v = [](int r) {
    if constexpr (F8) return f8_swizzle_tr<D>(r);
    else return lds_swizzle_tr<DL>(r);
  };
  // 16-bit layout: chunk c (16 bytes) of tile row r sits at chunk
  // c ^ lds_swizzle_rows<D>(r) in K (read by rows) and c ^ lds_swizzle_tr<D>(r)
  // in V (read transposed); both bank-conflict free.
  // Direct loads: load i of wave w fills LDS bytes [1 KB * (w*DNI + i), +1 KB)
  // of each buffer, lane l the 16 bytes at l*16; the lane's source offset
  // (without the tile's first key) is precomputed.
  int dma_k[DNI], dma_v[DNI];
#pragma unroll
  for (int i = 0; i < DNI; ++i) {
    const int q = (wave * DNI + i) * 64 + lane;   // physical chunk index in the tile
    const int row = q / CPR, pc = q % CPR;
    // logical chunks past the row (D = 80, 96) get an offset past every
    // resource range (2^31 plus a tile offset below 2^31: no wrap), so the
    // load writes zeros
    const int lk = pc ^ swz_k(row), lv = pc ^ swz_v(row);
    dma_k[i] = lk < CPRG ? (row * D + lk * VEC) * ESZ : int(0x80000000u);
    dma_v[i] = lv < CPRG ? (row * D + lv * VEC) * ESZ : int(0x80000000u);
  }
  // K operand reads: lane (row ln of a 32-key block, lane half g) reads
  // logical chunk 2*st + g.
  // (FP8: one 16-byte read feeds two MFMA steps, its first 8 bytes the
  // contraction slots of step 2p and its last 8 those of step 2p+1, so read p
  // takes chunk 2p + g; Q is loaded in the same order)
  int k_off[VTR ? NKO : 1];
#pragma unroll
  for (int st = 0; st < (VTR ? NKO : 1); ++st) {
    k_off[st] = ln * RB + (((2 * st + g) ^ swz_k(ln)) * 16);
    // (kept whole: split into its row and chunk parts, each read would cost
    // two adds instead of one)
    if (FA_OPAQUE_KOFF) asm volatile("" : "+v"(k_off[st]));
  }
  // Transposed V reads (ds_read_b64_tr_b16): within each 16-lane group, lane
  // 4a+b receives element b of the 8-byte chunks read by lanes a, a+4, a+8,
  // a+12.  So lane s of the group reads row 4g + s/4 (and 8 rows further for
  // the second read) of the 16-key group, at column 32*db + 16*(lane/16 % 2) +
  // 4*(s % 4); it then holds 4 consecutive keys of column 32*db + lane % 32.
  int v_off[VTR ? NDB : 1];
#pragma unroll
  for (int db = 0; db < (VTR ? NDB : 1); ++db) {
    const int r = 4 * g + ((lane >> 2) & 3);
    const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    v_off[db] = r * RB + ((c ^ swz_v(r)) * 16) + 8 * (lane & 1);
    if constexpr (F8) {
      // ds_read_b64_tr_b8: within each 16-lane group, lane 8a+b receives byte
      // b of the 8-byte chunks read by lanes a, a+2, ..., a+14.  Lane 16m+r
      // (a = r % 2, j = r / 2) reads key row 4*(m/2) + j (j < 4) or + j + 4
      // of the 16-key group, bytes 8a.. of chunk 2*db + m % 2; lane L then
      // holds column 32*db + L % 32 for keys k16+4g+0..3, k16+4g+8..11 (g =
      // L / 32): the order of P in the S^T registers.
      const int m = lane >> 4, r16 = lane & 15, a = r16 & 1, jj = r16 >> 1;
      const int rr = 4 * (m >> 1) + (jj < 4 ? jj : jj + 4);
      const int cc = 2 * db + (m & 1);
      v_off[db] = rr * RB + ((cc ^ swz_v(rr)) * 16) + 8 * a;
    }
  }

  // Issue the direct LDS loads of tile j into buffer buf (16-bit types); the
  // wave index is taken as a scalar, so the destination (M0) is scalar work.
  // KVPOL is the loads' cache policy (see launch_one).
  const int wave_s = FA_SCALAR_WAVE ? __builtin_amdgcn_readfirstlane(wave) : wave;
  const int half_s = KH == 2 ? __builtin_amdgcn_readfirstlane(half) : 0;
  T* const smem_h = smem + half_s * 2 * BUF;   // this key half's two buffers
  auto dma_tile = [&](int j, int buf) {
    if constexpr (VTR) {
      char* base = reinterpret_cast<char*>(smem_h + buf * BUF);
      const int soff = j * BN * D * ESZ;
#pragma unroll
      for (int i = 0; i < DNI; ++i) {
        char* dst = base + (wave_s * DNI + i) * 1024;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          // (a const copy: with the array element itself as the argument the
          // host pass silently emits no launch stub for the kernel)
          const __amdgpu_buffer_rsrc_t kr = kl_rs[l];
          if constexpr (BIAS)
            dma16_asm<KVPOL>(kr, (lds_void*)(dst + l * KT * ESZ), unsigned(dma_k[i]),
                             unsigned(soff));
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(dst + l * KT * ESZ), 16,
                                                     unsigned(dma_k[i]), unsigned(soff), 0, KVPOL);
        }
        if constexpr (BIAS)
          dma16_asm<KVPOL>(v_rs, (lds_void*)(dst + KTL * ESZ), unsigned(dma_v[i]), unsigned(soff));
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rs, (lds_void*)(dst + KTL * ESZ), 16,
                                                   unsigned(dma_v[i]), unsigned(soff), 0, KVPOL);
      }
    }
  };

  // Logit tiles through LDS (BLDS).  Load t (0..3) of a tile brings rows
  // 8t .. 8t+7 of the wave's 32, lane l the 16-byte chunk (l & 7) of row
  // 8t + (l >> 3), stored at chunk (l & 7) ^ ((row >> 1) & 7) of that row in
  // LDS: 16 lanes reading one chunk of 16 consecutive rows then hit 16
  // distinct bank groups.
  char* const bias_lds = reinterpret_cast<char*>(smem + KV_ELEMS) + (BLDS ? wave_s * BTILE : 0);
  int bdma_off[BLDS ? 4 : 1];
  if constexpr (BLDS) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 8 * t + (lane >> 3);
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);
      bdma_off[t] = ((wq0 - q_blk + r) * p.Nk + chunk * 8) * ESZ;
    }
  }
  auto dma_bias = [&](int j) {
    if constexpr (BLDS) {
      char* dst = bias_lds;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dma16_asm<0>(b_rs, (lds_void*)(dst + t * 1024), unsigned(bdma_off[t]),
                                  unsigned(j * BN * ESZ));
    }
  };
  // the lane's keys of the tile, as the 16-byte global loads give them:
  // keys 32kb + 16h + 8g + 0..7 of row ln (chunk 4kb + 2h + g)
  auto read_bias = [&](BiasVec (&dst)[QB][NKB][4]) {
    if constexpr (BLDS) {
      const char* src = bias_lds + ln * (BN * 2);
      const int sw = (ln >> 1) & 7;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (((4 * kb + 2 * h + g) ^ sw) * 16));
          dst[0][kb][2 * h] = u32x2{raw[0], raw[1]};
          dst[0][kb][2 * h + 1] = u32x2{raw[2], raw[3]};
        }
    }
  };

  // fp32: global -> registers (the LDS store follows the compute of the tile)
  auto gload = [&](int j) {
    if constexpr (!VTR) {
    const int key0 = j * BN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx / (D / VEC), col = (cidx % (D / VEC)) * VEC;
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(k_rs, ((key0 + row) * D + col) * ESZ, 0, 0);
    }
#pragma unroll
      for (int i = 0; i < VTPT; ++i) {
        const int t = tid + i * kThreads;
        const int kg = t % (BN / 4), dc = t / (BN / 4);
        if (VTASKS % kThreads == 0 || t < VTASKS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            vreg[i][r] = __builtin_amdgcn_raw_buffer_load_b128(
                v_rs, ((key0 + kg * 4 + r) * D + dc * VEC) * ESZ, 0, 0);
          }
        }
      }
    }
  };

  auto sstore = [&](int buf) {
    if constexpr (VTR) return;  // the direct loads already wrote the tile
    T* sK = smem + buf * BUF;
    T* sV = sK + KTL;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx / (D / VEC), col = (cidx % (D / VEC)) * VEC;
      *reinterpret_cast<u32x4*>(sK + row * KSTR + col) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VTPT; ++i) {
      const int t = tid + i * kThreads;
      const int kg = t % (BN / 4), dc = t / (BN / 4);
      if (VTASKS % kThreads == 0 || t < VTASKS) {
        T* dst = sV + (dc * VEC) * VSTR + vt_pos_of_group(kg);
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            *reinterpret_cast<u32x4*>(dst + e * VSTR) =
                u32x4{vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
          }
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const int w = e >> 1;
            u32 lo, hi;
            if (e & 1) {
              lo = (vreg[i][0][w] >> 16) | (vreg[i][1][w] & 0xffff0000u);
              hi = (vreg[i][2][w] >> 16) | (vreg[i][3][w] & 0xffff0000u);
            } else {
              lo = (vreg[i][0][w] & 0xffffu) | (vreg[i][1][w] << 16);
              hi = (vreg[i][2][w] & 0xffffu) | (vreg[i][3][w] << 16);
            }
            *reinterpret_cast<u32x2*>(dst + e * VSTR) = u32x2{lo, hi};
          }
        }
      }
    }
  };

  // ---- online-softmax state --------------------------------------------------
  // m_ref: the reference max the exponents are taken against (base-2 logit
  // units, same in both lane halves).  It is raised only when a tile's row
  // max exceeds it by more than kTau, so p = 2^(t - m_ref) <= 2^kTau and the
  // rescale of the accumulator is skipped for most tiles.  O = acc / l and
  // LSE = m_ref + log2(l) do not depend on which reference is used.
  float m_ref[QB], l_run[QB];
  f32x16 acc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    l_run[qb] = 0.f;  // this lane's share of the running row sum
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x16{};
  }

  // (called from two loops in the BLDS instances; inlined at both)
  auto compute = [&](int j, int buf) __attribute__((always_inline)) {
    const T* sK = smem_h + buf * BUF;
    const T* sV = sK + KTL;
    const int key0 = j * BN;

    // S^T = K_j Q^T  (rows: keys of the tile, columns: 32 query rows per block)
    // (a chain sums the products of all its layers into the same registers)
    f32x16 s[QB][NKB];
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Frag kf;
        if constexpr (F8) {
          const char* src = reinterpret_cast<const char*>(sK + l * KT) + kb * 32 * RB + k_off[st / 2];
          const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
          kf = (st % 2 == 0) ? __builtin_bit_cast(Frag, u32x2{raw[0], raw[1]})
                             : __builtin_bit_cast(Frag, u32x2{raw[2], raw[3]});
        } else if constexpr (F32) {
          kf = sK[(kb * 32 + ln) * KSTR + st * KS + g * KP];
        } else {
          const char* src = reinterpret_cast<const char*>(sK + l * KT) + kb * 32 * RB + k_off[st];
          kf = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(src));
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = E::mma(kf, qf[l][qb][st], (l == 0 && st == 0) ? f32x16{} : s[qb][kb]);
      }
    }

    // Register r of block kb holds key key0 + kb*32 + 8*(r/4) + 4*g + r%4 of row qi.
    float m_tile[QB];
    bool grow_any = false;
    swap_bias_halves();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (BIAS) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[qb][kb][r] = fmaf(s[qb][kb][r], scale_abs, bias_at(qb, kb, r));
      }
      const bool need_mask =
          (key0 + BN > p.Nk) ||
          (CAUSAL && key0 + BN - 1 > pos_min(wq0 + 32 * qb, wq0 + 32 * qb + 31)) ||
          (W > 0 && key0 <= pos_max(wq0 + 32 * qb, wq0 + 32 * qb + 31) - W);
      if (need_mask) {
        // Register r of block kb holds the key at a constant offset from the
        // lane's first key key0 + 4g; the visible keys are those at offsets
        // in [lo, hi): below Nk, not after the row's position (causal), and
        // not W or more before it (window).
        const int first = key0 + 4 * g;
        const int hi = (CAUSAL ? min(p.Nk, qpos[qb] + 1) : p.Nk) - first;
        const int lo = qpos[qb] - W + 1 - first;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            const bool dead = off >= hi || (W > 0 && off < lo);
            if (dead) s[qb][kb][r] = -INFINITY;
          }
      }
      // row max over the tile: in-lane, then across the two lane halves
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = partner_max(mx);
      m_tile[qb] = mx * ce;  // ce > 0, so max(s)*ce = max(s*ce)
      grow_any = grow_any || (m_tile[qb] > m_ref[qb] + kTauT);  // -inf + kTau stays -inf
    }
    if (__builtin_amdgcn_ballot_w64(grow_any) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool grow = m_tile[qb] > m_ref[qb] + kTauT;
        // rows that grow: alpha = 2^(m_ref - m_tile), which is 0 while m_ref = -inf
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref[qb] - m_tile[qb]) : 1.f;
        m_ref[qb] = grow ? m_tile[qb] : m_ref[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      }
    }

    // p = 2^(t - m_ref); row sums; P rounded to the input type for the P.V product
    float rs[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float neg_m = (m_ref[qb] == -INFINITY) ? 0.f : kPShift - m_ref[qb];  // no exp(-inf + inf)
      rs[qb] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = fmaf(s[qb][kb][r], ce, neg_m);
          const float e = __builtin_amdgcn_exp2f(x);
          s[qb][kb][r] = e;
          rs[qb] += e;
        }
      l_run[qb] += rs[qb];
    }

    // O^T += V_j^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (F32) {
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
          const int pos = kb * 32 + (cc >> 3) * 16 + 8 * g + (cc & 7);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const float vf = sV[(db * 32 + ln) * VSTR + pos];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = E::mma(vf, s[qb][kb][cc], acc[qb][db]);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Frag pf[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            f32x8 pv;
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = s[qb][kb][8 * h + i];
            pf[qb] = E::pack8(pv);
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            // The 8 keys lane half g feeds this MFMA are k16+4g+0..3, then
            // k16+4g+8..11 (k16 = first key of the 16-key group), the order
            // the S^T registers hold P in.  Each transposed read gives every
            // lane 4 consecutive keys of its column d = 32*db + lane%32.
            const char* src = reinterpret_cast<const char*>(sV) + (kb * 32 + 16 * h) * RB + v_off[db];
            Frag vf;
            if constexpr (F8) {
              vf = __builtin_bit_cast(Frag, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src));
            } else {
              const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)src);
              const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + 8 * RB));
              const u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
              vf = __builtin_bit_cast(Frag, u32x4{lw[0], lw[1], hw[0], hw[1]});
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = E::mma(vf, pf[qb], acc[qb][db]);
          }
        }
      }
    }
  };

  // ---- main loop: double-buffered K/V tiles -------------------------------------
  // Tile j+1 is requested (into the other LDS buffer, or into registers for
  // fp32) before tile j is computed; one barrier per tile.  The buffer being
  // filled was last read in the previous iteration, before its barrier.
  // KH = 2: the first half takes tiles [j_begin, j_begin + n/2), the second
  // the rest; both run ceil(n/2) iterations so that every wave reaches every
  // barrier (the first half idles through the last one when n is odd).
  int t_begin = j_begin, t_end = j_end;
  if constexpr (KH == 2) {
    const int mid = j_begin + (j_end - j_begin) / 2;
    if (half_s == 0) t_end = mid;
    else t_begin = mid;
  }
  const int iters = KH == 2 ? (j_end - j_begin + 1) / 2 : j_end - j_begin;
  // Logits.  BLDS instances, rows that allow 16-byte loads: tile j+1's go
  // HBM -> LDS as soon as tile j's are in registers; each wave reads only its
  // own region, so the tile barrier is not needed for them, and the wait
  // before it covers them.  BLDS instances, other rows: each tile's are
  // loaded when it is computed (one register set).  Other instances: tile
  // j+1's are loaded into registers while tile j is computed.
  // (whether a wave works on a tile is the same in all its lanes; read from
  // lane 0 so that the branches on it are scalar)
  auto active_s = [&](int jj) {
    const bool a = jj < t_end && wave_has_rows &&
                   (!CAUSAL || (jj * BN <= wave_pos_max && jj * BN + BN - 1 >= wave_key_lo));
    return __builtin_amdgcn_readfirstlane(int(a)) != 0;
  };
  if (BLDS && p.bias_vec) {
    if (iters > 0) {
      dma_tile(t_begin, 0);
      if (active_s(t_begin)) dma_bias(t_begin);
      __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      __syncthreads();
    }
    for (int it = 0; it < iters; ++it) {
      const int j = t_begin + it;
      const int cur = it & 1;
      if (j + 1 < t_end) dma_tile(j + 1, cur ^ 1);
      const bool act = active_s(j);
      if (act) {
        read_bias(bcur);
        // the reads are done before the region is refilled
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      }
      if (active_s(j + 1)) dma_bias(j + 1);
      if (act) compute(j, cur);
      __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      __syncthreads();
    }
  } else {
    if (iters > 0) {
      if (t_begin < t_end) dma_tile(t_begin, 0);
      gload(j_begin);
      if constexpr (BIAS && !BLDS) load_bias(bcur, j_begin);
      sstore(0);
      if constexpr (VTR) __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      __syncthreads();
    }
    for (int it = 0; it < iters; ++it) {
      const int j = t_begin + it;
      const int cur = it & 1;
      const bool has_tile = KH == 1 || j < t_end;
      const bool has_next = j + 1 < t_end;
      if (has_next) {
        dma_tile(j + 1, cur ^ 1);
        gload(j + 1);
      }
      // a wave skips tiles above its rows' diagonal and, with a window, tiles
      // wholly left of its rows' windows
      const bool active = has_tile && wave_has_rows &&
                          (!CAUSAL || (j * BN <= wave_pos_max && j * BN + BN - 1 >= wave_key_lo));
      if constexpr (BLDS) {
        if (active) load_bias(bcur, j);
      } else if constexpr (BIAS) {
        {
          const bool next_active =
              has_next && wave_has_rows &&
              (!CAUSAL || ((j + 1) * BN <= wave_pos_max && (j + 1) * BN + BN - 1 >= wave_key_lo));
          if (next_active) load_bias(bnext, j + 1);
        }
      }
      if (active) compute(j, cur);
      if constexpr (BIAS && !BLDS) {
        {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) bcur[qb][kb][q4] = bnext[qb][kb][q4];
        }
      }
      if (has_next) sstore(cur ^ 1);
      // the direct LDS loads of this wave are done before the barrier publishes them
      if constexpr (VTR) __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      __syncthreads();
    }
  }

  // ---- KH = 2: merge the second key half's state into the first ---------------
  // Both halves hold the same rows in the same lanes, so the merge is per lane:
  // with M = max(m0, m1), each side's sum and output are scaled by
  // 2^(m_side - M) (0 for a side that saw no key) and added -- the merge of
  // two partial states of the kwkr.cn tutorial, §2.2.  The LDS buffers are
  // free: the last iteration's barrier followed every wave's last read, and
  // no tile load is in flight.
  if constexpr (KH == 2) {
    float* xs = reinterpret_cast<float*>(smem) + wave * XN * 64 + lane;
    if (half == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float* x = xs + qb * (2 + 16 * NDB) * 64;
        x[0] = m_ref[qb];
        x[64] = l_run[qb];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[(2 + 16 * db + r) * 64] = acc[qb][db][r];
      }
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float* x = xs + qb * (2 + 16 * NDB) * 64;
      const float m1 = x[0], l1 = x[64];
      const float m = fmaxf(m_ref[qb], m1);
      const float a0 = m_ref[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[qb] - m);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      m_ref[qb] = m;
      l_run[qb] = l_run[qb] * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[qb][db][r] = acc[qb][db][r] * a0 + x[(2 + 16 * db + r) * 64] * a1;
    }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 -----------------------------
  // (key split: the same over the split's keys, O kept in fp32)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool row_ok = qi[qb] < n_rows;
    const float l_tot = partner_sum(l_run[qb]);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    // Lane half g holds d = 8*q4 + 4*g + 0..3 of each 32-wide block.  One swap
    // per word gives lane half 0 the 8 values d = 16*pr + 0..7 and lane half 1
    // d = 16*pr + 8..15, so each lane writes whole 16-byte (bf16/fp16) or
    // 32-byte (fp32) runs.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        f32x4 a4, b4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a4[e] = acc[qb][db][8 * pr + e] * inv;
          b4[e] = acc[qb][db][8 * pr + 4 + e] * inv;
        }
        const int col = db * 32 + 16 * pr + 8 * g;  // first of this lane's 8 columns
        OutT* dst = Oh + int64_t(qi[qb]) * D + col;
        if constexpr (OUT_F32) {
          const u32x4 aw = __builtin_bit_cast(u32x4, a4), bw = __builtin_bit_cast(u32x4, b4);
          u32x4 ao, bo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto r = __builtin_amdgcn_permlane32_swap(u32(aw[e]), u32(bw[e]), false, false);
            const u32 r0 = r[0], r1 = r[1];
            ao[e] = r0;
            bo[e] = r1;
          }
          if (row_ok && (D % 32 == 0 || col < D)) {
            reinterpret_cast<u32x4*>(dst)[0] = ao;
            reinterpret_cast<u32x4*>(dst)[1] = bo;
          }
        } else {
          const u32x2 aw = Elem<OutT>::narrow4(a4), bw = Elem<OutT>::narrow4(b4);
          u32x4 out;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const auto r = __builtin_amdgcn_permlane32_swap(u32(aw[e]), u32(bw[e]), false, false);
            const u32 r0 = r[0], r1 = r[1];
            out[e] = r0;
            out[2 + e] = r1;
          }
          if (row_ok && (D % 32 == 0 || col < D)) *reinterpret_cast<u32x4*>(dst) = out;
        }
      }
    if (row_ok && g == 0)
      Lh[qi[qb]] = (l_tot > 0.f) ? (m_ref[qb] - kPShift) * kLn2 + logf(l_tot) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Merge of normalised partial results (key-split path, and fa_merge).
// Row r of the result combines part_o[s][r][:] and part_lse[s][r] over the
// parts s: with M = max_s LSE_s and w_s = e^(LSE_s - M), O = sum_s w_s O_s /
// sum_s w_s and LSE = M + ln(sum_s w_s) -- the merge of the kwkr.cn tutorial,
// §2.2, for normalised states (state (m, l, o) = (LSE_s, 1, O_s)).  A part
// with LSE = -inf has weight 0 and its O is not read; with no finite part the
// row gets O = 0 and LSE = -inf.
//
// Layout: the output is a flat list of rows * D/4 items (a row and 4 of its
// columns).  A workgroup takes 64 consecutive items, one per lane, and its 4
// waves split the parts between them (wave w folds parts w, w+4, ...), so the
// loads of different parts are independent and many are in flight at once.
// Each wave's state (M_w, sum of weights, weighted sum) goes through LDS and
// wave 0 merges the four the same way.  HBM-bound: every partial is read once.
// ---------------------------------------------------------------------------
constexpr int kMergeWaves = 4;

template <typename T>
__global__ __launch_bounds__(kMergeWaves * 64) void fa_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int n_parts,
    int64_t rows, int d4, T* __restrict__ o, float* __restrict__ lse) {
  constexpr bool F32 = std::is_same<T, float>::value;
  __shared__ float s_m[kMergeWaves][64];
  __shared__ float s_w[kMergeWaves][64];
  __shared__ f32x4 s_a[kMergeWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t total = rows * d4;
  const int64_t D = int64_t(4) * d4;
  for (int64_t base = int64_t(blockIdx.x) * 64; base < total; base += int64_t(gridDim.x) * 64) {
    const int64_t t = base + lane;
    const bool ok = t < total;
    const int64_t row = ok ? t / d4 : 0;
    const int c4 = ok ? int(t - row * d4) : 0;
    // this wave's parts: max LSE, then weights and the weighted sum
    float m = -INFINITY;
    if (ok) {
#pragma unroll 8
      for (int sp = wave; sp < n_parts; sp += kMergeWaves)
        m = fmaxf(m, part_lse[sp * rows + row]);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (ok && m != -INFINITY) {
      // (every part's O is read, so that the loads of one wave's parts do not
      // wait on their LSE; an empty part's O, which may be any bits, is
      // selected away rather than multiplied by 0)
#pragma unroll 4
      for (int sp = wave; sp < n_parts; sp += kMergeWaves) {
        const float ls = part_lse[sp * rows + row];
        const f32x4 x = *reinterpret_cast<const f32x4*>(part_o + (sp * rows + row) * D + 4 * c4);
        const bool live = ls != -INFINITY;
        const float w = live ? __builtin_amdgcn_exp2f((ls - m) * kLog2e) : 0.f;
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = live ? fmaf(w, x[e], acc[e]) : acc[e];
      }
    }
    s_m[wave][lane] = m;
    s_w[wave][lane] = wsum;
    s_a[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && ok) {
      float mt = s_m[0][lane];
#pragma unroll
      for (int g = 1; g < kMergeWaves; ++g) mt = fmaxf(mt, s_m[g][lane]);
      f32x4 at = {0.f, 0.f, 0.f, 0.f};
      float wt = 0.f;
      if (mt != -INFINITY) {
#pragma unroll
        for (int g = 0; g < kMergeWaves; ++g) {
          const float mg = s_m[g][lane];
          if (mg == -INFINITY) continue;
          const float f = __builtin_amdgcn_exp2f((mg - mt) * kLog2e);
          const f32x4 ag = s_a[g][lane];
          wt = fmaf(f, s_w[g][lane], wt);
#pragma unroll
          for (int e = 0; e < 4; ++e) at[e] = fmaf(f, ag[e], at[e]);
        }
      }
      const float inv = wt > 0.f ? 1.f / wt : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) at[e] *= inv;
      T* dst = o + row * D + 4 * c4;
      if constexpr (F32) {
        *reinterpret_cast<f32x4*>(dst) = at;
      } else {
        *reinterpret_cast<u32x2*>(dst) = Elem<T>::narrow4(at);
      }
      if (c4 == 0) lse[row] = wt > 0.f ? mt + logf(wt) : -INFINITY;
    }
    __syncthreads();
  }
}

// Few partial results (up to kMergeFew): one lane per (row, 4 columns) loops
// over the parts itself, with no exchange between waves.  The arithmetic is
// the one above in the same order (with at most one part per wave there it
// is bit-identical); the split kernels' many-part decode merges keep the
// kernel above, which spreads the parts of a row over the waves.
constexpr int kMergeFew = 4;
template <typename T>
__global__ __launch_bounds__(256) void fa_merge_few_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int n_parts,
    int64_t rows, int d4, T* __restrict__ o, float* __restrict__ lse) {
  constexpr bool F32 = std::is_same<T, float>::value;
  const int64_t total = rows * d4;
  const int64_t D = int64_t(4) * d4;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * 256) {
    const int64_t row = t / d4;
    const int c4 = int(t - row * d4);
    float m = -INFINITY;
    for (int sp = 0; sp < n_parts; ++sp) m = fmaxf(m, part_lse[sp * rows + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
      for (int sp = 0; sp < n_parts; ++sp) {
        const float ls = part_lse[sp * rows + row];
        if (ls == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);
        const f32x4 x = *reinterpret_cast<const f32x4*>(part_o + (sp * rows + row) * D + 4 * c4);
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, x[e], acc[e]);
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= inv;
    T* dst = o + row * D + 4 * c4;
    if constexpr (F32) {
      *reinterpret_cast<f32x4*>(dst) = acc;
    } else {
      *reinterpret_cast<u32x2*>(dst) = Elem<T>::narrow4(acc);
    }
    if (c4 == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
  }
}

// Cache policy of the K/V tile loads: in the key split, when a KV head's
// packed rows fit one row block (decode-like shapes), every K/V tile is read
// by exactly one workgroup, and the loads carry the non-temporal hint (decode
// B8 20/4 heads, 32768 keys: 82.6 against 96.4 us); everywhere else other row
// blocks of the head re-read the tiles from L2, and the hint costs about 4%.
// The choice is a template argument: a branch on it inside the tile loop cost
// 1.3% on the split instances that do not take it.
template <typename T, int D, int BN, int QB, bool CAUSAL, bool BIAS, bool SPLIT,
          bool WINDOW = false, int NL = 1, int KH = 1>
hipError_t launch_one(const Params& p, unsigned grid, hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&p)};
  const void* fn = reinterpret_cast<const void*>(
      &fa_fwd_kernel<T, D, BN, QB, CAUSAL, BIAS, SPLIT, WINDOW, NL, 0, KH>);
  if constexpr (SPLIT && FA_SPLIT_KV_STREAM && !std::is_same<T, float>::value) {
    if (p.n_qtiles == 1)
      fn = reinterpret_cast<const void*>(
          &fa_fwd_kernel<T, D, BN, QB, CAUSAL, BIAS, SPLIT, WINDOW, NL, kPolicyNT, KH>);
  }
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads * KH), args, 0, stream);
}

// Chain instances.  Keys per tile: the K tiles of all layers and the V tile
// share each of the two LDS buffers, so tiles shrink to 32 keys where 64
// would leave room for fewer than two workgroups per CU.
template <typename T, int D, int NL>
hipError_t launch_chain_nl(const Params& p, unsigned grid, hipStream_t s, bool causal) {
  constexpr int BN = (D == 64 && NL == 2) ? 64 : 32;
  return causal ? launch_one<T, D, BN, 1, true, false, false, false, NL>(p, grid, s)
                : launch_one<T, D, BN, 1, false, false, false, false, NL>(p, grid, s);
}

template <typename T, int D>
hipError_t launch_chain_d(const Params& p, unsigned grid, hipStream_t s, bool causal, int nl) {
  switch (nl) {
    case 2: return launch_chain_nl<T, D, 2>(p, grid, s, causal);
    case 3: return launch_chain_nl<T, D, 3>(p, grid, s, causal);
    default: return launch_chain_nl<T, D, 4>(p, grid, s, causal);
  }
}

template <typename T>
hipError_t launch_chain_t(const Params& p, unsigned grid, hipStream_t s, int D, bool causal,
                          int nl) {
  switch (D) {
    case 64: return launch_chain_d<T, 64>(p, grid, s, causal, nl);
    case 80: return launch_chain_d<T, 80>(p, grid, s, causal, nl);
    case 96: return launch_chain_d<T, 96>(p, grid, s, causal, nl);
    default: return launch_chain_d<T, 128>(p, grid, s, causal, nl);
  }
}

template <typename T, int D, int BN, int QB, bool SPLIT>
hipError_t launch_d(const Params& p, unsigned grid, hipStream_t s, bool causal, bool bias) {
  if (causal) {
    if constexpr (!SPLIT) {
      if (p.window > 0)
        return bias ? launch_one<T, D, BN, QB, true, true, false, true>(p, grid, s)
                    : launch_one<T, D, BN, QB, true, false, false, true>(p, grid, s);
    }
    return bias ? launch_one<T, D, BN, QB, true, true, SPLIT>(p, grid, s)
                : launch_one<T, D, BN, QB, true, false, SPLIT>(p, grid, s);
  }
  return bias ? launch_one<T, D, BN, QB, false, true, SPLIT>(p, grid, s)
              : launch_one<T, D, BN, QB, false, false, SPLIT>(p, grid, s);
}

// Head dim 256 (16-bit, fused, no window): 32-key tiles, 64 KB of LDS per
// workgroup.  Without a bias two workgroups share a compute unit (256 VGPRs
// per lane); the bias tile's registers would spill there, so the bias
// instances take one workgroup per compute unit and the accumulator registers
// (B2 H16 S4096 causal: 322 us at two, 414 at one; with a bias, H8: 549 us
// spilling at two, 214 at one).
template <typename T, bool SPLIT>
hipError_t launch_d256(const Params& p, unsigned grid, hipStream_t s, bool causal, bool bias) {
  if constexpr (!SPLIT) {
    if (causal && p.window > 0)
      return bias ? launch_one<T, 256, 32, 1, true, true, false, true>(p, grid, s)
                  : launch_one<T, 256, 32, 1, true, false, false, true>(p, grid, s);
  }
  if (causal)
    return bias ? launch_one<T, 256, 32, 1, true, true, SPLIT>(p, grid, s)
                : launch_one<T, 256, 32, 1, true, false, SPLIT>(p, grid, s);
  return bias ? launch_one<T, 256, 32, 1, false, true, SPLIT>(p, grid, s)
              : launch_one<T, 256, 32, 1, false, false, SPLIT>(p, grid, s);
}

// 32-row query blocks per wave.  Two blocks (64 rows) halve the K/V operand
// reads per MFMA; they fit in registers only for 16-bit inputs without a bias
// tile, at D = 64 and (non-causal, 32-key tiles) at D = 128.  Every other
// instance keeps one, and so does the key-split path.
constexpr int query_blocks(int dtype, int D, bool bias, bool split, bool causal) {
  return split ? 1
               : dtype == FA_DTYPE_FP8_E4M3                   ? 1
               : (dtype != FA_DTYPE_FP32 && D == 64 && !bias) ? kQB64
               : (dtype != FA_DTYPE_FP32 && D == 128 && !bias && !causal) ? kQB128N
               : (D == 128) ? kQB128 : 1;
}

template <typename T, bool SPLIT>
hipError_t launch_t(const Params& p, unsigned grid, hipStream_t s, int D, bool causal, bool bias) {
  if (D == 64) {
    if constexpr (!std::is_same<T, float>::value && !SPLIT) {
      if (!bias) {
        if (causal && p.window > 0)
          return launch_one<T, 64, kBN64, kQB64, true, false, false, true, 1, FA_KH64>(p, grid,
                                                                                       s);
        return causal ? launch_one<T, 64, kBN64, kQB64, true, false, false, false, 1, FA_KH64>(
                            p, grid, s)
                      : launch_one<T, 64, kBN64, kQB64, false, false, false>(p, grid, s);
      }
    }
    return launch_d<T, 64, kBN64, 1, SPLIT>(p, grid, s, causal, bias);
  }
  if constexpr (!std::is_same<T, float>::value) {
    if (D == 80) return launch_d<T, 80, kBN128, 1, SPLIT>(p, grid, s, causal, bias);
    if (D == 96) return launch_d<T, 96, kBN128, 1, SPLIT>(p, grid, s, causal, bias);
    if (D == 256) return launch_d256<T, SPLIT>(p, grid, s, causal, bias);
  }
  if constexpr (SPLIT) {
    // (32-key tiles without a bias, 64 with one)
    constexpr int BS = FA_SPLIT_BN128;
    if (causal)
      return bias ? launch_one<T, 128, kBN128, 1, true, true, true>(p, grid, s)
                  : launch_one<T, 128, BS, 1, true, false, true>(p, grid, s);
    return bias ? launch_one<T, 128, kBN128, 1, false, true, true>(p, grid, s)
                : launch_one<T, 128, BS, 1, false, false, true>(p, grid, s);
  } else {
    if constexpr (!std::is_same<T, float>::value) {
      if (!bias && !causal) return launch_one<T, 128, kBN128N, kQB128N, false, false, false>(p, grid, s);
    }
    return launch_d<T, 128, kBN128, kQB128, SPLIT>(p, grid, s, causal, bias);
  }
}

Params make_params(const LaunchArgs& a, int rows_per_block, int n_rows) {
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.bias = a.bias;
  p.o = a.o;
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.BH = a.B * a.Hq;
  p.group = a.Hq / a.Hkv;
  p.n_qtiles = (n_rows + rows_per_block - 1) / rows_per_block;
  // The kernel folds the scale into base-2 exponents and needs a positive
  // factor: a negative scale is realised by flipping the sign of Q (exact), and
  // a zero (or vanishing) one by a factor so small that every finite logit
  // times it rounds to 0 in float32 -- the same uniform softmax.
  float c = fabsf(a.scale) * kLog2e;
  if (!(c >= 1e-30f)) c = 1e-30f;
  p.c = c;
  p.scale_abs = fmaxf(fabsf(a.scale), 1e-30f / kLog2e);
  const bool neg = a.scale < 0.f;
  p.q_sign = !neg                          ? 0u
             : a.dtype == FA_DTYPE_FP32     ? 0x80000000u
             : a.dtype == FA_DTYPE_FP8_E4M3 ? 0x80808080u
                                            : 0x80008000u;
  p.bias_vec = (a.dtype == FA_DTYPE_FP32) ? (a.Nk % 4) == 0 : (a.Nk % 8) == 0;
  p.window = a.window;
  for (int l = 0; l < kMaxChainLayers; ++l) p.chain_q[l] = p.chain_k[l] = nullptr;
  p.n_splits = 1;
  p.part_rows = 0;
  return p;
}

// FP8 inputs: fused forward without a bias, D = 64 or 128 (checked by the API).
hipError_t launch_f8(const Params& p, unsigned grid, hipStream_t s, int D, bool causal) {
  using F8 = fp8e4m3;
  if (causal && p.window > 0)
    return D == 64 ? launch_one<F8, 64, 64, 1, true, false, false, true>(p, grid, s)
                   : launch_one<F8, 128, 64, 1, true, false, false, true>(p, grid, s);
  if (D == 64)
    return causal ? launch_one<F8, 64, 64, 1, true, false, false, false, 1, FA_KH64_F8>(p, grid,
                                                                                         s)
                  : launch_one<F8, 64, 64, 1, false, false, false>(p, grid, s);
  return causal ? launch_one<F8, 128, 64, 1, true, false, false>(p, grid, s)
                : launch_one<F8, 128, 64, 1, false, false, false>(p, grid, s);
}

// FP8 key split (the decode step over an FP8 KV cache): 64-key tiles, fp32
// partials like the 16-bit instances; the merge writes a bf16 O.
hipError_t launch_f8_split(const Params& p, unsigned grid, hipStream_t s, int D, bool causal) {
  using F8 = fp8e4m3;
  if (D == 64)
    return causal ? launch_one<F8, 64, 64, 1, true, false, true>(p, grid, s)
                  : launch_one<F8, 64, 64, 1, false, false, true>(p, grid, s);
  return causal ? launch_one<F8, 128, 64, 1, true, false, true>(p, grid, s)
                : launch_one<F8, 128, 64, 1, false, false, true>(p, grid, s);
}

template <bool SPLIT>
hipError_t dispatch(const Params& p, unsigned grid, const LaunchArgs& a) {
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  const bool bias = a.bias != nullptr;
  if (a.dtype == FA_DTYPE_FP8_E4M3)
    return SPLIT ? launch_f8_split(p, grid, s, a.D, a.causal) : launch_f8(p, grid, s, a.D, a.causal);
  switch (a.dtype) {
    case FA_DTYPE_BF16: return launch_t<__bf16, SPLIT>(p, grid, s, a.D, a.causal, bias);
    case FA_DTYPE_FP16: return launch_t<_Float16, SPLIT>(p, grid, s, a.D, a.causal, bias);
    default: return launch_t<float, SPLIT>(p, grid, s, a.D, a.causal, bias);
  }
}

hipError_t merge(const float* part_o, const float* part_lse, int n_parts, int64_t rows, int D,
                 void* o, float* lse, int dtype, hipStream_t s) {
  const int d4 = D / 4;
  const int64_t total = rows * d4;
  if (n_parts <= kMergeFew) {
    // one lane per item, up to 32 workgroups per CU; the kernel strides over the rest
    const int64_t want_few = (total + 255) / 256;
    const unsigned grid_few = unsigned(want_few < 8192 ? want_few : 8192);
    switch (dtype) {
      case FA_DTYPE_BF16:
        fa_merge_few_kernel<__bf16><<<grid_few, 256, 0, s>>>(part_o, part_lse, n_parts, rows, d4,
                                                             static_cast<__bf16*>(o), lse);
        break;
      case FA_DTYPE_FP16:
        fa_merge_few_kernel<_Float16><<<grid_few, 256, 0, s>>>(
            part_o, part_lse, n_parts, rows, d4, static_cast<_Float16*>(o), lse);
        break;
      default:
        fa_merge_few_kernel<float><<<grid_few, 256, 0, s>>>(part_o, part_lse, n_parts, rows, d4,
                                                            static_cast<float*>(o), lse);
        break;
    }
    return hipGetLastError();
  }
  // one workgroup per 64 items, up to 64 per CU; the kernel strides over the rest
  const int64_t want = (total + 63) / 64;
  const unsigned grid = unsigned(want < 16384 ? want : 16384);
  const dim3 block(kMergeWaves * 64);
  switch (dtype) {
    case FA_DTYPE_BF16:
      fa_merge_kernel<__bf16><<<grid, block, 0, s>>>(part_o, part_lse, n_parts, rows, d4,
                                                     static_cast<__bf16*>(o), lse);
      break;
    case FA_DTYPE_FP16:
      fa_merge_kernel<_Float16><<<grid, block, 0, s>>>(part_o, part_lse, n_parts, rows, d4,
                                                       static_cast<_Float16*>(o), lse);
      break;
    default:
      fa_merge_kernel<float><<<grid, block, 0, s>>>(part_o, part_lse, n_parts, rows, d4,
                                                    static_cast<float*>(o), lse);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int launch_forward(const LaunchArgs& a) {
  const int bm = kWaves * 32 * query_blocks(a.dtype, a.D, a.bias != nullptr, false, a.causal);
  const Params p = make_params(a, bm, a.Nq);
  const unsigned grid = unsigned(p.n_qtiles) * unsigned(p.BH);
  return dispatch<false>(p, grid, a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int launch_forward_split(const LaunchArgs& a, int n_splits, void* workspace) {
  const int group = a.Hq / a.Hkv;
  const int64_t part_rows = int64_t(a.B) * a.Hq * a.Nq;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             split_partial_o_bytes(part_rows, a.D, n_splits));
  LaunchArgs pa = a;
  pa.o = part_o;
  pa.lse = part_lse;
  Params p = make_params(pa, kWaves * 32, group * a.Nq);
  p.n_splits = n_splits;
  p.part_rows = part_rows;
  const unsigned grid = unsigned(p.n_qtiles) * unsigned(n_splits) * unsigned(a.B * a.Hkv);
  if (dispatch<true>(p, grid, pa) != hipSuccess) return FA_ERR_HIP;
  // (FP8 inputs give a bf16 O)
  const int out_dtype = a.dtype == FA_DTYPE_FP8_E4M3 ? int(FA_DTYPE_BF16) : a.dtype;
  return merge(part_o, part_lse, n_splits, part_rows, a.D, a.o, a.lse, out_dtype,
               static_cast<hipStream_t>(a.stream)) == hipSuccess
             ? FA_OK
             : FA_ERR_HIP;
}

int launch_forward_chain(const LaunchArgs& a, const void* const* q_layers,
                         const void* const* k_layers, int n_layers) {
  if (n_layers == 1) return launch_forward(a);
  Params p = make_params(a, kWaves * 32, a.Nq);
  for (int l = 0; l < kMaxChainLayers; ++l) {
    p.chain_q[l] = l < n_layers ? q_layers[l] : nullptr;
    p.chain_k[l] = l < n_layers ? k_layers[l] : nullptr;
  }
  const unsigned grid = unsigned(p.n_qtiles) * unsigned(p.BH);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  const hipError_t e = a.dtype == FA_DTYPE_BF16
                           ? launch_chain_t<__bf16>(p, grid, s, a.D, a.causal, n_layers)
                           : launch_chain_t<_Float16>(p, grid, s, a.D, a.causal, n_layers);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Allocation-free key split: the partials live in a static device array of
// FA_SPLIT_SCRATCH_BYTES (each GPU the library runs on holds its own copy for
// the life of the process).  On the host the array's name is only a stand-in
// for its device address, so the address is taken once per device with
// hipGetSymbolAddress, with that device current, and the kernels receive it
// as their workspace pointer.
// ---------------------------------------------------------------------------
}  // namespace fa

static __device__ __attribute__((aligned(256))) unsigned char scratch[FA_SPLIT_SCRATCH_BYTES];

namespace fa {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device); nullptr if the runtime cannot give it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

int launch_forward_split_noalloc(const LaunchArgs& a, int n_splits) {
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return FA_ERR_HIP;
  return launch_forward_split(a, n_splits, ws);
}

int launch_merge(const float* part_o, const float* part_lse, int n_parts, int64_t rows, int D,
                 void* o, float* lse, int dtype, void* stream) {
  return merge(part_o, part_lse, n_parts, rows, D, o, lse, dtype,
               static_cast<hipStream_t>(stream)) == hipSuccess
             ? FA_OK
             : FA_ERR_HIP;
}

}  // namespace fa

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
//    the 1-D grid lists the heaviest causal row blocks first, and consecutive
//    blocks walk the heads so that a head's row blocks share one XCD when the
//    head count is a multiple of 8;
//  * each wave computes the transposed score block S^T = K . Q^T with
//    32x32 MFMAs (bf16/fp16: v_mfma_f32_32x32x16, fp32: v_mfma_f32_32x32x2f32),
//    so one lane holds one query row and 16 of the 32 keys of a block: row max
//    and row sum are in-lane reductions plus one v_permlane32_swap;
//  * the output is accumulated transposed too, O^T += V^T . P^T, so the same
//    lane owns the same query row in S^T and in O^T: the online-softmax
//    rescale is a per-lane scalar and P feeds the MFMA B operand straight from
//    the S^T registers without any shuffle;
//  * K tiles sit in LDS row-major, V tiles transposed (d-major) with the keys
//    of each 16-key group reordered so that every MFMA operand read is one
//    16-byte ds_read per lane; rows are padded by 16 bytes so that 32 lanes
//    reading 32 rows hit distinct banks;
//  * two LDS buffers: tile j+1 is fetched from global memory into registers
//    while tile j is being computed, then written to the other buffer; one
//    barrier per tile;
//  * exp is the hardware base-2 exponential with scale*log2(e) folded into one
//    FMA; masks are applied only on tiles that cross the causal diagonal or
//    the end of the keys, and tiles wholly above the diagonal are skipped.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef uint32_t u32;
typedef uint16_t u16;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kQW = 32;                // query rows per wave
constexpr int kBM = kWaves * kQW;      // query rows per workgroup
constexpr int kBN = 64;                // keys per K/V tile
constexpr int kThreads = kWaves * 64;
static_assert(kBM == kRowsPerBlock, "grid-size validation assumes this block height");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element traits: MFMA shape, operand fragment type and conversions.
// KP = contraction values one lane supplies to one MFMA.
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static constexpr int KP = 8;
  using Frag = bf16x8;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag pack8(f32x8 x) {
    return __builtin_convertvector(x, bf16x8);
  }
  static __device__ __forceinline__ float widen(u32 bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
  }
  static __device__ __forceinline__ u32x2 narrow4(f32x4 x) {
    return __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
  }
};

template <>
struct Elem<_Float16> {
  static constexpr int KP = 8;
  using Frag = f16x8;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag pack8(f32x8 x) {
    return __builtin_convertvector(x, f16x8);
  }
  static __device__ __forceinline__ float widen(u32 bits16) {
    return float(__builtin_bit_cast(_Float16, u16(bits16)));
  }
  static __device__ __forceinline__ u32x2 narrow4(f32x4 x) {
    return __builtin_bit_cast(u32x2, __builtin_convertvector(x, f16x4));
  }
};

template <>
struct Elem<float> {
  static constexpr int KP = 1;
  using Frag = float;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

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
  int n_qtiles;  // ceil(Nq / kBM)
  float c;       // |scale| * log2(e), never 0 (see the launcher)
  u32 q_sign;    // sign bits XORed into Q when scale < 0
  int bias_vec;  // bias rows allow 4-element vector loads
};

// Key position inside a V^T tile row.  Within each group of 16 keys the 4-key
// runs are stored in the order 0,2,1,3, so that the 8 keys one lane half feeds
// to a P.V MFMA (keys 0-3 and 8-11, or 4-7 and 12-15) are contiguous.
__device__ __forceinline__ int vt_pos_of_group(int kg) {  // kg = key / 4
  const int r = kg & 3;
  const int sigma = (r == 1) ? 2 : (r == 2) ? 1 : r;
  return (kg >> 2) * 16 + sigma * 4;
}

// {own value, value of lane l^32} in some order, via v_permlane32_swap.  The
// two results are copied out of the returned vector as values before being
// reinterpreted: applying __builtin_bit_cast to the element lvalue r[1] reads
// the vector's first element instead (seen with this ROCm clang).
__device__ __forceinline__ void own_and_partner(float x, float& a, float& b) {
  const u32 xi = __builtin_bit_cast(u32, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  const u32 r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ float partner_max(float x) {
  float a, b;
  own_and_partner(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float partner_sum(float x) {
  float a, b;
  own_and_partner(x, a, b);
  return a + b;
}

template <typename T, int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(Params p) {
  using E = Elem<T>;
  using Frag = typename E::Frag;
  constexpr bool F32 = std::is_same<T, float>::value;
  constexpr int KP = E::KP;
  constexpr int KS = 2 * KP;         // contraction length of one MFMA
  constexpr int NS = D / KS;         // MFMAs per 32x32 score block
  constexpr int ESZ = sizeof(T);
  constexpr int VEC = 16 / ESZ;      // elements per 16-byte vector
  constexpr int KSTR = D + VEC;      // K tile row stride, elements
  constexpr int VSTR = kBN + VEC;    // V^T tile row stride, elements
  constexpr int KT = kBN * KSTR;     // elements per K buffer
  constexpr int VT = D * VSTR;       // elements per V^T buffer
  constexpr int NKB = kBN / 32;      // 32-key blocks per tile
  constexpr int NDB = D / 32;        // 32-wide column blocks of the output
  constexpr int KCH = kBN * D / VEC / kThreads;           // K vectors per thread
  constexpr int VTASKS = (kBN / 4) * (D / VEC);           // 4-key x VEC-column tasks
  constexpr int VTPT = (VTASKS + kThreads - 1) / kThreads;
  static_assert(KCH * kThreads * VEC == kBN * D, "K tile must split evenly");

  __shared__ __attribute__((aligned(16))) T smem[2 * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;

  const int bh = int(blockIdx.x % unsigned(p.BH));
  const int rank = int(blockIdx.x / unsigned(p.BH));
  const int tile = CAUSAL ? (p.n_qtiles - 1 - rank) : rank;
  const int b = bh / p.Hq, hq = bh - b * p.Hq, hk = hq / p.group;

  const int64_t kv_head = int64_t(b) * p.Hkv + hk;
  const T* __restrict__ Qh = static_cast<const T*>(p.q) + int64_t(bh) * p.Nq * D;
  const T* __restrict__ Kh = static_cast<const T*>(p.k) + kv_head * p.Nk * D;
  const T* __restrict__ Vh = static_cast<const T*>(p.v) + kv_head * p.Nk * D;
  T* __restrict__ Oh = static_cast<T*>(p.o) + int64_t(bh) * p.Nq * D;
  float* __restrict__ Lh = p.lse + int64_t(bh) * p.Nq;

  const int q_blk = tile * kBM;
  const int wq0 = q_blk + wave * kQW;     // first row of this wave
  const int qi = wq0 + ln;                // the row this lane owns
  const bool row_ok = qi < p.Nq;
  const bool wave_has_rows = wq0 < p.Nq;
  const int wq_last = min(wq0 + kQW, p.Nq) - 1;
  const int blk_last = min(q_blk + kBM, p.Nq) - 1;

  int n_kv = (p.Nk + kBN - 1) / kBN;
  if (CAUSAL) n_kv = min(n_kv, blk_last / kBN + 1);

  // ---- Q fragments: B operand of S^T = K Q^T, loaded once --------------------
  Frag qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int64_t off = int64_t(qi) * D + s * KS + g * KP;
    if constexpr (F32) {
      const u32 raw = row_ok ? __builtin_bit_cast(u32, Qh[off]) : 0u;
      qf[s] = __builtin_bit_cast(float, raw ^ p.q_sign);
    } else {
      u32x4 raw = row_ok ? *reinterpret_cast<const u32x4*>(Qh + off) : u32x4{0, 0, 0, 0};
      raw ^= p.q_sign;
      qf[s] = __builtin_bit_cast(Frag, raw);
    }
  }

  // ---- bias row pointer and per-tile register block -------------------------
  const T* __restrict__ brow = nullptr;
  if constexpr (BIAS) {
    brow = static_cast<const T*>(p.bias) + (int64_t(bh) * p.Nq + (row_ok ? qi : 0)) * p.Nk;
  }
  // bias values for this lane's 4-key runs: [kb][q4] -> 4 elements
  using BiasVec = typename std::conditional<F32, f32x4, u32x2>::type;
  BiasVec bcur[NKB][4], bnext[NKB][4];

  auto load_bias = [&](BiasVec (&dst)[NKB][4], int j) {
    if constexpr (BIAS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int key = j * kBN + kb * 32 + 8 * q4 + 4 * g;
          BiasVec val{};
          if (row_ok) {
            if (p.bias_vec && key + 3 < p.Nk) {
              val = __builtin_nontemporal_load(reinterpret_cast<const BiasVec*>(brow + key));
            } else {
              if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (key + e < p.Nk) ? brow[key + e] : 0.f;
              } else {
                const u16* b16 = reinterpret_cast<const u16*>(brow);
                u32 w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (key + e < p.Nk) ? u32(b16[key + e]) : 0u;
                val = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
              }
            }
          }
          dst[kb][q4] = val;
        }
      }
    }
  };
  auto bias_at = [&](const BiasVec (&src)[NKB][4], int kb, int r) -> float {
    if constexpr (F32) {
      return src[kb][r >> 2][r & 3];
    } else {
      const u32 w = src[kb][r >> 2][(r & 3) >> 1];
      return E::widen((r & 1) ? (w >> 16) : (w & 0xffffu));
    }
  };

  // ---- K/V staging through registers -----------------------------------------
  u32x4 kreg[KCH];
  u32x4 vreg[VTPT][4];

  auto gload = [&](int j) {
    const int key0 = j * kBN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / VEC), col = (c % (D / VEC)) * VEC;
      const int key = key0 + row;
      kreg[i] = (key < p.Nk) ? *reinterpret_cast<const u32x4*>(Kh + int64_t(key) * D + col)
                             : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VTPT; ++i) {
      const int t = tid + i * kThreads;
      const int kg = t % (kBN / 4), dc = t / (kBN / 4);
      if (VTASKS % kThreads == 0 || t < VTASKS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + kg * 4 + r;
          vreg[i][r] = (key < p.Nk)
                           ? *reinterpret_cast<const u32x4*>(Vh + int64_t(key) * D + dc * VEC)
                           : u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto sstore = [&](int buf) {
    T* sK = smem + buf * (KT + VT);
    T* sV = sK + KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / VEC), col = (c % (D / VEC)) * VEC;
      *reinterpret_cast<u32x4*>(sK + row * KSTR + col) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VTPT; ++i) {
      const int t = tid + i * kThreads;
      const int kg = t % (kBN / 4), dc = t / (kBN / 4);
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

  // ---- online-softmax state ---------------------------------------------------
  float m_run = -INFINITY;  // running row max, base-2 logit units (same in both lane halves)
  float l_run = 0.f;        // this lane's share of the running row sum
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const float c = p.c;

  auto compute = [&](int j, int buf) {
    const T* sK = smem + buf * (KT + VT);
    const T* sV = sK + KT;
    const int key0 = j * kBN;

    // S^T = K_j Q^T  (rows: keys of the tile, columns: this wave's 32 query rows)
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const T* src = sK + (kb * 32 + ln) * KSTR + st * KS + g * KP;
        Frag kf;
        if constexpr (F32) {
          kf = *src;
        } else {
          kf = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(src));
        }
        s[kb] = E::mma(kf, qf[st], s[kb]);
      }
    }

    // Register r of block kb holds key key0 + kb*32 + 8*(r/4) + 4*g + r%4 of row qi.
    if constexpr (BIAS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = fmaf(s[kb][r], c, bias_at(bcur, kb, r) * kLog2e);
    }
    const bool need_mask = (key0 + kBN > p.Nk) || (CAUSAL && key0 + kBN - 1 > wq0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool dead = key >= p.Nk || (CAUSAL && key > qi);
          if (dead) s[kb][r] = -INFINITY;
        }
    }

    // Row max over the tile: in-lane over 2*16 values, then across the lane halves.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = partner_max(mx);
    const float m_tile = BIAS ? mx : mx * c;  // c > 0, so max(s)*c = max(s*c)
    const float m_new = fmaxf(m_run, m_tile);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no exp(-inf + inf)
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    const float neg_m = -m_use;

    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = BIAS ? (s[kb][r] + neg_m) : fmaf(s[kb][r], c, neg_m);
        const float e = __builtin_amdgcn_exp2f(x);
        s[kb][r] = e;
        rs += e;
      }
    l_run = fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

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
            acc[db] = E::mma(vf, s[kb][cc], acc[db]);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x8 pv;
#pragma unroll
          for (int i = 0; i < 8; ++i) pv[i] = s[kb][8 * h + i];
          const Frag pf = E::pack8(pv);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const T* src = sV + (db * 32 + ln) * VSTR + kb * 32 + 16 * h + 8 * g;
            const Frag vf = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(src));
            acc[db] = E::mma(vf, pf, acc[db]);
          }
        }
      }
    }
  };

  // ---- main loop: double-buffered K/V tiles -----------------------------------
  if (n_kv > 0) {
    gload(0);
    if constexpr (BIAS) load_bias(bcur, 0);
    sstore(0);
    __syncthreads();
  }
  for (int j = 0; j < n_kv; ++j) {
    const int cur = j & 1;
    const bool has_next = j + 1 < n_kv;
    if (has_next) gload(j + 1);
    const bool active = wave_has_rows && (!CAUSAL || j * kBN <= wq_last);
    if constexpr (BIAS) {
      const bool next_active = has_next && wave_has_rows && (!CAUSAL || (j + 1) * kBN <= wq_last);
      if (next_active) load_bias(bnext, j + 1);
    }
    if (active) compute(j, cur);
    if constexpr (BIAS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) bcur[kb][q4] = bnext[kb][q4];
    }
    if (has_next) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = m ln2 + ln l ---------------------------------
  const float l_tot = partner_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (row_ok) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        f32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = acc[db][4 * q4 + e] * inv;
        T* dst = Oh + int64_t(qi) * D + d0;
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(dst) = o4;
        } else {
          *reinterpret_cast<u32x2*>(dst) = E::narrow4(o4);
        }
      }
    if (g == 0) Lh[qi] = (l_tot > 0.f) ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL, bool BIAS>
hipError_t launch_one(const Params& p, unsigned grid, hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<T, D, CAUSAL, BIAS>),
                         dim3(grid), dim3(kThreads), args, 0, stream);
}

template <typename T, int D>
hipError_t launch_d(const Params& p, unsigned grid, hipStream_t s, bool causal, bool bias) {
  if (causal) {
    return bias ? launch_one<T, D, true, true>(p, grid, s) : launch_one<T, D, true, false>(p, grid, s);
  }
  return bias ? launch_one<T, D, false, true>(p, grid, s) : launch_one<T, D, false, false>(p, grid, s);
}

template <typename T>
hipError_t launch_t(const Params& p, unsigned grid, hipStream_t s, int D, bool causal, bool bias) {
  return D == 64 ? launch_d<T, 64>(p, grid, s, causal, bias)
                 : launch_d<T, 128>(p, grid, s, causal, bias);
}

}  // namespace

int launch_forward(const LaunchArgs& a) {
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
  p.n_qtiles = (a.Nq + kBM - 1) / kBM;
  // The kernel folds the scale into base-2 exponents and needs a positive
  // factor: a negative scale is realised by flipping the sign of Q (exact), and
  // a zero (or vanishing) one by a factor so small that every finite logit
  // times it rounds to 0 in float32 -- the same uniform softmax.
  float c = fabsf(a.scale) * kLog2e;
  if (!(c >= 1e-30f)) c = 1e-30f;
  p.c = c;
  const bool neg = a.scale < 0.f;
  p.q_sign = !neg ? 0u : (a.dtype == FA_DTYPE_FP32 ? 0x80000000u : 0x80008000u);
  p.bias_vec = (a.Nk % 4) == 0;
  const unsigned grid = unsigned(p.n_qtiles) * unsigned(p.BH);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  const bool bias = a.bias != nullptr;
  hipError_t err;
  switch (a.dtype) {
    case FA_DTYPE_BF16: err = launch_t<__bf16>(p, grid, s, a.D, a.causal, bias); break;
    case FA_DTYPE_FP16: err = launch_t<_Float16>(p, grid, s, a.D, a.causal, bias); break;
    default: err = launch_t<float>(p, grid, s, a.D, a.causal, bias); break;
  }
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa

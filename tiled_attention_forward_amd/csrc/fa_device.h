// Device-side helpers shared by the forward (fa_fwd.hip) and backward
// (fa_bwd.hip) kernels: vector types, the MFMA element traits, raw buffer
// resources and the lane-half exchange.  Internal, not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt = 0 only: vector
// memory counter bits [3:0] and [15:14] zero, expcnt [6:4] and lgkmcnt [11:8]
// at their maxima (no wait).
constexpr int kWaitVmem0 = 0x0F70;
// waiting for lgkmcnt = 0 only (LDS reads): vmcnt and expcnt at their maxima
constexpr int kWaitLgkm0 = 0xC07F;
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

// OCP FP8 E4M3 (bias 7, 3 mantissa bits, no infinity, largest finite 448), the
// gfx950 native 8-bit float.  A one-byte storage type; values are only ever
// touched as bytes, by the matrix cores and by v_cvt_pk_fp8_f32.
struct fp8e4m3 {
  uint8_t bits;
};

// FP8 operands of v_mfma_f32_32x32x16_fp8_fp8 are laid out like the 16-bit
// ones of the 32x32x16 instructions (lane l: row l % 32, contraction values
// 8 * (l / 32) .. + 7), one byte each: 8 bytes per lane.
template <>
struct Elem<fp8e4m3> {
  static constexpr int KP = 8;
  using Frag = long;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
  }
  // 8 floats -> 8 bytes, value i in byte i (round to nearest even)
  static __device__ __forceinline__ Frag pack8(f32x8 x) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
    return __builtin_bit_cast(Frag, u32x2{u32(lo), u32(hi)});
  }
};

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

// LDS tiles of 16-bit K, V, Q or dO rows are stored unpadded, the 16-byte
// chunk c of tile row r at chunk c ^ lds_swizzle<D>(r).  The LDS serves 256
// bytes per cycle (64 banks of 4 bytes): a ds_read_b128 serves 16 lanes per
// cycle, a ds_read_b64_tr_b16 32 lanes.  The swizzle keeps both patterns the
// kernels use free of bank conflicts:
//  * row reads: 16 lanes read the same logical chunk of 16 consecutive rows;
//  * transposed reads: 32 lanes read 4 consecutive rows, 4 adjacent chunks each.
// With D = 64 a row is 128 bytes, so even and odd rows sit in different bank
// halves and the swizzle needs only bits 1-3 of r; with D = 128 a row covers
// all 64 banks and it uses bits 0-3.  Only r mod 16 matters.
template <int D>
__device__ __forceinline__ int lds_swizzle(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

// Tiles read one way only can use a swizzle for that pattern alone:
// lds_swizzle_rows<D> for row reads (16 distinct bank groups over 16 rows),
// lds_swizzle_tr<D> for transposed reads.  The latter ignores bit 3 of r, so
// the second transposed read of a 16-row group (rows +8) sits at a fixed
// 8-row byte offset from the first.
// Rows of 256 or 512 bytes (D = 128, 256) start on the same bank, so both use
// the same values (chunk indices stay inside the row: XOR values below 16).
template <int D>
__device__ __forceinline__ int lds_swizzle_rows(int r) {
  if constexpr (D == 64) return (r >> 1) & 7;
  return r & 15;
}
template <int D>
__device__ __forceinline__ int lds_swizzle_tr(int r) {
  if constexpr (D == 64) return ((r >> 1) & 1) << 2;
  return (r & 3) << 2;
}

// FP8 tiles (rows of D bytes: 4 chunks at D = 64, 8 at D = 128).
//  * row reads (ds_read_b128, 16 lanes per cycle, 16 consecutive rows, one
//    logical chunk): a 64-byte row covers 16 banks, so rows r and r+4 start
//    on the same bank: chunk c ^ ((r >> 2) & 3); a 128-byte row covers 32:
//    chunk c ^ ((r >> 1) & 7), as for 16-bit rows of 64 elements;
//  * transposed reads (ds_read_b64_tr_b8, 32 lanes per cycle): 8 rows
//    {0..3, 8..11} (+ a multiple of 4) of two adjacent chunks, both halves of
//    each; rows r and r+8 must land apart (64-byte rows: chunk c ^ 2 for the
//    second 8 rows), and at 128 bytes rows 2 apart too.
template <int D>
__device__ __forceinline__ int f8_swizzle_rows(int r) {
  if constexpr (D == 64) return (r >> 2) & 3;
  return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int f8_swizzle_tr(int r) {
  if constexpr (D == 64) return ((r >> 3) & 1) << 1;
  return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// (the hardware range check), so tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           0x00020000);
}

// Workgroup ids are dealt round-robin to the 8 XCDs, each with its own L2.
// Renumber so that the ids one XCD receives are consecutive: logical id
// x*(full/8) + i for the i-th id of XCD x.  Used where all workgroups carry
// equal work, so that the blocks of one head (consecutive logical ids) run on
// one XCD at the same time and share its L2 copy of the head's operands.  The
// last nblk % 8 ids keep their number.
__device__ __forceinline__ unsigned xcd_contiguous(unsigned id, unsigned nblk) {
  const unsigned full = nblk & ~7u;
  return id < full ? (id & 7u) * (full >> 3) + (id >> 3) : id;
}

// Causal grids list their units rank-major (unit = rank * units_per_rank + u)
// with `group` workgroups per unit, e.g. the query heads of one KV head.  The
// ids come in runs of 8*group; in run k the id at offset r is member r/8 of
// unit 8k + r%8, so the members of a unit all go to one XCD, one after the
// other.  group = 1 is the identity; a tail shorter than a run keeps the plain
// order (unit = id / group).
struct UnitMember {
  unsigned unit, member;
};
__device__ __forceinline__ UnitMember xcd_group_units(unsigned id, unsigned nblk, unsigned group) {
  const unsigned run = 8u * group, full = nblk - nblk % run;
  if (id < full) {
    const unsigned r = id % run;
    return {(id / run) * 8u + (r & 7u), r >> 3};
  }
  return {id / group, id % group};
}

}  // namespace fa

// Device helpers for the gfx950 codec kernels: fragment types, bf16 / fp16
// conversions, the cross-lane transposes and the register butterflies of the
// Walsh-Hadamard transform.
//
// Lane layout used by every codec kernel ("four lanes per block"): a wave
// handles 16 blocks at a time; lane l works on block row r = l & 15 and holds
// E = d/4 of its values, quarter g = l >> 4.  This is the row layout of the
// 16x16 MFMA operands (row r lives in lanes r, r+16, r+32, r+48), so the
// residual and key projections feed the matrix cores without any reshuffle.
//
// The d-point Walsh-Hadamard transform H = H2 (x) ... (x) H2 is a butterfly
// along every bit of the element index.  Bits held in the register index are
// transformed in registers; the two bits held in lane bits 4 and 5 are first
// moved into the register index with v_permlane16_swap / v_permlane32_swap
// (one instruction per register pair), which transposes a lane bit with a
// register bit.  Measured semantics on gfx950: swap(x, y) exchanges x in the
// odd 16-lane rows (upper 32-lane half) with y in the even rows (lower half).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
// two fp32 -> packed bf16 pair in one v_cvt_pk_bf16_f32 (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const b2 b = __builtin_convertvector((f2){lo, hi}, b2);
  return __builtin_bit_cast(uint32_t, b);
}
// fp32 -> fp16 bits, round to nearest even, overflow to +-inf (v_cvt_f16_f32)
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Sum of squares of the E register values, accumulated as eight interleaved partial
// sums combined pairwise (keeps the fp32 rounding error of a block norm near 1e-7).
template <int E>
__device__ __forceinline__ float tree_sumsq(const float (&v)[E]) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v[i] * v[i];
#pragma unroll
  for (int j = 8; j < E; ++j) acc[j & 7] = fmaf(v[j], v[j], acc[j & 7]);
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// Butterfly along register-index bit K: (a, b) -> (a + b, a - b).
template <int E, int K>
__device__ __forceinline__ void bfly(float (&v)[E]) {
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (j & (1 << K)) continue;
    const float a = v[j], b = v[j | (1 << K)];
    v[j] = a + b;
    v[j | (1 << K)] = a - b;
  }
}

// Transpose register-index bit K with lane bit 4 (16-lane rows).
template <int E, int K>
__device__ __forceinline__ void xch16(float (&v)[E]) {
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (j & (1 << K)) continue;
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j | (1 << K)]),
                                              false, false);
    v[j] = __uint_as_float(r[0]);
    v[j | (1 << K)] = __uint_as_float(r[1]);
  }
}

// Transpose register-index bit K with lane bit 5 (32-lane halves).
template <int E, int K>
__device__ __forceinline__ void xch32(float (&v)[E]) {
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (j & (1 << K)) continue;
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j | (1 << K)]),
                                              false, false);
    v[j] = __uint_as_float(r[0]);
    v[j | (1 << K)] = __uint_as_float(r[1]);
  }
}

// Largest value over the four lanes of a block row (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum of a value over the four lanes of a block row (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int E> struct Log2;
template <> struct Log2<16> { static constexpr int v = 4; };
template <> struct Log2<32> { static constexpr int v = 5; };
template <> struct Log2<64> { static constexpr int v = 6; };
template <> struct Log2<128> { static constexpr int v = 7; };

// ---------------------------------------------------------------------------------------------
// Element maps.  "load layout": register j of lane quarter g holds element
// e = (j & 7) + 8 g + 32 (j >> 3), so the four lanes of a block read 64
// contiguous bytes per 16-byte load.  The quantize transform ends in the
// "contiguous layout": quarter g holds the E consecutive elements starting at
// E * qpos(g), register j at offset cperm(j).  Dequantize starts from the
// contiguous layout with identity order and ends in the load layout with a
// permuted chunk order (dq_out_chunk).
// ---------------------------------------------------------------------------------------------
__host__ __device__ constexpr int load_e(int g, int j) { return (j & 7) + 8 * g + 32 * (j >> 3); }

template <int D>
__host__ __device__ constexpr int qpos(int g) {
  return D == 64 ? (((g & 1) << 1) | (g >> 1)) : g;
}

// Offset, inside the lane's contiguous run, of register j after the forward transform.
template <int D>
__host__ __device__ constexpr int cperm(int j) {
  // D=64, 128: identity.  D=256: reg bits (3,4,5) hold element bits (5,3,4).
  // D=512: reg bits (3,4,5,6) hold element bits (5,6,3,4).
  return D == 256 ? ((j & 7) | (((j >> 3) & 1) << 5) | (((j >> 4) & 1) << 3) | (((j >> 5) & 1) << 4))
       : D == 512 ? ((j & 7) | (((j >> 3) & 1) << 5) | (((j >> 4) & 1) << 6) | (((j >> 5) & 1) << 3) |
                     (((j >> 6) & 1) << 4))
                  : j;
}

// Forward transform for quantize: load layout in, contiguous layout out.  STAGE0 = false
// skips the butterfly along register bit 0 (done by the caller while unpacking).
template <int D, bool STAGE0 = true>
__device__ __forceinline__ void wht_forward(float (&v)[D / 4]) {
  constexpr int E = D / 4;
  if constexpr (STAGE0) bfly<E, 0>(v);
  bfly<E, 1>(v); bfly<E, 2>(v);
  bfly<E, 3>(v);
  if constexpr (E >= 32) bfly<E, 4>(v);
  if constexpr (E >= 64) bfly<E, 5>(v);
  if constexpr (E >= 128) bfly<E, 6>(v);
  if constexpr (D == 64) {
    // reg3 <-> e5 / lane4 <-> e3: swap, transform e3; then e4 (lane5) through reg3 and back
    xch16<E, 3>(v); bfly<E, 3>(v);
    xch32<E, 3>(v); bfly<E, 3>(v); xch32<E, 3>(v);
  } else {
    constexpr int KA = Log2<E>::v - 2;   // register bit holding element bit log2(D)-2
    constexpr int KB = Log2<E>::v - 1;   // register bit holding element bit log2(D)-1
    xch16<E, KA>(v); bfly<E, KA>(v);
    xch32<E, KB>(v); bfly<E, KB>(v);
  }
}

// Inverse transform for dequantize (H is symmetric, so the same butterflies):
// contiguous layout in (quarter g holds e = E g + j), load layout out.
template <int D>
__device__ __forceinline__ void wht_dequant(float (&v)[D / 4]) {
  constexpr int E = D / 4;
  bfly<E, 0>(v); bfly<E, 1>(v); bfly<E, 2>(v); bfly<E, 3>(v);
  if constexpr (E >= 32) bfly<E, 4>(v);
  if constexpr (E >= 64) bfly<E, 5>(v);
  if constexpr (E >= 128) bfly<E, 6>(v);
  if constexpr (D == 64) {
    xch16<E, 3>(v); bfly<E, 3>(v);   // lane4 <- e3, reg3 <- e4
    xch32<E, 3>(v); bfly<E, 3>(v);   // lane5 <- e4, reg3 <- e5
  } else {
    xch16<E, 3>(v); bfly<E, 3>(v);   // lane4 <- e3, reg3 <- e(L-2)
    xch32<E, 4>(v); bfly<E, 4>(v);   // lane5 <- e4, reg4 <- e(L-1)
  }
}

// After wht_dequant, register chunk s (registers 8s..8s+7) of quarter g holds
// elements 8 g + dq_out_chunk(s) + 0..7.
template <int D>
__host__ __device__ constexpr int dq_out_chunk(int s) {
  // chunk-index bits: (s0, s1, s2, s3) = register bits (3, 4, 5, 6)
  return D == 64 ? 32 * s
       : D == 128 ? 32 * s
       : D == 256 ? (((s & 1) << 6) | (((s >> 1) & 1) << 7) | (((s >> 2) & 1) << 5))
                  : (((s & 1) << 7) | (((s >> 1) & 1) << 8) | (((s >> 2) & 1) << 5) | (((s >> 3) & 1) << 6));
}

// The register chunk whose elements follow those of chunk s (dq_out_chunk + 32): chunks s
// and dq_partner(s), s with dq_out_chunk(s) a multiple of 64, make up one 128-byte line of
// bf16 output.
template <int D>
__host__ __device__ constexpr int dq_partner(int s) {
  for (int t = 0; t < D / 32; ++t)
    if (dq_out_chunk<D>(t) == dq_out_chunk<D>(s) + 32) return t;
  return -1;
}

// The quantize kernel takes the rotated residual rho (contiguous layout, registers
// renamed to offset order) back through the dequantize butterflies: register chunk k
// (registers 8k .. 8k+7) of quarter g then holds elements 8 res_col8(k) + 0..7 of
// H rho = d D r.  For d = 64 the contiguous layout keeps element bits 4 and 5 in lane
// bits 5 and 4, which swaps those two bits of the dequantize output map.
template <int D>
__host__ __device__ constexpr int res_col8(int g, int k) {
  return D == 64 ? ((g & 1) | (k << 1) | ((g >> 1) << 2)) : g + dq_out_chunk<D>(k) / 8;
}

}  // namespace pqd

// gfx950 kernels of the block codec and the QJL sketch.
//
// Every kernel is persistent: each wave walks over tiles of 16 blocks (keys)
// with a grid stride, so the per-workgroup set-up (codebook, search grid and
// projection matrix staged in LDS) is paid once per workgroup.
#include <algorithm>
#include <type_traits>

#include "pq_device.h"
#include "pq_internal.h"

using namespace pqd;
using pqi::CodecTables;

namespace {

constexpr int kThreads = 256;             // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;

// Persistent grids: workgroups per CU for each kernel (a wave then walks over
// n_tiles / (4 * grid) tiles, prefetching the next one).
#ifndef PQ_QUANT_WG_PER_CU
#define PQ_QUANT_WG_PER_CU 4
#endif
#ifndef PQ_DEQUANT_WG_PER_CU
#define PQ_DEQUANT_WG_PER_CU 4
#endif
#ifndef PQ_QUANT_WAVES_PER_EU
#define PQ_QUANT_WAVES_PER_EU 1
#endif
#ifndef PQ_RB_WPE
#define PQ_RB_WPE 4              // rotated-basis quantize: waves per SIMD
#endif
#ifndef PQ_RB_WG
#define PQ_RB_WG 1               // ... and workgroups per CU sharing them
#endif
constexpr int kRbThreads = 256 * PQ_RB_WPE / PQ_RB_WG;
#ifndef PQ_LOOKUP_BATCH
#define PQ_LOOKUP_BATCH 8        // grid lookups of the code decision in flight at once
#endif
#ifndef PQ_LOOKUP_BATCH_QJL
#define PQ_LOOKUP_BATCH_QJL 2    // ... with the QJL stage at d <= 128 (16-byte entries; twice that above)
#endif
#ifndef PQ_SKETCH_WG_PER_CU
#define PQ_SKETCH_WG_PER_CU 2
#endif

// ------------------------------------------------------------------------------------------
// LDS set-up shared by quantize and dequantize
// ------------------------------------------------------------------------------------------
// One entry per thread step; the nearest boundary of every cell comes with the tables.
__device__ void build_search_grid(const CodecTables& t, uint4* tab) {
  const int rep_shift = t.nrep == 16 ? 4 : 0;
  for (int i = threadIdx.x; i < t.ncell * t.nrep; i += blockDim.x) {
    const int best = t.cell_best[i >> rep_shift];
    tab[i] = make_uint4(__float_as_uint(t.beta[best]), (uint32_t)best, __float_as_uint(t.cent[best]),
                        __float_as_uint(t.cent[best + 1]));
  }
}

// Walsh-Hadamard operand fragments of the d = 128 rotation on the bf16 matrix cores.  H's entry
// (k, n) is (-1)^popcount(k & n).  Output row tile t (coordinates 16 t + 0..15) and K step s
// (elements 32 s + 0..31) take the block of H that is H's block (s = 0, t & 1) times
// (-1)^popcount(s & (t >> 1)), since k = 32 s + kk and n = 16 t + nn share bits 5 and 6 only
// through s and t >> 1.  So four fragments cover every (s, t): fragment f = (t & 1) + 2 neg, as
// the A operand of v_mfma_f32_16x16x32_bf16 (lane l: row nn = l & 15, K = 8 (l >> 4) + 0..7),
// entries +-1.0 in bf16, written to hf[f * 64 + lane].
constexpr int kHfBytes = 4 * 64 * 16;
constexpr int kSmBytes = 4 * 4 * 16;     // sign words of the rotated-basis kernel at d = 128

__device__ void build_wht_frags(uint4* hf) {
  for (int i = threadIdx.x; i < 4 * 64; i += blockDim.x) {
    const int f = i >> 6, l = i & 63, t0 = f & 1, neg = f >> 1;
    const int nn = l & 15, gk = l >> 4;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = 8 * gk + 2 * p + h;               // K index inside the step
        const int par = (__popc(kk & nn) + (((kk >> 4) & 1) & t0) + neg) & 1;
        word |= (par ? 0xBF80u : 0x3F80u) << (16 * h);
      }
      w[p] = word;
    }
    hf[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Adding 2^23 to a float in [0, 2^23) rounds it to an integer held in the low
// mantissa bits: the search-grid cell of y is the bit pattern of
// med3(fma(y, 1/w, half + 2^23), 2^23, 2^23 + ncell - 1) minus that of 2^23.
constexpr float kMagic = 8388608.0f;
constexpr uint32_t kMagicBits = 0x4B000000u;


__device__ void copy_centroids(const CodecTables& t, float* cent) {
  for (int k = threadIdx.x; k <= t.nbound; k += blockDim.x) cent[k] = t.cent[k];
}

// Dequantize at d = 512 on the fp16 matrix cores.  Every centroid as an fp16 high part
// and the fp16 rounding of the rest (22 significant bits), packed (high | low << 16); and the two
// A fragments of the inverse transform: element bits 3, 4, 5 and the two top bits are summed by
// v_mfma_f32_16x16x32_f16 (K index 8 gk + jj: jj holds element bits 3..5, gk the top two; output
// row nn, tile t0: bits 3, 4 = nn >> 2, bit 5 = nn & 1, the top two = (nn >> 1) & 1 and t0), the
// remaining element bits by butterflies over the K steps.  Entries +-1.0 in fp16.
__device__ void build_dq_mr_tables(const CodecTables& t, uint32_t* cpair, uint4* hfd) {
  for (int k = threadIdx.x; k <= t.nbound; k += blockDim.x) {
    const float c = t.cent[k];
    const _Float16 hi = (_Float16)c;
    const _Float16 lo = (_Float16)(c - (float)hi);
    cpair[k] = (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
  }
  for (int i = threadIdx.x; i < 2 * 64; i += blockDim.x) {
    const int t0 = i >> 6, l = i & 63, nn = l & 15, gk = l >> 4;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int jj = 2 * p + h;
        const int par = ((jj & 1) & ((nn >> 2) & 1)) + (((jj >> 1) & 1) & ((nn >> 3) & 1)) + (((jj >> 2) & 1) & (nn & 1)) +
                        ((gk & 1) & ((nn >> 1) & 1)) + (((gk >> 1) & 1) & t0);
        word |= ((par & 1) ? 0xBC00u : 0x3C00u) << (16 * h);
      }
      w[p] = word;
    }
    hfd[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Projection matrix G (m x D bf16) staged in LDS, rows >= m zero.  16-byte chunk c
// of row n is stored at chunk position c ^ (n & SW) so that the 16 rows read by
// one 16-lane group hit 16 different bank groups.
template <int D>
__device__ __forceinline__ int g_swizzle(int n, int c) {
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int SW = CPR < 16 ? CPR - 1 : 15;
  return n * CPR + (c ^ (n & SW));
}

// Rows [row0, row0 + rows) of G into the swizzled LDS buffer gb (rows >= m zero), each
// 16-byte chunk passed through cvt(chunk, sign byte of its 8 columns).  A thread first
// issues BATCH loads, clamped in bounds so that none waits behind a branch, and only then
// converts and stores them: the loads of a batch are in flight together.
template <int D, int BATCH, typename Cvt>
__device__ __forceinline__ void stage_rows(const uint16_t* proj, const uint8_t* signs, int m, int row0, int rows,
                                           uint4* gb, Cvt cvt) {
  constexpr int CPR = D / 8;
  const uint4* src = reinterpret_cast<const uint4*>(proj);
  const int total = rows * CPR, nt = blockDim.x;
  for (int i0 = threadIdx.x; i0 < total; i0 += BATCH * nt) {
    uint4 b[BATCH];
    uint32_t sb[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = min(i0 + u * nt, total - 1);
      const int n = min(row0 + i / CPR, m - 1);
      b[u] = src[n * CPR + i % CPR];
      sb[u] = signs ? signs[i % CPR] : 0u;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = i0 + u * nt;
      if (i < total) {
        const int nl = i / CPR, c = i % CPR;
        gb[g_swizzle<D>(nl, c)] = row0 + nl < m ? cvt(b[u], sb[u]) : make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <int D>
__device__ void stage_projection(const uint16_t* proj, int m, int m_pad, uint4* gl) {
  stage_rows<D, 8>(proj, nullptr, m, 0, m_pad, gl, [](const uint4& b, uint32_t) { return b; });
}

// fp16 copy of a bf16 pair of G scaled by 2^10 (exact for |G| >= 2^-24; the bf16
// mantissa fits in fp16), with the sign of element 2t (2t+1) flipped when bit 2t
// (2t+1) of the sign byte sb is set.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_signed(uint32_t w, uint32_t sb, int t) {
  w ^= (((sb >> (2 * t)) & 1u) << 15) | (((sb >> (2 * t + 1)) & 1u) << 31);
  const _Float16 lo = (_Float16)(bf16_lo(w) * 1024.0f);
  const _Float16 hi = (_Float16)(bf16_hi(w) * 1024.0f);
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// A 16-byte chunk of G (8 columns, whose rotation signs are the bits of sb) as the same
// columns of G D in fp16, scaled by 2^10.  Byte c of the sign mask covers columns 8c..8c+7.
__device__ __forceinline__ uint4 gd_f16(const uint4& b, uint32_t sb) {
  return make_uint4(bf16x2_to_f16x2_signed(b.x, sb, 0), bf16x2_to_f16x2_signed(b.y, sb, 1),
                    bf16x2_to_f16x2_signed(b.z, sb, 2), bf16x2_to_f16x2_signed(b.w, sb, 3));
}
__device__ __forceinline__ uint4 gd_chunk_f16(const uint4* src, const uint8_t* signs, int cpr, int n, int c) {
  return gd_f16(src[n * cpr + c], signs[c]);
}

template <int D, bool G_LDS>
__device__ __forceinline__ f16x8 load_gfrag_f16(const uint4* gl, const uint16_t* proj, const uint8_t* signs, int m,
                                                int row, int col8) {
  uint4 w;
  if constexpr (G_LDS) {
    w = gl[g_swizzle<D>(row, col8)];
  } else {
    w = make_uint4(0, 0, 0, 0);
    if (row < m) w = gd_chunk_f16(reinterpret_cast<const uint4*>(proj), signs, D / 8, row, col8);
  }
  return __builtin_bit_cast(f16x8, w);
}

template <int D, bool G_LDS>
__device__ __forceinline__ bf16x8 load_gfrag(const uint4* gl, const uint16_t* proj, int m, int row, int col8) {
  uint4 w;
  if constexpr (G_LDS) {
    w = gl[g_swizzle<D>(row, col8)];
  } else {
    w = make_uint4(0, 0, 0, 0);
    if (row < m) w = reinterpret_cast<const uint4*>(proj)[row * (D / 8) + col8];
  }
  return __builtin_bit_cast(bf16x8, w);
}

// Sign bits of four 16-column N tiles nt0 .. nt0+3 of G x for 16 blocks (or keys), from
// MFMAs with G rows as the A operand and the 16 blocks as B: acc[q][i] of lane
// (block r, quarter gg) is p[r][16 (nt0 + q) + 4 gg + i].  A bit is p > 0, read off the
// fp32 pattern as med3(int, 0, 1) (+0 and -0 give 0).  Lane quarter gg builds byte q of
// its word from its 4 bits (nibble gg of the 16-bit chunk of N tile nt0 + q); one
// permlane16 swap pairs quarters (0,1) and (2,3) into the even and odd output bytes,
// one permlane32 swap brings both to every quarter, and two byte permutes interleave
// them.  Returns the 8 output bytes (bits 64 (nt0/4) .. +63, LSB first) in every lane
// of block r.
// Byte q (low nibble) of the word: the four bits of N tile nt0 + q held by this lane.
__device__ __forceinline__ uint32_t sign_nibble(const f32x4& acc, int q) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = __float_as_int(acc[i]);
    x |= (uint32_t)min(max(v, 0), 1) << (8 * q + i);
  }
  return x;
}

__device__ __forceinline__ uint2 sign_bytes_of(uint32_t x) {
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t z = a[0] | (a[1] << 4);          // quarters (0,1): even bytes, (2,3): odd bytes
  const auto b = __builtin_amdgcn_permlane32_swap(z, z, false, false);
  const uint32_t E = b[0], O = b[1];
  return make_uint2(__builtin_amdgcn_perm(O, E, 0x05010400u), __builtin_amdgcn_perm(O, E, 0x07030602u));
}

__device__ __forceinline__ uint2 sign_bytes4(const f32x4 (&acc)[4]) {
  return sign_bytes_of(sign_nibble(acc[0], 0) | sign_nibble(acc[1], 1) | sign_nibble(acc[2], 2) |
                       sign_nibble(acc[3], 3));
}

// Lane quarter 0 of block row r writes the 8 bytes at byte 2 nt0 of that row (fewer at
// the end of a row of mb bytes).
__device__ __forceinline__ void store_sign_bytes(uint2 w, int lane, int64_t row0, int64_t nrows, uint8_t* bits,
                                                 int mb, int nt0) {
  const int64_t row = row0 + (lane & 15);
  const int byte0 = 2 * nt0;
  if ((lane >> 4) != 0 || row >= nrows) return;
  uint8_t* dst = bits + row * (int64_t)mb + byte0;
  if ((mb & 7) == 0 && byte0 + 8 <= mb) {
    *reinterpret_cast<uint2*>(dst) = w;
  } else {
    for (int j = 0; j < 8 && byte0 + j < mb; ++j) dst[j] = (uint8_t)((j < 4 ? w.x : w.y) >> (8 * (j & 3)));
  }
}

// Inverse of cperm (a permutation of register-index bits), in closed form so that it folds
// to a constant inside unrolled loops.
template <int D>
__host__ __device__ constexpr int cperm_inv(int o) {
  return D == 256 ? ((o & 7) | (((o >> 5) & 1) << 3) | (((o >> 3) & 1) << 4) | (((o >> 4) & 1) << 5))
       : D == 512 ? ((o & 7) | (((o >> 5) & 1) << 3) | (((o >> 6) & 1) << 4) | (((o >> 3) & 1) << 5) |
                     (((o >> 4) & 1) << 6))
                  : o;
}

// ------------------------------------------------------------------------------------------
// Quantize (+ optional QJL residual stage)
// ------------------------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D, bool IN_BF16>
__device__ __forceinline__ void load_tile(uint4 (&raw)[IN_BF16 ? D / 32 : D / 16], const void* x, int64_t T,
                                          int64_t n_blocks, int64_t full_tiles, int r, int g) {
  constexpr int NR = IN_BF16 ? D / 32 : D / 16;
  const int64_t blk = T * 16 + r;
  const uint4* src = IN_BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + blk * D)
                             : reinterpret_cast<const uint4*>(static_cast<const float*>(x) + blk * D);
  // lane-quarter g reads elements 32 s + 8 g .. +8 (16 bytes of bf16, 32 of fp32)
  auto idx = [&](int i) { return IN_BF16 ? 4 * i + g : 8 * (i >> 1) + 2 * g + (i & 1); };
  // streamed once: non-temporal loads keep the caches for the tables
  auto ld = [&](int i) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + idx(i));
    return make_uint4(w.x, w.y, w.z, w.w);
  };
  if (T < full_tiles) {                       // uniform: every row of the tile exists
#pragma unroll
    for (int i = 0; i < NR; ++i) raw[i] = ld(i);
  } else {
    const bool valid = blk < n_blocks;
#pragma unroll
    for (int i = 0; i < NR; ++i) raw[i] = valid ? ld(i) : make_uint4(0, 0, 0, 0);
  }
}


// x0 s0 + x1 s1 for bf16 pairs x = (x0, x1), s = (s0, s1): the three-operand form of
// v_dot2_f32_bf16 with an inline zero addend (the builtin is lowered to the accumulating
// two-operand form, which needs the zero moved into the destination first).
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t s) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(s));
  return r;
}

// Two fp32 values -> packed fp16 high parts (round to nearest even).
__device__ __forceinline__ uint32_t split_hi_f16x2(float x0, float x1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 h = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, h);
}
// Low parts fp16(x - hi): v_fma_mix computes x - hi exactly from the fp16 hi and
// the fp32 x and rounds once to fp16, writing the low or the high half.
__device__ __forceinline__ uint32_t split_lo_f16x2(uint32_t hp, float x0, float x1) {
  uint32_t lo;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lo) : "v"(hp), "v"(x0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(lo) : "v"(hp), "v"(x1));
  return lo;
}

// A d/8-byte sign mask read as D/32 dwords (the grouped calls require 4-byte aligned masks), and
// byte i of it.
template <int D>
struct SignWords {
  uint32_t w[D / 32];
  __device__ __forceinline__ void load(const uint8_t* signs) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) w[i] = reinterpret_cast<const uint32_t*>(signs)[i];
  }
  // byte 4 dw + g (dw a compile-time index, g = 0..3 the lane quarter)
  __device__ __forceinline__ uint32_t byte(int dw, int g) const { return (w[dw] >> (8 * g)) & 0xffu; }
};

// Bit-packed code runs: a lane's run of codes is a little-endian bit stream of B bits per
// code.  NB bytes of it move as the widest accesses the run's alignment allows (a run starts
// at a multiple of NB bytes).
template <int NB>
__device__ __forceinline__ void store_code_bytes(uint8_t* dst, const uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i)
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (NB % 8 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) reinterpret_cast<uint2*>(dst)[i] = make_uint2(w[2 * i], w[2 * i + 1]);
  } else if constexpr (NB % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) reinterpret_cast<uint32_t*>(dst)[i] = w[i];
  } else {
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
  }
}
template <int NB>
__device__ __forceinline__ void load_code_bytes(const uint8_t* src, bool valid, uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4 x = valid ? reinterpret_cast<const uint4*>(src)[i] : make_uint4(0, 0, 0, 0);
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  } else if constexpr (NB % 8 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) {
      const uint2 x = valid ? reinterpret_cast<const uint2*>(src)[i] : make_uint2(0, 0);
      w[2 * i] = x.x; w[2 * i + 1] = x.y;
    }
  } else if constexpr (NB % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) w[i] = valid ? reinterpret_cast<const uint32_t*>(src)[i] : 0u;
  } else {
#pragma unroll
    for (int i = 0; i < (NB + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < NB / 2; ++i)
      w[i >> 1] |= (uint32_t)(valid ? reinterpret_cast<const uint16_t*>(src)[i] : 0) << (16 * (i & 1));
  }
}
// Code j of a B-bit stream held in dwords (B <= 8; a code may straddle two dwords).
template <int B, int N>
__device__ __forceinline__ uint32_t stream_code(const uint32_t (&w)[N], int j) {
  const int pos = B * j, k = pos >> 5, sh = pos & 31;
  uint32_t c = w[k] >> sh;
  if (sh + B > 32) c |= w[k + 1] << (32 - sh);
  return c & ((1u << B) - 1u);
}

// MODE: 0 = search grid stored once, 1 = replicated per lane of a 16-lane LDS group,
// 2 = codes bit-packed, the grid's replication read from the tables at run time
// RB: the QJL projection runs in the rotated basis, p = G r = (G D H) rho / d, from rows of
// G D H staged in LDS as fp16 high and low fragments (no inverse transform of the residual)
template <int D, bool IN_BF16, bool QJL, bool G_LDS, int MODE, bool RB = false>
struct Quantizer {
  static constexpr bool REP = MODE == 1;
  static constexpr bool PK = MODE == 2;
  static constexpr int E = D / 4;
  static constexpr int KS = D / 32;                         // MFMA K steps per block
  static constexpr int NR = IN_BF16 ? D / 32 : D / 16;      // 16-byte loads per lane per tile
  static constexpr uint32_t kRepShift = REP ? 8u : 4u;      // log2(bytes per cell)

  // d = 128 bf16 blocks (without a projection, or with the rotated-basis one): the rotation on
  // the bf16 matrix cores (the products x_k D_k H(k, n) are exact; only the fp32 sums round)
  static constexpr bool MR = IN_BF16 && ((D == 128 && (!QJL || RB)) || D == 256);
  // d = 256: the result is moved to the contiguous layout of the butterflies (MRT), so that
  // the codes, the inverse transform of the residual and the projections stay as they are
  static constexpr bool MRT = MR && D == 256;

  const pqi::QuantArgs& a;
  const unsigned char* smem;
  const uint4* gl;
  const uint4* hf = nullptr;          // the Walsh-Hadamard fragments in LDS (MR)
  // rotation signs of this lane's element pairs: per pair, the sign bits of its two elements
  // (bits 15 and 31: ORed with a bf16 scale in both halves they make the +-rscale pair of the
  // first butterfly; for fp32 input they flip the values directly); for d = 512 only the sign
  // bytes (elements 32 s + 8 g .. +7) are held and the pairs are formed when used, which keeps
  // 48 registers free
  static constexpr bool kCompactSigns = D == 512;
  // the rotated-basis kernel on the matrix cores keeps the sign words in LDS instead (sml:
  // [quarter g][K step s] as 16 bytes, the xor masks of chunk s of the load layout)
  static constexpr bool SM_LDS = MR && QJL && RB;
  uint32_t smask[SM_LDS ? 1 : (kCompactSigns ? D / 32 : E / 2)];
  const uint4* sml = nullptr;
  int lane, r, g, m, m_pad, mb;
  float inv_w, offM, topM, inv_sqrt_d;
  uint32_t lane_off, rep_shift;
  // the tensor being quantized: codes and norms out, its block count (retarget() switches)
  uint8_t* codes;
  uint16_t* norms;
  int64_t n_blocks;

  // pair p holds elements load_e(g, 2p) and +1: bits 2 (p & 3) and 2 (p & 3) + 1 of sign
  // byte 4 (p >> 2) + g
  __device__ __forceinline__ void load_signs(const uint8_t* signs) {
    if constexpr (kCompactSigns) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) smask[s] = signs[4 * s + g];
    } else {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const uint32_t b = signs[4 * s + g];
#pragma unroll
        for (int t = 0; t < 4; ++t) smask[4 * s + t] = (((b >> (2 * t)) & 1u) << 15) | (((b >> (2 * t + 1)) & 1u) << 31);
      }
    }
  }

  // another tensor of the same codec (grouped calls): its signs (loaded ahead), outputs and
  // block count
  __device__ __forceinline__ void retarget(const SignWords<D>& sw, uint8_t* c, uint16_t* nm, int64_t nb) {
    if constexpr (kCompactSigns) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) smask[s] = sw.byte(s, g);
    } else {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const uint32_t b = sw.byte(s, g);
#pragma unroll
        for (int t = 0; t < 4; ++t) smask[4 * s + t] = (((b >> (2 * t)) & 1u) << 15) | (((b >> (2 * t + 1)) & 1u) << 31);
      }
    }
    codes = c;
    norms = nm;
    n_blocks = nb;
  }

  __device__ Quantizer(const pqi::QuantArgs& args, const unsigned char* sm, const uint4* g_lds)
      : a(args), smem(sm), gl(g_lds) {
    lane = threadIdx.x & 63;
    r = lane & 15;
    g = lane >> 4;
    m = a.m;
    m_pad = (m + 15) & ~15;
    mb = m >> 3;
    codes = a.codes;
    norms = a.norms;
    n_blocks = a.n_blocks;
    if (a.signs && !SM_LDS) load_signs(a.signs);
    inv_w = a.t.cell_inv_w;
    offM = (float)a.t.half + kMagic;
    topM = kMagic + (float)(a.t.ncell - 1);
    inv_sqrt_d = 1.0f / sqrtf((float)D);
    const bool rep = PK ? a.t.nrep == 16 : REP;
    rep_shift = PK ? (rep ? 8u : 4u) : kRepShift;
    lane_off = (rep ? 16u * (uint32_t)(lane & 15) : 0u) - (kMagicBits << rep_shift);
  }

  // Codes and norm of the tile's 16 blocks (stored), and with the QJL stage the residual
  // norm (stored) and the rotated residual left in v, scaled by a power of two.

  // the value described above for element pair p (registers 2p, 2p+1 of the load layout)
  __device__ __forceinline__ uint32_t sgn(int p) const {
    if constexpr (kCompactSigns) {
      const uint32_t b = (smask[p >> 2] >> (2 * (p & 3))) & 3u;
      return ((b & 1u) << 15) | ((b & 2u) << 30);
    } else {
      return smask[p];
    }
  }

  // v = H (D x) for the 16 blocks of a tile of bf16 input on the matrix cores (MR): the signs D
  // flip the input's sign bits (then addw raises the exponent fields of both bf16 halves), the
  // B operand of K step s is chunk s of the load layout (lane
  // (r, g): elements 32 s + 8 g + 0..7 of block r), and output tile t leaves coordinate
  // 16 t + 4 g + i of block r in register 4 t + i.  With MRT the two top bits of t are then
  // exchanged with the lane bits 4 and 5 and the registers renamed: the contiguous layout.
  __device__ __forceinline__ void rotate_mfma(const uint4 (&w)[NR], float (&v)[E], uint32_t addw = 0) const {
    constexpr int KSM = D / 32, MT = D / 16;
    bf16x8 b[KSM];
#pragma unroll
    for (int s = 0; s < KSM; ++s) {
      uint4 sm;
      if constexpr (SM_LDS) sm = sml[g * KSM + s];
      else sm = make_uint4(sgn(4 * s), sgn(4 * s + 1), sgn(4 * s + 2), sgn(4 * s + 3));
      b[s] = __builtin_bit_cast(bf16x8, make_uint4((w[s].x ^ sm.x) + addw, (w[s].y ^ sm.y) + addw,
                                                   (w[s].z ^ sm.z) + addw, (w[s].w ^ sm.w) + addw));
    }
    f32x4 acc[MT];
    // one fragment live at a time: fragment f serves the (s, t) with t & 1 = f & 1 and
    // popcount(s & (t >> 1)) odd exactly when f > 1; s = 0 comes first for every t
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, hf[f * 64 + lane]);
#pragma unroll
      for (int s = 0; s < KSM; ++s)
#pragma unroll
        for (int t = f & 1; t < MT; t += 2)
          if ((__builtin_popcount(s & (t >> 1)) & 1) == (f >> 1))
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h, b[s], s == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[t],
                                                              0, 0, 0);
    }
    if constexpr (MRT) {
      constexpr int L = Log2<E>::v;
      float u[E];
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) u[4 * t + i] = acc[t][i];
      xch16<E, L - 2>(u);
      xch32<E, L - 1>(u);
      // register j now holds offset (j & 3) + 4 (bit L-2) + 8 (bit L-1) + 16 (bits 2..L-3) of
      // the lane's run; the contiguous layout keeps offset o in register cperm_inv(o)
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int o = (j & 3) | (((j >> (L - 2)) & 1) << 2) | (((j >> (L - 1)) & 1) << 3) |
                      (((j >> 2) & ((1 << (L - 4)) - 1)) << 4);
        v[cperm_inv<D>(o)] = u[j];
      }
    } else {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * t + i] = acc[t][i];
    }
  }

  // The code words of the matrix-core layout (word t: codes of coordinates 16 t + 4 g + 0..3)
  // to the contiguous layout (word w: codes 32 g + 4 w + 0..3): a 4 x 4 transpose of word pairs
  // over the block's four lanes, lane bit 4 with word bit 1 and lane bit 5 with word bit 2,
  // then a renaming of the words.
  __device__ __forceinline__ void codes_to_runs(uint32_t (&cw)[E / 4]) const {
    static_assert(E == 32, "d = 128 only");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & 2) continue;
      auto x = __builtin_amdgcn_permlane16_swap(cw[j], cw[j | 2], false, false);
      cw[j] = x[0];
      cw[j | 2] = x[1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & 4) continue;
      auto x = __builtin_amdgcn_permlane32_swap(cw[j], cw[j | 4], false, false);
      cw[j] = x[0];
      cw[j | 4] = x[1];
    }
    uint32_t o[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) o[w] = cw[((w >> 2) & 1) | ((w & 1) << 1) | (((w >> 1) & 1) << 2)];
#pragma unroll
    for (int w = 0; w < 8; ++w) cw[w] = o[w];
  }

  __device__ __forceinline__ void decide(const uint4 (&raw)[NR], int64_t T, float (&v)[E]) {
    const int64_t blk = T * 16 + r;
    const bool valid = blk < n_blocks;
    // The block norm comes first, from the raw values, so that the rotation can run on x scaled
    // by rscale = 2^e (a power of two that brings n into [1, 2)): for bf16 input the scale rides
    // on the +-1 sign pairs of the first butterfly (exact products), so z' = rscale H (D x)
    // needs no per-element rescale, and the residual z' - rscale n16 c sits near 1 for the
    // fp16 split of the QJL stage.
    float ss;
    if constexpr (IN_BF16) {
      typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
      float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x2 x = __builtin_bit_cast(bf16x2, w[u]);
          sq[u] = __builtin_amdgcn_fdot2_f32_bf16(x, x, sq[u], false);
        }
      }
      ss = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    } else {
      float sq[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sq[i] = 0.0f;
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const uint32_t f[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) sq[(4 * s + t) & 7] = fmaf(__uint_as_float(f[t]), __uint_as_float(f[t]), sq[(4 * s + t) & 7]);
      }
      ss = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
    }
    ss = sum4(ss);
    float n = sqrtf(ss);
    uint16_t n16 = f32_to_f16(n);
    // e in [-126, 126]: blocks with a norm below 2^-126 keep the largest scale that stays finite
    int e = n > 0.0f ? min(max(-ilogbf(n), -126), 126) : 0;
    [[maybe_unused]] float nr_far = -1.0f;
    if constexpr (!MR) {
      // a norm outside [2^-60, 2^61): the sum of squares may have left the fp32 range, so it is
      // taken again from the entries scaled by 2^-k, k the exponent of the block's largest entry
      // (the four lanes of a block take this branch together)
      if (!(ss >= 0x1p-120f && ss < 0x1p122f)) {
        auto ent = [&](int i) {          // entry i of this lane, i < 4 NR (fp32) or 8 NR (bf16)
          const uint4& q = raw[IN_BF16 ? i >> 3 : i >> 2];
          const int w = IN_BF16 ? (i >> 1) & 3 : i & 3;
          const uint32_t x = w == 0 ? q.x : w == 1 ? q.y : w == 2 ? q.z : q.w;
          return IN_BF16 ? ((i & 1) ? bf16_hi(x) : bf16_lo(x)) : __uint_as_float(x);
        };
        constexpr int NE = IN_BF16 ? 8 * NR : 4 * NR;
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < NE; ++i) mx = fmaxf(mx, fabsf(ent(i)));
        mx = max4(mx);
        const int k = mx > 0.0f ? ilogbf(mx) : 0;
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
          const float t = ldexpf(ent(i), -k);
          sq = fmaf(t, t, sq);
        }
        const float nq = sqrtf(sum4(sq));
        n = ldexpf(nq, k);
        n16 = f32_to_f16(n);
        e = nq > 0.0f ? min(max(-(ilogbf(nq) + k), -126), 126) : 0;
        nr_far = ldexpf(nq, k + e);      // n 2^e without leaving the fp32 range
      }
    }
    const float rscale = __uint_as_float((uint32_t)(127 + e) << 23);
    // On the matrix cores (MR) a block whose norm lies in [2^-60, 2^12) (without the QJL stage
    // [2^-60, 2^61)) goes in scaled by 2^es, es = max(e, 0): for e > 0 the exponent fields of its
    // bf16 entries are raised by e (the same integer add that follows the sign flip; exact for
    // normal entries, since no entry exceeds the norm, and a zero or subnormal entry becomes at
    // most 2^-66 of the scaled norm).  No product or sum can then leave the fp32 range, and the
    // QJL residual (at most 9 n per coordinate) stays inside the fp16 range for the split.
    // Other blocks (a sum of squares that underflowed or overflowed included) go in scaled by
    // 2^-k, k the exponent of their largest entry, rounded to bf16, with their norm taken again
    // from the scaled entries.  es is the exponent of the scale v carries.
    constexpr float kSsHi = QJL ? 0x1p24f : 0x1p122f;
    const bool pre = MR && !(ss >= 0x1p-120f && ss < kSsHi);
    float nr = nr_far >= 0.0f ? nr_far : n * rscale;             // the norm on v's axis
    float nsc = f16_to_f32(n16) * rscale;                         // the stored norm, on v's axis
    [[maybe_unused]] int es = e;
    [[maybe_unused]] uint32_t addw = 0;                           // exponent raise of both halves
    [[maybe_unused]] uint4 w[MR ? NR : 1];
    if constexpr (MR) {
#pragma unroll
      for (int i = 0; i < NR; ++i) w[i] = raw[i];
      es = max(e, 0);
      const float sc = __uint_as_float((uint32_t)(127 + es) << 23);
      nr = n * sc;
      nsc = f16_to_f32(n16) * sc;
      addw = (uint32_t)es * 0x00800080u;
      if (pre) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const uint32_t q[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(q[u])), fabsf(bf16_hi(q[u]))));
        }
        mx = max4(mx);                     // the block's four lanes take this branch together
        const int k = mx > 0.0f ? ilogbf(mx) : 0;
        auto sc2 = [&](uint32_t x) { return pack_bf16x2(ldexpf(bf16_lo(x), -k), ldexpf(bf16_hi(x), -k)); };
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          w[i] = make_uint4(sc2(w[i].x), sc2(w[i].y), sc2(w[i].z), sc2(w[i].w));
          const uint32_t q[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) sq = fmaf(bf16_lo(q[u]), bf16_lo(q[u]), fmaf(bf16_hi(q[u]), bf16_hi(q[u]), sq));
        }
        const float nq = sqrtf(sum4(sq));  // the norm of the scaled block
        n = ldexpf(nq, k);
        n16 = f32_to_f16(n);
        nr = nq;
        nsc = ldexpf(f16_to_f32(n16), -k);
        es = -k;
        addw = 0;
      }
    }
    // scaled coordinate -> grid cells (a guess of the cell, the decision below is exact: a
    // one-ulp reciprocal moves only values within an ulp of a cell edge to the neighbouring
    // cell, whose entry decides them the same way unless a boundary sits on that edge)
    const float a_w = nr > 0.0f ? inv_w * __builtin_amdgcn_rcpf(nr) : 0.0f;

    if constexpr (MR) {
      rotate_mfma(w, v, addw);             // v = 2^es H (D x)
    } else if constexpr (IN_BF16) {
      // signs, bf16 -> fp32, the scale and the first butterfly (register bit 0 pairs the two
      // halves of a word) in two dot products per pair: (x0 D0 + x1 D1, x0 D0 - x1 D1) rscale
      const uint32_t scw = ((uint32_t)(127 + e) << 7) * 0x10001u;   // bf16 rscale in both halves
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int p = 4 * s + u;
          const uint32_t sp = sgn(p) | scw;
          v[2 * p] = dot2_bf16(w[u], sp);
          v[2 * p + 1] = dot2_bf16(w[u], sp ^ 0x80000000u);
        }
      }
      wht_forward<D, false>(v);            // v = z' = rscale H (D x)
    } else {
#pragma unroll
      for (int s = 0; s < NR / 2; ++s) {
        const uint32_t f[8] = {raw[2 * s].x, raw[2 * s].y, raw[2 * s].z, raw[2 * s].w,
                               raw[2 * s + 1].x, raw[2 * s + 1].y, raw[2 * s + 1].z, raw[2 * s + 1].w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t sp = sgn(4 * s + t / 2);
          const uint32_t sm = (t & 1) ? (sp & 0x80000000u) : (sp << 16);
          v[8 * s + t] = __uint_as_float(f[t] ^ sm) * rscale;
        }
      }
      wht_forward<D>(v);                   // v = z' = rscale H (D x)
    }

    // code: y = z' / nr lies above boundary beta exactly when z' - beta nr > 0 (one fma, one
    // rounding); the grid cell comes from z' a_w; with the QJL stage the scaled residual
    // rho = z' - rscale n16 c[code] (= rscale H D r) replaces z' in v
    uint32_t cw[E / 4];
#pragma unroll
    for (int w = 0; w < E / 4; ++w) cw[w] = 0;
    // PQ_LOOKUP_BATCH grid lookups in flight: a batch issues all its LDS reads before it reads
    // the first of them (bounds the registers the scheduler may tie up)
    constexpr int LB = QJL ? (D <= 128 ? PQ_LOOKUP_BATCH_QJL : 2 * PQ_LOOKUP_BATCH_QJL) : PQ_LOOKUP_BATCH;
    using TE = typename std::conditional<QJL, u32x4, u32x2>::type;
#pragma unroll
    for (int j0 = 0; j0 < E; j0 += LB) {
      TE te[LB];
#pragma unroll
      for (int jj = 0; jj < LB; ++jj) {
        const float u = __builtin_amdgcn_fmed3f(fmaf(v[j0 + jj], a_w, offM), kMagic, topM);
        const uint32_t addr = (__float_as_uint(u) << (PK ? rep_shift : kRepShift)) + lane_off;
        te[jj] = *static_cast<const TE*>(__builtin_assume_aligned(smem + addr, sizeof(TE)));
      }
#pragma unroll
      for (int jj = 0; jj < LB; ++jj) {
        const int j = j0 + jj;
        asm("" : "+v"(te[jj]));            // keep the cell as one LDS read of the whole entry
        uint32_t code;
        if constexpr (QJL) {
          const bool gt = fmaf(-__uint_as_float(te[jj].x), nr, v[j]) > 0.0f;
          code = te[jj].y + (gt ? 1u : 0u);
          const float c = __uint_as_float(gt ? te[jj].w : te[jj].z);
          v[j] = fmaf(-nsc, c, v[j]);
          asm volatile("" : "+v"(v[j]));   // keep the residual next to its lookup
        } else {
          code = te[jj].y + (fmaf(-__uint_as_float(te[jj].x), nr, v[j]) > 0.0f ? 1u : 0u);
        }
        const int o = cperm<D>(j);
        cw[o >> 2] |= code << (8 * (o & 3));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // materialise the packed codes here: otherwise the whole decision chain sinks into
    // the store branch below and keeps every lookup result live until then
#pragma unroll
    for (int w = 0; w < E / 4; ++w) asm volatile("" : "+v"(cw[w]));
    if constexpr (MR && !MRT) codes_to_runs(cw);
    if constexpr (PK) {
      // bit-packed codes: the lane's run of E codes is E pbits / 8 contiguous bytes
      switch (a.pbits) {
        case 1: store_packed<1>(cw, blk, valid); break;
        case 2: store_packed<2>(cw, blk, valid); break;
        case 3: store_packed<3>(cw, blk, valid); break;
        case 4: store_packed<4>(cw, blk, valid); break;
        case 5: store_packed<5>(cw, blk, valid); break;
        case 6: store_packed<6>(cw, blk, valid); break;
        default: store_packed<7>(cw, blk, valid); break;
      }
      if (valid && g == 0) norms[blk] = n16;
    } else if constexpr (D == 128) {
      // a block's codes are one 128-byte line, two 16-byte pieces per lane: the neighbouring
      // blocks r & ~1 and r | 1 (lanes l, l ^ 1) trade pieces so that each store writes
      // whole lines (half-line stores reach HBM as partial lines)
      const bool odd = r & 1;
      const int64_t blk_e = T * 16 + (r & ~1);
      u32x4 x, y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(odd ? cw[i] : cw[4 + i]), 0xB1, 0xF, 0xF, true);
        x[i] = odd ? recv : cw[i];
        y[i] = odd ? cw[4 + i] : recv;
      }
      u32x4* dst = reinterpret_cast<u32x4*>(codes + blk_e * D + E * qpos<D>(g) + (odd ? 16 : 0));
      if (blk_e < n_blocks) dst[0] = x;
      if (blk_e + 1 < n_blocks) dst[D / 16] = y;
      if (valid && g == 0) norms[blk] = n16;
    } else if (valid) {
      uint4* dst = reinterpret_cast<uint4*>(codes + blk * D + E * qpos<D>(g));
#pragma unroll
      for (int w = 0; w < E / 16; ++w)
        dst[w] = make_uint4(cw[4 * w + 0], cw[4 * w + 1], cw[4 * w + 2], cw[4 * w + 3]);
      if (g == 0) norms[blk] = n16;
    }

    if constexpr (QJL) {
      const float rss = sum4(tree_sumsq<E>(v));
      // ||r|| = ||H D r|| / sqrt(d); the product with 2^-e is the exact quotient by rscale
      const float rn = MR ? ldexpf(sqrtf(rss) * inv_sqrt_d, -es)
                          : sqrtf(rss) * __uint_as_float((uint32_t)(127 - e) << 23) * inv_sqrt_d;
      if (valid && g == 0) a.rnorms[blk] = f32_to_f16(rn);
    }
  }

  // The lane's E byte codes (cw, run order) packed at B bits each and stored at their place
  // in the block's bit stream: the run starts E qpos(g) codes into the block.
  template <int B>
  __device__ __forceinline__ void store_packed(const uint32_t (&cw)[E / 4], int64_t blk, bool valid) {
    constexpr int NB = E * B / 8;                         // packed bytes of the run
    uint32_t pw[(NB + 3) / 4];
#pragma unroll
    for (int i = 0; i < (NB + 3) / 4; ++i) pw[i] = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t c = (cw[i >> 2] >> (8 * (i & 3))) & 0xffu;
      const int pos = B * i, k = pos >> 5, sh = pos & 31;
      pw[k] |= c << sh;
      if (sh + B > 32) pw[k + 1] |= c >> (32 - sh);
    }
    if (valid) store_code_bytes<NB>(codes + blk * (D * B / 8) + E * qpos<D>(g) * B / 8, pw);
  }

  // The rotated residual back in the block's coordinates, w = H rho = d D r (times the
  // power-of-two scale), split into fp16 high and low parts (22 significant bits) as MFMA
  // B fragments: register chunk k of quarter g holds columns 8 res_col8(g, k) + 0..7.
  // The signs D are folded into the staged copy of G, so the products give a positive
  // multiple of G r.
  __device__ __forceinline__ void residual_frags(const float (&v)[E], u32x4 (&ahi)[KS], u32x4 (&alo)[KS]) {
    float w[E];
#pragma unroll
    for (int i = 0; i < E; ++i) w[i] = v[cperm_inv<D>(i)];
    wht_dequant<D>(w);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x0 = w[8 * k + 2 * t], x1 = w[8 * k + 2 * t + 1];
        const uint32_t hp = split_hi_f16x2(x0, x1);
        ahi[k][t] = hp;
        alo[k][t] = split_lo_f16x2(hp, x0, x1);
      }
    }
  }

  // The scaled rotated residual (registers in run order) split into fp16 high and low parts
  // (22 significant bits) as MFMA B fragments: K step k takes registers 8 k .. 8 k + 7.
  __device__ __forceinline__ void rotated_frags(const float (&v)[E], u32x4 (&bhi)[KS], u32x4 (&blo)[KS]) const {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x0 = v[8 * k + 2 * t], x1 = v[8 * k + 2 * t + 1];
        const uint32_t hp = split_hi_f16x2(x0, x1);
        bhi[k][t] = hp;
        blo[k][t] = split_lo_f16x2(hp, x0, x1);
      }
    }
  }

  // Rows of G D H into LDS for the rotated-basis projection: row i of G D H is H (D g_i), the
  // transform decide() applies to a block, so a wave takes 16 rows of G at a time as a tile of
  // blocks (rows >= m are zero), applies the signs and the forward transform (no scale), and
  // stores register chunk k of each lane as fragment (row tile, k, lane), high parts first, then
  // the low parts: the same element order as the residual fragments.
  __device__ void stage_rotated(uint4* gp, int wv, int waves) const {
    const int nt = m_pad >> 4;
    uint4* glo = gp + (size_t)nt * KS * 64;
    for (int rt = wv; rt < nt; rt += waves) {
      uint4 raw[D / 32];
      load_tile<D, true>(raw, a.proj, rt, m, m >> 4, r, g);
      float v[E];
      if constexpr (MR) {
        rotate_mfma(raw, v);
        u32x4 hi[KS], lo[KS];
        rotated_frags(v, hi, lo);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          gp[((size_t)rt * KS + k) * 64 + lane] = make_uint4(hi[k][0], hi[k][1], hi[k][2], hi[k][3]);
          glo[((size_t)rt * KS + k) * 64 + lane] = make_uint4(lo[k][0], lo[k][1], lo[k][2], lo[k][3]);
        }
        continue;
      }
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int p = 4 * s + u;
          const uint32_t sp = sgn(p) | 0x3F803F80u;           // +-1.0 pairs
          v[2 * p] = dot2_bf16(w[u], sp);
          v[2 * p + 1] = dot2_bf16(w[u], sp ^ 0x80000000u);
        }
      }
      wht_forward<D, false>(v);
      u32x4 hi[KS], lo[KS];
      rotated_frags(v, hi, lo);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        gp[((size_t)rt * KS + k) * 64 + lane] = make_uint4(hi[k][0], hi[k][1], hi[k][2], hi[k][3]);
        glo[((size_t)rt * KS + k) * 64 + lane] = make_uint4(lo[k][0], lo[k][1], lo[k][2], lo[k][3]);
      }
    }
  }

  // Sign bits of G r from the scaled rotated residual: three products per K step (high x high,
  // high x low, low x high) against the staged rows of G D H; the positive factors rscale / d
  // do not change a sign.  Output layout as in project().
  __device__ __forceinline__ void project_rotated(const u32x4 (&bhi)[KS], const u32x4 (&blo)[KS], int64_t T) {
    const int nt = m_pad >> 4;
    const uint4* glo = gl + (size_t)nt * KS * 64;
    for (int nt0 = 0; nt0 < nt; nt0 += 4) {
      f32x4 acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (nt0 + q < nt) {
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            const f16x8 ah = __builtin_bit_cast(f16x8, gl[((size_t)(nt0 + q) * KS + k) * 64 + lane]);
            const f16x8 al = __builtin_bit_cast(f16x8, glo[((size_t)(nt0 + q) * KS + k) * 64 + lane]);
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(f16x8, bhi[k]), acc[q], 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(f16x8, blo[k]), acc[q], 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, __builtin_bit_cast(f16x8, bhi[k]), acc[q], 0, 0, 0);
          }
        }
      }
      store_sign_bytes(sign_bytes4(acc), lane, T * 16, n_blocks, a.qbits, mb, nt0);
    }
  }

  // The rotated residual back in the block's coordinates, unsplit (see residual_frags).
  __device__ __forceinline__ void residual_block(float (&v)[E]) {
    float w[E];
#pragma unroll
    for (int i = 0; i < E; ++i) w[i] = v[cperm_inv<D>(i)];
    wht_dequant<D>(w);
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = w[i];
  }

  // Sign bits of N tiles [nt_begin, nt_end) (nt_begin a multiple of 4).  G rows come from
  // the LDS buffer gb, whose row 0 is row row0 of G, or (without LDS) from global memory.
  template <bool FROM_LDS>
  __device__ __forceinline__ void project(const u32x4 (&ahi)[KS], const u32x4 (&alo)[KS], int64_t T,
                                          const uint4* gb, int row0, int nt_begin, int nt_end) {
    for (int nt0 = nt_begin; nt0 < nt_end; nt0 += 4) {
      f32x4 acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (nt0 + 4 <= nt_end) {
        // four N tiles: their products interleaved, so that no product waits for the one before
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          f16x8 b[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = 16 * (nt0 + q) + r;
            if constexpr (FROM_LDS) b[q] = __builtin_bit_cast(f16x8, gb[g_swizzle<D>(row - row0, res_col8<D>(g, k))]);
            else b[q] = load_gfrag_f16<D, false>(gb, a.proj, a.signs, m, row, res_col8<D>(g, k));
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[q], __builtin_bit_cast(f16x8, ahi[k]), acc[q], 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[q], __builtin_bit_cast(f16x8, alo[k]), acc[q], 0, 0, 0);
        }
        store_sign_bytes(sign_bytes4(acc), lane, T * 16, n_blocks, a.qbits, mb, nt0);
        continue;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (nt0 + q < nt_end) {
          const int row = 16 * (nt0 + q) + r;
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            f16x8 b;
            if constexpr (FROM_LDS) b = __builtin_bit_cast(f16x8, gb[g_swizzle<D>(row - row0, res_col8<D>(g, k))]);
            else b = load_gfrag_f16<D, false>(gb, a.proj, a.signs, m, row, res_col8<D>(g, k));
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, __builtin_bit_cast(f16x8, ahi[k]), acc[q], 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, __builtin_bit_cast(f16x8, alo[k]), acc[q], 0, 0, 0);
          }
        }
      }
      store_sign_bytes(sign_bytes4(acc), lane, T * 16, n_blocks, a.qbits, mb, nt0);
    }
  }

  // the QJL projection of a tile whose codes decide() has taken (rotated basis)
  __device__ __forceinline__ void project_tile(const float (&v)[E], int64_t T) {
    u32x4 bhi[KS], blo[KS];
    rotated_frags(v, bhi, blo);
    project_rotated(bhi, blo, T);
  }

  __device__ __forceinline__ void tile(const uint4 (&raw)[NR], int64_t T) {
    float v[E];
    decide(raw, T, v);
    if constexpr (QJL && RB) {
      project_tile(v, T);
    } else if constexpr (QJL) {
      u32x4 ahi[KS], alo[KS];
      residual_frags(v, ahi, alo);
      project<G_LDS>(ahi, alo, T, gl, 0, 0, m_pad >> 4);
    }
  }
};

// Rows [row0, row0 + rows) of G D as fp16 scaled by 2^10 (rows >= m zero), swizzled rows
// of D/8 16-byte chunks, into gb.
template <int D>
__device__ void stage_projection_rows(const uint16_t* proj, const uint8_t* signs, int m, int row0, int rows,
                                      uint4* gb) {
  stage_rows<D, 8>(proj, signs, m, row0, rows, gb, [](const uint4& b, uint32_t sb) { return gd_f16(b, sb); });
}

// THREADS = 512 when G takes most of the LDS: one workgroup per CU then still runs two waves
// per SIMD.  RB (rotated-basis projection, G D H in LDS): sixteen-wave workgroups, one per CU
// (four waves per SIMD), so the grid and G D H are built once per CU.
template <int D, bool IN_BF16, bool QJL, bool G_LDS, int MODE, int THREADS = kThreads, bool RB = false>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(RB ? (MODE == 2 ? 3 : PQ_RB_WPE) : (THREADS == 512 ? 2 : PQ_QUANT_WAVES_PER_EU))))
void pq_quantize_kernel(const pqi::QuantArgs a) {
  using Q = Quantizer<D, IN_BF16, QJL, G_LDS, MODE, RB>;
  constexpr int WAVES = THREADS / 64;
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* tab = reinterpret_cast<uint4*>(smem);
  uint4* gl = reinterpret_cast<uint4*>(smem + a.t.ncell * a.t.nrep * 16);
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t full_tiles = a.n_blocks >> 4;
  const int64_t n_waves = (int64_t)gridDim.x * WAVES;
  int64_t T = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  uint4 raw[Q::NR];
  // the first tile's input is requested before the tables are built: its latency overlaps
  // that work
  if constexpr (Q::NR <= 4)
    if (T < n_tiles) load_tile<D, IN_BF16>(raw, a.x, T, a.n_blocks, full_tiles, threadIdx.x & 15, (threadIdx.x >> 4) & 3);
  build_search_grid(a.t, tab);
  Q q(a, smem, gl);
  if constexpr (Q::MR) {
    // the Walsh-Hadamard fragments after the grid and G D H
    const size_t gbytes = QJL && RB ? (size_t)q.m_pad * D * 4 : QJL && G_LDS ? (size_t)q.m_pad * D * 2 : 0;
    uint4* hfp = reinterpret_cast<uint4*>(smem + a.t.ncell * a.t.nrep * 16 + gbytes);
    build_wht_frags(hfp);
    q.hf = hfp;
    if constexpr (Q::SM_LDS) {
      // the sign words after the fragments: entry g * (D / 32) + s, word t = pair 4 s + t of quarter g
      uint4* sm = hfp + kHfBytes / 16;
      for (int i = threadIdx.x; i < 4 * (D / 32); i += blockDim.x) {
        const int gq = i / (D / 32), st = i % (D / 32);
        const uint32_t b = a.signs[4 * st + gq];
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = (((b >> (2 * t)) & 1u) << 15) | (((b >> (2 * t + 1)) & 1u) << 31);
        sm[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      q.sml = sm;
    }
  }
  if constexpr (QJL && RB && Q::NR <= 4) {
    // the search grid first; the rows of G D H are then built (by the first waves) while
    // every wave takes the codes of its first tile, and only that tile's projection waits
    // for them
    __syncthreads();
    q.stage_rotated(gl, threadIdx.x >> 6, WAVES);
    uint4 nxt[Q::NR];
    if (T + n_waves < n_tiles) load_tile<D, IN_BF16>(nxt, a.x, T + n_waves, a.n_blocks, full_tiles, q.r, q.g);
    const bool first = T < n_tiles;
    float v[Q::E];
    if (first) q.decide(raw, T, v);
    __syncthreads();
    if (first) q.project_tile(v, T);
    for (T += n_waves; T < n_tiles; T += n_waves) {
#pragma unroll
      for (int i = 0; i < Q::NR; ++i) raw[i] = nxt[i];
      if (T + n_waves < n_tiles) load_tile<D, IN_BF16>(nxt, a.x, T + n_waves, a.n_blocks, full_tiles, q.r, q.g);
      q.tile(raw, T);
    }
    return;
  }
  if constexpr (QJL && RB) q.stage_rotated(gl, threadIdx.x >> 6, WAVES);
  else if constexpr (QJL && G_LDS) stage_projection_rows<D>(a.proj, a.signs, a.m, 0, (a.m + 15) & ~15, gl);
  __syncthreads();

  if constexpr (Q::NR <= 4) {
    // the next tile's input is loaded before this tile is processed (16 more registers; a
    // two-buffer unrolled loop would save the copies but pushes the kernel into spills)
    for (; T < n_tiles; T += n_waves) {
      uint4 nxt[Q::NR];
      if (T + n_waves < n_tiles) load_tile<D, IN_BF16>(nxt, a.x, T + n_waves, a.n_blocks, full_tiles, q.r, q.g);
      q.tile(raw, T);
#pragma unroll
      for (int i = 0; i < Q::NR; ++i) raw[i] = nxt[i];
    }
  } else {
    // several waves per SIMD overlap one wave's loads with another's arithmetic
    for (; T < n_tiles; T += n_waves) {
      load_tile<D, IN_BF16>(raw, a.x, T, a.n_blocks, full_tiles, q.r, q.g);
      q.tile(raw, T);
    }
  }
}

// Quantize with a QJL projection too large to keep in LDS (config 5: m = d = 512 would need
// 512 KiB).  A workgroup quantizes one tile per wave; each wave writes its tile's
// block-coordinate residual (rotation signs applied, D w = d r times the power-of-two scale)
// to LDS as fp16 high and low MFMA B fragments.  The workgroup then multiplies G by the
// residuals of all its tiles: wave w takes the groups of four N tiles w, w + WAVES, ...,
// reads their G fragments straight from L2 into registers (bf16 -> fp16, two K steps ahead),
// and every G fragment feeds 2 x 4 tiles of MFMAs while every residual fragment read from
// LDS feeds four N tiles.  bf16 values in the fp16 normal range convert exactly; smaller ones
// keep fp16's absolute precision (6e-8), far below what decides a sign.
// eight waves where two per SIMD fit in the register file, else four with all of it
template <int D>
constexpr int chunk_threads() { return D <= 128 ? 512 : 256; }
#ifndef PQ_CHUNK_GDEPTH
#define PQ_CHUNK_GDEPTH 3
#endif
// LDS bytes of the residual fragments of one workgroup
template <int D>
constexpr size_t chunk_frag_bytes() { return (size_t)(chunk_threads<D>() / 64) * (D / 32) * 2 * 64 * 16; }

__device__ __forceinline__ f16x8 bf16x8_to_f16(const uint4& b) {
  const u32x4 h = {split_hi_f16x2(bf16_lo(b.x), bf16_hi(b.x)), split_hi_f16x2(bf16_lo(b.y), bf16_hi(b.y)),
                   split_hi_f16x2(bf16_lo(b.z), bf16_hi(b.z)), split_hi_f16x2(bf16_lo(b.w), bf16_hi(b.w))};
  return __builtin_bit_cast(f16x8, h);
}

template <int D, bool IN_BF16, int MODE>
__global__ __launch_bounds__(chunk_threads<D>()) __attribute__((amdgpu_waves_per_eu(chunk_threads<D>() / 256)))
void pq_quantize_chunked_kernel(const pqi::QuantArgs a) {
  using Q = Quantizer<D, IN_BF16, true, true, MODE>;
  constexpr int THREADS = chunk_threads<D>();
  constexpr int WAVES = THREADS / 64;
  constexpr int KS = Q::KS;
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* tab = reinterpret_cast<uint4*>(smem);
  u32x4* rf = reinterpret_cast<u32x4*>(smem + a.t.ncell * a.t.nrep * 16);   // [WAVES][KS][2][64]
  build_search_grid(a.t, tab);
  Q q(a, smem, nullptr);
  if constexpr (Q::MR) {
    // the Walsh-Hadamard fragments after the residual fragments
    uint4* hfp = reinterpret_cast<uint4*>(smem + a.t.ncell * a.t.nrep * 16 + chunk_frag_bytes<D>());
    build_wht_frags(hfp);
    q.hf = hfp;
  }
  const int lane = q.lane, r = q.r, g = q.g, wv = threadIdx.x >> 6;
  // rotation signs of this lane's residual registers: chunk k holds columns 8 res_col8(g, k) + 0..7
  uint32_t rsg[(KS + 3) / 4];
#pragma unroll
  for (int k = 0; k < (KS + 3) / 4; ++k) rsg[k] = 0;
#pragma unroll
  for (int k = 0; k < KS; ++k) rsg[k >> 2] |= (uint32_t)a.signs[res_col8<D>(g, k)] << (8 * (k & 3));
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t full_tiles = a.n_blocks >> 4;
  const int64_t n_groups = (n_tiles + WAVES - 1) / WAVES;
  const int m = a.m, ngrp = (q.m_pad + 63) >> 6;                    // groups of four N tiles
  const uint4* gsrc = reinterpret_cast<const uint4*>(a.proj);
  for (int64_t TG = blockIdx.x; TG < n_groups; TG += gridDim.x) {   // uniform over the workgroup
    const int64_t T = TG * WAVES + wv;                               // may lie past the end: no stores
    __syncthreads();                                                  // search grid built / fragments consumed
    {
      uint4 raw[Q::NR];
      load_tile<D, IN_BF16>(raw, a.x, T, a.n_blocks, full_tiles, r, g);
      float v[Q::E];
      q.decide(raw, T, v);
      q.residual_block(v);
      u32x4* my = rf + (size_t)wv * KS * 2 * 64;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        u32x4 hi, lo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t s0 = (rsg[k >> 2] >> (8 * (k & 3) + 2 * t)) & 1u;
          const uint32_t s1 = (rsg[k >> 2] >> (8 * (k & 3) + 2 * t + 1)) & 1u;
          const float x0 = __uint_as_float(__float_as_uint(v[8 * k + 2 * t]) ^ (s0 << 31));
          const float x1 = __uint_as_float(__float_as_uint(v[8 * k + 2 * t + 1]) ^ (s1 << 31));
          hi[t] = split_hi_f16x2(x0, x1);
          lo[t] = split_lo_f16x2(hi[t], x0, x1);
        }
        my[(2 * k) * 64 + lane] = hi;
        my[(2 * k + 1) * 64 + lane] = lo;
      }
    }
    __syncthreads();                                                  // every tile's fragments written
    for (int grp = wv; grp < ngrp; grp += WAVES) {
      // G fragment (N tile 4 grp + j, K step k): row 16 (4 grp + j) + r, columns 8 res_col8(g, k) + 0..7;
      // rows past m read row m - 1 (their signs are not stored)
      auto gload = [&](int k, uint4 (&ga)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = min(16 * (4 * grp + j) + r, m - 1);
          ga[j] = gsrc[(int64_t)row * (D / 8) + res_col8<D>(g, k)];
        }
      };
#pragma unroll
      for (int t0 = 0; t0 < WAVES; t0 += 4) {
        f32x4 acc[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[tt][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // G fragments PQ_CHUNK_GDEPTH K steps ahead, residual fragments one K step ahead
        constexpr int GD = PQ_CHUNK_GDEPTH;
        uint4 ga[GD][4];
#pragma unroll
        for (int k = 0; k < GD && k < KS; ++k) gload(k, ga[k]);
        auto bload = [&](int k, f16x8 (&b)[4][2]) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const u32x4* f = rf + ((size_t)(t0 + tt) * KS + k) * 2 * 64 + lane;
            b[tt][0] = __builtin_bit_cast(f16x8, f[0]);
            b[tt][1] = __builtin_bit_cast(f16x8, f[64]);
          }
        };
        f16x8 bc[4][2];
        bload(0, bc);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          f16x8 af[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) af[j] = bf16x8_to_f16(ga[k % GD][j]);
          if (k + GD < KS) gload(k + GD, ga[k % GD]);
          f16x8 bn[4][2];
          if (k + 1 < KS) bload(k + 1, bn);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[tt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[j], bc[tt][0], acc[tt][j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[tt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[j], bc[tt][1], acc[tt][j], 0, 0, 0);
          }
          if (k + 1 < KS) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) { bc[tt][0] = bn[tt][0]; bc[tt][1] = bn[tt][1]; }
          }
          __builtin_amdgcn_sched_barrier(0);                          // keeps the loads where they are issued
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          store_sign_bytes(sign_bytes4(acc[tt]), lane, (TG * WAVES + t0 + tt) * 16, a.n_blocks, a.qbits, q.mb, 4 * grp);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Dequantize.  Outputs are written with non-temporal stores: they stream to HBM without
// displacing the codes and tables in the caches.
// ------------------------------------------------------------------------------------------
// One tensor's dequantize state in a wave: codes, norms and output of the tensor and the
// output sign masks of this lane (register chunk s holds elements 8 g + dq_out_chunk(s) + 0..7).
template <int D, bool OUT_BF16, int PB>
struct Dequantizer {
  static constexpr int E = D / 4;
  static constexpr int CB = PB ? PB : 8;                     // bits per stored code (PB = 0: a byte each)
  static constexpr int NB = E * CB / 8;                      // code bytes of the lane's run
  static constexpr int NQ = (NB + 3) / 4;                    // ... as dwords
  // d = 512: the inverse transform on the fp16 matrix cores (MR), output chunk c of a lane
  // (elements 32 c + 8 g + 0..7) in registers 8 c + 0..7, see inverse_mfma().  (At d = 256 the
  // same form was faster with byte codes, 70 against 78 us at config 5, but slower with packed
  // codes, 65-70 against 59 us; byte and packed codes dequantize through one form, so d = 256
  // keeps the butterflies.)
  static constexpr bool MR = D == 512;
  const float* cent;
  const uint32_t* cpair = nullptr;   // MR: centroid fp16 high | low << 16
  const uint4* hfd = nullptr;        // MR: the two A fragments
  int r, g;
  uint32_t smask[E / 2];
  const uint8_t* codes;
  const uint16_t* norms;
  void* out;
  int64_t n_blocks;

  // output elements 8 g + out_chunk(s) + 0..7 are register chunk s
  static __host__ __device__ constexpr int out_chunk(int s) { return MR ? 32 * s : dq_out_chunk<D>(s); }

  __device__ __forceinline__ void retarget(const uint8_t* signs, const uint8_t* c, const uint16_t* nm, void* o,
                                           int64_t nb) {
    // byte loads (the mask may sit at any address): register chunk s is output elements
    // 8 g + out_chunk(s) + 0..7, sign byte g + out_chunk(s) / 8
#pragma unroll
    for (int s = 0; s < E / 8; ++s) set_chunk(s, signs[g + out_chunk(s) / 8]);
    codes = c;
    norms = nm;
    out = o;
    n_blocks = nb;
  }
  __device__ __forceinline__ void set_chunk(int s, uint32_t b) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t s0 = (b >> (2 * t)) & 1u, s1 = (b >> (2 * t + 1)) & 1u;
      smask[4 * s + t] = OUT_BF16 ? ((s0 << 15) | (s1 << 31)) : (s0 | (s1 << 1));
    }
  }
  __device__ __forceinline__ void retarget(const SignWords<D>& sw, const uint8_t* c, const uint16_t* nm, void* o,
                                           int64_t nb) {
    // register chunk s is output elements 8 g + out_chunk(s) + 0..7: sign byte g + out_chunk(s) / 8
#pragma unroll
    for (int s = 0; s < E / 8; ++s) set_chunk(s, sw.byte(out_chunk(s) / 32, g));
    codes = c;
    norms = nm;
    out = o;
    n_blocks = nb;
  }

  // the lane's run: codes E g .. E g + E - 1 of block 16 T + r (a CB-bit stream)
  __device__ __forceinline__ void load(uint32_t (&q)[NQ], uint16_t& nb, int64_t T) const {
    const int64_t blk = T * 16 + r;
    const bool valid = blk < n_blocks;
    load_code_bytes<NB>(codes + blk * (D * CB / 8) + E * g * CB / 8, valid, q);
    nb = valid ? norms[blk] : (uint16_t)0;
  }

  // MR: the lane's run (elements E g + j) as the B operand: K step s takes registers
  // (s & 7) + 8 jj + 64 (s >> 3), jj = 0..7 (element bits 3..5), so the products sum element bits
  // 3..5 and the lane bits; partial sums of K step s land in registers 8 s + 4 t0 + i, and
  // butterflies over s (register bits 3 and up) finish the transform.  Afterwards register
  // 8 (8 s_hi + b) + 4 t0 + i holds output element b + 8 g + 32 c, c = i0 + 2 i1 + 4 t0 (d = 256)
  // or i0 + 2 s_hi + 4 i1 + 8 t0 (d = 512); the registers are then renamed to chunk order.
  __device__ __forceinline__ void inverse_mfma(const uint32_t (&q)[NQ], float (&v)[E]) const {
    constexpr int KSD = E / 8;
    float u[E];
    const f16x8 h0 = __builtin_bit_cast(f16x8, hfd[lane_id()]);
    const f16x8 h1 = __builtin_bit_cast(f16x8, hfd[64 + lane_id()]);
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      uint32_t cp[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) cp[jj] = cpair[stream_code<CB>(q, (s & 7) + 8 * jj + 64 * (s >> 3))];
      u32x4 bh, bl;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        bh[p] = __builtin_amdgcn_perm(cp[2 * p + 1], cp[2 * p], 0x05040100u);   // high parts
        bl[p] = __builtin_amdgcn_perm(cp[2 * p + 1], cp[2 * p], 0x07060302u);   // low parts
      }
      f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h0, __builtin_bit_cast(f16x8, bh), f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h1, __builtin_bit_cast(f16x8, bh), f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h0, __builtin_bit_cast(f16x8, bl), a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(h1, __builtin_bit_cast(f16x8, bl), a1, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[8 * s + i] = a0[i];
        u[8 * s + 4 + i] = a1[i];
      }
    }
    bfly<E, 3>(u); bfly<E, 4>(u); bfly<E, 5>(u);
    if constexpr (D == 512) bfly<E, 6>(u);
    // rename: chunk c, element b of the chunk -> register 8 c + b
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = j & 3, t0 = (j >> 2) & 1, b = (j >> 3) & 7, sh = j >> 6;
      const int c = D == 256 ? (i & 1) + 2 * (i >> 1) + 4 * t0 : (i & 1) + 2 * sh + 4 * (i >> 1) + 8 * t0;
      v[8 * c + b] = u[j];
    }
  }
  static __device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

  __device__ __forceinline__ void tile(const uint32_t (&q)[NQ], uint16_t nb, int64_t T) const {
    float v[E];
    const float scale = f16_to_f32(nb) * (1.0f / (float)D);
    if constexpr (MR) {
      inverse_mfma(q, v);
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = cent[stream_code<CB>(q, j)];
      wht_dequant<D>(v);
    }

    // Stores write whole 128-byte lines: a line of a block is two 16-byte pieces (a, b) in
    // each of its four lanes; the neighbouring blocks r & ~1 and r | 1 (lanes l, l ^ 1) trade
    // pieces, so that one store writes block r & ~1's line from both lanes and the next
    // block r | 1's.  Half-line stores would reach HBM as partial lines.
    const bool odd = r & 1;
    const int64_t blk_e = T * 16 + (r & ~1);
    const bool ok_e = blk_e < n_blocks, ok_o = blk_e + 1 < n_blocks;
    auto put = [&](auto* row_e, const u32x4& pa, const u32x4& pb, int off_a, int off_b) {
      u32x4 x, y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(odd ? pa[i] : pb[i]), 0xB1, 0xF, 0xF, true);
        x[i] = odd ? recv : pa[i];                                    // block r & ~1: its a, then its b
        y[i] = odd ? pb[i] : recv;                                    // block r | 1
      }
      const int off = odd ? off_b : off_a;
      if (ok_e) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(row_e + off));
      if (ok_o) __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(row_e + D + off));
    };
    if constexpr (OUT_BF16) {
      uint16_t* row_e = static_cast<uint16_t*>(out) + blk_e * D + 8 * g;
      auto pack = [&](int s) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = pack_bf16x2(v[8 * s + 2 * t] * scale, v[8 * s + 2 * t + 1] * scale) ^ smask[4 * s + t];
        return w;
      };
      // chunk s and chunk partner(s) hold the two halves of one output line
#pragma unroll
      for (int s = 0; s < E / 8; ++s)
        if (out_chunk(s) % 64 == 0)
          put(row_e, pack(s), pack(MR ? s + 1 : dq_partner<D>(s)), out_chunk(s), out_chunk(s) + 32);
    } else {
      float* row_e = static_cast<float*>(out) + blk_e * D + 8 * g;
#pragma unroll
      for (int s = 0; s < E / 8; ++s) {
        float f[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t sb = (smask[4 * s + t / 2] >> (t & 1)) & 1u;
          f[t] = __uint_as_float(__float_as_uint(v[8 * s + t] * scale) ^ (sb << 31));
        }
        const u32x4 pa = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
        const u32x4 pb = {__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7])};
        put(row_e, pa, pb, out_chunk(s), out_chunk(s) + 4);
      }
    }
  }
};

template <int D, bool OUT_BF16, int PB>
__global__ __launch_bounds__(kThreads) void pq_dequantize_kernel(const pqi::DequantArgs a) {
  using DQ = Dequantizer<D, OUT_BF16, PB>;
  __shared__ float cent[1 << pqi::kMaxBits];
  __shared__ uint32_t cpair[DQ::MR ? 1 << pqi::kMaxBits : 1];
  __shared__ uint4 hfd[DQ::MR ? 128 : 1];
  copy_centroids(a.t, cent);
  if constexpr (DQ::MR) build_dq_mr_tables(a.t, cpair, hfd);
  __syncthreads();

  DQ dq;
  dq.cent = cent;
  dq.cpair = cpair;
  dq.hfd = hfd;
  dq.r = threadIdx.x & 15;
  dq.g = (threadIdx.x & 63) >> 4;
  dq.retarget(a.signs, a.codes, a.norms, a.out, a.n_blocks);

  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t n_waves = (int64_t)gridDim.x * kWaves;
  int64_t T = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  uint32_t q[DQ::NQ];
  uint16_t nb;
  dq.load(q, nb, T);
  for (; T < n_tiles; T += n_waves) {
    uint32_t qn[DQ::NQ];
    uint16_t nbn;
    dq.load(qn, nbn, T + n_waves);                   // the next tile's codes (zero past the end)
    dq.tile(q, nb, T);
#pragma unroll
    for (int w = 0; w < DQ::NQ; ++w) q[w] = qn[w];
    nb = nbn;
  }
}

// ------------------------------------------------------------------------------------------
// Grouped codec over many tensors in one launch (a weight set streamed in one pass): the
// tensors are listed in a device table and their tiles numbered in table order; wave w takes
// the chunks of C consecutive tiles w, w + n_waves, ... and a cursor that only moves forward
// finds each tile's tensor from the table's block counts (uniform loads).  Dequantize, bound by
// memory, strides over the whole set in chunks of PQ_MANY_CHUNK tiles (as the single-tensor
// kernels stride over one tensor) and loads the next tile's record with its codes; quantize,
// bound by vector issue, gives each wave one contiguous range, so it changes tensor at most a
// few times.
// ------------------------------------------------------------------------------------------
#ifndef PQ_MANY_CHUNK
#define PQ_MANY_CHUNK 2
#endif
#ifndef PQ_MANY_WG_PER_CU
#define PQ_MANY_WG_PER_CU 4      // grouped quantize: workgroups per CU
#endif
__device__ __forceinline__ int64_t tiles_of(int64_t n_blocks) { return (n_blocks + 15) >> 4; }

struct ManyCursor {
  const pqi::TensorDesc* tab;
  int ti;                     // current tensor
  int64_t base, end;          // its global tile range [base, end)
  __device__ __forceinline__ void init(const pqi::TensorDesc* t) {
    tab = t;
    ti = 0;
    base = 0;
    end = tiles_of(tab[0].n_blocks);
  }
  // move to the tensor holding global tile Tg (Tg never decreases); true when it changed
  __device__ __forceinline__ bool seek(int64_t Tg) {
    bool moved = false;
    while (Tg >= end) {
      base = end;
      ++ti;
      end = base + tiles_of(tab[ti].n_blocks);
      moved = true;
    }
    return moved;
  }
};

__device__ __forceinline__ int64_t many_total(const pqi::TensorDesc* tab, int n_tensors) {
  int64_t total = 0;
  for (int i = 0; i < n_tensors; ++i) total += tiles_of(tab[i].n_blocks);
  return total;
}

// global tile of step k of wave w: chunk w + (k / C) n_waves, tile k % C of the chunk
__device__ __forceinline__ int64_t many_tile(int64_t w, int64_t k, int64_t n_waves, int64_t C) {
  return (w + (k / C) * n_waves) * C + k % C;
}

// The record of the tensor a tile belongs to, read one tile ahead (with its sign words) so that
// a change of tensor never waits on a load.
template <int D>
struct ManyRecord {
  const void* x;
  uint8_t* codes;
  uint16_t* norms;
  void* out;
  int64_t n_blocks, base;
  SignWords<D> sw;
  __device__ __forceinline__ void read(const pqi::TensorDesc* tab, const ManyCursor& c) {
    x = tab[c.ti].x;
    codes = tab[c.ti].codes;
    norms = tab[c.ti].norms;
    out = tab[c.ti].out;
    n_blocks = tab[c.ti].n_blocks;
    base = c.base;
    sw.load(tab[c.ti].signs);
  }
};

template <int D, bool IN_BF16, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PQ_QUANT_WAVES_PER_EU)))
void pq_quantize_many_kernel(const pqi::QuantArgs a, const pqi::TensorDesc* tab, int n_tensors) {
  using Q = Quantizer<D, IN_BF16, false, false, MODE>;
  extern __shared__ __align__(16) unsigned char smem[];
  build_search_grid(a.t, reinterpret_cast<uint4*>(smem));
  uint4* hfp = reinterpret_cast<uint4*>(smem + a.t.ncell * a.t.nrep * 16);   // after the grid (MR)
  if constexpr (Q::MR) build_wht_frags(hfp);
  __syncthreads();
  Q q(a, smem, nullptr);
  if constexpr (Q::MR) q.hf = hfp;
  const int64_t total = many_total(tab, n_tensors);
  const int64_t n_waves = (int64_t)gridDim.x * kWaves;
  const int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  // one contiguous range per wave (few tensor changes; four waves per SIMD hide the loads)
  const int64_t t0 = total * w / n_waves, t1 = total * (w + 1) / n_waves;
  if (t0 >= t1) return;
  ManyCursor cur;
  cur.init(tab);
  cur.seek(t0);
  ManyRecord<D> rc;
  rc.read(tab, cur);
  q.retarget(rc.sw, rc.codes, rc.norms, rc.n_blocks);
  for (int64_t T = t0; T < t1; ++T) {
    if (cur.seek(T)) {
      rc.read(tab, cur);
      q.retarget(rc.sw, rc.codes, rc.norms, rc.n_blocks);
    }
    uint4 raw[Q::NR];
    load_tile<D, IN_BF16>(raw, rc.x, T - rc.base, rc.n_blocks, rc.n_blocks >> 4, q.r, q.g);
    q.tile(raw, T - rc.base);
  }
}

template <int D, bool OUT_BF16, int PB>
__global__ __launch_bounds__(kThreads) void pq_dequantize_many_kernel(const pqi::DequantArgs a, const pqi::TensorDesc* tab,
                                                                      int n_tensors) {
  using DQ = Dequantizer<D, OUT_BF16, PB>;
  __shared__ float cent[1 << pqi::kMaxBits];
  __shared__ uint32_t cpair[DQ::MR ? 1 << pqi::kMaxBits : 1];
  __shared__ uint4 hfd[DQ::MR ? 128 : 1];
  copy_centroids(a.t, cent);
  if constexpr (DQ::MR) build_dq_mr_tables(a.t, cpair, hfd);
  __syncthreads();
  DQ dq;
  dq.cent = cent;
  dq.cpair = cpair;
  dq.hfd = hfd;
  dq.r = threadIdx.x & 15;
  dq.g = (threadIdx.x & 63) >> 4;
  const int64_t total = many_total(tab, n_tensors);
  const int64_t n_waves = (int64_t)gridDim.x * kWaves;
  const int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  constexpr int64_t C = PQ_MANY_CHUNK;
  ManyCursor cur;
  cur.init(tab);
  int64_t k = 0, T = many_tile(w, 0, n_waves, C);
  if (T >= total) return;
  cur.seek(T);
  ManyRecord<D> rc, rn;
  rc.read(tab, cur);
  dq.retarget(rc.sw, rc.codes, rc.norms, rc.out, rc.n_blocks);
  // the lane's codes and norm of tile Tg of the tensor of record r (zero past its end)
  auto load = [&](uint32_t (&q)[DQ::NQ], uint16_t& nb, const ManyRecord<D>& r, int64_t Tg) {
    const int64_t blk = (Tg - r.base) * 16 + dq.r;
    const bool valid = blk < r.n_blocks;
    load_code_bytes<DQ::NB>(r.codes + blk * (D * DQ::CB / 8) + DQ::E * dq.g * DQ::CB / 8, valid, q);
    nb = valid ? r.norms[blk] : (uint16_t)0;
  };
  uint32_t q[DQ::NQ];
  uint16_t nb;
  load(q, nb, rc, T);
  while (true) {
    const int64_t Tn = many_tile(w, k + 1, n_waves, C);
    const bool more = Tn < total;
    const bool moved = more && cur.seek(Tn);
    if (moved) rn.read(tab, cur);
    uint32_t qn[DQ::NQ];
    uint16_t nbn = 0;
    if (more) load(qn, nbn, moved ? rn : rc, Tn);
    dq.tile(q, nb, T - rc.base);
    if (!more) break;
    if (moved) {
      rc = rn;
      dq.retarget(rc.sw, rc.codes, rc.norms, rc.out, rc.n_blocks);
    }
    T = Tn;
    ++k;
#pragma unroll
    for (int i = 0; i < DQ::NQ; ++i) q[i] = qn[i];
    nb = nbn;
  }
}

// ------------------------------------------------------------------------------------------
// QJL key sketch: norm + sign(G k), keys feed the MFMA directly (bf16 products are exact).
// A wave takes NT key tiles per pass, so every G fragment read from LDS feeds NT MFMAs;
// G rows are the A operand so that each lane ends with projections of its own key, and
// the sign bits of each N tile are taken as soon as it is done (16 live accumulators).
// Eight waves per workgroup share one LDS copy of G.
// ------------------------------------------------------------------------------------------
#ifndef PQ_SKETCH_THREADS
#define PQ_SKETCH_THREADS 512
#endif
#ifndef PQ_SKETCH_WAVES_PER_EU
#define PQ_SKETCH_WAVES_PER_EU 4
#endif
constexpr int kSketchThreads = PQ_SKETCH_THREADS;

// The keys of pass P (NT tiles of 16) as MFMA B fragments: lane quarter g holds elements
// 32 s + 8 g .. +7 of key row r of each tile (zero past the last key).  SPLIT: the keys are
// masked to their group's outlier channels (part 1) or to the other channels (part 0) as they
// are loaded, so norm and signs are those of the masked key.  STREAM: non-temporal loads.
template <int D, int NT, bool SPLIT, bool STREAM = true>
__device__ __forceinline__ void sketch_load_keys(bf16x8 (&kf)[NT][D / 32], const pqi::SketchArgs& a, int64_t P,
                                                 int r, int g) {
  constexpr int KS = D / 32;
  const int64_t n_keys = a.n_keys;
  const bool full = (P + 1) * NT * 16 <= n_keys;          // uniform
  // SPLIT: (head, token) of the pass's first key, once per pass
  int64_t head0 = 0, tok0 = 0;
  if constexpr (SPLIT) {
    head0 = (P * NT * 16) / a.seq_len;
    tok0 = P * NT * 16 - head0 * a.seq_len;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t key = (P * NT + t) * 16 + r;
    const bool valid = full || key < n_keys;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.keys + key * D);
    // element 8 s + i of this lane (column 32 s + 8 g + i) is an outlier channel of the key's
    // group when bit 8 s + i of om is set
    uint32_t om[(KS * 8 + 31) / 32];
    if constexpr (SPLIT) {
#pragma unroll
      for (int w = 0; w < (KS * 8 + 31) / 32; ++w) om[w] = 0;
      // the key's (head, token): at most NT 16 tokens past the pass's first key (keys past the
      // end take the last key's group)
      int64_t head = head0, tok = tok0 + t * 16 + r;
      while (tok >= a.seq_len) {
        tok -= a.seq_len;
        ++head;
      }
      if (!valid) {
        head = n_keys / a.seq_len - 1;
        tok = a.seq_len - 1;
      }
      const int64_t grp = a.seq_len <= 0xFFFFFFFFll ? (int64_t)((uint32_t)tok / (uint32_t)a.group_size)
                                                    : tok / a.group_size;
      const uint8_t* ix = a.oidx + (head * a.n_groups + grp) * a.n_out;
#pragma unroll 8
      for (int j = 0; j < a.n_out; ++j) {
        const int c = ix[j];
        if (((c >> 3) & 3) == g) {
          const int b = 8 * (c >> 5) + (c & 7);
#pragma unroll
          for (int w = 0; w < (KS * 8 + 31) / 32; ++w) om[w] |= (b >> 5) == w ? 1u << (b & 31) : 0u;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (valid) w = STREAM ? __builtin_nontemporal_load(src + 4 * s + g) : src[4 * s + g];
      if constexpr (SPLIT) {
        const uint32_t bs = om[(8 * s) >> 5] >> ((8 * s) & 31);      // this chunk's 8 bits
        const uint32_t keep = a.part ? bs : ~bs;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          w[u] &= ((keep >> (2 * u)) & 1u ? 0x0000FFFFu : 0u) | ((keep >> (2 * u + 1)) & 1u ? 0xFFFF0000u : 0u);
      }
      kf[t][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// The squared norm of this lane's key of tile t (all four quarters summed).
template <int D, int NT>
__device__ __forceinline__ float sketch_sumsq(const bf16x8 (&kf)[NT][D / 32], int t) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  float ss = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const u32x4 w = __builtin_bit_cast(u32x4, kf[t][s]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // element copied to a scalar first: a bit cast of the vector element itself
      // is lowered to a read of element 0 by this compiler
      const uint32_t wu = w[u];
      const bf16x2 h = __builtin_bit_cast(bf16x2, wu);
      ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
    }
  }
  return sum4(ss);
}

template <int D, bool G_LDS, bool SPLIT>
__global__ __launch_bounds__(kSketchThreads) __attribute__((amdgpu_waves_per_eu(PQ_SKETCH_WAVES_PER_EU)))
void qjl_sketch_kernel(const pqi::SketchArgs a) {
  constexpr int KS = D / 32;
#ifndef PQ_SKETCH_NT128
#define PQ_SKETCH_NT128 4
#endif
  constexpr int NT = (D <= 128 && G_LDS) ? PQ_SKETCH_NT128 : (D <= 256 ? 2 : 1);
  constexpr int WAVES = kSketchThreads / 64;
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* gl = reinterpret_cast<uint4*>(smem);
  const int m = a.m, m_pad = (m + 15) & ~15, mb = m >> 3;
  if constexpr (G_LDS) {
    stage_projection<D>(a.proj, m, m_pad, gl);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int ntiles = m_pad >> 4;
  const int64_t n_keys = a.n_keys;
  const int64_t n_tiles = (n_keys + 15) >> 4;
  const int64_t n_pass = (n_tiles + NT - 1) / NT;
  const int64_t wave_id = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * WAVES;

  for (int64_t P = wave_id; P < n_pass; P += n_waves) {
    bf16x8 kf[NT][KS];
    sketch_load_keys<D, NT, SPLIT>(kf, a, P, r, g);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t key = (P * NT + t) * 16 + r;
      const float ss = sketch_sumsq<D, NT>(kf, t);
      if (key < n_keys && g == 0) a.norms[key] = f32_to_f16(sqrtf(ss));
    }
    for (int nt0 = 0; nt0 < ntiles; nt0 += 4) {
      uint32_t x[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) x[t] = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (nt0 + q < ntiles) {                               // uniform
          const int row = 16 * (nt0 + q) + r;
          f32x4 acc[NT];
          const bf16x8 b0 = load_gfrag<D, G_LDS>(gl, a.proj, m, row, g);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, kf[t][0], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
          for (int s = 1; s < KS; ++s) {
            const bf16x8 b = load_gfrag<D, G_LDS>(gl, a.proj, m, row, 4 * s + g);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, kf[t][s], acc[t], 0, 0, 0);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) x[t] |= sign_nibble(acc[t], q);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        store_sign_bytes(sign_bytes_of(x[t]), lane, (P * NT + t) * 16, n_keys, a.bits, mb, nt0);
    }
  }
}

// ------------------------------------------------------------------------------------------
// QJL key sketch for m a multiple of 128 with G in LDS.  Row 128 c + 8 p + q of G is output row
// p of N tile q (0..7) of row group c, so at the end of a row group lane quarter g of key r holds
// the signs of rows 128 c + 32 g .. + 31 of that key as one word in bit order (byte i: rows
// 128 c + 8 (4 g + i) + 0..7), stored without any exchange between lanes.  A sign is read from
// the fp16 conversion of a projection rounded toward zero (which keeps the sign of every
// nonzero value); one byte permute gathers the four signs of an accumulator.  The keys of the
// wave's next pass are loaded while this pass is computed.
// ------------------------------------------------------------------------------------------
#ifndef PQ_SKETCH8_NT
#define PQ_SKETCH8_NT 2                                     // key tiles per pass (d <= 128; half that above)
#endif
#ifndef PQ_SKETCH8_WAVES_PER_EU
#define PQ_SKETCH8_WAVES_PER_EU 4
#endif
#ifndef PQ_SKETCH8_WG_PER_CU
#define PQ_SKETCH8_WG_PER_CU 2
#endif
#ifndef PQ_SKETCH8_THREADS
#define PQ_SKETCH8_THREADS 512
#endif
constexpr int kSketch8Threads = PQ_SKETCH8_THREADS;
template <int D>
constexpr int sketch8_nt() { return D <= 128 ? PQ_SKETCH8_NT : (PQ_SKETCH8_NT + 1) / 2; }

// LDS position of 16-byte chunk c of G row n: the rows 8 p + q (p = 0..15) that one 16-lane
// group reads together land on 16 different bank groups (8 for d = 64)
template <int D>
__device__ __forceinline__ int g_swizzle8(int n, int c) {
  constexpr int CPR = D / 8;
  constexpr int SW = CPR < 16 ? CPR - 1 : 15;
  return n * CPR + (c ^ ((n >> 3) & SW));
}

// Sign bits of the four projections of an accumulator at the top bit of each byte (1 where
// the projection is negative or -0).
__device__ __forceinline__ uint32_t sign_tops(const f32x4& acc) {
  const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(acc[0], acc[1]));
  const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(acc[2], acc[3]));
  return __builtin_amdgcn_perm(h23, h01, 0x07050301u);
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(kSketch8Threads) __attribute__((amdgpu_waves_per_eu(PQ_SKETCH8_WAVES_PER_EU)))
void qjl_sketch_rows_kernel(const pqi::SketchArgs a) {
  constexpr int KS = D / 32;
  constexpr int NT = sketch8_nt<D>();
  constexpr int WAVES = kSketch8Threads / 64;
  constexpr int CPR = D / 8;
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* gl = reinterpret_cast<uint4*>(smem);
  const int m = a.m, mb = m >> 3, ngrp = m >> 7;
  {
    // G into LDS, four chunks in flight per thread
    const uint4* src = reinterpret_cast<const uint4*>(a.proj);
    const int total = m * CPR;
    constexpr int S = kSketch8Threads;
    int i = threadIdx.x;
    for (; i + 3 * S < total; i += 4 * S) {
      const uint4 b0 = src[i], b1 = src[i + S], b2 = src[i + 2 * S], b3 = src[i + 3 * S];
      gl[g_swizzle8<D>(i / CPR, i % CPR)] = b0;
      gl[g_swizzle8<D>((i + S) / CPR, (i + S) % CPR)] = b1;
      gl[g_swizzle8<D>((i + 2 * S) / CPR, (i + 2 * S) % CPR)] = b2;
      gl[g_swizzle8<D>((i + 3 * S) / CPR, (i + 3 * S) % CPR)] = b3;
    }
    for (; i < total; i += S) gl[g_swizzle8<D>(i / CPR, i % CPR)] = src[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n_keys = a.n_keys;
  const int64_t n_pass = (n_keys + 16 * NT - 1) / (16 * NT);
  const int64_t n_waves = (int64_t)gridDim.x * WAVES;
  int64_t P = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  if (P >= n_pass) return;                                  // no barrier follows
  bf16x8 kf[NT][KS];
  sketch_load_keys<D, NT, SPLIT, false>(kf, a, P, r, g);
  for (; P < n_pass; P += n_waves) {
    const bool more = P + n_waves < n_pass;
    bf16x8 kn[NT][KS];
    if (more) sketch_load_keys<D, NT, SPLIT, false>(kn, a, P + n_waves, r, g);
    uint32_t live[NT];                                      // all ones unless the key is zero
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t key = (P * NT + t) * 16 + r;
      const float ss = sketch_sumsq<D, NT>(kf, t);
      if (key < n_keys && g == 0) a.norms[key] = f32_to_f16(sqrtf(ss));
      live[t] = ss > 0.0f ? ~0u : 0u;
    }
    for (int c = 0; c < ngrp; ++c) {
      uint32_t neg[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) neg[t] = 0;
      // N tile q: MFMA row r is G row 128 c + 8 r + q
      auto project = [&](int q, f32x4 (&acc)[NT]) {
        const int row = 128 * c + 8 * r + q;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, gl[g_swizzle8<D>(row, 4 * s + g)]);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, kf[t][s], s ? acc[t] : f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                             0, 0, 0);
        }
      };
      // the products of N tile q + 1 are issued before the signs of N tile q are read off
      f32x4 acc[2][NT];
      project(0, acc[0]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q < 7) project(q + 1, acc[(q + 1) & 1]);
        // projection rows 128 c + 8 (4 g + i) + q: sign of row i at bit 8 i + q
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          neg[t] |= (sign_tops(acc[q & 1][t]) >> (7 - q)) & (0x01010101u << q);
          // taken here: otherwise the sign reads sink into the store branch below and keep
          // every accumulator of the row group live until then
          asm volatile("" : "+v"(neg[t]));
        }
        __builtin_amdgcn_sched_barrier(0);                  // one N tile in flight: bounds the live accumulators
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int64_t key = (P * NT + t) * 16 + r;
        if (key < n_keys)
          *reinterpret_cast<uint32_t*>(a.bits + key * mb + 16 * c + 4 * g) = ~neg[t] & live[t];
      }
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[t][s] = kn[t][s];
    }
  }
}

// ------------------------------------------------------------------------------------------
// Outlier channels: one wave per (head, group of group_size tokens).  Lane l holds channels
// D/64 l .. D/64 (l+1) - 1 and sums their squares over the group's tokens in fp32; then
// n_out rounds each take the wave-wide maximum of (sum of squares, lower channel first) as
// one 64-bit key (the fp32 pattern of a non-negative sum orders as an integer).
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void qjl_outlier_kernel(const pqi::OutlierArgs a) {
  constexpr int CPL = D / 64;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= a.n_heads * a.n_groups) return;                     // whole waves only
  const int64_t head = wid / a.n_groups, grp = wid % a.n_groups;
  const int64_t t0 = grp * a.group_size, t1 = min(t0 + (int64_t)a.group_size, a.seq_len);
  float ss[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) ss[c] = 0.0f;
  const uint16_t* base = a.keys + (head * a.seq_len) * D + CPL * lane;
  // eight tokens' loads in flight at a time (clamped to the group, masked when past it)
  for (int64_t t = t0; t < t1; t += 8) {
    uint16_t x[8][CPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t* p = base + min(t + u, t1 - 1) * D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) x[u][c] = p[c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = t + u < t1 ? 1.0f : 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float v = bf16_to_f32(x[u][c]) * w;
        ss[c] = fmaf(v, v, ss[c]);
      }
    }
  }
  uint32_t taken = 0;
  uint8_t* out = a.oidx + wid * a.n_out;
  for (int j = 0; j < a.n_out; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint64_t k = ((taken >> c) & 1u) ? 0ull
                         : ((uint64_t)__float_as_uint(ss[c]) << 32) | (uint64_t)(0xFFFFu - (CPL * lane + c));
      best = k > best ? k : best;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), off), lo = __shfl_xor((uint32_t)best, off);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      best = o > best ? o : best;
    }
    const int ch = 0xFFFF - (int)(best & 0xFFFFu);
    if (ch / CPL == lane) taken |= 1u << (ch % CPL);
    if (lane == 0) out[j] = (uint8_t)ch;
  }
}

// ------------------------------------------------------------------------------------------
// Query projection sq = G q (fp32) on the bf16 matrix cores: one wave per 16 x 16 tile of
// (query, projection row); the bf16 products are exact and accumulate in fp32.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void qjl_project_kernel(const pqi::ProjectArgs a) {
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int64_t q0 = (int64_t)blockIdx.x * 16;
  const int n0 = blockIdx.y * 16;
  const int d = a.d;
  const int64_t qrow = q0 + r;
  const int nrow = n0 + r;
  const uint4* qs = reinterpret_cast<const uint4*>(a.q + qrow * d);
  const uint4* gs = reinterpret_cast<const uint4*>(a.proj + (int64_t)nrow * d);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < d / 32; ++s) {
    const uint4 qa = qrow < a.n_q ? qs[4 * s + g] : make_uint4(0, 0, 0, 0);
    const uint4 gb = nrow < a.m ? gs[4 * s + g] : make_uint4(0, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa), __builtin_bit_cast(bf16x8, gb),
                                                 acc, 0, 0, 0);
  }
  // acc[i] = sq[q0 + 4 g + i][n0 + r]
  if (nrow < a.m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t qi = q0 + 4 * g + i;
      if (qi < a.n_q)
        a.sq[(qi / a.rows_per_group) * a.group_stride + (qi % a.rows_per_group) * a.m + nrow] = acc[i];
    }
  }
}

// ------------------------------------------------------------------------------------------
// QJL score for grouped-query attention on the int8 matrix cores.
//
// sum_i (2 b_i - 1) sq_i = 2 sum_i b_i sq_i - sum_i sq_i.  Each projected query
// is quantized to integers Q_i = rint(sq_i / s), s = max|sq| / kLimbRange, and
// split into three int8 limbs Q = 16384 h2 + 128 h1 + h0; the bit vectors,
// expanded to bytes {0, 1}, meet the limbs in v_mfma_i32_16x16x64_i8 with exact
// int32 accumulation.  A rows: 4 query heads x 4 slots (h2, h1, h0, 0); B columns:
// 16 keys.  Lane group gq holds bits [m/4 gq, m/4 (gq+1)) of its key, K step k the
// 16 bits from m/4 gq + 16 k.  The limbs are built once per workgroup in LDS in
// A-fragment order (K step k, lane L: 16 bytes at 16 (64 k + L)).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t spread_nibble(uint32_t nib) {
  // 4 bits -> 4 bytes of value 0/1 (bit j -> byte j)
  return (nib * 0x204081u) & 0x01010101u;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_sum(int x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}


__device__ __forceinline__ int limb_of(int Q, int l) {
  const int h2 = (int)rintf((float)Q * (1.0f / 16384.0f));
  const int rem = Q - 16384 * h2;
  const int h1 = (int)rintf((float)rem * (1.0f / 128.0f));
  const int h0 = rem - 128 * h1;
  return l == 0 ? h2 : l == 1 ? h1 : h0;
}

// The 2 KS bytes of packed key bits of lane group gq (K steps 0 .. KS-1, 16 bits each).
template <int KS>
__device__ __forceinline__ void load_key_bits(const uint8_t* kb, bool valid, uint32_t (&w)[(KS + 1) / 2]) {
#pragma unroll
  for (int j = 0; j < (KS + 1) / 2; ++j) w[j] = 0;
  if (!valid) return;
  if constexpr (KS % 8 == 0) {
#pragma unroll
    for (int j = 0; j < KS / 8; ++j) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb) + j);
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
  } else if constexpr (KS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < KS / 4; ++j) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(kb) + j);
      w[2 * j] = v.x; w[2 * j + 1] = v.y;
    }
  } else if constexpr (KS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < KS / 2; ++j) w[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb) + j);
  } else {
#pragma unroll
    for (int k = 0; k < KS; ++k)
      w[k >> 1] |= (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(kb) + k) << (16 * (k & 1));
  }
}

template <int KS, bool ADD>
#ifndef PQ_SCORE_TILES
#define PQ_SCORE_TILES 4         // key tiles of a QJL score iteration (the next ones load meanwhile)
#endif
__global__ __launch_bounds__(kThreads) void qjl_score_kernel(const pqi::ScoreArgs a, int chunks_per_group) {
  constexpr int m = 64 * KS, mb = m >> 3;
  const int group = a.q_heads / a.kv_heads;
  const int grp = blockIdx.x / chunks_per_group;          // (batch, kv head) pair
  const int chunk = blockIdx.x % chunks_per_group;
  const int b = grp / a.kv_heads, gk = grp % a.kv_heads;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;

  __shared__ i32x4 frag[KS * 64];
  __shared__ float scl[4];
  __shared__ int isum[4];
  for (int i = threadIdx.x; i < KS * 64; i += blockDim.x) frag[i] = i32x4{0, 0, 0, 0};
  __syncthreads();
  // wave wv quantizes query head wv of the group into A rows 4 wv + limb
  if (wv < group) {
    const float* src = a.sq + ((int64_t)b * a.q_heads + gk * group + wv) * m;
    float x[KS];                                          // element lane + 64 j of the head
#pragma unroll
    for (int j = 0; j < KS; ++j) x[j] = src[lane + 64 * j];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < KS; ++j) amax = fmaxf(amax, fabsf(x[j]));
    const float s = wave_max(amax) / pqi::kLimbRange;
    const float inv_s = s > 0.0f ? 1.0f / s : 0.0f;
    int acc = 0;
    unsigned char* fb = reinterpret_cast<unsigned char*>(frag);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int e = lane + 64 * j;
      const int Q = (int)rintf(x[j] * inv_s);
      acc += Q;
      const int gq = e / (m / 4), k = (e % (m / 4)) >> 4, i = e & 15;
#pragma unroll
      for (int l = 0; l < 3; ++l) fb[(k * 64 + 16 * gq + 4 * wv + l) * 16 + i] = (unsigned char)(limb_of(Q, l) & 0xff);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      scl[wv] = s;
      isum[wv] = acc;
    }
  }
  __syncthreads();

  const int r = lane & 15, gq = lane >> 4;
  i32x4 af[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) af[k] = frag[k * 64 + lane];

  const int64_t T = a.n_keys;
  const uint8_t* bits = a.bits + (int64_t)grp * T * mb;
  const uint16_t* norms = a.norms + (int64_t)grp * T;
  const float c0 = 1.2533141373155003f / (float)m;        // sqrt(pi/2) / m
  const bool out_lane = gq < group;
  const int h_out = gk * group + (out_lane ? gq : 0);
  float* out = a.scores + ((int64_t)b * a.q_heads + h_out) * T;
  const float s_out = out_lane ? scl[gq] * c0 : 0.0f;
  const float sumq_out = out_lane ? (float)isum[gq] : 0.0f;

  // A wave takes 32 keys at a time as two 16-key tiles, the even keys and the odd keys, so
  // that lane (gq, r) ends with keys 2r and 2r + 1 and stores them together: 16 lanes write
  // a whole 128-byte line of a query head's scores.  U tiles (U/2 pairs) per iteration, the
  // next U tiles' bits and norms in flight meanwhile.
  constexpr int U = PQ_SCORE_TILES;
  const int64_t n_pairs = (T + 31) >> 5;
  const int64_t stride = (int64_t)chunks_per_group * kWaves;
  // loads of clamped keys (always in bounds, no branches, so several stay in flight); a
  // key past the end only feeds its own output column, which is not stored
  auto fetch = [&](int64_t p0, uint32_t (&w)[U][(KS + 1) / 2], uint16_t (&nu)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = min((p0 + (u >> 1) * stride) * 32 + 2 * r + (u & 1), T - 1);
      load_key_bits<KS>(bits + key * mb + (mb >> 2) * gq, true, w[u]);
      nu[u] = norms[key];
    }
  };
  const bool pairs_aligned = (T & 1) == 0;                // float2 stores stay 8-byte aligned
  uint32_t wn[U][(KS + 1) / 2];
  uint16_t nn[U];
  int64_t pair = (int64_t)chunk * kWaves + wv;
  fetch(pair, wn, nn);
  for (; pair < n_pairs; pair += (U / 2) * stride) {
    uint32_t w[U][(KS + 1) / 2];
    uint16_t nu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      nu[u] = nn[u];
#pragma unroll
      for (int j = 0; j < (KS + 1) / 2; ++j) w[u][j] = wn[u][j];
    }
    fetch(pair + (U / 2) * stride, wn, nn);
#pragma unroll
    for (int up = 0; up < U / 2; ++up) {
      const int64_t pp = pair + up * stride;
      if (pp >= n_pairs) break;                                       // uniform
      float val[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int u = 2 * up + sub;
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const uint32_t w16 = (w[u][k >> 1] >> (16 * (k & 1))) & 0xffffu;
          const i32x4 bf = {(int)spread_nibble(w16 & 0xf), (int)spread_nibble((w16 >> 4) & 0xf),
                            (int)spread_nibble((w16 >> 8) & 0xf), (int)spread_nibble(w16 >> 12)};
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[k], bf, acc, 0, 0, 0);
        }
        // lane (gq, key): acc[l] = sum_i bit_i * limb_l of query head gq.  S = sum_i bit_i Q_i
        // is exact in int32 (|S| <= m * kLimbRange < 2^31); 2 S - sum Q then carries one fp32
        // rounding.
        const int S = acc[0] * 16384 + acc[1] * 128 + acc[2];
        val[sub] = f16_to_f32(nu[u]) * s_out * fmaf(2.0f, (float)S, -sumq_out);
      }
      const int64_t key = pp * 32 + 2 * r;
      if (out_lane) {
        if (pairs_aligned && key + 1 < T) {
          float2* o = reinterpret_cast<float2*>(out + key);
          if constexpr (ADD) {
            const float2 prev = *o;
            *o = make_float2(prev.x + val[0], prev.y + val[1]);
          } else {
            *o = make_float2(val[0], val[1]);
          }
        } else {
          if (key < T) out[key] = ADD ? out[key] + val[0] : val[0];
          if (key + 1 < T) out[key + 1] = ADD ? out[key + 1] + val[1] : val[1];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Two-stage score: query preparation
//
// For every query row r of a KV head: qrot = H (D q) and sq = G q in fp32, then both are
// quantized to integers Q = rint(v / s), s = max|v| / kLimbRange, split into three int8
// limbs Q = 16384 h2 + 128 h1 + h0, and written in the A-fragment order of
// v_mfma_i32_16x16x64_i8: limb l, K step k is a 1 KiB block whose 16 bytes at 16 L
// (lane L = 16 gq + r) are elements 64 k + 16 gq + 0..15 (code term) or
// (m/4) gq + 16 k + 0..15 (QJL term) of row r.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pq_query_rotate_kernel(const pqi::QueryPrepArgs a) {
  const int h = blockIdx.x / pqi::kScoreRows, r = blockIdx.x % pqi::kScoreRows;
  const int d = a.d, m = a.m;
  unsigned char* base = a.prep + (int64_t)h * pqi::prep_head_bytes(d, m);
  float* qrot = reinterpret_cast<float*>(base) + (int64_t)r * d;
  float* sq = reinterpret_cast<float*>(base + pqi::prep_off_sq(d)) + (int64_t)r * m;
  __shared__ float v[512];
  const bool live = r < a.n_q;
  const uint16_t* q = a.q + ((int64_t)h * a.n_q + r) * d;
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float x = live ? bf16_to_f32(q[e]) : 0.0f;
    if ((a.signs[e >> 3] >> (e & 7)) & 1) x = -x;
    v[e] = x;
  }
  __syncthreads();
  // in-place Walsh-Hadamard butterflies in Sylvester order
  for (int half = 1; half < d; half <<= 1) {
    for (int t = threadIdx.x; t < d / 2; t += blockDim.x) {
      const int i = (t / half) * 2 * half + (t % half);
      const float x0 = v[i], x1 = v[i + half];
      v[i] = x0 + x1;
      v[i + half] = x0 - x1;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < d; e += blockDim.x) qrot[e] = v[e];
  // G q of the live rows comes from the projection kernel; the padding rows stay zero
  if (!live)
    for (int n = threadIdx.x; n < m; n += blockDim.x) sq[n] = 0.0f;
}


// One workgroup per (head, 1024-word slice of the fragments): every workgroup finds the 32
// row scales itself, the first slice of a head also stores them.
constexpr int kPrepWordsPerGroup = 1024;

__global__ __launch_bounds__(256) void pq_query_quant_kernel(const pqi::QueryPrepArgs a, int slices) {
  const int h = blockIdx.x / slices, slice = blockIdx.x % slices;
  const int d = a.d, m = a.m;
  unsigned char* base = a.prep + (int64_t)h * pqi::prep_head_bytes(d, m);
  const float* qrot = reinterpret_cast<const float*>(base);
  const float* sq = reinterpret_cast<const float*>(base + pqi::prep_off_sq(d));
  float* scale_out = reinterpret_cast<float*>(base + pqi::prep_off_meta(d, m));    // [2][16]
  int* isum_out = reinterpret_cast<int*>(base + pqi::prep_off_meta(d, m) + 128);    // [2][16]
  __shared__ float scale[2 * pqi::kScoreRows];
  // row scales: 16 threads per query row (a quarter of a wave), both terms in turn
  const int row = threadIdx.x >> 4, sub = threadIdx.x & 15;
  for (int term = 0; term < 2; ++term) {
    const int len = term == 0 ? d : m;
    const float* src = term == 0 ? qrot + (int64_t)row * d : sq + (int64_t)row * m;
    float amax = 0.0f;
    for (int e = sub; e < len; e += 16) amax = fmaxf(amax, fabsf(src[e]));
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const float sc = amax / pqi::kLimbRange;
    const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
    int acc = 0;
    for (int e = sub; e < len; e += 16) acc += (int)rintf(src[e] * inv);
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 16);
    if (sub == 0) {
      const int job = term * pqi::kScoreRows + row;
      scale[job] = inv;                                  // the reciprocal, used below
      if (slice == 0) {
        scale_out[job] = sc;
        isum_out[job] = acc;
      }
    }
  }
  __syncthreads();
  // fragment bytes, one 32-bit word (4 consecutive K elements) per thread step
  const int kc = d / 64, kq = m / 64;
  uint32_t* fc = reinterpret_cast<uint32_t*>(base + pqi::prep_off_frag_c(d, m));
  uint32_t* fq = reinterpret_cast<uint32_t*>(base + pqi::prep_off_frag_q(d, m));
  const int words_c = 3 * kc * 256, words_q = 3 * kq * 256;
  const int w_end = min(words_c + words_q, (slice + 1) * kPrepWordsPerGroup);
  for (int wi = slice * kPrepWordsPerGroup + threadIdx.x; wi < w_end; wi += blockDim.x) {
    const bool qjl = wi >= words_c;
    const int w = qjl ? wi - words_c : wi;
    const int blk = w >> 8, inblk = w & 255;          // 1 KiB block = 256 words
    const int nk = qjl ? kq : kc;
    const int l = blk / nk, k = blk % nk;
    const int L = inblk >> 2, byte0 = 4 * (inblk & 3);
    const int r = L & 15, gq = L >> 4;
    const float* src = qjl ? sq + (int64_t)r * m : qrot + (int64_t)r * d;
    const float inv = scale[(qjl ? pqi::kScoreRows : 0) + r];
    uint32_t word = 0;
    for (int b = 0; b < 4; ++b) {
      const int i = byte0 + b;
      const int e = qjl ? (m / 4) * gq + 16 * k + i : 64 * k + 16 * gq + i;
      word |= (uint32_t)(limb_of((int)rintf(src[e] * inv), l) & 0xff) << (8 * b);
    }
    (qjl ? fq : fc)[w] = word;
  }
}

// ------------------------------------------------------------------------------------------
// Two-stage score on the int8 matrix cores.
//
// score = n16/d <qrot, c[code]> + rnorm16 sqrt(pi/2)/m <sq, 2 b - 1>.  The codebook is
// antisymmetric and code 2^b-1-k is the bitwise complement of k, so c[code] is a sum of
// odd Walsh functions of the code bits: c[code] = sum_p alpha_p s_p(code) with
// s_p = 2 u_p - 1, u_p = parity(code & mask_p).  Each <qrot, s_p> is then an exact
// integer product of the query limbs with 0/1 bytes, like the QJL term.  A rows: the 16
// query rows; B columns: 16 tokens; lane (token r, group gq) holds code bytes
// 64 k + 16 gq + 0..15 of its token.
// ------------------------------------------------------------------------------------------
// Bytes {0, 1}: parity of (code & mask) for the four codes of w (mask folds to a constant
// once the plane loop is unrolled).
__device__ __forceinline__ int plane_bytes(uint32_t w, uint32_t mask) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (mask & (1u << i)) x ^= w >> i;
  return (int)(x & 0x01010101u);
}

__device__ __forceinline__ i32x4 plane_frag(const uint4& w, uint32_t mask) {
  return i32x4{plane_bytes(w.x, mask), plane_bytes(w.y, mask), plane_bytes(w.z, mask), plane_bytes(w.w, mask)};
}

// KQT: 0 = no QJL term, D/64 = the QJL term with m = d (bits of a key loaded as one vector),
// -1 = any other m (bits read per K step).  PK: codes bit-packed at BITS bits; a lane's 16
// codes of a K step are 2 BITS bytes of the token's stream, unpacked to bytes when used.
template <int D, int BITS, int KQT, bool PK>
__global__ __launch_bounds__(kThreads) void pq_score_kernel(const pqi::TwoStageArgs a, int chunks_per_group) {
  constexpr int KC = D / 64;
  constexpr int NP = 1 << (BITS - 1);
  constexpr bool QJL = KQT != 0;
  constexpr int KQB = KQT > 0 ? KQT : 1;                  // register words for the fixed-m bits
  const int m = QJL ? a.m : 0;
  const int KQ = m >> 6, mb = m >> 3;
  const int grp = blockIdx.x / chunks_per_group, chunk = blockIdx.x % chunks_per_group;

  extern __shared__ __align__(16) unsigned char smem[];
  const unsigned char* src = a.prep + (int64_t)grp * pqi::prep_head_bytes(D, m);
  {
    const int64_t off = pqi::prep_off_meta(D, m);
    const int nbytes = (int)(pqi::prep_head_bytes(D, m) - off);
    const uint4* s4 = reinterpret_cast<const uint4*>(src + off);
    uint4* d4 = reinterpret_cast<uint4*>(smem);
    for (int i = threadIdx.x; i < nbytes / 16; i += blockDim.x) d4[i] = s4[i];
  }
  __syncthreads();
  const float* scale = reinterpret_cast<const float*>(smem);
  const int* isum = reinterpret_cast<const int*>(smem + 128);
  const i32x4* fc = reinterpret_cast<const i32x4*>(smem + 256);
  const i32x4* fq = fc + 3 * KC * 64;

  const int lane = threadIdx.x & 63;
  const int r = lane & 15, gq = lane >> 4;
  const int64_t T = a.n_tok;
  const uint8_t* codes = a.codes + (int64_t)grp * T * (PK ? D * BITS / 8 : D);
  const uint16_t* norms = a.norms + (int64_t)grp * T;
  const uint8_t* qbits = QJL ? a.qbits + (int64_t)grp * T * mb : nullptr;
  const uint16_t* rnorms = QJL ? a.rnorms + (int64_t)grp * T : nullptr;
  float* out = a.scores + (int64_t)grp * a.n_q * T;
  const double cq = QJL ? 1.2533141373155003 / (double)m : 0.0;     // sqrt(pi/2) / m

  // one tile's inputs; tokens past the end are clamped to the last token (always in bounds,
  // no branches); such a token only feeds its own output column, which is not stored
  constexpr int PW = PK ? (2 * BITS + 3) / 4 : 4;       // dwords of a lane's 16 codes
  struct Inputs {
    uint32_t cw[KC][PW];
    uint32_t qb[(KQB + 1) / 2];
    uint16_t n16, rn16;
  };
  auto fetch = [&](int64_t tok_u, Inputs& in) {
    const int64_t tok = min(tok_u, T - 1);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if constexpr (PK) {
        load_code_bytes<2 * BITS>(codes + tok * (D * BITS / 8) + (64 * k + 16 * gq) * BITS / 8, true, in.cw[k]);
      } else {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + tok * D + 64 * k + 16 * gq));
        in.cw[k][0] = w.x; in.cw[k][1] = w.y; in.cw[k][2] = w.z; in.cw[k][3] = w.w;
      }
    }
    in.n16 = norms[tok];
    if constexpr (QJL) in.rn16 = rnorms[tok];
    if constexpr (KQT > 0) load_key_bits<KQT>(qbits + tok * mb + (mb >> 2) * gq, true, in.qb);
  };

  // the first term's plane weights and the QJL factor in fp32: the integer sums are exact, and
  // an fp32 combination of them lies within ~1e-6 of the scores' L1 size
  float alpha_f[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) alpha_f[p] = (float)a.alpha[p];
  const float cqf = (float)cq;

  // the scores of the 16 tokens of one tile for this lane's four query rows
  auto score_tile = [&](const Inputs& in, int64_t tok, float (&val)[4]) {
    i32x4 acc[NP][3];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int l = 0; l < 3; ++l) acc[p][l] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const i32x4 a0 = fc[(0 * KC + k) * 64 + lane];
      const i32x4 a1 = fc[(1 * KC + k) * 64 + lane];
      const i32x4 a2 = fc[(2 * KC + k) * 64 + lane];
      uint4 cb;                                           // the 16 codes as bytes
      if constexpr (PK) {
        uint32_t u[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) u[i >> 2] |= stream_code<BITS>(in.cw[k], i) << (8 * (i & 3));
        cb = make_uint4(u[0], u[1], u[2], u[3]);
      } else {
        cb = make_uint4(in.cw[k][0], in.cw[k][1], in.cw[k][2], in.cw[k][3]);
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const i32x4 b = plane_frag(cb, pqi::plane_mask(BITS, p));
        acc[p][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b, acc[p][0], 0, 0, 0);
        acc[p][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b, acc[p][1], 0, 0, 0);
        acc[p][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b, acc[p][2], 0, 0, 0);
      }
      // d = 512: one K chunk's fragments live at a time (two waves per SIMD instead of one)
      if constexpr (D >= 512) __builtin_amdgcn_sched_barrier(0);
    }
    i32x4 accq[3] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
    auto qstep = [&](int k, uint32_t w16) {
      const i32x4 b = {(int)spread_nibble(w16 & 0xf), (int)spread_nibble((w16 >> 4) & 0xf),
                       (int)spread_nibble((w16 >> 8) & 0xf), (int)spread_nibble(w16 >> 12)};
      accq[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fq[(0 * KQ + k) * 64 + lane], b, accq[0], 0, 0, 0);
      accq[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fq[(1 * KQ + k) * 64 + lane], b, accq[1], 0, 0, 0);
      accq[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fq[(2 * KQ + k) * 64 + lane], b, accq[2], 0, 0, 0);
    };
    if constexpr (KQT > 0) {
#pragma unroll
      for (int k = 0; k < KQT; ++k) qstep(k, (in.qb[k >> 1] >> (16 * (k & 1))) & 0xffffu);
    } else if constexpr (KQT < 0) {
      const uint8_t* kb = qbits + min(tok, T - 1) * mb + (mb >> 2) * gq;
      for (int k = 0; k < KQ; ++k) qstep(k, *reinterpret_cast<const uint16_t*>(kb + 2 * k));
    }
    const float n16 = f16_to_f32(in.n16) * (1.0f / (float)D);
    const float rn = QJL ? f16_to_f32(in.rn16) * cqf : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = min(4 * gq + i, 15);
      // 2 S - isum = sum_e Q_e (2 u_e - 1) is an int32 (|.| <= sum |Q_e| < 2^31): formed in
      // wrapping 32-bit arithmetic from the limb sums, exact, then one conversion per plane
      float first = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t S = 16384u * (uint32_t)acc[p][0][i] + 128u * (uint32_t)acc[p][1][i] + (uint32_t)acc[p][2][i];
        first = fmaf(alpha_f[p], (float)(int)(2u * S - (uint32_t)isum[qi]), first);
      }
      float v = n16 * scale[qi] * first;
      if constexpr (QJL) {
        const uint32_t S = 16384u * (uint32_t)accq[0][i] + 128u * (uint32_t)accq[1][i] + (uint32_t)accq[2][i];
        v = fmaf(rn * scale[16 + qi], (float)(int)(2u * S - (uint32_t)isum[16 + qi]), v);
      }
      val[i] = v;
    }
  };

  // A wave takes 32 tokens at a time as two tiles, the even tokens and the odd tokens, so that
  // lane (gq, r) ends with tokens 2r and 2r + 1 of its query rows and stores them together:
  // 16 lanes write a whole 128-byte line of a query row.  One tile's inputs are in flight
  // while the other is scored.
  const int64_t n_pairs = (T + 31) >> 5;
  const int64_t stride = (int64_t)chunks_per_group * kWaves;
  const bool pairs_aligned = (T & 1) == 0;               // a query row's pair starts 8-byte aligned
  int64_t pair = (int64_t)chunk * kWaves + (threadIdx.x >> 6);
  Inputs nxt;
  if (pair < n_pairs) fetch(32 * pair + 2 * r, nxt);
  for (; pair < n_pairs; pair += stride) {
    float val[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const Inputs in = nxt;
      if (sub == 0) fetch(32 * pair + 2 * r + 1, nxt);
      else if (pair + stride < n_pairs) fetch(32 * (pair + stride) + 2 * r, nxt);   // uniform
      score_tile(in, 32 * pair + 2 * r + sub, val[sub]);
      // the scores are taken here: otherwise their arithmetic sinks to the paired store below
      // and keeps every accumulator of the first tile live through the second
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(val[sub][i]));
      __builtin_amdgcn_sched_barrier(0);                  // one tile's products live at a time
    }
    const int64_t tok = 32 * pair + 2 * r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = 4 * gq + i;
      if (qi < a.n_q) {
        float* o = out + (int64_t)qi * T + tok;
        if (pairs_aligned && tok + 1 < T) {
          *reinterpret_cast<float2*>(o) = make_float2(val[0][i], val[1][i]);
        } else {
          if (tok < T) o[0] = val[0][i];
          if (tok + 1 < T) o[1] = val[1][i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode attention over the quantized cache, fused: every key code is scored and every value
// code accumulated in one pass, and nothing is decoded to memory.
//
// A wave takes a range of 16-token tiles of one KV head, the head's 16 query rows and one
// slice of attn_cols(d) value columns.  The scores are the two-stage products above with the
// operands swapped, so they come out transposed: lane (query c = lane & 15, g = lane >> 4)
// holds the scores of tokens 4 g + i, i = 0..3, which is the A-operand layout of
// v_mfma_f32_16x16x16_f16 for the probability tile P[query][token].  The dequantized value is
// linear in its centroid vector, so
//     sum_t p_t vhat_t = D . H (sum_t p_t n16_t / d . c[code_t]),
// and the wave accumulates O = P' C on the matrix cores in the rotated basis
// (P'[q][t] = p_qt n16_t / d, C[t][e] = c[code_te]); the combine kernel applies the inverse
// rotation once per query.  P' and C enter as fp16 hi + lo pairs (products hi.hi + hi.lo +
// lo.hi), about 22 significant bits each.  Value column e of N-tile j sits in lane n = lane & 15
// as e = (d/16) n + slice * NT + j, so a lane reads NT consecutive codes of a token.  Softmax
// is online in base 2 (logits times log2 e).
// ------------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

__device__ __forceinline__ uint32_t f16_split_pair(float x0, float x1, uint32_t& lo) {
  const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
  const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  return (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
}

__device__ __forceinline__ f16x4 as_f16x4(uint32_t w0, uint32_t w1) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  return __builtin_bit_cast(f16x4, (u32x2){w0, w1});
}

// Byte k of x as a 32-bit value (one v_perm_b32: selector 0x0c is a zero byte).
__device__ __forceinline__ uint32_t byte_at(uint32_t x, int k) {
  return __builtin_amdgcn_perm(0u, x, 0x0c0c0c00u | (uint32_t)k);
}

template <int D, int BITS, int KQT, bool PK>
__global__ __launch_bounds__(kThreads) void pq_attend_kernel(const pqi::AttnArgs a) {
  constexpr int KC = D / 64;
  constexpr int NP = 1 << (BITS - 1);
  constexpr bool QJL = KQT != 0;
  constexpr int KQB = KQT > 0 ? KQT : 1;
  constexpr int DC = pqi::attn_cols(D), CS = D / DC, NT = DC / 16, RUN = D / 16;
  constexpr uint32_t CMASK = (1u << BITS) - 1u;
  const int m = QJL ? a.m : 0;
  const int KQ = m >> 6, mb = m >> 3;
  // workgroup = (head, column slice, group of kWaves ranges); wave = one range
  const int grp = blockIdx.x % a.n_parts;
  const int cs = (blockIdx.x / a.n_parts) % CS;
  const int head = blockIdx.x / (a.n_parts * CS);
  const int wv = (int)(threadIdx.x >> 6);
  const int range = grp * kWaves + wv;
  const bool live = range < a.n_ranges;

  // LDS: the value centroids as a fixed array (a code times 4 is its entry's address, with
  // no base to add), the query fragments of the head after them
  __shared__ uint32_t ctab[1 << pqi::kMaxScoreBits];
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t meta = pqi::prep_off_meta(D, m);
  const int nbytes = (int)(pqi::prep_head_bytes(D, m) - meta);
  {
    const uint4* s4 = reinterpret_cast<const uint4*>(a.prep + (int64_t)head * pqi::prep_head_bytes(D, m) + meta);
    uint4* d4 = reinterpret_cast<uint4*>(smem);
    for (int i = threadIdx.x; i < nbytes / 16; i += blockDim.x) d4[i] = s4[i];
  }
  // value centroids as fp16 pairs, hi | lo << 16
  if (threadIdx.x < (1 << BITS)) {
    uint32_t lo;
    const uint32_t hi = f16_split_pair(a.vcent[threadIdx.x], 0.0f, lo);
    ctab[threadIdx.x] = (hi & 0xffffu) | (lo << 16);
  }
  __syncthreads();

  const float* scale = reinterpret_cast<const float*>(smem);
  const int* isum = reinterpret_cast<const int*>(smem + 128);
  const i32x4* fc = reinterpret_cast<const i32x4*>(smem + 256);
  const i32x4* fq = fc + 3 * KC * 64;

  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t T = a.n_tok;
  const int64_t n_tiles = (T + 15) >> 4;
  const int64_t t_begin = live ? (int64_t)range * a.tiles_per_range : 0;
  const int64_t t_end = live ? min(n_tiles, t_begin + a.tiles_per_range) : 0;
  const int64_t hoff = (int64_t)head * T;
  constexpr int RB = PK ? D * BITS / 8 : D;              // code bytes of a token
  const uint8_t* kcodes = a.k_codes + hoff * RB;
  const uint8_t* vcodes = a.v_codes + hoff * RB;
  const uint16_t* knorms = a.k_norms + hoff;
  const uint16_t* vnorms = a.v_norms + hoff;
  const uint8_t* qbits = QJL ? a.k_qbits + hoff * mb : nullptr;
  const uint16_t* rnorms = QJL ? a.k_rnorms + hoff : nullptr;
  const double cq = QJL ? 1.2533141373155003 / (double)m : 0.0;     // sqrt(pi/2) / m

  // one tile's inputs; tokens past the end are clamped to the last token (always in bounds),
  // and their probabilities are set to zero.  The key inputs of the next tile are fetched once
  // the current ones are used (they load during the softmax and the value product), the value
  // inputs once the value product is done (they load during the next scores): one copy of each
  // is live at a time.
  constexpr int PW = PK ? (2 * BITS + 3) / 4 : 4;       // dwords of a lane's 16 key codes
  constexpr int VL = NT * BITS;                          // bits of a lane's packed value-code run
  constexpr int VW = PK ? (VL + 31) / 32 : NT / 4;       // dwords of a lane's NT value codes
  struct KeyIn {
    uint32_t cw[KC][PW];
    uint32_t qb[(KQB + 1) / 2];
    uint16_t kn, rn;      // key norm and residual norm of token r of the tile (raw loads: no
                          // arithmetic on them here, which would wait for the whole fetch)
  };
  struct ValIn {
    uint32_t vr[4][VW];
    uint16_t vn;          // value norm of token r of the tile
  };
  auto fetch_k = [&](int64_t tile, KeyIn& in) {
    const int64_t tok = min(tile * 16 + r, T - 1);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if constexpr (PK) {
        load_code_bytes<2 * BITS>(kcodes + tok * RB + (64 * k + 16 * g) * BITS / 8, true, in.cw[k]);
      } else {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kcodes + tok * RB + 64 * k + 16 * g));
        in.cw[k][0] = w.x; in.cw[k][1] = w.y; in.cw[k][2] = w.z; in.cw[k][3] = w.w;
      }
    }
    in.kn = knorms[tok];
    if constexpr (QJL) in.rn = rnorms[tok];
    if constexpr (KQT > 0) load_key_bits<KQT>(qbits + tok * mb + (mb >> 2) * g, true, in.qb);
  };
  auto fetch_v = [&](int64_t tile, ValIn& in) {
    in.vn = vnorms[min(tile * 16 + r, T - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t vt = min(tile * 16 + 4 * g + i, T - 1);
      const int e0 = RUN * r + cs * NT;                  // first value column of the lane
      if constexpr (PK) {
        // the dwords holding bits s .. s + VL - 1 of the token's stream, shifted down by s
        const uint32_t* row = reinterpret_cast<const uint32_t*>(vcodes + vt * RB);
        const int s = e0 * BITS, k0 = s >> 5, kl = (s + VL - 1) >> 5;
        uint32_t w[VW + 1];
#pragma unroll
        for (int u = 0; u <= VW; ++u) w[u] = row[min(k0 + u, kl)];
#pragma unroll
        for (int u = 0; u < VW; ++u) in.vr[i][u] = __builtin_amdgcn_alignbit(w[u + 1], w[u], (uint32_t)(s & 31));
      } else {
#pragma unroll
        for (int u = 0; u < VW; u += 2) {
          if (u + 1 < VW) {
            const uint2 w = *reinterpret_cast<const uint2*>(vcodes + vt * RB + e0 + 4 * u);
            in.vr[i][u] = w.x; in.vr[i][u + 1] = w.y;
          } else {
            in.vr[i][u] = *reinterpret_cast<const uint32_t*>(vcodes + vt * RB + e0 + 4 * u);
          }
        }
      }
    }
  };

  const float isc = scale[r], isq = QJL ? scale[16 + r] : 0.0f;
  const int sum_c = isum[r], sum_q = QJL ? isum[16 + r] : 0;
  float mx = -INFINITY, ls = 0.0f;
  f32x4 o[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  KeyIn kin;
  ValIn vin;
  if (live) {                                            // every live range holds at least one tile
    fetch_k(t_begin, kin);
    fetch_v(t_begin, vin);
  }
  for (int64_t tile = t_begin; tile < t_end; ++tile) {
    // the query fragments are read from LDS in every tile rather than held in registers
    // across the loop (3 (d + m) / 16 registers that would cost the wave its occupancy)
    asm volatile("" ::: "memory");
    // next tile, or this one again on the last pass: the fetches stay unconditional, so the
    // count of loads in flight is the same on every path and each wait covers only its data
    const int64_t nt = tile + 1 < t_end ? tile + 1 : tile;
    // --- scores S^T: rows = tokens, columns = queries
    i32x4 acc[NP][3];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int l = 0; l < 3; ++l) acc[p][l] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const i32x4 a0 = fc[(0 * KC + k) * 64 + lane];
      const i32x4 a1 = fc[(1 * KC + k) * 64 + lane];
      const i32x4 a2 = fc[(2 * KC + k) * 64 + lane];
      uint4 cb;
      if constexpr (PK) {
        uint32_t u[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) u[i >> 2] |= stream_code<BITS>(kin.cw[k], i) << (8 * (i & 3));
        cb = make_uint4(u[0], u[1], u[2], u[3]);
      } else {
        cb = make_uint4(kin.cw[k][0], kin.cw[k][1], kin.cw[k][2], kin.cw[k][3]);
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const i32x4 b = plane_frag(cb, pqi::plane_mask(BITS, p));
        acc[p][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a0, acc[p][0], 0, 0, 0);
        acc[p][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a1, acc[p][1], 0, 0, 0);
        acc[p][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a2, acc[p][2], 0, 0, 0);
      }
    }
    i32x4 accq[3] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
    auto qstep = [&](int k, uint32_t w16) {
      const i32x4 b = {(int)spread_nibble(w16 & 0xf), (int)spread_nibble((w16 >> 4) & 0xf),
                       (int)spread_nibble((w16 >> 8) & 0xf), (int)spread_nibble(w16 >> 12)};
      accq[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, fq[(0 * KQ + k) * 64 + lane], accq[0], 0, 0, 0);
      accq[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, fq[(1 * KQ + k) * 64 + lane], accq[1], 0, 0, 0);
      accq[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, fq[(2 * KQ + k) * 64 + lane], accq[2], 0, 0, 0);
    };
    if constexpr (KQT > 0) {
#pragma unroll
      for (int k = 0; k < KQT; ++k) qstep(k, (kin.qb[k >> 1] >> (16 * (k & 1))) & 0xffffu);
    } else if constexpr (KQT < 0) {
      const uint8_t* kb = qbits + min(tile * 16 + r, T - 1) * mb + (mb >> 2) * g;
      for (int k = 0; k < KQ; ++k) qstep(k, *reinterpret_cast<const uint16_t*>(kb + 2 * k));
    }
    // --- logits of query r at tokens 4 g + i (base 2); the norms come from the lanes that
    // fetched those tokens
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t kn = (uint32_t)__shfl((int)((uint32_t)kin.kn | (QJL ? (uint32_t)kin.rn << 16 : 0u)), 4 * g + i);
      // 2 S - isum = sum_e Q_e (2 u_e - 1) is an int32 (|.| <= sum |Q_e| < 2^31): formed in
      // wrapping 32-bit arithmetic from the limb sums, exact, then one conversion per plane
      double first = 0.0;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t S = 16384u * (uint32_t)acc[p][0][i] + 128u * (uint32_t)acc[p][1][i] + (uint32_t)acc[p][2][i];
        first += a.alpha[p] * (double)(int)(2u * S - (uint32_t)sum_c);
      }
      double val = (double)f16_to_f32((uint16_t)(kn & 0xffffu)) / (double)D * (double)isc * first;
      if constexpr (QJL) {
        const uint32_t S = 16384u * (uint32_t)accq[0][i] + 128u * (uint32_t)accq[1][i] + (uint32_t)accq[2][i];
        val += (double)f16_to_f32((uint16_t)(kn >> 16)) * cq * (double)isq * (double)(int)(2u * S - (uint32_t)sum_q);
      }
      z[i] = tile * 16 + 4 * g + i < T ? (float)(val * a.scale_log2) : -INFINITY;
    }
    fetch_k(nt, kin);
    asm volatile("" ::: "memory");                      // issue those loads here, not after the product
    // --- online softmax; every tile holds a live token, so the tile maximum is finite
    float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(mx, mt);
    const float al = exp2f(mx - mn);
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = exp2f(z[i] - mn);
    ls = ls * al + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    mx = mn;
    if (__any(al != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(al, 4 * g + i);          // scale of query row 4 g + i
#pragma unroll
        for (int j = 0; j < NT; ++j) o[j][i] *= ai;
      }
    }
    // --- P' = p . n16_v / d as fp16 hi + lo
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t vn = (uint32_t)__shfl((int)vin.vn, 4 * g + i);
      w[i] = pv[i] * (f16_to_f32((uint16_t)vn) * (1.0f / (float)D));
    }
    uint32_t pl0, pl1;
    const uint32_t ph0 = f16_split_pair(w[0], w[1], pl0);
    const uint32_t ph1 = f16_split_pair(w[2], w[3], pl1);
    const f16x4 Ah = as_f16x4(ph0, ph1), Al = as_f16x4(pl0, pl1);
    // --- O += P' C, N-tile by N-tile; byte codes are masked and scaled by 4 a dword at a
    // time, so each entry address is one byte extract
    uint32_t va[4][VW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int u = 0; u < VW; ++u) va[i][u] = PK ? vin.vr[i][u] : (vin.vr[i][u] & (CMASK * 0x01010101u)) << 2;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      uint32_t t4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (a byte select per code is faster up to d = 256; at d = 512, at one wave per SIMD,
        // the compiler's shift-and-mask measured faster)
        const uint32_t addr = PK ? stream_code<BITS>(va[i], j) * 4u
                                 : D >= 512 ? __builtin_amdgcn_ubfe(va[i][j >> 2], 8 * (j & 3), 8) : byte_at(va[i][j >> 2], j & 3);
        t4[i] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(ctab) + addr);
      }
      const f16x4 Bh = as_f16x4(__builtin_amdgcn_perm(t4[1], t4[0], 0x05040100u),
                                __builtin_amdgcn_perm(t4[3], t4[2], 0x05040100u));
      const f16x4 Bl = as_f16x4(__builtin_amdgcn_perm(t4[1], t4[0], 0x07060302u),
                                __builtin_amdgcn_perm(t4[3], t4[2], 0x07060302u));
      o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ah, Bh, o[j], 0, 0, 0);
      o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ah, Bl, o[j], 0, 0, 0);
      o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(Al, Bh, o[j], 0, 0, 0);
    }
    fetch_v(nt, vin);
  }
  // merge the kWaves ranges of the workgroup (a wave without tiles holds max -inf, sum 0, O 0)
  // into one partial result: rescale to the common maximum, then sum in a fixed order through
  // two LDS slots (waves 2, 3 into 0, 1; then wave 1 into 0).  The prep region is reused.
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  __syncthreads();
  float* xm = reinterpret_cast<float*>(smem);           // [kWaves][16] maxima, then [kWaves][16] sums
  float* slot = xm + 2 * kWaves * 16;                    // [2][16][DC]
  if (g == 0) {
    xm[wv * 16 + r] = mx;
    xm[(kWaves + wv) * 16 + r] = ls;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qr = 4 * g + i;
    float M = xm[qr];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, xm[w * 16 + qr]);
    const float f = exp2f(xm[wv * 16 + qr] - M);        // 0 for a wave without tiles
#pragma unroll
    for (int j = 0; j < NT; ++j) o[j][i] *= f;
  }
  auto put = [&](float* dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NT; j += 4)
        *reinterpret_cast<float4*>(dst + (4 * g + i) * DC + NT * r + j) =
            make_float4(o[j][i], o[j + 1][i], o[j + 2][i], o[j + 3][i]);
  };
  auto add = [&](const float* src) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NT; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + (4 * g + i) * DC + NT * r + j);
        o[j][i] += v.x; o[j + 1][i] += v.y; o[j + 2][i] += v.z; o[j + 3][i] += v.w;
      }
  };
  if (wv >= 2) put(slot + (wv - 2) * 16 * DC);
  __syncthreads();
  if (wv < 2) add(slot + wv * 16 * DC);
  __syncthreads();
  if (wv == 1) put(slot);
  __syncthreads();
  if (wv == 0) {
    add(slot);
    const int64_t part = (int64_t)head * a.n_parts + grp;
    if (cs == 0 && g == 0) {
      float M = xm[r], L = 0.0f;
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, xm[w * 16 + r]);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) L += xm[(kWaves + w) * 16 + r] * exp2f(xm[w * 16 + r] - M);
      reinterpret_cast<float2*>(a.work_ml)[part * 16 + r] = make_float2(M, L);
    }
    float* po = a.work_o + part * 16 * D + RUN * r + cs * NT;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NT; j += 4)
        *reinterpret_cast<float4*>(po + (4 * g + i) * D + j) = make_float4(o[j][i], o[j + 1][i], o[j + 2][i], o[j + 3][i]);
  }
}

// Merge the partial results of one (head, query) with the unquantized window, rotate back and
// normalise.
constexpr int kCombineThreads = 512;

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) r += red[w];
  return r;
}

template <int D>
__global__ __launch_bounds__(kCombineThreads) void pq_attend_combine_kernel(const pqi::AttnArgs a) {
  const int h = blockIdx.x / a.n_q, qi = blockIdx.x % a.n_q;
  const int R = a.n_parts, W = (int)a.n_win;
  const int tid = threadIdx.x;
  __shared__ float x[D];
  __shared__ float ew[pqi::kAttnMaxWin];
  __shared__ float red_f[kCombineThreads / 64];
  __shared__ double red_d[kCombineThreads / 64];
  extern __shared__ float wr[];                          // [R] weights of the partials
  // window logits (base 2): tpt threads per window token (neighbouring lanes, at most 16), each
  // summing every tpt-th 8-value chunk; the query in LDS as fp32
  if (W > 0) {
    const uint16_t* q = a.q + ((int64_t)h * a.n_q + qi) * D;
    for (int e = tid; e < D; e += kCombineThreads) x[e] = bf16_to_f32(q[e]);
    __syncthreads();
    int tpt = 1;
    while (tpt < 16 && tpt * 2 * W <= kCombineThreads) tpt *= 2;
    const int part = tid % tpt;
    // the lanes of a token group run the same trips (they share w), so the group's shuffles
    // below always find their partners active
    for (int w = tid / tpt; w < W; w += kCombineThreads / tpt) {
      const uint4* kw = reinterpret_cast<const uint4*>(a.k_win + ((int64_t)h * W + w) * D);
      // products of bf16 values are exact in fp32; the sums run in double
      double s0 = 0.0, s1 = 0.0;
#pragma unroll 4
      for (int c = part; c < D / 8; c += tpt) {
        const uint4 u = kw[c];
        const float* qq = x + 8 * c;
        s0 += (double)(qq[0] * bf16_lo(u.x)) + (double)(qq[2] * bf16_lo(u.y));
        s1 += (double)(qq[1] * bf16_hi(u.x)) + (double)(qq[3] * bf16_hi(u.y));
        s0 += (double)(qq[4] * bf16_lo(u.z)) + (double)(qq[6] * bf16_lo(u.w));
        s1 += (double)(qq[5] * bf16_hi(u.z)) + (double)(qq[7] * bf16_hi(u.w));
      }
      double sw = s0 + s1;
      for (int o = 1; o < tpt; o <<= 1) sw += __shfl_xor(sw, o);
      if (part == 0) ew[w] = (float)(sw * a.scale_log2);
    }
  }
  __syncthreads();
  const float2* ml = reinterpret_cast<const float2*>(a.work_ml) + (int64_t)h * R * 16 + qi;
  float mloc = -INFINITY;
  for (int t = tid; t < R; t += kCombineThreads) mloc = fmaxf(mloc, ml[t * 16].x);
  for (int t = tid; t < W; t += kCombineThreads) mloc = fmaxf(mloc, ew[t]);
  const float M = block_max(mloc, red_f);
  double lsum = 0.0;
  for (int t = tid; t < R; t += kCombineThreads) {
    const float2 v = ml[t * 16];
    const float f = exp2f(v.x - M);
    wr[t] = f;
    lsum += (double)f * (double)v.y;
  }
  for (int t = tid; t < W; t += kCombineThreads) {
    const float f = exp2f(ew[t] - M);
    ew[t] = f;
    lsum += (double)f;
  }
  const double L = block_sum(lsum, red_d);               // its barriers also publish wr and ew
  // weighted sum of the partial outputs: thread (column group cg, row class par) sums float4
  // columns over partials par, par + NPAR, ...; the row classes meet in LDS
  constexpr int C4 = D / 4, NPAR = kCombineThreads / C4;
  __shared__ float4 red4[NPAR][C4];
  const int cg = tid % C4, par = tid / C4;
  {
    const float4* po4 = reinterpret_cast<const float4*>(a.work_o + (int64_t)h * R * 16 * D + (int64_t)qi * D);
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
    for (int t = par; t < R; t += NPAR) {
      const float4 v = po4[(int64_t)t * 16 * C4 + cg];
      const float w = wr[t];
      acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
    }
    red4[par][cg] = acc;
  }
  __syncthreads();
  for (int e = tid; e < D; e += kCombineThreads) {
    float v = 0.0f;
    for (int p = 0; p < NPAR; ++p) v += reinterpret_cast<const float*>(red4[p])[e];
    x[e] = v;
  }
  __syncthreads();
  // inverse rotation: Walsh-Hadamard butterflies in Sylvester order
  for (int half = 1; half < D; half <<= 1) {
    for (int t = tid; t < D / 2; t += kCombineThreads) {
      const int i = (t / half) * 2 * half + (t % half);
      const float x0 = x[i], x1 = x[i + half];
      x[i] = x0 + x1;
      x[i + half] = x0 - x1;
    }
    __syncthreads();
  }
  // window values, same thread layout (four bf16 columns per load)
  {
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const uint2* vw = reinterpret_cast<const uint2*>(a.v_win + (int64_t)h * W * D);
#pragma unroll 8
    for (int w = par; w < W; w += NPAR) {
      const uint2 u = vw[(int64_t)w * C4 + cg];
      const float f = ew[w];
      acc.x = fmaf(f, bf16_lo(u.x), acc.x); acc.y = fmaf(f, bf16_hi(u.x), acc.y);
      acc.z = fmaf(f, bf16_lo(u.y), acc.z); acc.w = fmaf(f, bf16_hi(u.y), acc.w);
    }
    red4[par][cg] = acc;
  }
  __syncthreads();
  float* out = a.out + ((int64_t)h * a.n_q + qi) * D;
  for (int e = tid; e < D; e += kCombineThreads) {
    float v = ((a.v_signs[e >> 3] >> (e & 7)) & 1) ? -x[e] : x[e];
    for (int p = 0; p < NPAR; ++p) v += reinterpret_cast<const float*>(red4[p])[e];
    out[e] = (float)((double)v / L);
  }
}

// ------------------------------------------------------------------------------------------
// Block-diagonal rotation (block sizes that are not powers of two).  One wave per block with a
// grid stride; the block lives in LDS as fp32 (d floats per wave), each power-of-two part is
// transformed by in-LDS butterflies (a wave's LDS operations complete in program order, so no
// barrier is needed between stages), and the per-part factor sqrt(d / d_k) comes from a table
// shared by the workgroup.  Codes by bisection over the boundaries (count of boundaries below).
// ------------------------------------------------------------------------------------------
// Elements live in LDS with 4 words of padding after every 64: element e at word bd_pad(e),
// so that lanes reading 64 consecutive elements each (the lowest stages) start on different
// bank groups.
__device__ __forceinline__ int bd_pad(int e) { return e + ((e >> 6) << 2); }
// LDS words of one block (per wave)
__host__ __device__ constexpr int bd_words(int d) { return d + (d >> 6) * 4 + 4; }

// R stages of the butterfly of one part (offset o, size s) starting at element bit b0 >= 6:
// each lane takes groups of 2^R elements spaced 2^b0 apart (padded spacing 2^b0 + 2^(b0-4)),
// transforms them in registers and writes them back (R stages per LDS round trip instead of
// one).
template <int R, int QG>
__device__ __forceinline__ void bd_pass(float* xb, int o, int s, int b0, int lane) {
  const int groups = s >> R;
  const int step = (1 << b0) + (1 << (b0 - 4));
  // QG groups per lane at a time: all their reads are issued before any write
  for (int t0 = 0; t0 < groups; t0 += 64 * QG) {
    float v[QG][1 << R];
    int i0[QG];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int t = min(t0 + 64 * q + lane, groups - 1);
      i0[q] = bd_pad(o + ((t >> b0) << (b0 + R)) + (t & ((1 << b0) - 1)));
#pragma unroll
      for (int k = 0; k < (1 << R); ++k) v[q][k] = xb[i0[q] + k * step];
    }
#pragma unroll
    for (int q = 0; q < QG; ++q)
#pragma unroll
      for (int h = 1; h < (1 << R); h <<= 1)
#pragma unroll
        for (int k = 0; k < (1 << R); ++k)
          if (!(k & h)) {
            const float x0 = v[q][k], x1 = v[q][k + h];
            v[q][k] = x0 + x1;
            v[q][k + h] = x0 - x1;
          }
#pragma unroll
    for (int q = 0; q < QG; ++q)
      if (t0 + 64 * q + lane < groups)
#pragma unroll
        for (int k = 0; k < (1 << R); ++k) xb[i0[q] + k * step] = v[q][k];
  }
  __builtin_amdgcn_wave_barrier();
}

// The first log2(G) stages of a part: each lane takes G consecutive elements (16-byte LDS
// accesses; the padding puts the lanes of a 16-lane group on different bank groups) and
// transforms them in registers.
template <int G>
__device__ __forceinline__ void bd_pass_low(float* xb, int o, int s, int lane) {
  if (lane < s / G) {
    float4* p = reinterpret_cast<float4*>(xb + bd_pad(o + lane * G));
    float v[G];
#pragma unroll
    for (int q = 0; q < G / 4; ++q) {
      const float4 w = p[q];
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
#pragma unroll
    for (int h = 1; h < G; h <<= 1)
#pragma unroll
      for (int k = 0; k < G; ++k)
        if (!(k & h)) {
          const float x0 = v[k], x1 = v[k + h];
          v[k] = x0 + x1;
          v[k + h] = x0 - x1;
        }
#pragma unroll
    for (int q = 0; q < G / 4; ++q) p[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
  __builtin_amdgcn_wave_barrier();
}

// Walsh-Hadamard transform of every power-of-two part of the block in LDS (parts largest
// first, as d's binary expansion): the six lowest stages per lane in registers, then three
// stages per pass over groups whose lanes touch consecutive words.
template <int QG>
__device__ __forceinline__ void bd_butterflies(float* xb, int d, int lane) {
  int o = 0;
  for (int b = 31 - __builtin_clz((unsigned)d); b >= 0; --b) {
    if (!((d >> b) & 1)) continue;
    const int s = 1 << b;
    if (s == 32) {
      bd_pass_low<32>(xb, o, s, lane);
    } else {
      bd_pass_low<64>(xb, o, s, lane);
      int b0 = 6;
      for (; b0 + 3 <= b; b0 += 3) bd_pass<3, QG>(xb, o, s, b0, lane);
      if (b - b0 == 2) bd_pass<2, QG>(xb, o, s, b0, lane);
      else if (b - b0 == 1) bd_pass<1, QG>(xb, o, s, b0, lane);
    }
    o += s;
  }
}

// weight sqrt(d / d_k) of the part (of d's binary expansion, largest first) that holds element e
__device__ __forceinline__ float bd_part_weight(int e, int d) {
  int o = 0;
  for (int b = 31 - __builtin_clz((unsigned)d); b >= 0; --b) {
    if (!((d >> b) & 1)) continue;
    const int s = 1 << b;
    if (e < o + s) return sqrtf((float)d / (float)s);
    o += s;
  }
  return 0.0f;
}

// Quantize: global accesses are 16 bytes per lane, the next block's loads issued before this
// block is transformed.  Codes come from the search grid of the N(0,1) codebook (one LDS read
// per coordinate, as the power-of-two codec): each lane codes four consecutive coordinates at
// a time (conflict-free 16-byte LDS reads, one 4-byte store of codes, consecutive across lanes).
template <bool IN_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(IN_BF16 ? 3 : 1)))
void pq_quantize_bd_kernel(const pqi::BdArgs a) {
  constexpr int CH = IN_BF16 ? 8 : 4;                    // input values per 16-byte load
  constexpr int ML = pqi::kBdMaxD / CH / 64;             // loads per lane per block, at most
  constexpr int MG = pqi::kBdMaxD / 256;                 // groups of four coordinates per lane, at most
  extern __shared__ __align__(16) unsigned char bsmem[];
  const int d = a.d, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ncell = a.ncell, nrep = a.nrep;
  uint2* tab = reinterpret_cast<uint2*>(bsmem);           // [ncell][nrep] (boundary, its index)
  float* gwt = reinterpret_cast<float*>(bsmem + (((size_t)ncell * nrep * 8 + 15) & ~(size_t)15));  // [d / 4]
  float* xb = gwt + ((d / 4 + 3) & ~3) + wv * bd_words(d);
  // search grid: cell k (centre (k - half) w) holds the boundary nearest to its centre
  for (int i = threadIdx.x; i < ncell * nrep; i += blockDim.x) {
    const float c = (float)(i / nrep - a.half) * a.cell_w;
    int best = 0;
    float bd = fabsf(a.beta[0] - c);
    for (int j = 1; j < (1 << a.bits) - 1; ++j) {
      const float dd = fabsf(a.beta[j] - c);
      if (dd < bd) { bd = dd; best = j; }
    }
    tab[i] = make_uint2(__float_as_uint(a.beta[best]), (uint32_t)best);
  }
  const int rep_shift = nrep == 16 ? 7 : 3;               // log2(bytes per cell)
  const uint32_t lane_off = (nrep == 16 ? 8u * (uint32_t)(lane & 15) : 0u) - (kMagicBits << rep_shift);
  const float offM = (float)a.half + kMagic, topM = kMagic + (float)(ncell - 1), inv_w = a.cell_inv_w;
  // the part weight of each group of four coordinates
  for (int i = threadIdx.x; i < d / 4; i += blockDim.x) gwt[i] = bd_part_weight(4 * i, d);
  __syncthreads();
  const int nch = d / CH, ng = d / 4;
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  auto fetch = [&](int64_t blk, uint4 (&raw)[ML]) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.x) +
                                                      min(blk, a.n_blocks - 1) * d * (IN_BF16 ? 2 : 4));
#pragma unroll
    for (int u = 0; u < ML; ++u) {
      const int c = lane + 64 * u;
      raw[u] = c < nch ? src[c] : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 raw[ML];
  fetch((int64_t)blockIdx.x * 4 + wv, raw);
  for (int64_t blk = (int64_t)blockIdx.x * 4 + wv; blk < a.n_blocks; blk += n_waves) {
    double ss = 0.0;
#pragma unroll
    for (int u = 0; u < ML; ++u) {
      const int c = lane + 64 * u;
      if (c < nch) {
        float v[CH];
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int j = 0; j < CH; ++j)
          v[j] = IN_BF16 ? ((j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1])) : __uint_as_float(w[j]);
        const uint32_t sb = a.signs[(c * CH) >> 3] >> ((c * CH) & 7);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          ss += (double)v[j] * (double)v[j];
          if ((sb >> j) & 1) v[j] = -v[j];
        }
        float4* dst = reinterpret_cast<float4*>(xb + bd_pad(c * CH));
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    }
    fetch(blk + n_waves, raw);
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float n = (float)sqrt(ss);
    const float inv = n > 0.0f ? 1.0f / n : 0.0f;
    bd_butterflies<2>(xb, d, lane);
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + blk * d);
#pragma unroll 4
    for (int u = 0; u < MG; ++u) {
      const int c = lane + 64 * u;
      if (c < ng) {
        const float4 xv = *reinterpret_cast<const float4*>(xb + bd_pad(4 * c));
        const float sc = gwt[c] * inv;
        const float y[4] = {xv.x * sc, xv.y * sc, xv.z * sc, xv.w * sc};
        uint32_t pk = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float cu = __builtin_amdgcn_fmed3f(fmaf(y[j], inv_w, offM), kMagic, topM);
          const uint2 te = tab[((__float_as_uint(cu) << rep_shift) + lane_off) >> 3];
          pk |= (te.y + (y[j] > __uint_as_float(te.x) ? 1u : 0u)) << (8 * j);
        }
        dst[c] = pk;
      }
    }
    if (lane == 0) a.norms[blk] = f32_to_f16((float)sqrt(ss));
    __builtin_amdgcn_wave_barrier();
  }
}

// Dequantize: centroids times the part weight into LDS, the butterflies, then sign, scale and
// the store, 16 bytes per lane.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void pq_dequantize_bd_kernel(const pqi::BdArgs a) {
  constexpr int CH = OUT_BF16 ? 8 : 4;                   // output values per 16-byte store
  constexpr int ML = pqi::kBdMaxD / 16 / 64;
  extern __shared__ __align__(16) unsigned char bsmem[];
  const int d = a.d, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __shared__ float cent[1 << pqi::kMaxBits];
  float* xb = reinterpret_cast<float*>(bsmem) + wv * bd_words(d);
  const uint32_t cmask = (1u << a.bits) - 1u;
  for (int j = threadIdx.x; j < (1 << a.bits); j += blockDim.x) cent[j] = a.cent[j];
  // the part weight of each 16-code chunk this lane stages
  float cw[ML];
#pragma unroll
  for (int u = 0; u < ML; ++u) cw[u] = bd_part_weight(min(16 * (lane + 64 * u), d - 1), d);
  __syncthreads();
  const int n16 = d / 16, nch = d / CH;
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  // the next block's codes load while this one is transformed and written
  auto fetch = [&](int64_t blk, uint4 (&raw)[ML]) {
    const uint4* src = reinterpret_cast<const uint4*>(a.ccodes + min(blk, a.n_blocks - 1) * d);
#pragma unroll
    for (int u = 0; u < ML; ++u) {
      const int c = lane + 64 * u;
      raw[u] = c < n16 ? src[c] : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 raw[ML];
  fetch((int64_t)blockIdx.x * 4 + wv, raw);
  for (int64_t blk = (int64_t)blockIdx.x * 4 + wv; blk < a.n_blocks; blk += n_waves) {
#pragma unroll
    for (int u = 0; u < ML; ++u) {
      const int c = lane + 64 * u;
      if (c < n16) {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        const float wq = cw[u];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          reinterpret_cast<float4*>(xb + bd_pad(16 * c))[q] =
              make_float4(cent[w[q] & cmask] * wq, cent[(w[q] >> 8) & cmask] * wq,
                          cent[(w[q] >> 16) & cmask] * wq, cent[(w[q] >> 24) & cmask] * wq);
      }
    }
    fetch(blk + n_waves, raw);
    bd_butterflies<4>(xb, d, lane);
    const float scale = f16_to_f32(a.cnorms[blk]) * (1.0f / (float)d);
#pragma unroll
    for (int u = 0; u < pqi::kBdMaxD / CH / 64; ++u) {
      const int c = lane + 64 * u;
      if (c < nch) {
        float v[CH];
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) {
          const float4 xv = reinterpret_cast<const float4*>(xb + bd_pad(CH * c))[q];
          v[4 * q] = xv.x; v[4 * q + 1] = xv.y; v[4 * q + 2] = xv.z; v[4 * q + 3] = xv.w;
        }
        const uint32_t sb = a.signs[(c * CH) >> 3] >> ((c * CH) & 7);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          v[j] *= scale;
          if ((sb >> j) & 1) v[j] = -v[j];
        }
        uint4 o;
        if constexpr (OUT_BF16) {
          o = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7]));
        } else {
          o = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
        }
        reinterpret_cast<uint4*>(static_cast<unsigned char*>(a.out) + blk * d * (OUT_BF16 ? 2 : 4))[c] = o;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------------------------------
// Dense rotation with the sphere-coordinate codebook: y = Pi x / ||x||, codes against that
// codebook, xhat = n16 Pi^T c.  One wave per block (grid stride); the workgroup holds Pi in LDS
// (transposed for quantize, so lane i reads row i of Pi as consecutive words across lanes);
// the products of fp32 inputs are exact in double and summed in double, and the code is decided
// on that double y against the double boundaries (each held as an fp32 pair beta + beta_lo,
// 48 significant bits).
// ------------------------------------------------------------------------------------------
// PI_GLOBAL (d whose Pi does not fit in LDS, up to 512): every lane reads its own rows of Pi
// from global memory (L2-resident: at most 1 MiB) instead of the LDS copy.
template <bool IN_BF16, bool PI_GLOBAL>
__global__ __launch_bounds__(256) void pq_quantize_dense_kernel(const pqi::BdArgs a) {
  extern __shared__ float dsm[];                         // [d][d] Pi^T (in LDS), then [4 waves][d] blocks
  __shared__ double beta[(1 << pqi::kMaxBits) - 1];
  const int d = a.d, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float* pit = dsm;
  float* xb = dsm + (PI_GLOBAL ? 0 : d * d) + wv * d;
  if constexpr (!PI_GLOBAL)
    for (int idx = threadIdx.x; idx < d * d; idx += blockDim.x) pit[(idx % d) * d + idx / d] = a.rot[idx];
  for (int j = threadIdx.x; j < (1 << a.bits) - 1; j += blockDim.x) beta[j] = (double)a.beta[j] + (double)a.beta_lo[j];
  __syncthreads();
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  for (int64_t blk = (int64_t)blockIdx.x * 4 + wv; blk < a.n_blocks; blk += n_waves) {
    double ss = 0.0;
    for (int e = lane; e < d; e += 64) {
      const float v = IN_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[blk * d + e])
                              : static_cast<const float*>(a.x)[blk * d + e];
      ss += (double)v * (double)v;
      xb[e] = v;
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < d; i += 64) {
      double s0 = 0.0, s1 = 0.0;
      if constexpr (PI_GLOBAL) {
        // row i of Pi (rot is 4-byte aligned)
        const float* row = a.rot + (int64_t)i * d;
        for (int j = 0; j < d; j += 2) {
          s0 += (double)row[j] * (double)xb[j];
          s1 += (double)row[j + 1] * (double)xb[j + 1];
        }
      } else {
        for (int j = 0; j < d; j += 2) {
          s0 += (double)pit[j * d + i] * (double)xb[j];
          s1 += (double)pit[(j + 1) * d + i] * (double)xb[j + 1];
        }
      }
      const double y = (s0 + s1) * inv;
      int code = 0;
      for (int step = 1 << (a.bits - 1); step > 0; step >>= 1)
        if (y > beta[code + step - 1]) code += step;
      a.codes[blk * d + i] = (uint8_t)code;
    }
    if (lane == 0) a.norms[blk] = f32_to_f16((float)sqrt(ss));
    __builtin_amdgcn_wave_barrier();
  }
}

// PI_GLOBAL: Pi read from global memory (rows i, consecutive columns across the lanes).
template <bool OUT_BF16, bool PI_GLOBAL>
__global__ __launch_bounds__(256) void pq_dequantize_dense_kernel(const pqi::BdArgs a) {
  extern __shared__ float dsm[];                         // [d][d] Pi (in LDS), then [4 waves][d] centroids
  __shared__ float cent[1 << pqi::kMaxBits];
  const int d = a.d, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float* pi = PI_GLOBAL ? a.rot : dsm;
  float* cb = dsm + (PI_GLOBAL ? 0 : d * d) + wv * d;
  const uint32_t cmask = (1u << a.bits) - 1u;
  if constexpr (!PI_GLOBAL)
    for (int idx = threadIdx.x; idx < d * d; idx += blockDim.x) dsm[idx] = a.rot[idx];
  for (int j = threadIdx.x; j < (1 << a.bits); j += blockDim.x) cent[j] = a.cent[j];
  __syncthreads();
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  for (int64_t blk = (int64_t)blockIdx.x * 4 + wv; blk < a.n_blocks; blk += n_waves) {
    for (int i = lane; i < d; i += 64) cb[i] = cent[a.ccodes[blk * d + i] & cmask];
    const float n16 = f16_to_f32(a.cnorms[blk]);
    __builtin_amdgcn_wave_barrier();
    for (int j = lane; j < d; j += 64) {
      float s0 = 0.0f, s1 = 0.0f;
      for (int i = 0; i < d; i += 2) {
        s0 = fmaf(pi[i * d + j], cb[i], s0);
        s1 = fmaf(pi[(i + 1) * d + j], cb[i + 1], s1);
      }
      const float v = n16 * (s0 + s1);
      if (OUT_BF16) static_cast<uint16_t*>(a.out)[blk * d + j] = f32_to_bf16(v);
      else static_cast<float*>(a.out)[blk * d + j] = v;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Quantize on the fp32 matrix cores (fp32 blocks, and bf16 ones whose input or codes are not
// 16-byte aligned): a wave takes 16 blocks, Y (16 x d) = X (16 x d) Pi^T with
// v_mfma_f32_16x16x4f32 (layout as the dequantize kernel below, Pi^T in LDS).  A block of
// extreme norm is staged scaled by a power of two that brings its norm into [1, 2) (exact;
// products of tiny blocks would otherwise fall into fp32's subnormal range).  An fp32 sum of d
// products is then within d 2^-24 ||x|| of the exact one, so a coordinate of y = Y / ||x||
// farther than twice that from every boundary takes the same code as the exact value; the few
// nearer ones are recomputed from LDS with exact products summed in double and decided against
// the double boundaries, as the one-wave kernel.
constexpr int kDenseQWaves = 8;                         // waves sharing one LDS copy of Pi^T

template <bool IN_BF16, int D, bool VEC>
__global__ __launch_bounds__(64 * kDenseQWaves) void pq_quantize_dense_mfma_kernel(const pqi::BdArgs a) {
  constexpr int PS = D + 16;                             // LDS row stride of Pi^T
  constexpr int XS = D + 4;                              // LDS row stride of the blocks: rows 4 banks apart
  constexpr int NT = D / 16;
  constexpr float EPS = 2.0f * (float)D / 16777216.0f;   // twice the fp32 sum's error bound
  extern __shared__ __align__(16) float dsm[];           // [D][PS] Pi^T, [waves][16][XS] x, then the grid
  __shared__ float beta[(1 << pqi::kMaxBits) - 1];
  __shared__ double beta_d[(1 << pqi::kMaxBits) - 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nb = (1 << a.bits) - 1;
  float* xs = dsm + D * PS + wv * 16 * XS;
  uint4* gtab = reinterpret_cast<uint4*>(dsm + D * PS + kDenseQWaves * 16 * XS);
  for (int idx = threadIdx.x; idx < D * D; idx += blockDim.x) dsm[(idx % D) * PS + idx / D] = a.rot[idx];
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    beta[j] = a.beta[j];
    beta_d[j] = (double)a.beta[j] + (double)a.beta_lo[j];
  }
  // search grid over the codebook's boundaries (cells narrower than the smallest gap): cell k,
  // centre (k - half) w, holds its nearest boundary, that boundary's index and the boundaries on
  // either side of it (+-inf past the ends), so a code and its two enclosing boundaries come
  // from one 16-byte read
  const int ncell = a.ncell;
  for (int i = threadIdx.x; i < ncell; i += blockDim.x) {
    const float c = (float)(i - a.half) * a.cell_w;
    int best = 0;
    float bd = fabsf(a.beta[0] - c);
    for (int j = 1; j < nb; ++j) {
      const float dd = fabsf(a.beta[j] - c);
      if (dd < bd) { bd = dd; best = j; }
    }
    gtab[i] = make_uint4(__float_as_uint(a.beta[best]), (uint32_t)best,
                         __float_as_uint(best > 0 ? a.beta[best - 1] : -INFINITY),
                         __float_as_uint(best + 1 < nb ? a.beta[best + 1] : INFINITY));
  }
  __syncthreads();
  const float offM = (float)a.half + kMagic, topM = kMagic + (float)(ncell - 1), inv_w = a.cell_inv_w;
  // code of y with its two enclosing boundaries (lo < y <= hi in exact arithmetic)
  auto decide = [&](float y, float& lo, float& hi) {
    int code;
    if (ncell > 0) {
      const float u = __builtin_amdgcn_fmed3f(fmaf(y, inv_w, offM), kMagic, topM);
      const uint4 e = gtab[__float_as_uint(u) - kMagicBits];
      const float bb = __uint_as_float(e.x);
      const bool gt = y > bb;
      code = (int)e.y + (gt ? 1 : 0);
      lo = gt ? bb : __uint_as_float(e.z);
      hi = gt ? __uint_as_float(e.w) : bb;
    } else {
      code = 0;
      for (int step = 1 << (a.bits - 1); step > 0; step >>= 1)
        if (y > beta[code + step - 1]) code += step;
      lo = code > 0 ? beta[code - 1] : -INFINITY;
      hi = code < nb ? beta[code] : INFINITY;
    }
    return code;
  };
  auto decide_d = [&](double y) {
    int code = 0;
    for (int step = 1 << (a.bits - 1); step > 0; step >>= 1)
      if (y > beta_d[code + step - 1]) code += step;
    return code;
  };
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t n_waves = (int64_t)gridDim.x * kDenseQWaves;
  for (int64_t tile = (int64_t)blockIdx.x * kDenseQWaves + wv; tile < n_tiles; tile += n_waves) {
    // block r of the tile: lane group g stages a quarter of the row in LDS and sums its squares
    const int64_t blk = min(tile * 16 + r, a.n_blocks - 1);
    double ss = 0.0;
    if constexpr (VEC) {
      // 16-byte loads: chunk c = g + 4 u of the row (8 bf16 or 4 fp32 values)
      constexpr int CH = IN_BF16 ? 8 : 4;
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.x) +
                                                        blk * D * (IN_BF16 ? 2 : 4));
      uint4 w[D / CH / 4];
#pragma unroll
      for (int u = 0; u < D / CH / 4; ++u) w[u] = src[g + 4 * u];
#pragma unroll
      for (int u = 0; u < D / CH / 4; ++u) {
        const int c = g + 4 * u;
        float v[CH];
        const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int j = 0; j < CH; ++j)
          v[j] = IN_BF16 ? ((j & 1) ? bf16_hi(ww[j >> 1]) : bf16_lo(ww[j >> 1])) : __uint_as_float(ww[j]);
#pragma unroll
        for (int j = 0; j < CH; ++j) ss += (double)v[j] * (double)v[j];
        float4* dst = reinterpret_cast<float4*>(xs + r * XS + c * CH);
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    } else {
      for (int e = g; e < D; e += 4) {
        const float v = IN_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[blk * D + e])
                                : static_cast<const float*>(a.x)[blk * D + e];
        xs[r * XS + e] = v;
        ss += (double)v * (double)v;
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);                            // the block's sum in all four lanes
    // a block whose norm lies outside [2^-60, 2^60] is staged scaled by 2^-floor(log2 ||x||)
    // (the four lanes of a block split its elements); inside that range no fp32 product or sum leaves the
    // normal range and the block is used as it is
    const int e0 = ss > 0.0 ? ilogb(sqrt(ss)) : 0;
    const int ex = e0 < -60 || e0 > 60 ? -e0 : 0;
    if (ex != 0) {
      const double scd = ldexp(1.0, ex);
      __builtin_amdgcn_wave_barrier();
      for (int e = g; e < D; e += 4) xs[r * XS + e] = (float)((double)xs[r * XS + e] * scd);
    }
    __builtin_amdgcn_wave_barrier();
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int s = 0; s < D / 4; ++s) {
      const float av = xs[r * XS + 4 * s + g];
      const float* prow = dsm + (4 * s + g) * PS + r;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, prow[16 * t], acc[t], 0, 0, 0);
    }
    // lane (column n = 16 t + r, group g) holds blocks 4 g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bl = 4 * g + i;
      const int64_t b = tile * 16 + bl;
      const double sb = __shfl(ss, bl);                 // lane bl holds block bl's sum
      const int exb = __shfl(ex, bl);
      // 1 / ||x_scaled|| = 1 / (||x|| 2^ex): y is the same whether x is scaled or not
      const double invd = sb > 0.0 ? 1.0 / (sqrt(sb) * ldexp(1.0, exb)) : 0.0;
      const float inv = (float)invd;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = 16 * t + r;
        const float y = acc[t][i] * inv;
        float lo, hi;
        int code = decide(y, lo, hi);
        if (fabsf(y - lo) < EPS || fabsf(y - hi) < EPS) {
          double s0 = 0.0, s1 = 0.0;
          for (int j = 0; j < D; j += 2) {
            s0 += (double)dsm[j * PS + n] * (double)xs[bl * XS + j];
            s1 += (double)dsm[(j + 1) * PS + n] * (double)xs[bl * XS + j + 1];
          }
          code = decide_d((s0 + s1) * invd);
        }
        if (b < a.n_blocks) a.codes[b * D + n] = (uint8_t)code;
      }
      if (r == 0 && b < a.n_blocks) a.norms[b] = f32_to_f16((float)sqrt(sb));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Quantize bf16 blocks with the dense rotation on the bf16 matrix cores.  Pi is split exactly
// into three bf16 parts, Pi = hi + mid + lo (each the round-to-nearest of what the parts before
// it leave, so mid + lo and then hi + (mid + lo) give Pi back exactly in fp32).  A wave takes 16
// blocks and forms Y^T (d x 16) = (hi + mid) X^T, two 16x16x32 products per K step: lane (r, g)
// holds block r's values k = 32 u + 8 g .. + 7 straight from its 16-byte loads (the B operand as
// loaded) and receives y[16 t + 4 g + i] of block r, so each lane decides four consecutive codes
// of one block per column tile with that block's own 1 / ||x||.  Leaving lo out moves y by at most
// 2^-16 ||x||; with the fp32 accumulation and normalisation this bounds |y - y_exact| by the
// kernel's eps.  A code whose y lies within eps of its nearest boundary is queued and decided
// again in fp64 from the block as loaded (kept in LDS) and Pi = hi + (mid + lo), d / 8 lanes per
// queued code; after a tile's decisions its near codes go to the queue, which is drained when the
// next round of them may not fit and at the end.
constexpr int kDenseBWaves = 8;
constexpr int kDenseBQueue = 64;                         // queued codes per wave

template <int D>
struct DenseBLayout {
  static constexpr int KC = D / 8;                       // 16-byte k chunks of a row
  static constexpr int NT = D / 16;                      // column tiles of 16 outputs
  static constexpr int U = D / 32;                       // K steps of the 16x16x32 product
  static constexpr int XR = 2 * D + 16;                  // bytes per staged block (rows 4 banks apart)
  static constexpr int CR = D + 16;                      // bytes per code row
  static constexpr size_t PART = (size_t)KC * D * 16;    // one bf16 part of Pi as [kc][n] 16-byte chunks
  static constexpr size_t WAVE = 16 * XR + 16 * CR + kDenseBQueue * 4;
  static constexpr size_t bytes(int ncell) { return 3 * PART + kDenseBWaves * WAVE + (size_t)ncell * 8; }
};

// sum of a double over each aligned group of N lanes (every lane of the group gets it)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
template <int N>
__device__ __forceinline__ double sum_lanes_f64(double v) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  v += dpp_f64<0xB1>(v);                                 // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);                                 // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);                                // row_half_mirror: the other quad
  if constexpr (N == 16) v += dpp_f64<0x140>(v);         // row_mirror: the other half row
  return v;
}

template <int D>
__global__ __launch_bounds__(64 * kDenseBWaves) void pq_quantize_dense_bf16_kernel(const pqi::BdArgs a, float eps) {
  using L = DenseBLayout<D>;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  constexpr int NT = L::NT, U = L::U, XR = L::XR, CR = L::CR, KC = L::KC;
  extern __shared__ __align__(16) unsigned char dsb[];
  __shared__ double beta_d[(1 << pqi::kMaxBits) - 1];
  uint4* phi = reinterpret_cast<uint4*>(dsb);
  uint4* pmid = phi + KC * D;
  uint4* plo = pmid + KC * D;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  unsigned char* xs = dsb + 3 * L::PART + wv * L::WAVE;  // [16][XR] the wave's blocks as loaded
  unsigned char* cb = xs + 16 * XR;                       // [16][CR] their codes
  uint32_t* queue = reinterpret_cast<uint32_t*>(cb + 16 * CR);
  uint2* gtab = reinterpret_cast<uint2*>(dsb + 3 * L::PART + kDenseBWaves * L::WAVE);
  const int nb = (1 << a.bits) - 1;
  // chunk (kc, n) of each part holds Pi[n][8 kc .. 8 kc + 7]
  for (int idx = threadIdx.x; idx < KC * D; idx += blockDim.x) {
    const int n = idx / KC, kc = idx % KC;
    const float* src = a.rot + (size_t)n * D + 8 * kc;
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v0 = src[2 * j], v1 = src[2 * j + 1];
      h[j] = pack_bf16x2(v0, v1);
      const float r0 = v0 - bf16_lo(h[j]), r1 = v1 - bf16_hi(h[j]);
      m[j] = pack_bf16x2(r0, r1);
      l[j] = pack_bf16x2(r0 - bf16_lo(m[j]), r1 - bf16_hi(m[j]));
    }
    phi[kc * D + n] = make_uint4(h[0], h[1], h[2], h[3]);
    pmid[kc * D + n] = make_uint4(m[0], m[1], m[2], m[3]);
    plo[kc * D + n] = make_uint4(l[0], l[1], l[2], l[3]);
  }
  for (int j = threadIdx.x; j < nb; j += blockDim.x) beta_d[j] = (double)a.beta[j] + (double)a.beta_lo[j];
  // search grid: cell k, centre (k - half) w, holds its nearest boundary and that boundary's
  // index.  Cells are narrower than 0.9 of the smallest gap and eps is below a twentieth of it,
  // so a y within eps of any boundary is within eps of its cell's one.
  const int ncell = a.ncell;
  for (int i = threadIdx.x; i < ncell; i += blockDim.x) {
    const float c = (float)(i - a.half) * a.cell_w;
    int best = 0;
    float bd = fabsf(a.beta[0] - c);
    for (int j = 1; j < nb; ++j) {
      const float dd = fabsf(a.beta[j] - c);
      if (dd < bd) { bd = dd; best = j; }
    }
    gtab[i] = make_uint2(__float_as_uint(a.beta[best]), (uint32_t)best);
  }
  __syncthreads();
  const float offM = (float)a.half + kMagic, topM = kMagic + (float)(ncell - 1), inv_w = a.cell_inv_w;
  const uint32_t last_cell = (uint32_t)(ncell - 1);

  // decide the queued codes again in fp64: KC lanes per code, one 8-value chunk of k each.
  // With best the index of the boundary b next to y, the code is best + (y > b), and y > b is
  // taken from the sign of dot and of b and from dot^2 against b^2 ||x||^2 (no root or quotient)
  auto drain = [&](int cnt) {
    asm volatile("" ::: "memory");
    constexpr int PER = 64 / KC;                         // codes per pass
    const int G = lane / KC, j = lane % KC;
    for (int q0 = 0; q0 < cnt; q0 += PER) {
      const int qi = q0 + G;
      const bool valid = qi < cnt;
      const uint32_t e = queue[valid ? qi : q0];
      const int b = e & 15, n = (e >> 4) & 127;
      const int best = (int)cb[b * CR + n] - (int)(e >> 11);   // the fast code less its side bit
      const double bd = beta_d[best];
      const uint4 xv = *reinterpret_cast<const uint4*>(xs + b * XR + j * 16);
      const uint4 hv = phi[j * D + n], mv = pmid[j * D + n], lv = plo[j * D + n];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, hw[4] = {hv.x, hv.y, hv.z, hv.w};
      const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w}, lw[4] = {lv.x, lv.y, lv.z, lv.w};
      double dot = 0.0, sq = 0.0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = bf16_lo(xw[w]), x1 = bf16_hi(xw[w]);
        const float p0 = bf16_lo(hw[w]) + (bf16_lo(mw[w]) + bf16_lo(lw[w]));   // Pi exactly
        const float p1 = bf16_hi(hw[w]) + (bf16_hi(mw[w]) + bf16_hi(lw[w]));
        dot = fma((double)x0, (double)p0, dot);
        dot = fma((double)x1, (double)p1, dot);
        sq = fma((double)x0, (double)x0, sq);
        sq = fma((double)x1, (double)x1, sq);
      }
      dot = sum_lanes_f64<KC>(dot);
      sq = sum_lanes_f64<KC>(sq);
      const double lhs = dot * dot, rhs = bd * bd * sq;
      bool gt;
      if (sq == 0.0) gt = 0.0 > bd;                      // y = 0
      else if (dot >= 0.0) gt = bd < 0.0 || lhs > rhs;
      else gt = bd < 0.0 && lhs < rhs;
      if (valid && j == 0) cb[b * CR + n] = (uint8_t)(best + (gt ? 1 : 0));
    }
    asm volatile("" ::: "memory");
  };

  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t n_waves = (int64_t)gridDim.x * kDenseBWaves;
  // block r of tile T, chunks k = 32 u + 8 g .. + 7 (the next tile's are loaded while this
  // tile's codes are decided)
  auto load_tile_x = [&](int64_t T, uint4 (&xw)[U]) {
    const int64_t blk = min(T * 16 + r, a.n_blocks - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + blk * D);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 v = __builtin_nontemporal_load(src + 4 * u + g);
      xw[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  uint4 xn[U];
  int64_t T = (int64_t)blockIdx.x * kDenseBWaves + wv;
  if (T < n_tiles) load_tile_x(T, xn);
  for (; T < n_tiles; T += n_waves) {
    uint4 xw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) xw[u] = xn[u];
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      *reinterpret_cast<uint4*>(xs + r * XR + (4 * u + g) * 16) = xw[u];
      const uint32_t w4[4] = {xw[u].x, xw[u].y, xw[u].z, xw[u].w};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w4[w]), __builtin_bit_cast(bf16x2, w4[w]), ss, false);
    }
    ss = sum4(ss);                                       // the block's sum, equal in its four lanes
    float inv;
    uint16_t n16;
    if (ss >= 0x1p-80f && ss <= 0x1p120f) {
      // fp32 products and sums stay normal for such blocks
      inv = __builtin_amdgcn_rsqf(ss);
      n16 = f32_to_f16(sqrtf(ss));
    } else {
      // zero, tiny or huge block: its norm in fp64, and the block scaled by 2^-floor(log2 ||x||)
      // (exact in bf16 but for values far below the norm, whose loss is below 2^-100 ||x||)
      double sd = 0.0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t w4[4] = {xw[u].x, xw[u].y, xw[u].z, xw[u].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const double v0 = bf16_lo(w4[w]), v1 = bf16_hi(w4[w]);
          sd = fma(v0, v0, fma(v1, v1, sd));
        }
      }
      sd += __shfl_xor(sd, 16);
      sd += __shfl_xor(sd, 32);
      const double nrm = sqrt(sd);
      n16 = f32_to_f16((float)nrm);
      inv = 0.0f;
      if (sd > 0.0) {
        const double sc = ldexp(1.0, -ilogb(nrm));
        inv = (float)(1.0 / (nrm * sc));
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint32_t w4[4] = {xw[u].x, xw[u].y, xw[u].z, xw[u].w};
#pragma unroll
          for (int w = 0; w < 4; ++w)
            w4[w] = pack_bf16x2((float)((double)bf16_lo(w4[w]) * sc), (float)((double)bf16_hi(w4[w]) * sc));
          xw[u] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
      }
    }
    // hi and mid products in accumulators of their own: the rounding of the mid sum is 2^-8
    // of the hi sum's
    f32x4 acc[NT], accm[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = accm[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bf16x8 xf = __builtin_bit_cast(bf16x8, xw[u]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 h = __builtin_bit_cast(bf16x8, phi[(4 * u + g) * D + 16 * t + r]);
        const bf16x8 m = __builtin_bit_cast(bf16x8, pmid[(4 * u + g) * D + 16 * t + r]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h, xf, acc[t], 0, 0, 0);
        accm[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m, xf, accm[t], 0, 0, 0);
      }
    }
    if (T + n_waves < n_tiles) load_tile_x(T + n_waves, xn);
    // codes: lane (r, g) holds y[16 t + 4 g + i] of block r.  Element e = 4 t + i of the lane
    // is bit 31 - e of near (within eps of its cell's boundary) and of side (above it).
    // the grid lookups of two column tiles are issued together, then used
    uint32_t near = 0, side = 0;
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += 2) {
      float y[2][4];
      uint2 e[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[tt][i] = (acc[t0 + tt][i] + accm[t0 + tt][i]) * inv;
          const float cu = __builtin_amdgcn_fmed3f(fmaf(y[tt][i], inv_w, offM), kMagic, topM);
          const uint32_t ci = min(__float_as_uint(cu) - kMagicBits, last_cell);   // NaN stays in the table
          e[tt][i] = gtab[ci];
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bb = __uint_as_float(e[tt][i].x);
          const uint32_t gt = y[tt][i] > bb ? 1u : 0u;
          word |= (e[tt][i].y + gt) << (8 * i);
          near = 2 * near + (fabsf(y[tt][i] - bb) < eps ? 1u : 0u);
          side = 2 * side + gt;
        }
        *reinterpret_cast<uint32_t*>(cb + r * CR + 16 * (t0 + tt) + 4 * g) = word;
      }
    }
    near <<= 32 - 4 * NT;
    side <<= 32 - 4 * NT;
    // queue the near codes, one per lane per round, draining whenever the next round may not fit
    if (__builtin_amdgcn_ballot_w64(near != 0)) {
      int cnt = 0;
      for (;;) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(near != 0);
        if (!m) break;
        if (cnt + __popcll(m) > kDenseBQueue) {
          drain(cnt);
          cnt = 0;
        }
        if (near) {
          const int e = __builtin_clz(near);
          near &= ~(0x80000000u >> e);
          const uint32_t gt = (side >> (31 - e)) & 1u;
          const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          queue[pos] = (uint32_t)r | ((uint32_t)(16 * (e >> 2) + 4 * g + (e & 3)) << 4) | (gt << 11);
        }
        cnt += __popcll(m);
      }
      drain(cnt);
    }
    asm volatile("" ::: "memory");
    // whole 16-byte pieces of the tile's code rows
#pragma unroll
    for (int c = 0; c < (16 * KC / 2) / 64; ++c) {
      const int piece = lane + 64 * c, row = piece / (D / 16), col = piece % (D / 16);
      const int64_t b = T * 16 + row;
      const uint4 v = *reinterpret_cast<const uint4*>(cb + row * CR + col * 16);
      if (b < a.n_blocks) *reinterpret_cast<uint4*>(a.codes + b * D + col * 16) = v;
    }
    if (g == 0 && T * 16 + r < a.n_blocks) a.norms[T * 16 + r] = n16;
    asm volatile("" ::: "memory");
  }
}

// Dequantize on the fp16 matrix cores.  2^6 Pi and 2^6 c are split into fp16 hi and lo parts
// (the scale keeps the lo parts in fp16's normal range; each split leaves at most 2^-22 of the
// value), and Xhat^T (d x 16) = 2^-12 n16 (Pi^T C^T) is formed from three 16x16x32 products per
// K step (hi hi, hi lo, lo hi; the lo lo term is below 2^-22 of the sum's terms).  Lane (r, g)
// builds block r's centroid fragment for rows n = 32 u + 8 g .. + 7 from eight code bytes and
// receives xhat[16 t + 4 g + i] of block r; the tile goes out through LDS as whole 16-byte
// pieces of its rows.
constexpr int kDenseDWaves = 8;

template <int D, bool OUT_BF16>
struct DenseDLayout {
  static constexpr int NC = D / 8;                       // 16-byte n chunks of a column
  static constexpr int OR = D * (OUT_BF16 ? 2 : 4) + 16; // bytes per staged output row
  static constexpr size_t PART = (size_t)NC * D * 16;    // one fp16 part of 2^6 Pi^T as [nc][k] chunks
  static constexpr size_t bytes() { return 2 * PART + (size_t)kDenseDWaves * 16 * OR; }
};

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kDenseDWaves) void pq_dequantize_dense_f16_kernel(const pqi::BdArgs a) {
  using L = DenseDLayout<D, OUT_BF16>;
  constexpr int NC = L::NC, NT = D / 16, U = D / 32, OR = L::OR;
  constexpr int PIECES = D * (OUT_BF16 ? 2 : 4) / 16;    // 16-byte pieces of an output row
  extern __shared__ __align__(16) unsigned char dsd[];
  __shared__ uint32_t chl[1 << pqi::kMaxBits];           // 2^6 c as fp16 hi | lo << 16
  uint4* qhi = reinterpret_cast<uint4*>(dsd);
  uint4* qlo = qhi + NC * D;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  unsigned char* stg = dsd + 2 * L::PART + wv * 16 * OR;
  // chunk (nc, k) holds 2^6 Pi[8 nc .. 8 nc + 7][k]
  for (int idx = threadIdx.x; idx < NC * D; idx += blockDim.x) {
    const int nc = idx / D, k = idx % D;
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v0 = 64.0f * a.rot[(size_t)(8 * nc + 2 * j) * D + k];
      const float v1 = 64.0f * a.rot[(size_t)(8 * nc + 2 * j + 1) * D + k];
      const uint16_t h0 = f32_to_f16(v0), h1 = f32_to_f16(v1);
      h[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      l[j] = (uint32_t)f32_to_f16(v0 - f16_to_f32(h0)) | ((uint32_t)f32_to_f16(v1 - f16_to_f32(h1)) << 16);
    }
    qhi[idx] = make_uint4(h[0], h[1], h[2], h[3]);
    qlo[idx] = make_uint4(l[0], l[1], l[2], l[3]);
  }
  for (int j = threadIdx.x; j < (1 << a.bits); j += blockDim.x) {
    const float v = 64.0f * a.cent[j];
    const uint16_t h = f32_to_f16(v);
    chl[j] = (uint32_t)h | ((uint32_t)f32_to_f16(v - f16_to_f32(h)) << 16);
  }
  __syncthreads();
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t n_waves = (int64_t)gridDim.x * kDenseDWaves;
  for (int64_t T = (int64_t)blockIdx.x * kDenseDWaves + wv; T < n_tiles; T += n_waves) {
    const int64_t blk = min(T * 16 + r, a.n_blocks - 1);
    uint2 cw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cw[u] = *reinterpret_cast<const uint2*>(a.ccodes + blk * D + 32 * u + 8 * g);
    const float scale = f16_to_f32(a.cnorms[blk]) * 0x1p-12f;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = chl[((j < 4 ? cw[u].x : cw[u].y) >> (8 * (j & 3))) & 0xff];
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bh[j] = __builtin_amdgcn_perm(e[2 * j + 1], e[2 * j], 0x05040100u);   // the two hi halves
        bl[j] = __builtin_amdgcn_perm(e[2 * j + 1], e[2 * j], 0x07060302u);   // the two lo halves
      }
      const f16x8 fh = __builtin_bit_cast(f16x8, make_uint4(bh[0], bh[1], bh[2], bh[3]));
      const f16x8 fl = __builtin_bit_cast(f16x8, make_uint4(bl[0], bl[1], bl[2], bl[3]));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f16x8 ah = __builtin_bit_cast(f16x8, qhi[(4 * u + g) * D + 16 * t + r]);
        const f16x8 al = __builtin_bit_cast(f16x8, qlo[(4 * u + g) * D + 16 * t + r]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, fh, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, fl, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, fh, acc[t], 0, 0, 0);
      }
    }
    // lane (r, g) holds xhat[16 t + 4 g + i] of block r
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v0 = acc[t][0] * scale, v1 = acc[t][1] * scale, v2 = acc[t][2] * scale, v3 = acc[t][3] * scale;
      if constexpr (OUT_BF16)
        *reinterpret_cast<uint2*>(stg + r * OR + (16 * t + 4 * g) * 2) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      else
        *reinterpret_cast<float4*>(stg + r * OR + (16 * t + 4 * g) * 4) = make_float4(v0, v1, v2, v3);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < 16 * PIECES / 64; ++c) {
      const int piece = lane + 64 * c, row = piece / PIECES, col = piece % PIECES;
      const int64_t b = T * 16 + row;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + row * OR + col * 16);
      if (b < a.n_blocks)
        *reinterpret_cast<uint4*>(static_cast<unsigned char*>(a.out) + (b * D) * (OUT_BF16 ? 2 : 4) + col * 16) = v;
    }
    asm volatile("" ::: "memory");
  }
}

// Dequantize on the fp32 matrix cores (output not 16-byte aligned): a wave takes 16 blocks,
// Xhat (16 x d) = C (16 x d) Pi with v_mfma_f32_16x16x4f32 (fp32 products and sums; the centroids are fp32 exact).  K step s takes
// k = 4 s + g in lane group g; Pi sits in LDS with a row stride of d + 16 words, so the four lane
// groups of a B operand read four different bank quarters.
template <bool OUT_BF16, int D>
__global__ __launch_bounds__(256) void pq_dequantize_dense_mfma_kernel(const pqi::BdArgs a) {
  constexpr int PS = D + 16;                             // LDS row stride of Pi
  constexpr int NT = D / 16;                             // N tiles
  extern __shared__ float dsm[];
  __shared__ float cent[1 << pqi::kMaxBits];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const uint32_t cmask = (1u << a.bits) - 1u;
  for (int idx = threadIdx.x; idx < D * D; idx += blockDim.x) dsm[(idx / D) * PS + idx % D] = a.rot[idx];
  for (int j = threadIdx.x; j < (1 << a.bits); j += blockDim.x) cent[j] = a.cent[j];
  __syncthreads();
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wv; tile < n_tiles; tile += n_waves) {
    // the codes of block r of the tile (all of them: lane group g uses bytes 4 s + g)
    const int64_t blk = min(tile * 16 + r, a.n_blocks - 1);
    uint32_t cw[D / 4];
    const uint4* src = reinterpret_cast<const uint4*>(a.ccodes + blk * D);
#pragma unroll
    for (int q = 0; q < D / 16; ++q) {
      const uint4 w = src[q];
      cw[4 * q] = w.x; cw[4 * q + 1] = w.y; cw[4 * q + 2] = w.z; cw[4 * q + 3] = w.w;
    }
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int s = 0; s < D / 4; ++s) {
      const float av = cent[(cw[s] >> (8 * g)) & cmask];
      const float* prow = dsm + (4 * s + g) * PS + r;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, prow[16 * t], acc[t], 0, 0, 0);
    }
    // lane (column n = r, group g) holds rows 4 g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t b = tile * 16 + 4 * g + i;
      if (b < a.n_blocks) {
        const float n16 = f16_to_f32(a.cnorms[b]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float v = n16 * acc[t][i];
          if (OUT_BF16) static_cast<uint16_t*>(a.out)[b * D + 16 * t + r] = f32_to_bf16(v);
          else static_cast<float*>(a.out)[b * D + 16 * t + r] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// launch helpers
// ------------------------------------------------------------------------------------------
int grid_for(int64_t n_tiles, const pqi::LaunchCfg& c, int per_cu) {
  int64_t want = (n_tiles + kWaves - 1) / kWaves;
  int64_t cap = (int64_t)c.cu_count * per_cu;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

template <int D, int MODE>
hipError_t launch_quantize_r(bool in_bf16, bool qjl, bool g_lds, int grid, size_t lds, const pqi::QuantArgs& a,
                             hipStream_t s) {
  if (!qjl) {
    if (in_bf16) hipLaunchKernelGGL((pq_quantize_kernel<D, true, false, false, MODE>), grid, kThreads, lds, s, a);
    else hipLaunchKernelGGL((pq_quantize_kernel<D, false, false, false, MODE>), grid, kThreads, lds, s, a);
  } else if (D <= 256 && g_lds && lds > 65536) {
    // one workgroup per CU: eight waves (d = 512 would spill at two waves per SIMD)
    if constexpr (D <= 256) {
      const int64_t n_tiles = (a.n_blocks + 15) >> 4;
      const int g8 = (int)std::max<int64_t>(1, std::min<int64_t>(grid, (n_tiles + 7) / 8));
      if (in_bf16) hipLaunchKernelGGL((pq_quantize_kernel<D, true, true, true, MODE, 512>), g8, 512, lds, s, a);
      else hipLaunchKernelGGL((pq_quantize_kernel<D, false, true, true, MODE, 512>), g8, 512, lds, s, a);
    }
  } else if (g_lds) {
    if (in_bf16) hipLaunchKernelGGL((pq_quantize_kernel<D, true, true, true, MODE>), grid, kThreads, lds, s, a);
    else hipLaunchKernelGGL((pq_quantize_kernel<D, false, true, true, MODE>), grid, kThreads, lds, s, a);
  } else {
    if (in_bf16) hipLaunchKernelGGL((pq_quantize_kernel<D, true, true, false, MODE>), grid, kThreads, lds, s, a);
    else hipLaunchKernelGGL((pq_quantize_kernel<D, false, true, false, MODE>), grid, kThreads, lds, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_quantize_d(bool in_bf16, const pqi::QuantArgs& a, const pqi::LaunchCfg& c, hipStream_t s) {
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int m_pad = (a.m + 15) & ~15;
  const size_t base = (size_t)a.t.ncell * a.t.nrep * 16;
  const size_t glb = (size_t)m_pad * D * 2;
  const bool qjl = a.m > 0;
  // G kept in LDS for the whole launch when it fits beside the search grid (several
  // workgroups per CU while it takes at most 64 KiB), else walked in chunks
  // bf16 blocks at d = 256 rotate on the matrix cores in every form: their fragments follow the
  // grid and G (or the residual fragments)
  const size_t hfx = D == 256 && in_bf16 ? kHfBytes : 0;
  const bool g_lds = qjl && base + glb + hfx <= (size_t)c.max_lds;
  const int mode = a.pbits ? 2 : (a.t.nrep == 16 ? 1 : 0);
  // rotated-basis projection when G D H (fp16 high + low) fits beside the grid: one
  // sixteen-wave workgroup per CU (four waves per SIMD at <= 128 VGPRs); packed codes hold
  // more registers and run four-wave workgroups, three per CU (three waves per SIMD)
  const size_t grb = (size_t)m_pad * D * 4;
  // (d <= 128: wider blocks hold too many registers at four waves per SIMD)
  if constexpr (D <= 128) {
    // bf16 blocks at d = 128 rotate on the matrix cores: their fragments follow G D H
    const size_t rb = base + grb + (D == 128 && in_bf16 ? kHfBytes + kSmBytes : 0);
    if (qjl && rb <= (size_t)c.max_lds && base + grb <= 98304 && (mode < 2 || 3 * rb <= (size_t)c.max_lds)) {
      const size_t lds = rb;
      if (mode == 2) {
        const int g4 = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)c.cu_count * 3, (n_tiles + 3) / 4));
        if (in_bf16) hipLaunchKernelGGL((pq_quantize_kernel<D, true, true, false, 2, 256, true>), g4, 256, lds, s, a);
        else hipLaunchKernelGGL((pq_quantize_kernel<D, false, true, false, 2, 256, true>), g4, 256, lds, s, a);
        return hipGetLastError();
      }
      constexpr int rbw = kRbThreads / 64;
      const int g16 = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)c.cu_count * PQ_RB_WG, (n_tiles + rbw - 1) / rbw));
#define PQ_RB_LAUNCH(MODE)                                                                                       \
  if (in_bf16) hipLaunchKernelGGL((pq_quantize_kernel<D, true, true, false, MODE, kRbThreads, true>), g16, kRbThreads, lds, s, a); \
  else hipLaunchKernelGGL((pq_quantize_kernel<D, false, true, false, MODE, kRbThreads, true>), g16, kRbThreads, lds, s, a);
      if (mode == 1) { PQ_RB_LAUNCH(1) }
      else { PQ_RB_LAUNCH(0) }
#undef PQ_RB_LAUNCH
      return hipGetLastError();
    }
  }
  if (qjl && !g_lds) {
    // residual fragments of every tile of the workgroup beside the search grid
    const size_t lds = base + chunk_frag_bytes<D>() + hfx;
    if (lds > (size_t)c.max_lds) return hipErrorInvalidConfiguration;
    const int64_t n_groups = (n_tiles + chunk_threads<D>() / 64 - 1) / (chunk_threads<D>() / 64);
    const int per_cu = std::max(1, (int)((size_t)c.max_lds / lds));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(n_groups, (int64_t)c.cu_count * per_cu));
#define PQ_CHUNK_LAUNCH(MODE)                                                                               \
  if (in_bf16) hipLaunchKernelGGL((pq_quantize_chunked_kernel<D, true, MODE>), grid, chunk_threads<D>(), lds, s, a); \
  else hipLaunchKernelGGL((pq_quantize_chunked_kernel<D, false, MODE>), grid, chunk_threads<D>(), lds, s, a);
    if (mode == 2) { PQ_CHUNK_LAUNCH(2) }
    else if (mode == 1) { PQ_CHUNK_LAUNCH(1) }
    else { PQ_CHUNK_LAUNCH(0) }
#undef PQ_CHUNK_LAUNCH
    return hipGetLastError();
  }
  // (bf16 blocks at d = 256, and without the projection at d = 128, rotate on the matrix cores:
  // fragments after the grid and G)
  const size_t lds = base + (g_lds ? glb : 0) + hfx + (!qjl && D == 128 && in_bf16 ? kHfBytes : 0);
  const int grid = grid_for(n_tiles, c, lds > 65536 ? 1 : PQ_QUANT_WG_PER_CU);
  if (mode == 2) return launch_quantize_r<D, 2>(in_bf16, qjl, g_lds, grid, lds, a, s);
  if (mode == 1) return launch_quantize_r<D, 1>(in_bf16, qjl, g_lds, grid, lds, a, s);
  return launch_quantize_r<D, 0>(in_bf16, qjl, g_lds, grid, lds, a, s);
}

template <int D>
hipError_t launch_dequantize_d(bool out_bf16, const pqi::DequantArgs& a, const pqi::LaunchCfg& c, hipStream_t s) {
  const int64_t n_tiles = (a.n_blocks + 15) >> 4;
  const int grid = grid_for(n_tiles, c, PQ_DEQUANT_WG_PER_CU);
#define PQ_DQ_LAUNCH(PB)                                                                         \
  if (out_bf16) hipLaunchKernelGGL((pq_dequantize_kernel<D, true, PB>), grid, kThreads, 0, s, a); \
  else hipLaunchKernelGGL((pq_dequantize_kernel<D, false, PB>), grid, kThreads, 0, s, a);
  switch (a.pbits) {
    case 0: PQ_DQ_LAUNCH(0) break;
    case 1: PQ_DQ_LAUNCH(1) break;
    case 2: PQ_DQ_LAUNCH(2) break;
    case 3: PQ_DQ_LAUNCH(3) break;
    case 4: PQ_DQ_LAUNCH(4) break;
    case 5: PQ_DQ_LAUNCH(5) break;
    case 6: PQ_DQ_LAUNCH(6) break;
    case 7: PQ_DQ_LAUNCH(7) break;
    default: return hipErrorInvalidValue;
  }
#undef PQ_DQ_LAUNCH
  return hipGetLastError();
}

template <int D>
hipError_t launch_sketch_d(const pqi::SketchArgs& a, const pqi::LaunchCfg& c, hipStream_t s) {
  const int64_t n_tiles = (a.n_keys + 15) >> 4;
  const int m_pad = (a.m + 15) & ~15;
  const size_t glb = (size_t)m_pad * D * 2;
  const bool g_lds = glb <= (size_t)c.max_lds && glb <= 65536;
  // m a multiple of 128 with G in LDS: the row-grouped kernel (bits are 16-byte aligned)
  if constexpr (D <= 256) {
    if (g_lds && a.m % 128 == 0) {
      const int64_t n_pass = (a.n_keys + 16 * sketch8_nt<D>() - 1) / (16 * sketch8_nt<D>());
      const int g8 = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)c.cu_count * PQ_SKETCH8_WG_PER_CU,
                                                                 (n_pass + kSketch8Threads / 64 - 1) / (kSketch8Threads / 64)));
      if (a.oidx) hipLaunchKernelGGL((qjl_sketch_rows_kernel<D, true>), g8, kSketch8Threads, glb, s, a);
      else hipLaunchKernelGGL((qjl_sketch_rows_kernel<D, false>), g8, kSketch8Threads, glb, s, a);
      return hipGetLastError();
    }
  }
  const int grid = grid_for(n_tiles, c, PQ_SKETCH_WG_PER_CU);
  if (a.oidx) {
    if (g_lds) hipLaunchKernelGGL((qjl_sketch_kernel<D, true, true>), grid, kSketchThreads, glb, s, a);
    else hipLaunchKernelGGL((qjl_sketch_kernel<D, false, true>), grid, kSketchThreads, 0, s, a);
  } else {
    if (g_lds) hipLaunchKernelGGL((qjl_sketch_kernel<D, true, false>), grid, kSketchThreads, glb, s, a);
    else hipLaunchKernelGGL((qjl_sketch_kernel<D, false, false>), grid, kSketchThreads, 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int BITS, bool PK>
hipError_t launch_two_stage_dbp(const pqi::TwoStageArgs& a, int grid, int cpg, size_t lds, hipStream_t s) {
  if (a.m == 0) hipLaunchKernelGGL((pq_score_kernel<D, BITS, 0, PK>), grid, kThreads, lds, s, a, cpg);
  else if (a.m == D) hipLaunchKernelGGL((pq_score_kernel<D, BITS, D / 64, PK>), grid, kThreads, lds, s, a, cpg);
  else hipLaunchKernelGGL((pq_score_kernel<D, BITS, -1, PK>), grid, kThreads, lds, s, a, cpg);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_two_stage_db(const pqi::TwoStageArgs& a, int grid, int cpg, size_t lds, hipStream_t s) {
  if (a.packed) return launch_two_stage_dbp<D, BITS, true>(a, grid, cpg, lds, s);
  return launch_two_stage_dbp<D, BITS, false>(a, grid, cpg, lds, s);
}

template <int D>
hipError_t launch_two_stage_d(int bits, const pqi::TwoStageArgs& a, int grid, int cpg, size_t lds, hipStream_t s) {
  switch (bits) {
    case 1: return launch_two_stage_db<D, 1>(a, grid, cpg, lds, s);
    case 2: return launch_two_stage_db<D, 2>(a, grid, cpg, lds, s);
    case 3: return launch_two_stage_db<D, 3>(a, grid, cpg, lds, s);
    case 4: return launch_two_stage_db<D, 4>(a, grid, cpg, lds, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int BITS, bool PK>
hipError_t launch_attend_dbp(const pqi::AttnArgs& a, int grid, size_t lds, hipStream_t s) {
  if (a.m == 0) hipLaunchKernelGGL((pq_attend_kernel<D, BITS, 0, PK>), grid, kThreads, lds, s, a);
  else if (a.m == D) hipLaunchKernelGGL((pq_attend_kernel<D, BITS, D / 64, PK>), grid, kThreads, lds, s, a);
  else hipLaunchKernelGGL((pq_attend_kernel<D, BITS, -1, PK>), grid, kThreads, lds, s, a);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_attend_db(const pqi::AttnArgs& a, int grid, size_t lds, hipStream_t s) {
  if (a.packed) return launch_attend_dbp<D, BITS, true>(a, grid, lds, s);
  return launch_attend_dbp<D, BITS, false>(a, grid, lds, s);
}

template <int D>
hipError_t launch_attend_d(int bits, const pqi::AttnArgs& a, hipStream_t s) {
  static_assert(kWaves == pqi::kAttnWaves, "ranges per workgroup");
  if (a.n_parts > 0) {
    const int grid = a.n_heads * (D / pqi::attn_cols(D)) * a.n_parts;
    const size_t lds = std::max<size_t>((size_t)(pqi::prep_head_bytes(D, a.m) - pqi::prep_off_meta(D, a.m)),
                                        pqi::attn_merge_lds(D));
    hipError_t e = hipErrorInvalidValue;
    switch (bits) {
      case 1: e = launch_attend_db<D, 1>(a, grid, lds, s); break;
      case 2: e = launch_attend_db<D, 2>(a, grid, lds, s); break;
      case 3: e = launch_attend_db<D, 3>(a, grid, lds, s); break;
      case 4: e = launch_attend_db<D, 4>(a, grid, lds, s); break;
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pq_attend_combine_kernel<D>, a.n_heads * a.n_q, kCombineThreads, (size_t)a.n_parts * 4, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Bandwidth probe with the traffic of dequantize and none of its arithmetic: every byte in is
// written back zero-extended to 16 bits (1 byte read, 2 written per value).  Lane i of a load
// takes 8 consecutive bytes and writes the 16 bytes they become, so every load and store
// instruction covers one contiguous run (whole lines); four of each in flight per thread,
// non-temporal as in dequantize.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ u32x4 widen8(const u32x2& a) {
  return u32x4{__builtin_amdgcn_perm(0u, a.x, 0x0c010c00u), __builtin_amdgcn_perm(0u, a.x, 0x0c030c02u),
               __builtin_amdgcn_perm(0u, a.y, 0x0c010c00u), __builtin_amdgcn_perm(0u, a.y, 0x0c030c02u)};
}

__global__ __launch_bounds__(256) void pq_stream_probe_kernel(const uint8_t* in, uint16_t* out, int64_t n) {
  const u32x2* src = reinterpret_cast<const u32x2*>(in);
  u32x4* dst = reinterpret_cast<u32x4*>(out);
  const int64_t n8 = n >> 3;                                // whole 8-byte runs
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    u32x2 a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(widen8(a[u]), dst + i + u * stride);
  }
  for (; i < n8; i += stride) __builtin_nontemporal_store(widen8(__builtin_nontemporal_load(src + i)), dst + i);
  // the last n mod 8 values
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < (n & 7)) out[8 * n8 + t] = in[8 * n8 + t];
}

}  // namespace

// The library is compiled as six units of this file (PQ_UNIT 0 .. 5) in parallel: the
// quantize kernels for d = 64, 128; those for d = 256, 512; everything else but the
// two-stage score, the attention and the grouped codec; the two-stage score; the fused decode
// attention; the grouped (many-tensor) codec.  Without
// PQ_UNIT one unit holds all of it.  Kernels are templates or file-local, so each unit
// carries only the kernels its launch functions instantiate (plus the few non-template ones).
#ifndef PQ_UNIT
#define PQ_UNIT -1
#endif

namespace pqi {

#if PQ_UNIT < 0 || PQ_UNIT == 0
hipError_t launch_quantize_lo(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s) {
  switch (d) {
    case 64: return launch_quantize_d<64>(in_bf16, a, c, s);
    case 128: return launch_quantize_d<128>(in_bf16, a, c, s);
  }
  return hipErrorInvalidValue;
}
#endif

#if PQ_UNIT < 0 || PQ_UNIT == 1
hipError_t launch_quantize_hi(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s) {
  switch (d) {
    case 256: return launch_quantize_d<256>(in_bf16, a, c, s);
    case 512: return launch_quantize_d<512>(in_bf16, a, c, s);
  }
  return hipErrorInvalidValue;
}
#endif

#if PQ_UNIT < 0 || PQ_UNIT == 2
hipError_t launch_query_prep(const QueryPrepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(pq_query_rotate_kernel, a.n_heads * kScoreRows, 256, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.m > 0 && a.n_q > 0) {
    // G q of every live row into the sq block of its head
    ProjectArgs pa;
    pa.q = a.q; pa.n_q = (int64_t)a.n_heads * a.n_q; pa.proj = a.proj;
    pa.sq = reinterpret_cast<float*>(a.prep + prep_off_sq(a.d));
    pa.d = a.d; pa.m = a.m; pa.rows_per_group = a.n_q; pa.group_stride = prep_head_bytes(a.d, a.m) / 4;
    e = launch_project(pa, s);
    if (e != hipSuccess) return e;
  }
  const int words = 3 * (a.d / 64 + a.m / 64) * 256;
  const int slices = (words + kPrepWordsPerGroup - 1) / kPrepWordsPerGroup;
  hipLaunchKernelGGL(pq_query_quant_kernel, a.n_heads * slices, 256, 0, s, a, slices);
  return hipGetLastError();
}

#endif  // PQ_UNIT 2

#if PQ_UNIT < 0 || PQ_UNIT == 3
hipError_t launch_two_stage(int d, int bits, const TwoStageArgs& a, const LaunchCfg& c, hipStream_t s) {
  const int64_t n_pairs = (a.n_tok + 31) >> 5;           // a wave takes 32 tokens at a time
  int64_t per_group = ((int64_t)c.cu_count * 2 + a.n_heads - 1) / a.n_heads;
  const int64_t max_per_group = (n_pairs + kWaves - 1) / kWaves;
  if (per_group > max_per_group) per_group = max_per_group;
  if (per_group < 1) per_group = 1;
  const int grid = (int)(per_group * a.n_heads);
  const size_t lds = (size_t)(prep_head_bytes(d, a.m) - prep_off_meta(d, a.m));
  switch (d) {
    case 64: return launch_two_stage_d<64>(bits, a, grid, (int)per_group, lds, s);
    case 128: return launch_two_stage_d<128>(bits, a, grid, (int)per_group, lds, s);
    case 256: return launch_two_stage_d<256>(bits, a, grid, (int)per_group, lds, s);
    case 512: return launch_two_stage_d<512>(bits, a, grid, (int)per_group, lds, s);
  }
  return hipErrorInvalidValue;
}
#endif  // PQ_UNIT 3

#if PQ_UNIT < 0 || PQ_UNIT == 4
hipError_t launch_attention(int d, int bits, const AttnArgs& a, hipStream_t s) {
  switch (d) {
    case 64: return launch_attend_d<64>(bits, a, s);
    case 128: return launch_attend_d<128>(bits, a, s);
    case 256: return launch_attend_d<256>(bits, a, s);
    case 512: return launch_attend_d<512>(bits, a, s);
  }
  return hipErrorInvalidValue;
}
#endif  // PQ_UNIT 4

#if PQ_UNIT < 0 || PQ_UNIT == 5
}  // namespace pqi
namespace {
template <int D>
hipError_t launch_quantize_many_d(bool in_bf16, const pqi::QuantArgs& a, const pqi::TensorDesc* tab, int n_tensors,
                                  const pqi::LaunchCfg& c, hipStream_t s) {
  // bf16 blocks at d = 128 and 256 rotate on the matrix cores: their fragments after the grid
  const size_t lds = (size_t)a.t.ncell * a.t.nrep * 16 + ((D == 128 || D == 256) && in_bf16 ? kHfBytes : 0);
  const int grid = c.cu_count * PQ_MANY_WG_PER_CU;
  const int mode = a.pbits ? 2 : (a.t.nrep == 16 ? 1 : 0);
#define PQ_MANY_Q(MODE)                                                                                          \
  if (in_bf16) hipLaunchKernelGGL((pq_quantize_many_kernel<D, true, MODE>), grid, kThreads, lds, s, a, tab, n_tensors); \
  else hipLaunchKernelGGL((pq_quantize_many_kernel<D, false, MODE>), grid, kThreads, lds, s, a, tab, n_tensors);
  if (mode == 2) { PQ_MANY_Q(2) }
  else if (mode == 1) { PQ_MANY_Q(1) }
  else { PQ_MANY_Q(0) }
#undef PQ_MANY_Q
  return hipGetLastError();
}

template <int D>
hipError_t launch_dequantize_many_d(bool out_bf16, const pqi::DequantArgs& a, const pqi::TensorDesc* tab, int n_tensors,
                                    const pqi::LaunchCfg& c, hipStream_t s) {
  const int grid = c.cu_count * PQ_DEQUANT_WG_PER_CU;
#define PQ_MANY_DQ(PB)                                                                                            \
  if (out_bf16) hipLaunchKernelGGL((pq_dequantize_many_kernel<D, true, PB>), grid, kThreads, 0, s, a, tab, n_tensors); \
  else hipLaunchKernelGGL((pq_dequantize_many_kernel<D, false, PB>), grid, kThreads, 0, s, a, tab, n_tensors);
  switch (a.pbits) {
    case 0: PQ_MANY_DQ(0) break;
    case 1: PQ_MANY_DQ(1) break;
    case 2: PQ_MANY_DQ(2) break;
    case 3: PQ_MANY_DQ(3) break;
    case 4: PQ_MANY_DQ(4) break;
    case 5: PQ_MANY_DQ(5) break;
    case 6: PQ_MANY_DQ(6) break;
    case 7: PQ_MANY_DQ(7) break;
    default: return hipErrorInvalidValue;
  }
#undef PQ_MANY_DQ
  return hipGetLastError();
}
}  // namespace
namespace pqi {
hipError_t launch_quantize_many(int d, bool in_bf16, const QuantArgs& a, const TensorDesc* tab, int n_tensors,
                                const LaunchCfg& c, hipStream_t s) {
  switch (d) {
    case 64: return launch_quantize_many_d<64>(in_bf16, a, tab, n_tensors, c, s);
    case 128: return launch_quantize_many_d<128>(in_bf16, a, tab, n_tensors, c, s);
    case 256: return launch_quantize_many_d<256>(in_bf16, a, tab, n_tensors, c, s);
    case 512: return launch_quantize_many_d<512>(in_bf16, a, tab, n_tensors, c, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize_many(int d, bool out_bf16, const DequantArgs& a, const TensorDesc* tab, int n_tensors,
                                  const LaunchCfg& c, hipStream_t s) {
  switch (d) {
    case 64: return launch_dequantize_many_d<64>(out_bf16, a, tab, n_tensors, c, s);
    case 128: return launch_dequantize_many_d<128>(out_bf16, a, tab, n_tensors, c, s);
    case 256: return launch_dequantize_many_d<256>(out_bf16, a, tab, n_tensors, c, s);
    case 512: return launch_dequantize_many_d<512>(out_bf16, a, tab, n_tensors, c, s);
  }
  return hipErrorInvalidValue;
}
#endif  // PQ_UNIT 5

#if PQ_UNIT < 0 || PQ_UNIT == 2
hipError_t launch_stream_probe(const uint8_t* in, uint16_t* out, int64_t n, const LaunchCfg& c, hipStream_t s) {
  const int64_t want = std::max<int64_t>(1, ((n >> 3) + 1023) / 1024);   // four runs per thread
  const int grid = (int)std::min<int64_t>(want, (int64_t)c.cu_count * 16);
  hipLaunchKernelGGL(pq_stream_probe_kernel, grid, 256, 0, s, in, out, n);
  return hipGetLastError();
}

hipError_t launch_quantize_bd(bool in_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s) {
  // the search grid, the weights of the groups of four, then one block of fp32 per wave
  const size_t lds = (((size_t)a.ncell * a.nrep * 8 + 15) & ~(size_t)15) +
                     (size_t)(((a.d / 4 + 3) & ~3) + 4 * bd_words(a.d)) * sizeof(float);
  if (lds > (size_t)c.max_lds) return hipErrorInvalidConfiguration;
  const int64_t want = (a.n_blocks + 3) / 4;
  const int per_cu = std::max(1, std::min(4, (int)((size_t)c.max_lds / lds)));
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)c.cu_count * per_cu));
  if (in_bf16) hipLaunchKernelGGL(pq_quantize_bd_kernel<true>, grid, 256, lds, s, a);
  else hipLaunchKernelGGL(pq_quantize_bd_kernel<false>, grid, 256, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_dequantize_bd(bool out_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s) {
  const size_t lds = (size_t)4 * bd_words(a.d) * sizeof(float);      // one padded block of fp32 per wave
  const int64_t want = (a.n_blocks + 3) / 4;
  const int per_cu = std::max(1, std::min(4, (int)((size_t)c.max_lds / (lds + 1024))));
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)c.cu_count * per_cu));
  if (out_bf16) hipLaunchKernelGGL(pq_dequantize_bd_kernel<true>, grid, 256, lds, s, a);
  else hipLaunchKernelGGL(pq_dequantize_bd_kernel<false>, grid, 256, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_dense(bool in_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s) {
  if (in_bf16 && (a.d == 64 || a.d == 128) && ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.codes)) & 15) == 0 &&
      a.ncell > 0) {
    // bf16 matrix cores.  |y - y_exact| in units of 2^-24 ||x||: 2^-16 for the part of Pi left
    // out; one ulp for each of the d additions of the hi accumulation (terms summing to at most
    // 1.004 ||x||) and of the mid one (2^-8 of that), one for their sum; and the fp32 norm (d / 8
    // dot2 roundings, the sum over four lanes, the rsqrt, the final product).  10% on top.  The
    // grid test needs eps under a twentieth of the smallest boundary gap.
    const double units = 257.0 + 2.016 * a.d + 2.0 + 1.01 * (a.d / 8.0 + 6.0);
    const float eps = (float)(1.1 * units * 0x1p-24);
    const int nb = (1 << a.bits) - 1;
    double gap = INFINITY;
    for (int k = 0; k + 1 < nb; ++k) gap = std::min(gap, (double)a.beta[k + 1] - (double)a.beta[k]);
    const size_t lds = a.d == 64 ? DenseBLayout<64>::bytes(a.ncell) : DenseBLayout<128>::bytes(a.ncell);
    const size_t stat = ((size_t)1 << kMaxBits) * sizeof(double);   // the kernel's fp64 boundaries
    if (lds + stat <= (size_t)c.max_lds && (nb == 1 || eps < 0.05 * gap)) {
      const int per_cu = (int)std::max<size_t>(1, (size_t)c.max_lds / (lds + stat));
      const int64_t n_tiles = (a.n_blocks + 15) >> 4;
      const int grid = (int)std::max<int64_t>(
          1, std::min<int64_t>((n_tiles + kDenseBWaves - 1) / kDenseBWaves, (int64_t)c.cu_count * per_cu));
      if (a.d == 64) hipLaunchKernelGGL((pq_quantize_dense_bf16_kernel<64>), grid, 64 * kDenseBWaves, lds, s, a, eps);
      else hipLaunchKernelGGL((pq_quantize_dense_bf16_kernel<128>), grid, 64 * kDenseBWaves, lds, s, a, eps);
      return hipGetLastError();
    }
  }
  if (a.d == 64 || a.d == 128) {
    // Pi^T, the waves' blocks and the search grid; without room for the grid the kernel bisects
    BdArgs g = a;
    const size_t base = ((size_t)a.d * (a.d + 16) + kDenseQWaves * 16 * (size_t)(a.d + 4)) * sizeof(float);
    if (base + (size_t)a.ncell * 16 > (size_t)c.max_lds) g.ncell = 0;
    const size_t lds = base + (size_t)g.ncell * 16;
    const int64_t n_tiles = (a.n_blocks + 15) >> 4;
    const int grid = (int)std::max<int64_t>(
        1, std::min<int64_t>((n_tiles + kDenseQWaves - 1) / kDenseQWaves, (int64_t)c.cu_count * 2));
    const bool vec = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;   // 16-byte loads of the rows
#define PQ_DENSE_MFMA(DD, V)                                                                                             \
    if (in_bf16) hipLaunchKernelGGL((pq_quantize_dense_mfma_kernel<true, DD, V>), grid, 64 * kDenseQWaves, lds, s, g);  \
    else hipLaunchKernelGGL((pq_quantize_dense_mfma_kernel<false, DD, V>), grid, 64 * kDenseQWaves, lds, s, g);
    if (a.d == 64) {
      if (vec) { PQ_DENSE_MFMA(64, true) } else { PQ_DENSE_MFMA(64, false) }
    } else {
      if (vec) { PQ_DENSE_MFMA(128, true) } else { PQ_DENSE_MFMA(128, false) }
    }
#undef PQ_DENSE_MFMA
    return hipGetLastError();
  }
  // Pi^T in LDS when it fits, else read from global memory
  const bool pg = ((size_t)a.d * a.d + 4 * (size_t)a.d) * sizeof(float) > (size_t)c.max_lds;
  const size_t lds = ((pg ? 0 : (size_t)a.d * a.d) + 4 * (size_t)a.d) * sizeof(float);
  const int64_t want = (a.n_blocks + 3) / 4;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)c.cu_count * 4));
  if (pg) {
    if (in_bf16) hipLaunchKernelGGL((pq_quantize_dense_kernel<true, true>), grid, 256, lds, s, a);
    else hipLaunchKernelGGL((pq_quantize_dense_kernel<false, true>), grid, 256, lds, s, a);
  } else {
    if (in_bf16) hipLaunchKernelGGL((pq_quantize_dense_kernel<true, false>), grid, 256, lds, s, a);
    else hipLaunchKernelGGL((pq_quantize_dense_kernel<false, false>), grid, 256, lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_dense(bool out_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s) {
  if ((a.d == 64 || a.d == 128) && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0) {
    size_t lds;
    if (a.d == 64) lds = out_bf16 ? DenseDLayout<64, true>::bytes() : DenseDLayout<64, false>::bytes();
    else lds = out_bf16 ? DenseDLayout<128, true>::bytes() : DenseDLayout<128, false>::bytes();
    const size_t stat = ((size_t)1 << kMaxBits) * sizeof(uint32_t);
    if (lds + stat <= (size_t)c.max_lds) {
      const int per_cu = (int)std::max<size_t>(1, (size_t)c.max_lds / (lds + stat));
      const int64_t n_tiles = (a.n_blocks + 15) >> 4;
      const int grid = (int)std::max<int64_t>(
          1, std::min<int64_t>((n_tiles + kDenseDWaves - 1) / kDenseDWaves, (int64_t)c.cu_count * per_cu));
#define PQ_DENSE_F16(DD)                                                                                               \
      if (out_bf16) hipLaunchKernelGGL((pq_dequantize_dense_f16_kernel<DD, true>), grid, 64 * kDenseDWaves, lds, s, a); \
      else hipLaunchKernelGGL((pq_dequantize_dense_f16_kernel<DD, false>), grid, 64 * kDenseDWaves, lds, s, a);
      if (a.d == 64) { PQ_DENSE_F16(64) } else { PQ_DENSE_F16(128) }
#undef PQ_DENSE_F16
      return hipGetLastError();
    }
  }
  if (a.d == 64 || a.d == 128) {
    const size_t lds = (size_t)a.d * (a.d + 16) * sizeof(float);
    const int64_t n_tiles = (a.n_blocks + 15) >> 4;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n_tiles + 3) / 4, (int64_t)c.cu_count * 2));
#define PQ_DENSE_MFMA(DD)                                                                                   \
    if (out_bf16) hipLaunchKernelGGL((pq_dequantize_dense_mfma_kernel<true, DD>), grid, 256, lds, s, a);  \
    else hipLaunchKernelGGL((pq_dequantize_dense_mfma_kernel<false, DD>), grid, 256, lds, s, a);
    if (a.d == 64) { PQ_DENSE_MFMA(64) } else { PQ_DENSE_MFMA(128) }
#undef PQ_DENSE_MFMA
    return hipGetLastError();
  }
  const bool pg = ((size_t)a.d * a.d + 4 * (size_t)a.d) * sizeof(float) > (size_t)c.max_lds;
  const size_t lds = ((pg ? 0 : (size_t)a.d * a.d) + 4 * (size_t)a.d) * sizeof(float);
  const int64_t want = (a.n_blocks + 3) / 4;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)c.cu_count * 4));
  if (pg) {
    if (out_bf16) hipLaunchKernelGGL((pq_dequantize_dense_kernel<true, true>), grid, 256, lds, s, a);
    else hipLaunchKernelGGL((pq_dequantize_dense_kernel<false, true>), grid, 256, lds, s, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((pq_dequantize_dense_kernel<true, false>), grid, 256, lds, s, a);
    else hipLaunchKernelGGL((pq_dequantize_dense_kernel<false, false>), grid, 256, lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s) {
  return d <= 128 ? launch_quantize_lo(d, in_bf16, a, c, s) : launch_quantize_hi(d, in_bf16, a, c, s);
}

hipError_t launch_dequantize(int d, bool out_bf16, const DequantArgs& a, const LaunchCfg& c, hipStream_t s) {
  switch (d) {
    case 64: return launch_dequantize_d<64>(out_bf16, a, c, s);
    case 128: return launch_dequantize_d<128>(out_bf16, a, c, s);
    case 256: return launch_dequantize_d<256>(out_bf16, a, c, s);
    case 512: return launch_dequantize_d<512>(out_bf16, a, c, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sketch(int d, const SketchArgs& a, const LaunchCfg& c, hipStream_t s) {
  switch (d) {
    case 64: return launch_sketch_d<64>(a, c, s);
    case 128: return launch_sketch_d<128>(a, c, s);
    case 256: return launch_sketch_d<256>(a, c, s);
    case 512: return launch_sketch_d<512>(a, c, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_outliers(const OutlierArgs& a, hipStream_t s) {
  const int64_t waves = a.n_heads * a.n_groups;
  const int grid = (int)((waves + 3) / 4);
  switch (a.d) {
    case 64: hipLaunchKernelGGL(qjl_outlier_kernel<64>, grid, 256, 0, s, a); break;
    case 128: hipLaunchKernelGGL(qjl_outlier_kernel<128>, grid, 256, 0, s, a); break;
    case 256: hipLaunchKernelGGL(qjl_outlier_kernel<256>, grid, 256, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_project(const ProjectArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_q + 15) / 16), (unsigned)((a.m + 15) / 16));
  hipLaunchKernelGGL(qjl_project_kernel, grid, 64, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, const LaunchCfg& c, hipStream_t s) {
  const int groups = a.batch * a.kv_heads;
  // PQ_SCORE_WG_PER_CU workgroups per CU, at most one wave per 32 keys
#ifndef PQ_SCORE_WG_PER_CU
#define PQ_SCORE_WG_PER_CU 4
#endif
  int64_t per_group = ((int64_t)c.cu_count * PQ_SCORE_WG_PER_CU + groups - 1) / groups;
  const int64_t n_pairs = (a.n_keys + 31) >> 5;             // a wave takes 32 keys at a time
  const int64_t max_per_group = (n_pairs + kWaves - 1) / kWaves;
  if (per_group > max_per_group) per_group = max_per_group;
  if (per_group < 1) per_group = 1;
  const int grid = (int)(per_group * groups);
  const int cpg = (int)per_group;
  switch (a.m >> 6) {
#define PQ_SCORE_CASE(K)                                                                          \
    case K:                                                                                       \
      if (a.accumulate) hipLaunchKernelGGL((qjl_score_kernel<K, true>), grid, kThreads, 0, s, a, cpg); \
      else hipLaunchKernelGGL((qjl_score_kernel<K, false>), grid, kThreads, 0, s, a, cpg);             \
      break;
    PQ_SCORE_CASE(1) PQ_SCORE_CASE(2) PQ_SCORE_CASE(3) PQ_SCORE_CASE(4)
    PQ_SCORE_CASE(5) PQ_SCORE_CASE(6) PQ_SCORE_CASE(7) PQ_SCORE_CASE(8)
    PQ_SCORE_CASE(9) PQ_SCORE_CASE(10) PQ_SCORE_CASE(11) PQ_SCORE_CASE(12)
    PQ_SCORE_CASE(13) PQ_SCORE_CASE(14) PQ_SCORE_CASE(15) PQ_SCORE_CASE(16)
#undef PQ_SCORE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#endif  // PQ_UNIT 2

}  // namespace pqi

/*
 * pq.h - C ABI of the MI355X (gfx950) block codec and QJL sketch library.
 *
 * The library implements one data-parallel path:
 *
 *   * the rotate-then-quantize block codec: per block of d = 2^k values the
 *     L2 norm is stored as fp16, the block is normalised, rotated by the
 *     randomized Walsh-Hadamard transform R = H.D/sqrt(d), scaled by sqrt(d)
 *     and every coordinate is replaced by the index of its nearest Lloyd-Max
 *     centroid for N(0,1) (eliza quantization README, PolarQuant, "Algorithm
 *     in one paragraph"; glq 0.7.2 README, "How it works" item 2);
 *   * its inverse, centroid lookup -> /sqrt(d) -> R^T -> *norm (same section);
 *   * the optional QJL residual stage: packed signs of a Gaussian projection
 *     of the quantization residual r plus fp16(||r||) (same section, the 1-bit
 *     QJL residual correction; turbopress 0.4.2 README, "Package layout",
 *     qjl.py);
 *   * the QJL key sketch, fp16(||k||) and packed sign(S k) (eliza quantization
 *     README, QJL, "Algorithm in one paragraph");
 *   * the QJL asymmetric estimator of <q, k> from the packed key bits and the
 *     two-stage estimator of <q, x> from codes + residual bits (same section);
 *
 * and around it: the codes bit-packed at their width, the QJL outlier-channel
 * split sketch, fused decode attention over a quantized cache with an
 * unquantized recent window, the codec with a block-diagonal rotation for block
 * sizes that are not powers of two, and the codec with a dense random rotation
 * and the sphere-coordinate codebook (each declaration below cites its passage).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Status      0 (PQ_OK) on success, a PQ_E* code otherwise.  Arguments are
 *               validated synchronously before any HIP call; an invalid call
 *               launches nothing and writes nothing.  PQ_EHIP means a HIP API
 *               call failed; its hipError_t is kept per thread and returned by
 *               pq_last_hip_error().
 *   Execution   device entry points enqueue kernels on `stream` (a hipStream_t;
 *               NULL = the legacy default stream) and return without waiting.
 *               Faults inside a kernel surface at the caller's next
 *               synchronisation.  Calls on one stream run in order.
 *   Memory      every pointer argument of a device entry point is device
 *               memory allocated and owned by the caller; the library allocates
 *               nothing, keeps no pointer after return and holds no mutable
 *               global state (pq_attention_noalloc aside: it works in a fixed
 *               array of the library, see there), so concurrent calls from
 *               several threads are safe.  Host helpers take host memory.
 *   Alignment   tensors must be aligned to 16 bytes, except `norms`,
 *               `rnorms` (2 bytes) and the sign mask (1 byte).
 *   Empty input n_blocks == 0 (or n_keys == 0, n_q == 0, batch == 0) returns
 *               PQ_OK once the size parameters are valid; pointers are then not
 *               examined (they may be NULL) and nothing is launched.
 *   Dtypes      bf16 and fp16 values are passed as their uint16 bit patterns.
 *               PQ_F32 = IEEE fp32, PQ_BF16 = bfloat16.
 *   Signs D     `signs` is a d/8-byte mask, bit j (least significant bit
 *               first) set means D_j = -1.
 *   Projection  `proj` is the Gaussian JL matrix G, m x d row-major bf16.
 *   Bits        QJL sign bits are packed 8 per byte, least significant bit
 *               first; bit value 1 means sign +1, a projection of exactly 0
 *               gives bit 0 (qjl_apply.py, `_qjl_decode_keys`): a zero key or
 *               zero residual gives all-zero bits.  Projections are summed in
 *               fp32, so a nonzero one that cancels to exactly 0 there lies far
 *               inside the parity band of the exact value and may read either
 *               way (the key sketch reads it as +1).
 *   Limits      d in {64, 128, 256, 512} unless an entry point states other
 *               sizes; bits in 1..8; m a multiple of 8 in [8, 1024] (QJL
 *               residual stage and key sketch), a multiple of 64 in [64, 1024]
 *               for the score entry points; block norms must be finite (a norm
 *               >= 65520 is stored as fp16 +inf).
 */
#ifndef PQ_H
#define PQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQ_ABI_VERSION 1

#define PQ_OK 0
#define PQ_EINVAL 1        /* bad pointer, size, alignment, dtype or parameter */
#define PQ_EUNSUPPORTED 2  /* valid request outside what the kernels implement */
#define PQ_EHIP 3          /* a HIP runtime call failed, see pq_last_hip_error() */
#define PQ_ETOOBIG 4       /* needs more than the fixed work array of pq_attention_noalloc */

/* bytes of the fixed device work array behind pq_attention_noalloc (one copy per device) */
#define PQ_ATTN_NOALLOC_MAX_WORK (16 << 20)

#define PQ_F32 0
#define PQ_BF16 1

/* ---------------------------------------------------------------- host side */

int pq_abi_version(void);

/* Static description of a status code.  Never NULL. */
const char* pq_strerror(int status);

/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int pq_last_hip_error(void);

/*
 * Lloyd-Max quantizer for N(0,1) at `bits` bits, as used by the kernels
 * (eliza quantization README, PolarQuant, "Algorithm in one paragraph":
 * iterative conditional-expectation centroids; turbopress 0.4.2 README,
 * "Package layout", codebooks.py: float64 fixed point).
 *   centroids   out, 2^bits ascending values (may be NULL)
 *   boundaries  out, 2^bits - 1 midpoints of adjacent centroids (may be NULL)
 *   mse         out, distortion E[(X - Q(X))^2] of the fixed point (may be NULL)
 * Returns PQ_EINVAL for bits outside 1..8.  Thread safe; the first call for a
 * bit width runs the fixed-point iteration (up to ~0.1 s at 8 bits).
 */
int pq_codebook(int bits, double* centroids, double* boundaries, double* mse);

/*
 * The seeded random quantities of the codec, rebuilt from a 64-bit seed on the host (the
 * seed is the state that must persist: eliza quantization README, TurboQuant, "CLI",
 * --base-seed with layer i using seed base_seed + i, and dequantizing with other signs
 * giving garbage; QJL, "CLI", --projection-seed; qjl_apply.py draws its JL matrix from a
 * seeded generator per layer).  The generator is frozen so that any implementation
 * reproduces the bytes:
 *   mix(z)   = z3 ^ (z3 >> 31), z3 = (z2 ^ (z2 >> 27)) * 0x94D049BB133111EB,
 *              z2 = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9          (SplitMix64, mod 2^64)
 *   stream (seed, tag) starts in state s = mix(seed ^ tag); its output i is
 *   mix(s + (i + 1) * 0x9E3779B97F4A7C15); tag 0x5349474E for signs, 0x50524F4A for G.
 * pq_make_signs: D_j = -1 exactly when the top bit of output j is set; mask (host, d/8 bytes,
 *   written whole) holds D_j as bit j%8 of byte j/8, the sign-mask layout every entry point
 *   takes.  d a multiple of 8 in 8 .. 65536.
 * qjl_make_projection: G (host, m*d bf16 bit patterns, row-major, written whole); element
 *   k = i*d + j.  Outputs 2p and 2p+1 give u = ((out >> 11) + 0.5) 2^-53 in (0, 1) and the
 *   Box-Muller pair sqrt(-2 ln u1) (cos, sin)(2 pi u2) in double, each rounded to the
 *   nearest bf16 (ties to even).  m, d in 1 .. 65536 with m*d even.
 * Both return PQ_EINVAL for a NULL pointer or sizes outside these ranges; they touch no
 * device and are thread safe.
 */
int pq_make_signs(uint64_t seed, int d, uint8_t* mask);
int qjl_make_projection(uint64_t seed, int m, int d, uint16_t* proj);

/* ---------------------------------------------------------------- device side */

/*
 * Quantize n_blocks consecutive blocks of d values (eliza quantization
 * README, PolarQuant, "Algorithm in one paragraph").
 *   in_dtype   PQ_F32 or PQ_BF16; x holds n_blocks*d values, block b at x + b*d
 *   signs      d/8-byte rotation sign mask (device)
 *   codes      out, n_blocks*d bytes: code[b*d + i] = #{j : y_i > beta_j} for the
 *              rotated, normalised, sqrt(d)-scaled coordinate y_i (Sylvester
 *              order), decided in fp32
 *   norms      out, n_blocks fp16: fp16(||x_b||) round-to-nearest-even
 *   m          0 = no QJL stage (proj, qjl_bits, rnorms must then be NULL);
 *              otherwise the number of residual projections
 *   proj       G, m x d bf16 (device)
 *   qjl_bits   out, n_blocks * m/8 bytes: sign bits of G r, the seeded
 *              Gaussian matrix applied to the residual r = x - dequantize(code,
 *              norm) in the block's own coordinates
 *   rnorms     out, n_blocks fp16: fp16(||r||)
 */
int pq_quantize(int d, int bits, int in_dtype, const void* x, int64_t n_blocks,
                const uint8_t* signs, int m, const uint16_t* proj,
                uint8_t* codes, uint16_t* norms, uint8_t* qjl_bits, uint16_t* rnorms,
                void* stream);

/*
 * Dequantize: xhat_b = norm_b/d * D * (H c[code_b]) (eliza quantization README,
 * PolarQuant, "Algorithm in one paragraph": lookup -> /sqrt(d) -> inverse
 * rotation -> *norm).  QJL bits are not used.
 *   codes      n_blocks*d bytes, each < 2^bits
 *   norms      n_blocks fp16
 *   out_dtype  PQ_F32 or PQ_BF16 (round to nearest even); out holds n_blocks*d
 */
int pq_dequantize(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                  const uint8_t* signs, int out_dtype, void* out, void* stream);

/*
 * pq_quantize / pq_dequantize with the codes bit-packed (eliza quantization
 * README, TurboQuant, "Algorithm in one paragraph", step 4: indices packed into
 * bytes, two per byte at 4 bits and four per byte at 2 bits; the same stream
 * carries any width).  Arguments, outputs other than the codes, and errors as in
 * pq_quantize / pq_dequantize, except:
 *   codes      n_blocks * d*bits/8 bytes (16-byte aligned); block b at
 *              codes + b*d*bits/8 is a little-endian bit stream: bit j of code i
 *              is stream bit bits*i + j, stream bit p is bit p%8 of byte p/8
 *              (at 4 bits code 2k is the low nibble of byte k; at 8 bits the
 *              layout of pq_quantize)
 */
int pq_quantize_packed(int d, int bits, int in_dtype, const void* x, int64_t n_blocks,
                       const uint8_t* signs, int m, const uint16_t* proj,
                       uint8_t* codes, uint16_t* norms, uint8_t* qjl_bits, uint16_t* rnorms,
                       void* stream);
int pq_dequantize_packed(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                         const uint8_t* signs, int out_dtype, void* out, void* stream);

/*
 * Grouped codec: many tensors of one codec quantized (or dequantized) in one launch, a whole
 * weight set streamed in one pass (eliza quantization README, PolarQuant, "Algorithm in one
 * paragraph": the procedure runs over every linear weight tensor of the model).  Each tensor is
 * one pq_tensor record of a table in DEVICE memory (caller-owned, read by the kernels, not by
 * the host); the tiles of all tensors are split over the grid in table order.
 *   x          quantize input: n_blocks*d values of in_dtype (16-byte aligned)
 *   codes      n_blocks*d bytes, or n_blocks*d*bits/8 bit-packed (packed = 1), 16-byte aligned:
 *              written by pq_quantize_many, read by pq_dequantize_many
 *   norms      n_blocks fp16 (2-byte aligned): written / read likewise
 *   signs      d/8-byte rotation sign mask of this tensor (device), 4-byte aligned
 *   out        dequantize output: n_blocks*d values of out_dtype (16-byte aligned); unused by
 *              pq_quantize_many (may be NULL)
 *   n_blocks   blocks of this tensor, >= 0 (a zero-block tensor is skipped)
 * The result equals one pq_quantize / pq_dequantize (or their packed forms) per tensor, with
 * no QJL stage.  The host validates d, bits, the dtype, packed, n_tensors and the table
 * pointer (8-byte aligned); the records themselves live in device memory and are not
 * checked: each must meet the conditions above, as for the single-tensor calls.
 */
typedef struct {
  const void* x;
  uint8_t* codes;
  uint16_t* norms;
  const uint8_t* signs;
  void* out;
  int64_t n_blocks;
} pq_tensor;

int pq_quantize_many(int d, int bits, int in_dtype, int packed, int n_tensors, const pq_tensor* table,
                     void* stream);
int pq_dequantize_many(int d, int bits, int out_dtype, int packed, int n_tensors, const pq_tensor* table,
                       void* stream);

/*
 * QJL key sketch (eliza quantization README, QJL, "Algorithm in one paragraph").
 *   keys       n_keys*d bf16, key t at keys + t*d
 *   proj       G, m x d bf16
 *   bits       out, n_keys * m/8 bytes: sign(G k) packed LSB-first
 *   norms      out, n_keys fp16: fp16(||k||)
 */
int qjl_sketch(int d, int m, const uint16_t* keys, int64_t n_keys, const uint16_t* proj,
               uint8_t* bits, uint16_t* norms, void* stream);

/*
 * Project queries through the JL matrix: sq[i] = G q_i in fp32 (the query side
 * of the QJL estimator, same section).
 *   q          n_q*d bf16;  sq  out, n_q*m fp32
 */
int qjl_project(int d, int m, const uint16_t* q, int64_t n_q, const uint16_t* proj, float* sq,
                void* stream);

/*
 * QJL asymmetric estimator for grouped-query attention (eliza quantization
 * README, QJL, "Algorithm in one paragraph"; GQA score kernel named there):
 *   scores[b][h][t] = norm[b][g][t] * sqrt(pi/2)/m * sum_i (2 bit_i - 1) sq[b][h][i]
 * with g = h / (q_heads / kv_heads).
 *   sq         batch*q_heads*m fp32 from qjl_project
 *   bits       batch*kv_heads*n_keys * m/8 bytes (layout [b][g][t][m/8])
 *   norms      batch*kv_heads*n_keys fp16
 *   scores     out, batch*q_heads*n_keys fp32
 * q_heads must be a multiple of kv_heads with q_heads/kv_heads <= 4.
 */
int qjl_score(int m, int batch, int kv_heads, int q_heads, int64_t n_keys, const float* sq,
              const uint8_t* bits, const uint16_t* norms, float* scores, void* stream);

/*
 * Outlier channels of the keys (eliza quantization README, QJL, "Algorithm in one
 * paragraph": a top-k outlier sketch per group of group_size consecutive tokens;
 * qjl_apply.py, calibrate_key_outliers: channel norms over the group's tokens, top-k
 * indices as uint8).  Per head and group of group_size consecutive tokens (the last
 * group may be shorter), the n_out channels of largest L2 norm over the group's
 * tokens, in decreasing norm (sums of squares in fp32; ties to the lower channel).
 *   d          64, 128 or 256 (indices are bytes); 512 -> PQ_EUNSUPPORTED
 *   keys       n_heads*seq_len*d bf16, head h, token t at keys + (h*seq_len + t)*d
 *   idx        out, n_heads * ceil(seq_len/group_size) * n_out bytes, [head][group][rank]
 *   n_out      1 .. d
 */
int qjl_outlier_channels(int d, const uint16_t* keys, int64_t n_heads, int64_t seq_len, int group_size,
                         int n_out, uint8_t* idx, void* stream);

/*
 * qjl_sketch of one part of each key, split by its group's outlier channels (idx as
 * written by qjl_outlier_channels): part 0 sketches the key with those channels set
 * to zero (with G = S, m projections), part 1 the key on those channels only (with
 * its own matrix S_o, dim_outlier = m projections).  bits and norms as in qjl_sketch,
 * over n_heads*seq_len keys.  The score of a key is the sum of the two estimators
 * (qjl_score on part 0, then qjl_score_add on part 1): q.k = q.k_in + q.k_out.
 *   d          64, 128 or 256; part 0 or 1; other arguments as above
 */
int qjl_sketch_split(int d, int m, const uint16_t* keys, int64_t n_heads, int64_t seq_len, int group_size,
                     int n_out, const uint8_t* idx, int part, const uint16_t* proj, uint8_t* bits,
                     uint16_t* norms, void* stream);

/*
 * qjl_score that adds its estimate to the scores already in `scores` (the second
 * term of the split estimator).  Arguments and errors as in qjl_score.
 */
int qjl_score_add(int m, int batch, int kv_heads, int q_heads, int64_t n_keys, const float* sq,
                  const uint8_t* bits, const uint16_t* norms, float* scores, void* stream);

/*
 * Two-stage estimator of <q, x> from the stored codes and QJL residual bits,
 * without reconstructing x (eliza quantization README, TurboQuant, "Algorithm in
 * one paragraph"; scores straight from the packed indices: same README, "Fused
 * TurboQuant"):
 *   score = n16/d * <H(D q), c[code]> + rnorm16 * sqrt(pi/2)/m * <G q, 2 b - 1>
 * where <H(D q), c[code]> n16/d = <q, dequantize(code, n16)> since H is symmetric.
 *
 * pq_query_prep_bytes: bytes of the prepared-query buffer for n_heads heads
 * (-1 for invalid d or m).  Per head, at stride pq_query_prep_bytes(d, m, 1):
 *   float qrot[16][d]   H (D q) of query row r, rows >= n_q zero
 *   float sq[16][m]     G q
 *   float scale[2][16], int32 isum[2][16], then int8 limb tiles (internal)
 *
 * pq_query_prep: fill that buffer.
 *   q          n_heads * n_q * d bf16, layout [head][query][d], 1 <= n_q <= 16
 *   signs      the rotation sign mask of the codes to be scored
 *   proj       G, m x d bf16 (NULL when m == 0)
 *   prep       out, pq_query_prep_bytes(d, m, n_heads) bytes, 16-byte aligned
 *
 * pq_score: scores[h][i][t] for every head h, query i < n_q and token t.
 *   codes      n_heads * n_tok * d bytes, layout [head][token][d] (pq_quantize output)
 *   norms      n_heads * n_tok fp16
 *   qjl_bits   n_heads * n_tok * m/8 bytes, rnorms n_heads * n_tok fp16 (both
 *              NULL when m == 0: the score is then the first term alone)
 *   scores     out, n_heads * n_q * n_tok fp32, layout [head][query][token]
 * Limits: bits in 1..4 (PQ_EUNSUPPORTED above), m a multiple of 64 with
 * d + m <= 1344, n_q <= 16 (call again for more queries).  The query terms are
 * carried as integers of 21 bits relative to their largest entry; the sums
 * over d and m are exact.
 */
int64_t pq_query_prep_bytes(int d, int m, int n_heads);
int pq_query_prep(int d, int m, int n_heads, int n_q, const uint16_t* q, const uint8_t* signs,
                  const uint16_t* proj, void* prep, void* stream);
int pq_score(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
             const uint8_t* codes, const uint16_t* norms, const uint8_t* qjl_bits, const uint16_t* rnorms,
             float* scores, void* stream);

/*
 * pq_score reading bit-packed codes (eliza README, TurboQuant, "Algorithm in one
 * paragraph", step 4; eliza README, "Fused TurboQuant": scores straight from the
 * packed indices).  As pq_score, except:
 *   codes      n_heads * n_tok * d*bits/8 bytes (16-byte aligned), each token's
 *              codes one little-endian bit stream as written by pq_quantize_packed
 */
int pq_score_packed(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                    const uint8_t* codes, const uint16_t* norms, const uint8_t* qjl_bits,
                    const uint16_t* rnorms, float* scores, void* stream);

/*
 * Decode attention over the quantized cache plus an unquantized recent window, fused
 * (eliza quantization README, TurboQuant, "Algorithm in one paragraph": the cache holds
 * codes and norms, decoded by centroid lookup and inverse rotation at attention time, the
 * last residual_length tokens unquantized; same README, "Fused TurboQuant": scores straight
 * from the stored codes; glq 0.7.2 README, "Inline-dequant E8 KV": K/V decoded inside the
 * attention kernel, each read once, no workspace of decoded vectors).  For every head h and
 * query row i < n_q:
 *   s_t = the pq_score estimate of <q, k_t> (t < n_tok), s_w = <q, k_win[w]> (w < n_win),
 *   p   = softmax(sm_scale * [s_t ; s_w]),
 *   out[h][i] = sum_t p_t dequantize(v_t) + sum_w p_w v_win[w].
 * The value codes are read once and never decoded to memory: the kernel sums
 * p_t n16_t / d c[code_t] in the rotated basis and rotates back once per query.
 *
 * pq_attention_work_bytes: bytes of the work buffer (partial maxima, sums and rotated
 * outputs of the fused kernel; 0 when n_tok == 0, -1 for invalid arguments).
 *
 * pq_attention:
 *   d, bits, m  the codec of the keys (bits 1..4; m = 0: no QJL residual); the values
 *               use the same d and bits without a residual
 *   prep        pq_query_prep of q with the KEY signs (and G when m > 0)
 *   k_codes     n_heads * n_tok * d bytes [head][token][d], 16-byte aligned
 *   k_norms     n_heads * n_tok fp16; k_qjl_bits n_heads * n_tok * m/8 bytes and
 *               k_rnorms n_heads * n_tok fp16 (both NULL when m == 0)
 *   v_codes, v_norms  the values, as k_codes and k_norms (pq_quantize with m = 0)
 *   v_signs     the rotation sign mask of the values, d/8 bytes of device memory
 *   n_win       window tokens, 0 .. 4096; k_win, v_win bf16 [head][n_win][d] (16-byte
 *               aligned), q the bf16 queries [head][n_q][d] (all three may be NULL when
 *               n_win == 0)
 *   sm_scale    softmax scale (finite; 1/sqrt(d) in the usual attention)
 *   work        pq_attention_work_bytes(d, n_heads, n_tok) bytes, 16-byte aligned,
 *               device memory; its contents on entry do not matter
 *   out         n_heads * n_q * d fp32, layout [head][query][d]
 * n_tok + n_win must be at least 1 (PQ_EINVAL); n_q <= 16 per call.  All device pointers
 * are caller-owned; the call is asynchronous on `stream` and allocates nothing.  Scores
 * carry pq_score's precision; the probabilities and centroids enter the matrix cores as
 * fp16 pairs (about 22 significant bits) and accumulate in fp32.
 */
int64_t pq_attention_work_bytes(int d, int n_heads, int64_t n_tok);
int pq_attention(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                 const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits, const uint16_t* k_rnorms,
                 const uint8_t* v_codes, const uint16_t* v_norms, const uint8_t* v_signs, int64_t n_win,
                 const uint16_t* k_win, const uint16_t* v_win, const uint16_t* q, float sm_scale, void* work,
                 float* out, void* stream);

/*
 * pq_attention over bit-packed key and value codes (d*bits/8 bytes per token, as written
 * by pq_quantize_packed; eliza README, TurboQuant, "Algorithm in one paragraph", step 4).
 */
int pq_attention_packed(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                        const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits,
                        const uint16_t* k_rnorms, const uint8_t* v_codes, const uint16_t* v_norms,
                        const uint8_t* v_signs, int64_t n_win, const uint16_t* k_win, const uint16_t* v_win,
                        const uint16_t* q, float sm_scale, void* work, float* out, void* stream);

/*
 * pq_attention / pq_attention_packed for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the work
 * buffer is not an argument but a fixed array of PQ_ATTN_NOALLOC_MAX_WORK bytes in device
 * memory that the library holds on every device it runs on until the process ends.  The
 * call allocates nothing and frees nothing.
 *   packed     0: byte codes (as pq_attention), 1: bit-packed codes (as pq_attention_packed)
 *   other arguments, outputs and errors as pq_attention without `work`
 * Returns PQ_ETOOBIG, launching nothing, when pq_attention_work_bytes(d, n_heads, n_tok)
 * exceeds PQ_ATTN_NOALLOC_MAX_WORK (8.4 MB at 8 heads x 65536 tokens, d = 256 or 512).
 * Every call on one device shares that device's array and leaves its partial results there
 * (their contents on entry do not matter): calls that overlap in time on one device -- on
 * two streams, or from two threads -- race and give undefined results; calls on one stream
 * run in order and are safe.  The first call on a device looks up the array's address
 * there (a HIP runtime call, made after the arguments are validated).
 */
int pq_attention_noalloc(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                         const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits,
                         const uint16_t* k_rnorms, const uint8_t* v_codes, const uint16_t* v_norms,
                         const uint8_t* v_signs, int64_t n_win, const uint16_t* k_win, const uint16_t* v_win,
                         const uint16_t* q, float sm_scale, int packed, float* out, void* stream);

/*
 * Block sizes that are not powers of two (glq 0.7.2 README, "Advanced / Bit widths": a size
 * split into power-of-two blocks, 2688 = 2048 + 512 + 128; turbopress 0.4.2 README, "Package
 * layout": block-diagonal Walsh-Hadamard times Rademacher signs).  The codec of pq_quantize
 * with R = blockdiag(H_{d_k} / sqrt(d_k)) diag(D), d_k the powers of two of d's binary
 * expansion, largest first:
 *   y_k = sqrt(d / d_k) H_k (D x)_k / ||x||,  code_i = #{j : y_i > beta_j},  n16 = fp16(||x||),
 *   xhat_k = n16 / sqrt(d d_k) . D_k * (H_k c_k).
 * For a power of two this is the pq_quantize codec (codes may differ from pq_quantize's only
 * where a coordinate lies on the fp32 rounding edge of a boundary).
 *   d          a multiple of 32 in 64 .. 4096 (PQ_EINVAL if not a multiple of 32,
 *              PQ_EUNSUPPORTED outside the range)
 *   bits       1 .. 8; no QJL residual stage
 *   x          n_blocks * d values, fp32 or bf16 (in_dtype), 16-byte aligned
 *   signs      d/8-byte rotation sign mask (device)
 *   codes      out, n_blocks * d bytes, 16-byte aligned; norms out, n_blocks fp16
 * pq_dequantize_bd: codes and norms as written above -> out, n_blocks * d values of
 * out_dtype (fp32 or bf16 RNE), 16-byte aligned.  Asynchronous on `stream`, no allocation.
 */
int pq_quantize_bd(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const uint8_t* signs,
                   uint8_t* codes, uint16_t* norms, void* stream);
int pq_dequantize_bd(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                     const uint8_t* signs, int out_dtype, void* out, void* stream);

/*
 * Dense random rotation with the sphere-coordinate codebook (eliza quantization README,
 * TurboQuant, "Algorithm in one paragraph": the unit vector is rotated by a fixed random
 * orthogonal matrix Pi drawn by QR with a sign fix; each coordinate then follows the law of one
 * coordinate of a uniform point on the sphere, density proportional to (1 - t^2)^((d-3)/2), and
 * is bucketed against that law's Lloyd-Max centroids; x comes back as ||x|| Pi^T c).
 *   y = Pi x / ||x||,  code_i = #{j : y_i > beta_j},  n16 = fp16(||x||),  xhat = n16 Pi^T c.
 * pq_sphere_codebook: that law's Lloyd-Max centroids (2^bits, ascending) and boundaries
 *   (2^bits - 1) for bits 1..8 and d >= 3, host arrays (either may be NULL).
 * pq_quantize_dense / pq_dequantize_dense:
 *   d          a multiple of 16 up to 512 (PQ_EINVAL / PQ_EUNSUPPORTED otherwise); d = 64 and
 *              128 run on the matrix cores (bf16 blocks with x and codes 16-byte aligned on the
 *              bf16 ones, Pi split exactly into bf16 parts; otherwise fp32 ones), other d one
 *              block per wave with Pi in LDS while it fits (d <= 192) and read from global
 *              memory above.  Every code is the fp64 decision: codes whose fast value lies
 *              within the kernels' error bound of a boundary are decided again in fp64
 *   bits       1 .. 8
 *   rot        Pi, d x d fp32 row-major, device memory (the caller draws it; any orthogonal
 *              matrix is accepted and not checked)
 *   x          n_blocks * d values, fp32 or bf16 (in_dtype); codes n_blocks * d bytes (16-byte
 *              aligned for pq_dequantize_dense); norms n_blocks fp16; out n_blocks * d values
 *              of out_dtype (fp32 or bf16 RNE)
 * Asynchronous on `stream`, no allocation.
 */
int pq_sphere_codebook(int bits, int d, double* centroids, double* boundaries);
int pq_quantize_dense(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const float* rot,
                      uint8_t* codes, uint16_t* norms, void* stream);
int pq_dequantize_dense(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                        const float* rot, int out_dtype, void* out, void* stream);

/*
 * Measurement aid, not part of the method: a stream with the memory traffic of dequantize
 * (one byte read and two written per value) and none of its arithmetic, the ceiling that
 * dequantize is measured against.  out[i] = in[i] zero-extended to 16 bits, i < n.
 *   in         n bytes (16-byte aligned);  out  n uint16 (16-byte aligned)
 * Asynchronous on `stream`, no allocation; PQ_EINVAL for n < 0 or a bad pointer.
 */
int pq_probe_stream(const uint8_t* in, uint16_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ_H */

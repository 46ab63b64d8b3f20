/*
 * kvq_oracle.h -- plain, slow CPU oracle for the Hadamard-rotated token-wise
 * INT4 paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this library: only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg do.  It shares no code, header, table
 * or constant with the GPU library; it is written from the method's
 * description alone.
 *
 * Method (what is computed):
 *   - "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM
 *     Serving" (summary page, Research Findings; idea page, Core Innovation):
 *     each new key/value vector is rotated by a block-diagonal Hadamard
 *     matrix and then quantized to 4 bits with one quantization group per
 *     token (per token and KV head); the kernel that does this writes
 *     straight into a paged KV-cache layout, and attention runs fused over
 *     the quantized paged cache.
 *   - "InnerQ" (Table 3): scale factors and zero points are kept as FP16.
 *   - "BitDecoding-FP4" (Abstract): Hadamard rotation is one of the tools
 *     that suppresses key outliers under token-wise scaling.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   R1  group = all head_dim channels of one (token, KV head, K|V) vector.
 *   R2  asymmetric: x_hat = code * scale + zero, zero = min, codes 0..15,
 *       scale = (max - min) / 15, both rounded to FP16 (round to nearest even).
 *   R3  Hadamard: Sylvester order H[i][j] = (-1)^popcount(i & j), block size b
 *       on contiguous channel blocks, normalised by the fp32 constant 1/sqrt(b);
 *       the fp32 butterfly runs stages h = 1, 2, 4, ..., b/2 in that order and
 *       the scale is applied after the last stage.  b = 0 means no rotation
 *       (plain INT4).
 *   R4  code = clamp(round_half_even((y - zero) * (1 / scale)), 0, 15), with
 *       1/scale and each product/difference rounded separately in fp32; a
 *       zero scale gives 1/scale = 0 (all codes 0).
 *   R5  the signed zero of min and of (max - min) is made +0 by adding +0.0f.
 *   R6  the query is rotated by the same block Hadamard so q.k is preserved;
 *       the attention output is returned in the original (un-rotated) basis.
 *   R9  INT8 variant ("GPU-Accelerated INT8 Quantization for KV Cache
 *       Compression in Large Language Models", Abstract, which gives no
 *       formula): the same token-wise asymmetric quantizer with 8-bit codes,
 *       codes 0..255, scale = (max - min) / 255, everything else as R2-R5.
 *   R10 per-block groups (a variant of R1; "InnerQ" Abstract
 *       and Figure 1 group along the inner dimension): one group per
 *       `group` consecutive channels of the rotated vector (normally the
 *       Hadamard block), each with its own fp16 scale and zero as in R2.
 *   R12 MXFP4 variant ("BitDecoding-FP4", Abstract: native FP4 KV cache with
 *       Hadamard rotation under token-wise scaling; the block format is the
 *       OCP microscaling MXFP4 one): each 32 consecutive channels of the
 *       rotated vector share an E8M0 scale 2^X with X = floor(log2 max|y|)
 *       - 2 (-127 for an all-zero block), and each element is y / 2^X
 *       rounded to the nearest E2M1 value {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 *       (ties to the code with mantissa bit 0, saturating at 6, sign only
 *       on nonzero codes).  Decoded value = E2M1 value * 2^X.
 *   R13 scale search for keys ("BitDecoding-FP4", Abstract: outlier-aware
 *       key quantization combines Hadamard rotation with a scale search under
 *       token-wise scaling; the pages give neither the grid nor the
 *       criterion): the token-wise INT4 quantizer of R2 is tried over the key
 *       vector's range [mn, mx] shrunk toward zero by alpha_j = (16 - j)/16,
 *       j = 0 .. 7 (mn * alpha_j and mx * alpha_j in fp32; elements outside
 *       the range are clamped by the codes' clamp), and the candidate with the
 *       smallest grid SSE wins (the smaller j on a tie; j = 0 is the plain
 *       quantizer).  Grid SSE: each element decoded as code * scale + zero
 *       (fp32, the product exact, the sum rounded once), its error rounded
 *       once in fp32, scaled by 2^k with k = 20 - ex where max |y| < 2^ex
 *       (frexp), rounded to an integer (ties to even), squared and summed in
 *       64-bit integers: exact, so the sum's order does not matter.  Values
 *       keep the plain quantizer.
 *   R14 hybrid symmetric/asymmetric per group ("InnerQ", Abstract and
 *       Figure 3: symmetric or asymmetric quantization chosen per group from
 *       the group's own statistics; the rule is not given): the asymmetric
 *       candidate is R2 over the group; the symmetric one has scale =
 *       fp16(amax / 7), amax = max |y|, and zero = -8 * scale (exact in
 *       fp16), so the levels (code - 8) * scale hold 0 and reach 7 * scale =
 *       amax; both take the codes of R4.  The symmetric one is kept when its
 *       grid SSE (as in R13) is not larger, and is then marked by setting the
 *       sign bit of the stored fp16 scale; a decoded element is code *
 *       |scale| + zero in both modes.  A group of zeros, or one whose
 *       symmetric scale is 0 or whose -8 * scale overflows fp16, stays
 *       asymmetric.
 *   R7  softmax scale is a parameter (normally 1/sqrt(head_dim)); grouped
 *       query attention maps query head h to KV head h / (Hq / Hkv); an empty
 *       sequence gives a zero output; slot < 0 means "do not store".
 *
 * Cache layout (the on-device format; both implementations follow this text):
 *   page size P = 16 tokens, head_dim D in {64, 128}.
 *   INT4 pool: [num_pages][num_kv_heads][slab], slab = P * (D + 8) bytes:
 *     bytes [0, P*D/2)        K codes, token-major: byte t*(D/2) + j holds
 *                             channel 2j in bits 0..3 and 2j+1 in bits 4..7.
 *     bytes [P*D/2, P*D)      V codes, channel-group-major: the 4-byte word
 *                             index n*P + t (n = 0 .. D/8-1) holds channels
 *                             8n .. 8n+7 of token t; its byte j holds channel
 *                             8n+2j in bits 0..3 and 8n+2j+1 in bits 4..7.
 *     bytes [P*D, P*D+4P)     K sidecar: token t -> fp16 scale at 4t, fp16 zero
 *                             at 4t+2 (little endian).
 *     bytes [P*D+4P, P*D+8P)  V sidecar, same form.
 *   INT8 pool (token-wise INT8 variant, reading R9): [num_pages][num_kv_heads]
 *   [slab], slab = P * (2*D + 8) bytes:
 *     bytes [0, P*D)          K codes, token-major: byte t*D + c = channel c.
 *     bytes [P*D, 2*P*D)      V codes: the 4-byte word index (n*P + t)*2 + h
 *                             (n = 0 .. D/8-1, h = 0, 1) holds channels
 *                             8n+4h .. 8n+4h+3 of token t, byte j = channel
 *                             8n+4h+j.
 *     bytes [2*P*D, +4P)      K sidecar as in the INT4 pool; then V sidecar.
 *   Grouped INT4 pool (R10, group size g dividing D, at least 16):
 *   [num_pages][num_kv_heads][slab], slab = P * (D + 8 * (D/g)) bytes:
 *     bytes [0, P*D/2)        K codes as in the INT4 pool.
 *     bytes [P*D/2, P*D)      V codes: the 4-byte word index n*P + t (n < D/8)
 *                             holds channels n + (D/8) j, j = 0..7, of token t
 *                             (nibble j: byte j/2, bits 4(j%2)..+3).
 *     bytes [P*D, +4P*D/g)    K sidecar: token t, group i -> fp16 scale at
 *                             4(t*(D/g) + i), fp16 zero 2 bytes later.
 *     then the V sidecar in the same form.  The scale's sign bit marks a
 *     symmetric group of the hybrid quantizer (R14); a decoded element is
 *     code * |scale| + zero.
 *   MXFP4 pool (R12): [num_pages][num_kv_heads][slab], slab = P * (D + D/16)
 *   bytes:
 *     bytes [0, P*D)          K and V E2M1 codes, placed as the grouped INT4
 *                             pool places its codes (nibble = sign << 3 |
 *                             magnitude code).
 *     bytes [P*D, +P*D/32)    K scales: byte t*(D/32) + i = E8M0 of token t,
 *                             channels 32i .. 32i+31.
 *     then the V scales in the same form.
 *   bf16 pool: [num_pages][num_kv_heads][slab], slab = 2 * P * D * 2 bytes:
 *     K: bf16 element index t*D + c (token-major);
 *     V: bf16 element index P*D + ((n*(P/4) + g)*8 + j)*4 + i for channel
 *        c = 8n + j and token t = 4g + i.
 *   A token in slot s lives in page s / P at offset s % P.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of k, v and q inputs: 0 = fp16, 1 = bf16 (bit patterns) */
enum { KVQO_F16 = 0, KVQO_BF16 = 1 };

/* ---- scalar formats -------------------------------------------------- */
uint16_t kvq_oracle_f32_to_f16(float x);    /* round to nearest even      */
float    kvq_oracle_f16_to_f32(uint16_t h); /* exact                      */
uint16_t kvq_oracle_f32_to_bf16(float x);   /* round to nearest even      */
float    kvq_oracle_bf16_to_f32(uint16_t h);/* exact                      */

/* fp32 normalisation constant of a Hadamard block (1/sqrt(b) in fp32). */
float kvq_oracle_block_scale(int32_t b);

/* ---- per-vector steps ------------------------------------------------ */
/* y = blockdiag(H_b / sqrt(b)) x in fp32 with the butterfly of R3.  b = 0
 * (or 1) copies x.  x and y may alias. */
void kvq_oracle_rotate(const float* x, float* y, int32_t d, int32_t b);

/* Token-wise asymmetric INT4 of one vector (R2, R4, R5): codes[d] in 0..15
 * (one per byte, unpacked), fp16 bit patterns of scale and zero. */
void kvq_oracle_quantize(const float* y, int32_t d, uint8_t* codes,
                         uint16_t* scale, uint16_t* zero);

/* The same with 8-bit codes 0..255 and scale (max - min) / 255 (R9). */
void kvq_oracle_quantize_int8(const float* y, int32_t d, uint8_t* codes,
                              uint16_t* scale, uint16_t* zero);

/* Grid SSE of R13/R14 for n elements under (codes, fp16 scale, fp16 zero),
 * on the grid 2^-k; and the k of R13/R14 for elements of magnitude at most
 * amax. */
int64_t kvq_oracle_grid_sse(const float* y, int32_t d, const uint8_t* codes, uint16_t scale,
                            uint16_t zero, int32_t k);
int32_t kvq_oracle_grid_exponent(float amax);

/* Token-wise INT4 of one key vector with the scale search of R13; returns
 * the chosen j (alpha = (16 - j) / 16). */
int32_t kvq_oracle_quantize_search(const float* y, int32_t d, uint8_t* codes,
                                   uint16_t* scale, uint16_t* zero);

/* Hybrid INT4 of one group of g values (R14); returns 1 for the symmetric
 * mode (its scale then carries the sign bit), 0 for the asymmetric one. */
int32_t kvq_oracle_quantize_hybrid(const float* y, int32_t g, uint8_t* codes,
                                   uint16_t* scale, uint16_t* zero);

/* E2M1 code of one value (R12) and the value of a code. */
uint8_t kvq_oracle_e2m1_encode(float v);
double  kvq_oracle_e2m1_decode(uint8_t code);

/* One MXFP4 block of n values (R12): codes and the E8M0 scale byte. */
void kvq_oracle_quantize_mx(const float* y, int32_t n, uint8_t* codes, uint8_t* scale_e8m0);

/* ---- cache steps ----------------------------------------------------- */
size_t kvq_oracle_int4_slab_bytes(int32_t page_size, int32_t head_dim);
size_t kvq_oracle_bf16_slab_bytes(int32_t page_size, int32_t head_dim);
size_t kvq_oracle_int8_slab_bytes(int32_t page_size, int32_t head_dim);
size_t kvq_oracle_int4g_slab_bytes(int32_t page_size, int32_t head_dim, int32_t group);
size_t kvq_oracle_mxfp4_slab_bytes(int32_t page_size, int32_t head_dim);

/* Rotate + quantize + scatter num_tokens tokens into the INT4 pool.
 * k, v: [num_tokens][token_stride] 16-bit elements of type dtype, the first
 * num_kv_heads*head_dim of each token used as [num_kv_heads][head_dim]. */
int32_t kvq_oracle_append_int4(uint8_t* pool, int32_t num_pages, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block,
                               const uint16_t* k, const uint16_t* v, int32_t dtype,
                               int64_t token_stride, const int32_t* slot_mapping,
                               int32_t num_tokens);

/* kvq_oracle_append_int4 with the keys quantized by the scale search of R13
 * (values by the plain quantizer); the same INT4 pool. */
int32_t kvq_oracle_append_int4_search(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                      const uint16_t* k, const uint16_t* v, int32_t dtype,
                                      int64_t token_stride, const int32_t* slot_mapping,
                                      int32_t num_tokens);

/* The same into the INT8 pool (R9). */
int32_t kvq_oracle_append_int8(uint8_t* pool, int32_t num_pages, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block,
                               const uint16_t* k, const uint16_t* v, int32_t dtype,
                               int64_t token_stride, const int32_t* slot_mapping,
                               int32_t num_tokens);

/* Rotate + per-group quantize (R10) + scatter into the grouped INT4 pool. */
int32_t kvq_oracle_append_int4g(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                int32_t group, const uint16_t* k, const uint16_t* v,
                                int32_t dtype, int64_t token_stride, const int32_t* slot_mapping,
                                int32_t num_tokens);

/* kvq_oracle_append_int4g with the hybrid per-group quantizer of R14 (K and
 * V); the same grouped pool, read with |scale|. */
int32_t kvq_oracle_append_int4g_hybrid(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                       int32_t group, const uint16_t* k, const uint16_t* v,
                                       int32_t dtype, int64_t token_stride,
                                       const int32_t* slot_mapping, int32_t num_tokens);

/* Rotate + MXFP4-quantize (R12) + scatter into the MXFP4 pool. */
int32_t kvq_oracle_append_mxfp4(uint8_t* pool, int32_t num_pages, int32_t page_size,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block,
                                const uint16_t* k, const uint16_t* v, int32_t dtype,
                                int64_t token_stride, const int32_t* slot_mapping,
                                int32_t num_tokens);

/* Copy num_tokens tokens into the bf16 pool (fp16 input is rounded to bf16). */
int32_t kvq_oracle_append_bf16(uint8_t* pool, int32_t num_pages, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim,
                               const uint16_t* k, const uint16_t* v, int32_t dtype,
                               int64_t token_stride, const int32_t* slot_mapping,
                               int32_t num_tokens);

/* Read back one decoded element (fp64) of the INT4 pool: kind 0 = K, 1 = V.
 * Returns code*scale + zero in the rotated basis; code, scale, zero out-params
 * may be NULL. */
double kvq_oracle_int4_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page, int32_t head, int32_t off,
                            int32_t kind, int32_t channel, int32_t* code,
                            uint16_t* scale, uint16_t* zero);
double kvq_oracle_int8_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page, int32_t head, int32_t off,
                            int32_t kind, int32_t channel, int32_t* code,
                            uint16_t* scale, uint16_t* zero);
double kvq_oracle_int4g_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                             int32_t head_dim, int32_t group, int32_t page, int32_t head,
                             int32_t off, int32_t kind, int32_t channel, int32_t* code,
                             uint16_t* scale, uint16_t* zero);
double kvq_oracle_mxfp4_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page, int32_t head, int32_t off,
                             int32_t kind, int32_t channel, int32_t* code, uint8_t* scale_e8m0);
double kvq_oracle_bf16_read(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page, int32_t head, int32_t off,
                            int32_t kind, int32_t channel);

/* Exact softmax attention in fp64 for one query token per sequence over the
 * paged INT4 cache (R6, R7).  q: [batch][num_q_heads][head_dim] 16-bit of
 * type dtype.  block_table: [batch][max_pages_per_seq].  out: fp64
 * [batch][num_q_heads][head_dim].  Only the (b, h) pairs with
 * mask == NULL or mask[b*num_q_heads + h] != 0 are computed (others are 0). */
int32_t kvq_oracle_decode_int4(const uint8_t* pool, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block,
                               const uint16_t* q, int32_t dtype, int32_t num_q_heads,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t batch, double sm_scale,
                               const uint8_t* mask, double* out);

/* The same over the INT8 pool. */
int32_t kvq_oracle_decode_int8(const uint8_t* pool, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block,
                               const uint16_t* q, int32_t dtype, int32_t num_q_heads,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t batch, double sm_scale,
                               const uint8_t* mask, double* out);

/* The same over the grouped INT4 pool. */
int32_t kvq_oracle_decode_int4g(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block, int32_t group, const uint16_t* q,
                                int32_t dtype, int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                double sm_scale, const uint8_t* mask, double* out);

/* The same over the MXFP4 pool. */
int32_t kvq_oracle_decode_mxfp4(const uint8_t* pool, int32_t page_size, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block, const uint16_t* q, int32_t dtype,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                double sm_scale, const uint8_t* mask, double* out);

/* The same over the bf16 pool (no rotation). */
int32_t kvq_oracle_decode_bf16(const uint8_t* pool, int32_t page_size,
                               int32_t num_kv_heads, int32_t head_dim,
                               const uint16_t* q, int32_t dtype, int32_t num_q_heads,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t batch, double sm_scale,
                               const uint8_t* mask, double* out);

/* Attention with high-precision windows ("InnerQ", Abstract and Figure 2):
 * for a sequence of length L the first w_sink tokens and the last w_recent
 * tokens are read as bf16 from `win_pool` (a bf16 pool in the layout above)
 * in the original basis with the un-rotated query; every other token is read
 * from the INT4 pool in the rotated basis with the rotated query.  One exact
 * fp64 softmax over all L tokens; the INT4 tokens' share of the output is
 * rotated back before the two shares are added.  Window position of token t:
 * t when t < w_sink, else w_sink + (t - w_sink) mod w_recent (a ring of the
 * recent tokens), found through `win_block_table` [batch][max_win_pages].
 * Reading R8: the windows hold unrotated bf16 copies (the rotation only
 * serves the 4-bit codes).  A negative id in either table is a page that is
 * not there: its tokens are left out of the softmax, as in the plain decode
 * (a row with no token left is zero). */
int32_t kvq_oracle_decode_windowed(const uint8_t* int4_pool, const uint8_t* win_pool,
                                   int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block, const uint16_t* q, int32_t dtype,
                                   int32_t num_q_heads, const int32_t* block_table,
                                   int32_t max_pages_per_seq, const int32_t* win_block_table,
                                   int32_t max_win_pages, const int32_t* seq_lens, int32_t batch,
                                   int32_t w_sink, int32_t w_recent, double sm_scale,
                                   const uint8_t* mask, double* out);

/* Brute-force twin of kvq_oracle_decode_int4: gathers each sequence's keys and
 * values into contiguous fp64 rows, rotates every decoded row back with the
 * explicit matrix (H_b/sqrt(b))^T, and attends with the un-rotated query.  A
 * separate code path, meant for tiny inputs. */
int32_t kvq_oracle_decode_int4_bruteforce(const uint8_t* pool, int32_t page_size,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block, const uint16_t* q, int32_t dtype,
                                          int32_t num_q_heads, const int32_t* block_table,
                                          int32_t max_pages_per_seq, const int32_t* seq_lens,
                                          int32_t batch, double sm_scale, double* out);

/* Number of OpenMP threads the oracle uses (for the CPU-baseline report). */
int32_t kvq_oracle_num_threads(void);
/* Threads the following calls use (n > 0; timing only, results do not change). */
void kvq_oracle_set_num_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif

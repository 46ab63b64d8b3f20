/*
 * kvq.h -- C ABI of libkvq.so: Hadamard-rotated token-wise INT4 paged KV
 * cache for AMD Instinct MI355X (gfx950).
 *
 * The method: "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for
 * Real-World LLM Serving" (summary page, Research Findings; idea page, Core
 * Innovation) quantizes each new key/value vector to 4 bits with one group per
 * token after a block-diagonal Hadamard rotation, with a fused kernel that
 * writes straight into a paged cache, and runs attention fused over the
 * quantized pages.  "InnerQ" (Table 3) keeps scale factors and zero points in
 * FP16.  "BitDecoding-FP4" (Abstract) uses Hadamard rotation against key
 * outliers under token-wise scaling and stacks the query heads of a GQA group
 * into one matrix product over each KV page.
 *
 * Conventions shared by every entry point
 *   - All buffer pointers are DEVICE pointers owned by the caller (allocated
 *     with hipMalloc or by a framework on the same device).  The library
 *     allocates nothing and keeps no mutable global state (a per-device CU
 *     count is cached).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream).  Calls are asynchronous, never synchronize, and are safe to make
 *     from several host threads.
 *   - Argument validation happens on the host before anything is enqueued; a
 *     non-OK status means nothing was launched.  kvq_last_error() then gives a
 *     thread-local description.  KVQ_ERR_HIP reports a launch failure.
 *   - Page size P is 16 tokens.  head_dim D is 64 or 128.
 *   - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *   - Inputs that are 16-bit floats are fp16 or bf16 bit patterns (kvq_dtype).
 *
 * INT4 page pool layout: [num_pages][num_kv_heads][slab] bytes with
 *   slab = P * (D + 8) bytes (2176 at D = 128, 1152 at D = 64):
 *     [0, P*D/2)         K codes, token-major: byte t*(D/2) + j holds channel
 *                        2j (bits 0..3) and 2j+1 (bits 4..7) of token t.
 *     [P*D/2, P*D)       V codes, grouped by 8 channels: 32-bit word n*P + t
 *                        (n < D/8) holds channels 8n..8n+7 of token t, byte j
 *                        of it channel 8n+2j (bits 0..3) and 8n+2j+1 (4..7).
 *     [P*D, P*D + 4P)    K sidecar: token t -> fp16 scale at 4t, fp16 zero at
 *                        4t+2 (little endian).
 *     [P*D + 4P, P*D+8P) V sidecar, same form.
 *   A decoded element is code * scale + zero, in the rotated basis.
 *
 * INT8 page pool layout (token-wise INT8 variant): [num_pages][num_kv_heads]
 *   [slab] bytes with slab = P * (2*D + 8) bytes (4224 at D = 128):
 *     [0, P*D)           K codes, token-major: byte t*D + c = channel c.
 *     [P*D, 2*P*D)       V codes: 32-bit word (n*P + t)*2 + h (n < D/8,
 *                        h < 2) holds channels 8n+4h .. 8n+4h+3 of token t,
 *                        byte j = channel 8n+4h+j.
 *     [2*P*D, +4P)       K sidecar as in the INT4 pool; then the V sidecar.
 *
 * Grouped INT4 page pool layout (one scale/zero per g channels, g = 32 or
 *   64): [num_pages][num_kv_heads][slab], slab = P * (D + 8 * (D/g)) bytes:
 *     [0, P*D/2)         K codes as in the INT4 pool.
 *     [P*D/2, P*D)       V codes: 32-bit word n*P + t (n < D/8) holds channels
 *                        n + (D/8) j, j = 0..7, of token t; byte j/2 holds
 *                        nibble j (j even: bits 0..3).
 *     [P*D, +4P*D/g)     K sidecar: token t, group i -> fp16 scale at byte
 *                        4 (t*(D/g) + i), fp16 zero 2 bytes later.
 *     then the V sidecar in the same form.  A set sign bit of a scale marks a
 *     group written in the symmetric form (kvq_append_paged_int4g_hybrid); a
 *     decoded element is code * |scale| + zero in either form.
 *
 * MXFP4 page pool layout: [num_pages][num_kv_heads][slab], slab = P * (D + D/16)
 *   bytes (2176 at D = 128):
 *     [0, P*D)           K and V E2M1 codes placed as in the grouped INT4 pool
 *                        (nibble = sign << 3 | magnitude code 0..7 for
 *                        0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *     [P*D, +P*D/32)     K scales: byte t*(D/32) + i is the E8M0 exponent
 *                        (2^(byte-127)) of token t, channels 32i .. 32i+31.
 *     then the V scales in the same form.
 *   A decoded element is E2M1 value * 2^(byte-127), in the rotated basis.
 *
 * bf16 page pool layout: [num_pages][num_kv_heads][slab], slab = 4*P*D bytes:
 *     K: bf16 element t*D + c (token-major);
 *     V: bf16 element P*D + ((n*(P/4) + g)*8 + j)*4 + i for channel c = 8n + j
 *        and token t = 4g + i.
 *
 * A token in slot s lives at page s / P, offset s % P.
 *
 * Device-side robustness: slots outside [0, num_pages*P) are skipped; page
 * table entries outside [0, num_pages) contribute nothing; seq_lens are
 * clamped to [0, max_seq_len].  These are safety nets, not features.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1

/* Bytes of the static device scratch of kvq_decode_attn_noalloc (64 MiB). */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size, misalignment       */
  KVQ_ERR_UNSUPPORTED = 2,       /* valid but not built: D, P, block, group    */
  KVQ_ERR_WORKSPACE_TOO_SMALL = 3,
  KVQ_ERR_HIP = 4                /* launch failed; detail in kvq_last_error()  */
} kvq_status;

typedef enum { KVQ_F16 = 0, KVQ_BF16 = 1 } kvq_dtype;

/* INT4 cache descriptor.  `pool` must be 16-byte aligned and hold
 * kvq_int4_page_bytes(page_size, num_kv_heads, head_dim) * num_pages bytes. */
typedef struct {
  void*   pool;
  int32_t num_pages;
  int32_t page_size;        /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
  int32_t hadamard_block;   /* 16, 32, 64 or 128 (dividing head_dim); 0 = plain INT4 */
} kvq_int4_cache;

/* INT8 cache descriptor: the same fields as the INT4 one; `pool` holds
 * kvq_int8_page_bytes(page_size, num_kv_heads, head_dim) * num_pages bytes. */
typedef struct {
  void*   pool;
  int32_t num_pages;
  int32_t page_size;        /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
  int32_t hadamard_block;   /* 16, 32, 64 or 128 (dividing head_dim); 0 = no rotation */
} kvq_int8_cache;

/* Grouped INT4 cache descriptor: the INT4 fields plus the group size; `pool`
 * holds kvq_int4g_page_bytes(page_size, num_kv_heads, head_dim, group_size)
 * * num_pages bytes. */
typedef struct {
  void*   pool;
  int32_t num_pages;
  int32_t page_size;        /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
  int32_t hadamard_block;   /* 16, 32, 64 or 128 (dividing head_dim); 0 = no rotation */
  int32_t group_size;       /* channels per scale/zero pair: 32 or 64 (<= head_dim) */
} kvq_int4g_cache;

/* MXFP4 cache descriptor: the INT4 fields; `pool` holds
 * kvq_mxfp4_page_bytes(page_size, num_kv_heads, head_dim) * num_pages bytes. */
typedef struct {
  void*   pool;
  int32_t num_pages;
  int32_t page_size;        /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 (decode: 128) */
  int32_t hadamard_block;   /* 16, 32, 64 or 128 (dividing head_dim); 0 = no rotation */
} kvq_mxfp4_cache;

/* bf16 cache descriptor (baseline).  `pool` 16-byte aligned,
 * kvq_bf16_page_bytes(...) * num_pages bytes. */
typedef struct {
  void*   pool;
  int32_t num_pages;
  int32_t page_size;        /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
} kvq_bf16_cache;

/* Bytes of one page (all KV heads) of each pool. */
size_t kvq_int4_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim);
size_t kvq_int8_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim);
size_t kvq_int4g_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                            int32_t group_size);
size_t kvq_mxfp4_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim);
size_t kvq_bf16_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim);

/*
 * kvq_append_paged -- write path (SAW-INT4 summary page, Research Findings:
 * the fused rotation-quantization kernel writing into the paged layout).
 *
 * For every token t < num_tokens with slot s = slot_mapping[t] >= 0, and every
 * KV head h, both for K (from `k`) and V (from `v`):
 *   x = widen(input[t*token_stride + h*D .. + D))       (exact, to fp32)
 *   y = blockdiag(H_b)/sqrt(b) x  with the fp32 butterfly, stages h = 1, 2, 4,
 *       ..., b/2 in ascending order, then one multiply by fp32(1/sqrt(b));
 *       skipped when hadamard_block == 0
 *   zero = fp16(min y + 0), scale = fp16(((max y - min y) + 0) / 15)
 *   code_d = clamp(round_half_even((y_d - zero) * (1/scale)), 0, 15),
 *            1/scale = 0 when scale == 0; every fp32 operation rounded once
 *   codes and (scale, zero) stored in page s/16, offset s%16 (layout above).
 * Codes and sidecars are bit-exact functions of the input.
 *
 * k, v:         device, [num_tokens][token_stride] elements of `dtype`, the
 *               first num_kv_heads*head_dim of each token used; 16-byte
 *               aligned, token_stride a multiple of 8, >= num_kv_heads*D and
 *               <= 2^24 (else KVQ_ERR_INVALID_ARGUMENT).
 * slot_mapping: device int32 [num_tokens]; two tokens of one call must not
 *               share a slot.
 * num_tokens:   >= 0 (0 launches nothing).
 */
kvq_status kvq_append_paged(const kvq_int4_cache* cache, const void* k, const void* v,
                            kvq_dtype dtype, int64_t token_stride,
                            const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * kvq_decode_attn -- read path (SAW-INT4 summary page: fused attention
 * execution over the paged quantized cache; BitDecoding-FP4 Abstract: GQA
 * query heads stacked into one product per KV page).
 *
 * For each sequence b < batch and query head h < num_q_heads, with L =
 * seq_lens[b] tokens whose pages are block_table[b][0 .. ceil(L/16)):
 *   q_rot = blockdiag(H_b)/sqrt(b) q[b][h]          (so q.k is preserved)
 *   s_i   = sm_scale * (q_rot . k_hat_i),  k_hat_i = code * scale + zero
 *   o_rot = sum_i softmax(s)_i v_hat_i
 *   out[b][h] = (blockdiag(H_b)/sqrt(b))^T o_rot    (original basis)
 * L = 0 gives a zero row.  Accuracy: within max-abs 2e-3 and relative L2
 * 1e-3 of exact fp64 attention over the same decoded cache.
 *
 * q:            device, [batch][num_q_heads][head_dim] of `dtype`, 16-byte aligned.
 * block_table:  device int32 [batch][max_pages_per_seq].  An entry of a
 *               sequence's range outside [0, num_pages) is a page that is
 *               not there: it is not read and its tokens are left out of the
 *               softmax (a row with no token left is zero).
 * seq_lens:     device int32 [batch], each <= max_seq_len.
 * max_seq_len:  host bound on seq_lens (sizes the split-K grid);
 *               max_pages_per_seq*16 >= max_seq_len.
 * sm_scale:     softmax scale (normally 1/sqrt(head_dim)), finite.
 * num_splits:   0 = choose automatically; otherwise the number of split-K
 *               partitions of the longest sequence (clamped to what fits;
 *               each partition holds a multiple of 4 pages, so the count
 *               used can be smaller).  A batch of at most 32 sequences cut
 *               into 16 or more partitions may have them grown on the
 *               device from the batch's total length, so that the busy
 *               ones stay about 512 workgroups' worth.  With 0, a batch of
 *               at least 256 (sequence, KV head) pairs whose longest
 *               sequence would be cut takes the stream-K mapping instead
 *               (this decode, the INT8 and the grouped INT4 ones): the
 *               batch's pages, one sequence after another (each sequence
 *               also counted as a fixed number of pages of work), are cut
 *               per KV head into ranges, one per workgroup the device holds
 *               at once (longer for the workgroups dispatched first on
 *               each CU, which the hardware issues first), and sequences
 *               met by several ranges are merged from their partials.  The partitioning changes only the
 *               rounding of the result.
 * out:          device fp32 [batch][num_q_heads][head_dim], 16-byte aligned.
 * workspace:    device scratch of at least kvq_decode_workspace_bytes(...)
 *               for the same arguments, 16-byte aligned; its contents are
 *               overwritten.  Calls that overlap on one workspace race.
 */
kvq_status kvq_decode_attn(const kvq_int4_cache* cache, const void* q, kvq_dtype dtype,
                           int32_t num_q_heads, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                           int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_decode_attn_noalloc -- kvq_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and accuracy
 * as kvq_decode_attn without the workspace: the split-K partials go to a
 * static device array of KVQ_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (its address is looked up on
 * the first call on each device, with that device current).  The call
 * allocates nothing.  A call whose plan needs more scratch than that (the
 * planned splits' partials, or with the stream-K mapping two partials per
 * range of the largest grid plus 8 bytes per sequence) returns
 * KVQ_ERR_WORKSPACE_TOO_SMALL before anything is launched.  Every call on a
 * GPU shares that GPU's scratch and the partials of one call are read only
 * by that call, so nothing needs clearing between calls; calls that overlap
 * on one GPU (other streams, other threads) race on it.
 */
kvq_status kvq_decode_attn_noalloc(const kvq_int4_cache* cache, const void* q, kvq_dtype dtype,
                                   int32_t num_q_heads, const int32_t* block_table,
                                   int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                   int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                   void* stream);

/* kvq_decode_workspace_bytes -- workspace of the split-K decode.  No passage
 * of the pages fixes how a decode is partitioned: splitting a sequence's
 * pages over workgroups and merging their partial softmax states (maximum,
 * sum, unnormalised output) by the log-sum-exp rule is this library's
 * design for long contexts and ragged batches, and the workspace holds
 * those partials.  Bytes the decodes of this header need for these
 * arguments (0 allowed): the larger of the planned splits' partials and, where the
 * stream-K mapping applies (num_splits 0, see kvq_decode_attn), its
 * partials -- (head_dim + 2) floats for two slots per query head and range
 * of a grid of at most 2048 workgroups rounded up to whole KV heads -- and
 * two int32 per sequence.  One size serves every decode of the header. */
size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t num_splits);

/*
 * kvq_decode_attn_windowed -- kvq_decode_attn with high-precision windows
 * ("InnerQ", Abstract and Figure 2: sink tokens and the most recent tokens
 * stay in high precision beside the quantized cache, and the output shares of
 * the two are formed apart and then combined).
 *
 * For a sequence of L tokens the first w_sink and the last w_recent tokens
 * are read from `window`, a bf16 pool holding unrotated copies of them, and
 * attended with the unrotated query; the tokens in between are read from the
 * INT4 cache as in kvq_decode_attn.  The result is the one softmax over all
 * L tokens (the INT4 share rotated back), obtained by the log-sum-exp merge
 * of the INT4 split partials and the window pass.  Two launches: one grid
 * of the window and INT4 workgroups stores every partial in the workspace
 * (the window's in the last slot of each row); the split merge then writes
 * `out`.
 *
 * Window layout: window position of token t is t when t < w_sink, else
 * w_sink + (t - w_sink) mod w_recent (a ring of the recent tokens: a new
 * token overwrites the one leaving the window); position i lives in page
 * window_table[b * max_window_pages + i / 16] at offset i % 16 of `window`.
 * The caller writes the window with kvq_append_paged_bf16 (and every token,
 * windowed or not, with kvq_append_paged).  Only the positions
 * [0, min(L, w_sink + w_recent)) are read.
 *
 * window_table: device int32 [batch][max_window_pages], max_window_pages*16
 *               >= w_sink + w_recent (may be null when both are 0).
 * w_sink, w_recent: >= 0.
 * workspace:    at least kvq_decode_windowed_workspace_bytes(...) (never 0).
 * Other arguments as kvq_decode_attn; the window pool must have the cache's
 * num_kv_heads and head_dim.
 */
kvq_status kvq_decode_attn_windowed(const kvq_int4_cache* cache, const kvq_bf16_cache* window,
                                    const void* q, kvq_dtype dtype, int32_t num_q_heads,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    const int32_t* window_table, int32_t max_window_pages,
                                    const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                    int32_t w_sink, int32_t w_recent, float sm_scale,
                                    int32_t num_splits, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Workspace bytes kvq_decode_attn_windowed needs: one partial per INT4
 * split and one for the window pass, batch * num_q_heads * (splits + 1) *
 * (head_dim + 2) floats (always > 0 for batch > 0). */
size_t kvq_decode_windowed_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_seq_len, int32_t num_splits);

/*
 * kvq_append_paged_int4_search -- kvq_append_paged with a scale search for
 * the keys ("BitDecoding-FP4", Abstract: outlier-aware key quantization
 * combines Hadamard rotation with a scale search under token-wise scaling).
 * After the rotation, each key vector's range [min y, max y] is shrunk
 * toward zero by alpha_j = (16 - j) / 16, j = 0 .. 7 (each end multiplied by
 * alpha_j in fp32), the token-wise quantizer of kvq_append_paged is applied
 * with each candidate range (elements outside it are clamped by the codes'
 * clamp), and the candidate with the smallest squared reconstruction error
 * is stored, the smaller j on a tie (j = 0 is kvq_append_paged's result).
 * The error is measured exactly on an integer grid: each element decoded as
 * code * scale + zero in fp32 (product exact, sum rounded once), its error
 * y - decoded rounded once, scaled by 2^(20 - ex) with max |y| < 2^ex,
 * rounded to an integer (ties to even), squared and summed in 64 bits.
 * Values are quantized as in kvq_append_paged.  The pool is the INT4 pool,
 * read by kvq_decode_attn; codes and sidecars are bit-exact functions of
 * the input.  Same arguments and rules as kvq_append_paged (about eight
 * quantizer passes per key vector: for caches whose keys carry outliers).
 */
kvq_status kvq_append_paged_int4_search(const kvq_int4_cache* cache, const void* k, const void* v,
                                        kvq_dtype dtype, int64_t token_stride,
                                        const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * Token-wise INT8 variant ("GPU-Accelerated INT8 Quantization for KV Cache
 * Compression in Large Language Models", Abstract: 8-bit KV codes), twice
 * the bytes of INT4 per token.  The quantizer is kvq_append_paged's with 255
 * levels:
 *   zero = fp16(min y + 0), scale = fp16(((max y - min y) + 0) / 255)
 *   code_d = clamp(round_half_even((y_d - zero) * (1/scale)), 0, 255)
 * after the same optional block Hadamard rotation; codes and sidecars are
 * bit-exact functions of the input.  kvq_decode_attn_int8 is kvq_decode_attn
 * over the INT8 pool (same arguments, accuracy and workspace size, from
 * kvq_decode_workspace_bytes).
 */
kvq_status kvq_append_paged_int8(const kvq_int8_cache* cache, const void* k, const void* v,
                                 kvq_dtype dtype, int64_t token_stride,
                                 const int32_t* slot_mapping, int32_t num_tokens, void* stream);
kvq_status kvq_decode_attn_int8(const kvq_int8_cache* cache, const void* q, kvq_dtype dtype,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped INT4 variant: the quantizer of kvq_append_paged applied to each
 * group of group_size consecutive channels of the rotated vector on its own
 * (one fp16 scale and zero per group: the grouping along the inner dimension
 * of "InnerQ", Abstract and Figure 1; with group_size = hadamard_block, one
 * group per Hadamard block).  An outlier channel then only widens its own
 * group's scale.  kvq_decode_attn_int4g is kvq_decode_attn over this pool
 * (same arguments, accuracy and workspace size).  Codes and sidecars are
 * bit-exact functions of the input.
 */
kvq_status kvq_append_paged_int4g(const kvq_int4g_cache* cache, const void* k, const void* v,
                                  kvq_dtype dtype, int64_t token_stride,
                                  const int32_t* slot_mapping, int32_t num_tokens, void* stream);
kvq_status kvq_decode_attn_int4g(const kvq_int4g_cache* cache, const void* q, kvq_dtype dtype,
                                 int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_append_paged_int4g_hybrid -- kvq_append_paged_int4g with the hybrid
 * quantizer ("InnerQ", Abstract and Figure 3: symmetric or asymmetric
 * quantization chosen for each group from the group's own statistics).  For
 * each group two candidates: the asymmetric one of kvq_append_paged_int4g,
 * and the symmetric one with scale = fp16(max |y| / 7) and zero = -8 * scale
 * (exact in fp16), whose levels (code - 8) * scale hold 0.  The symmetric one
 * is kept when its squared reconstruction error, measured on the integer
 * grid of kvq_append_paged_int4_search, is not larger; its scale is then
 * stored with the sign bit set.  A group of zeros, or one whose symmetric
 * scale is 0 in fp16 or whose -8 * scale is beyond fp16, stays asymmetric.
 * Read by kvq_decode_attn_int4g (which takes |scale|); codes and sidecars are
 * bit-exact functions of the input.  Same arguments and rules as
 * kvq_append_paged_int4g.
 */
kvq_status kvq_append_paged_int4g_hybrid(const kvq_int4g_cache* cache, const void* k, const void* v,
                                         kvq_dtype dtype, int64_t token_stride,
                                         const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * MXFP4 variant ("BitDecoding-FP4", Abstract: an FP4 KV cache with Hadamard
 * rotation under token-wise scaling; OCP microscaling block format): after the
 * optional block Hadamard rotation, each 32 channels of a vector share the
 * E8M0 scale 2^X with X = floor(log2(max |y|)) - 2 (-127 for a zero block),
 * and each element is y / 2^X rounded to the nearest E2M1 value (a tie goes
 * to the code with mantissa bit 0; 6 and above saturate to 6; the sign bit
 * only on nonzero codes).  Same bytes per token as INT4.  Codes and scales
 * are bit-exact functions of the input.  kvq_decode_attn_mxfp4 is
 * kvq_decode_attn over this pool (head_dim 128; same arguments, accuracy and
 * workspace size); its QK product runs on the block-scaled FP4 matrix
 * instruction of gfx950, its PV product on the bf16 one (V converted by the
 * FP4-to-bf16 instruction, exact).
 */
kvq_status kvq_append_paged_mxfp4(const kvq_mxfp4_cache* cache, const void* k, const void* v,
                                  kvq_dtype dtype, int64_t token_stride,
                                  const int32_t* slot_mapping, int32_t num_tokens, void* stream);
kvq_status kvq_decode_attn_mxfp4(const kvq_mxfp4_cache* cache, const void* q, kvq_dtype dtype,
                                 int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_append_paged_bf16 / kvq_decode_attn_bf16 -- the unquantized baseline
 * the quantized caches are measured against ("InnerQ", Table 4: the FP16
 * GEMV kernel as the latency baseline of the fused dequantize kernels;
 * "BitDecoding-FP4", Abstract: accuracy and serving throughput stated
 * relative to a BF16 KV cache).  Here the baseline cache holds bf16 (half
 * the bytes of fp32, the same as fp16) in the bf16 pool layout above.
 *
 * kvq_append_paged_bf16 copies K and V into the bf16 pool (fp16 input is
 * rounded to bf16, nearest even); same argument rules as kvq_append_paged.
 */
kvq_status kvq_append_paged_bf16(const kvq_bf16_cache* cache, const void* k, const void* v,
                                 kvq_dtype dtype, int64_t token_stride,
                                 const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* kvq_decode_attn_bf16: kvq_decode_attn over the bf16 pool (no rotation,
 * no dequantization: exact attention over the stored bf16 values up to fp32
 * rounding).  Same argument rules and workspace size; it always takes the
 * planned split mapping. */
kvq_status kvq_decode_attn_bf16(const kvq_bf16_cache* cache, const void* q, kvq_dtype dtype,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens,
                                int32_t batch, int32_t max_seq_len, float sm_scale,
                                int32_t num_splits, float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Static name of a status code. */
const char* kvq_status_string(kvq_status status);

/* Thread-local description of the last non-OK status returned on this thread
 * ("" if none).  Valid until the next call on the same thread. */
const char* kvq_last_error(void);

/* KVQ_ABI_VERSION of the built library. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif

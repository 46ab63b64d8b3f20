// C ABI of libkvq.so (declared in include/kvq.h): host-side validation, split
// planning and dispatch.  Nothing here allocates device memory or
// synchronizes; every launch goes to the caller's stream.
#include "kvq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kvq_internal.hpp"

// Split-K scratch of kvq_decode_attn_noalloc: a static device array, one copy
// on each GPU the library runs on, held until the process ends.  Host code
// never passes this name as an address (on the host it is only a stand-in);
// each device's address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace kvq {

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

kvq_status check_geometry(int32_t num_pages, int32_t page_size, int32_t hkv, int32_t d) {
  if (num_pages <= 0 || hkv <= 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "num_pages and num_kv_heads must be > 0");
  if (page_size != 16) return fail(KVQ_ERR_UNSUPPORTED, "page_size %d unsupported (only 16)", page_size);
  if (d != 64 && d != 128) return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d);
  return KVQ_OK;
}

kvq_status check_append(const void* pool, const void* k, const void* v, kvq_dtype dtype,
                        int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                        int32_t hkv, int32_t d) {
  if (num_tokens < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (dtype != KVQ_F16 && dtype != KVQ_BF16) return fail(KVQ_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (pool == nullptr) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache pool is null");
  if (!aligned16(pool)) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache pool not 16-byte aligned");
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping) return fail(KVQ_ERR_INVALID_ARGUMENT, "k, v or slot_mapping is null");
  if (!aligned16(k) || !aligned16(v)) return fail(KVQ_ERR_INVALID_ARGUMENT, "k or v not 16-byte aligned");
  if (!aligned4(slot_mapping)) return fail(KVQ_ERR_INVALID_ARGUMENT, "slot_mapping not 4-byte aligned");
  if (token_stride < static_cast<int64_t>(hkv) * d)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "token_stride %lld < num_kv_heads*head_dim", (long long)token_stride);
  if (token_stride % 8 != 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "token_stride must be a multiple of 8 elements");
  // the append kernel addresses a tile of 64 token rows with 32-bit offsets
  if (token_stride > (int64_t{1} << 24)) return fail(KVQ_ERR_INVALID_ARGUMENT, "token_stride above 2^24 elements");
  return KVQ_OK;
}

kvq_status check_decode(const void* pool, const void* q, kvq_dtype dtype, int32_t hq, int32_t hkv,
                        const int32_t* block_table, int32_t max_pages_per_seq,
                        const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                        float sm_scale, int32_t num_splits, const float* out) {
  if (dtype != KVQ_F16 && dtype != KVQ_BF16) return fail(KVQ_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (batch < 0 || max_seq_len < 0 || num_splits < 0)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "batch, max_seq_len and num_splits must be >= 0");
  if (hq <= 0 || hq % hkv != 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "num_q_heads %d not a multiple of num_kv_heads %d", hq, hkv);
  if (hq / hkv > 16) return fail(KVQ_ERR_UNSUPPORTED, "query group size %d > 16 unsupported", hq / hkv);
  if (!std::isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARGUMENT, "sm_scale not finite");
  if (pool == nullptr) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache pool is null");
  if (!aligned16(pool)) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache pool not 16-byte aligned");
  if (batch == 0) return KVQ_OK;
  if (!q || !block_table || !seq_lens || !out) return fail(KVQ_ERR_INVALID_ARGUMENT, "q, block_table, seq_lens or out is null");
  if (!aligned16(q) || !aligned16(out)) return fail(KVQ_ERR_INVALID_ARGUMENT, "q or out not 16-byte aligned");
  if (!aligned4(block_table) || !aligned4(seq_lens)) return fail(KVQ_ERR_INVALID_ARGUMENT, "block_table or seq_lens misaligned");
  if (max_pages_per_seq <= 0 || static_cast<int64_t>(max_pages_per_seq) * 16 < max_seq_len)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "max_pages_per_seq*16 < max_seq_len");
  return KVQ_OK;
}

}  // namespace

SplitPlan plan_splits(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t num_splits) {
  const int32_t pages_max = (max_seq_len + 15) / 16;
  if (pages_max <= 0) return SplitPlan{4, 1};
  int64_t s;
  if (num_splits > 0) {
    s = num_splits;
  } else {
    // Four-wave workgroups: about 512 of them (2 waves per SIMD) keep the
    // HBM busy.  The host does not see the lengths, only their maximum, and
    // in a ragged batch the longest sequence has to be cut finely or it
    // finishes long after the rest, while the empty splits of the shorter
    // sequences cost little: splits hold at most 256 pages.  Measured on
    // lognormal batches of 32 and 256 sequences (2x faster than 512-page
    // splits at 32) and on 8 x 131072 tokens (6% slower than the best split
    // count there).  At least 16 pages (one 4-page step per wave) per split.
    const int64_t units = static_cast<int64_t>(batch > 0 ? batch : 1) * hkv;
    const int64_t s_fill = (512 + units - 1) / units;
    const int64_t s_len = (pages_max + 255) / 256;
    s = s_len > s_fill ? s_len : s_fill;
    const int64_t min_len = (pages_max + 15) / 16;
    if (s > min_len) s = min_len;
  }
  const int64_t max_s = (pages_max + 3) / 4;   // at least one 4-page step per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  int64_t sp = (pages_max + s - 1) / s;
  sp = (sp + 3) / 4 * 4;
  s = (pages_max + sp - 1) / sp;
  return SplitPlan{static_cast<int32_t>(sp), static_cast<int32_t>(s)};
}

// The device may grow the splits (balanced_split_pages) for a small batch cut
// into many splits (16 or more: long contexts) whose whole work could exceed
// about 512 workgroups of the planned size; otherwise the plan stands and the
// kernels skip the scan of the lengths.
bool may_balance(int32_t batch, int32_t hkv, int32_t max_seq_len, const SplitPlan& p) {
  if (p.nsplit < 16 || batch > kBalanceMaxBatch) return false;
  const int64_t pages_max = (static_cast<int64_t>(max_seq_len) + 15) / 16;
  return pages_max * batch * hkv > static_cast<int64_t>(p.split_pages) * 512;
}

size_t workspace_bytes(int32_t batch, int32_t hq, int32_t d, const SplitPlan& p) {
  if (p.nsplit <= 1) return 0;   // unsplit work writes the output directly
  return static_cast<size_t>(batch) * hq * p.nsplit * (d + 2) * sizeof(float);
}

// Stream-K (the plain INT4-family decodes with an automatic plan): each
// workgroup of the grid takes an equal range of the batch's pages, so a
// ragged batch leaves none idle and none runs long.  Taken where the plan
// would cut the longest sequence (the grid is then sized for it, and most
// workgroups of a ragged batch have little or nothing to do) and the batch
// has at least 256 (sequence, KV head) pairs: measured on lognormal batches
// of the 70B-shaped layer, 10% faster at 32 sequences and 3% at 256, equal
// at 128, slower at 8 (ranges of a few pages, a partial per range); a batch
// of equal lengths cut once per sequence keeps the plan (no merge).  Its
// workspace: two partials per range and query head for the largest grid,
// and the merge's record of each sequence.
bool stream_call(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t num_splits) {
  const int64_t pages_max = (static_cast<int64_t>(max_seq_len) + 15) / 16;
  // the run of a KV head (pages plus a fixed cost per sequence) stays far
  // inside the device's 32-bit arithmetic
  const int64_t cost = std::max(kStreamItemCost1, kStreamItemCost2);
  return num_splits == 0 && static_cast<int64_t>(batch) * hkv >= 256 &&
         static_cast<int64_t>(batch) * (pages_max + cost) < (int64_t{1} << 30) &&
         plan_splits(batch, hkv, max_seq_len, 0).nsplit > 1;
}

int64_t stream_slots(int32_t hq, int32_t hkv) {   // partial rows of the largest grid
  return static_cast<int64_t>(hkv) * ((kStreamMaxWorkgroups + hkv - 1) / hkv) * 2 * (hq / hkv);
}

size_t stream_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t d) {
  return static_cast<size_t>(stream_slots(hq, hkv)) * (d + 2) * sizeof(float) +
         static_cast<size_t>(batch) * 2 * sizeof(int32_t);
}

namespace {

enum class Pool { kInt4, kInt8, kInt4g, kMxfp4, kBf16 };

kvq_status check_block(int32_t b, int32_t d) {
  if (!(b == 0 || b == 16 || b == 32 || b == 64 || b == 128) || b > d)
    return fail(KVQ_ERR_UNSUPPORTED, "hadamard_block %d unsupported for head_dim %d", b, d);
  return KVQ_OK;
}

kvq_status launch_decode(Pool kind, const void* pool, int32_t num_pages, int32_t hkv, int32_t d,
                         int32_t block, int32_t group, const void* q, kvq_dtype dtype, int32_t hq,
                         const int32_t* block_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                         float sm_scale, int32_t num_splits, float* out, void* workspace,
                         size_t workspace_bytes_given, void* stream) {
  kvq_status st = check_decode(pool, q, dtype, hq, hkv, block_table, max_pages_per_seq, seq_lens,
                               batch, max_seq_len, sm_scale, num_splits, out);
  if (st != KVQ_OK || batch == 0) return st;
  const bool quant = kind == Pool::kInt4 || kind == Pool::kInt8 || kind == Pool::kInt4g;
  const bool use_sk = quant && stream_call(batch, hkv, max_seq_len, num_splits);
  const SplitPlan plan = plan_splits(batch, hkv, max_seq_len, num_splits);
  if (!use_sk && static_cast<int64_t>(plan.nsplit) * hkv * batch > INT32_MAX)
    return fail(KVQ_ERR_UNSUPPORTED, "batch * num_kv_heads * splits above 2^31 workgroups");
  const size_t need = use_sk ? stream_workspace_bytes(batch, hq, hkv, d) : workspace_bytes(batch, hq, d, plan);
  if (workspace_bytes_given < need)
    return fail(KVQ_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes_given, need);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace)))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "workspace null or not 16-byte aligned");
  DecodeArgs a{};
  a.pool = static_cast<const uint8_t*>(pool);
  a.q = static_cast<const uint16_t*>(q);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.part_acc = static_cast<float*>(workspace);
  a.part_ml = static_cast<float*>(workspace) + static_cast<size_t>(batch) * hq * plan.nsplit * d;
  a.num_pages = num_pages;
  a.num_kv_heads = hkv;
  a.num_q_heads = hq;
  a.head_dim = d;
  a.block = block;
  a.bt_stride = max_pages_per_seq;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.split_pages = plan.split_pages;
  a.nsplit = plan.nsplit;
  a.sm_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  a.in_bf16 = dtype == KVQ_BF16;
  a.part_stride = plan.nsplit;
  a.group = group;
  a.balance = may_balance(batch, hkv, max_seq_len, plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_sk) {
    const int bits = kind == Pool::kInt8 ? 8 : 4;
    const int gs = kind == Pool::kInt4g ? group : 0;
    int32_t ranges = 0, per_slot = 1;
    hipError_t e = stream_ranges(a, bits, gs, &ranges, &per_slot);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
    const int64_t slots = stream_slots(hq, hkv);
    a.sk_ranges = ranges;
    a.sk_per_slot = per_slot;
    a.part_acc = static_cast<float*>(workspace);
    a.part_ml = static_cast<float*>(workspace) + slots * d;
    a.sk_rec = reinterpret_cast<int32_t*>(static_cast<float*>(workspace) + slots * (d + 2));
    a.balance = 0;
    // the merge's lanes per row: about the ranges a sequence meets (at most
    // the ranges, or one per 16 pages and one more; a ranges-per-sequence
    // share of the batch on average)
    const int64_t pages_max = (static_cast<int64_t>(max_seq_len) + 15) / 16;
    int64_t est = std::min<int64_t>(ranges, (pages_max + 15) / 16 + 1);
    est = std::min<int64_t>(est, (4 * static_cast<int64_t>(ranges) + batch - 1) / batch + 2);
    a.part_stride = static_cast<int32_t>(est);
    e = launch_decode_quant_stream(a, bits, gs, s);
    if (e == hipSuccess) e = launch_reduce(a, s);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return KVQ_OK;
  }
  hipError_t e = kind == Pool::kInt4    ? launch_decode_int4(a, s)
                 : kind == Pool::kInt8  ? launch_decode_int8(a, s)
                 : kind == Pool::kInt4g ? launch_decode_int4g(a, s)
                 : kind == Pool::kMxfp4 ? launch_decode_mxfp4(a, s)
                                        : launch_decode_bf16(a, s);
  if (e == hipSuccess && plan.nsplit > 1) e = launch_reduce(a, s);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

// The address of this device's copy of `scratch`, looked up once per device
// with that device current (the caller's), then kept.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" {

size_t kvq_int4_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  if (page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return static_cast<size_t>(num_kv_heads) * page_size * (head_dim + 8);
}

size_t kvq_bf16_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  if (page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return static_cast<size_t>(num_kv_heads) * page_size * head_dim * 4;
}

size_t kvq_int8_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  if (page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return static_cast<size_t>(num_kv_heads) * page_size * (2 * head_dim + 8);
}

size_t kvq_mxfp4_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  if (page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 32 != 0) return 0;
  return static_cast<size_t>(num_kv_heads) * page_size * (head_dim + head_dim / 16);
}

size_t kvq_int4g_page_bytes(int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                            int32_t group_size) {
  if (page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || group_size <= 0 ||
      head_dim % group_size != 0)
    return 0;
  return static_cast<size_t>(num_kv_heads) * page_size * (head_dim + 8 * (head_dim / group_size));
}

}  // extern "C"

namespace kvq {
namespace {

// The quantizing append shared by the INT4 and INT8 pools (same descriptor
// fields, different code width).
int32_t group_of(const kvq_int4_cache*) { return 0; }
int32_t group_of(const kvq_int8_cache*) { return 0; }
int32_t group_of(const kvq_int4g_cache* c) { return c->group_size; }
int32_t group_of(const kvq_mxfp4_cache*) { return 32; }

template <class Cache>
kvq_status check_quant_cache(const Cache* cache, Pool kind) {
  if (cache == nullptr) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache descriptor is null");
  kvq_status st = check_geometry(cache->num_pages, cache->page_size, cache->num_kv_heads, cache->head_dim);
  if (st != KVQ_OK) return st;
  st = check_block(cache->hadamard_block, cache->head_dim);
  if (st != KVQ_OK) return st;
  if (kind == Pool::kInt4g) {
    const int32_t gs = group_of(cache);
    if (!(gs == 32 || gs == 64) || gs > cache->head_dim)
      return fail(KVQ_ERR_UNSUPPORTED, "group_size %d unsupported for head_dim %d (32 or 64)", gs,
                  cache->head_dim);
  }
  return KVQ_OK;
}

template <class Cache>
kvq_status append_quant(const Cache* cache, Pool kind, const void* k, const void* v, kvq_dtype dtype,
                        int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                        void* stream, int32_t mode = kQuantPlain) {
  kvq_status st = check_quant_cache(cache, kind);
  if (st != KVQ_OK) return st;
  st = check_append(cache->pool, k, v, dtype, token_stride, slot_mapping, num_tokens,
                    cache->num_kv_heads, cache->head_dim);
  if (st != KVQ_OK || num_tokens == 0) return st;
  AppendArgs a{};
  a.pool = static_cast<uint8_t*>(cache->pool);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.slot_mapping = slot_mapping;
  a.token_stride = token_stride;
  a.num_tokens = num_tokens;
  a.num_pages = cache->num_pages;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.block = cache->hadamard_block;
  a.in_bf16 = dtype == KVQ_BF16;
  a.group = group_of(cache);
  a.mode = mode;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = kind == Pool::kInt8    ? launch_append_int8(a, s)
                       : kind == Pool::kInt4g ? launch_append_int4g(a, s)
                       : kind == Pool::kMxfp4 ? launch_append_mxfp4(a, s)
                                              : launch_append_int4(a, s);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

template <class Cache>
kvq_status decode_quant(const Cache* cache, Pool kind, const void* q, kvq_dtype dtype,
                        int32_t num_q_heads, const int32_t* block_table, int32_t max_pages_per_seq,
                        const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                        int32_t num_splits, float* out, void* workspace,
                        size_t workspace_bytes_given, void* stream) {
  kvq_status st = check_quant_cache(cache, kind);
  if (st != KVQ_OK) return st;
  if (kind == Pool::kMxfp4 && cache->head_dim != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "MXFP4 decode is built for head_dim 128 only");
  return launch_decode(kind, cache->pool, cache->num_pages, cache->num_kv_heads, cache->head_dim,
                       cache->hadamard_block, group_of(cache), q, dtype,
                       num_q_heads, block_table, max_pages_per_seq, seq_lens, batch, max_seq_len,
                       sm_scale, num_splits, out, workspace, workspace_bytes_given, stream);
}

}  // namespace
}  // namespace kvq

extern "C" {

kvq_status kvq_append_paged(const kvq_int4_cache* cache, const void* k, const void* v,
                            kvq_dtype dtype, int64_t token_stride, const int32_t* slot_mapping,
                            int32_t num_tokens, void* stream) {
  return append_quant(cache, Pool::kInt4, k, v, dtype, token_stride, slot_mapping, num_tokens, stream);
}

kvq_status kvq_append_paged_int4_search(const kvq_int4_cache* cache, const void* k, const void* v,
                                        kvq_dtype dtype, int64_t token_stride,
                                        const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  return append_quant(cache, Pool::kInt4, k, v, dtype, token_stride, slot_mapping, num_tokens, stream,
                      kQuantKeySearch);
}

kvq_status kvq_append_paged_int8(const kvq_int8_cache* cache, const void* k, const void* v,
                                 kvq_dtype dtype, int64_t token_stride,
                                 const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  return append_quant(cache, Pool::kInt8, k, v, dtype, token_stride, slot_mapping, num_tokens, stream);
}

kvq_status kvq_append_paged_mxfp4(const kvq_mxfp4_cache* cache, const void* k, const void* v,
                                  kvq_dtype dtype, int64_t token_stride,
                                  const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  return append_quant(cache, Pool::kMxfp4, k, v, dtype, token_stride, slot_mapping, num_tokens, stream);
}

kvq_status kvq_append_paged_int4g(const kvq_int4g_cache* cache, const void* k, const void* v,
                                  kvq_dtype dtype, int64_t token_stride,
                                  const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  return append_quant(cache, Pool::kInt4g, k, v, dtype, token_stride, slot_mapping, num_tokens, stream);
}

kvq_status kvq_append_paged_int4g_hybrid(const kvq_int4g_cache* cache, const void* k, const void* v,
                                         kvq_dtype dtype, int64_t token_stride,
                                         const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  return append_quant(cache, Pool::kInt4g, k, v, dtype, token_stride, slot_mapping, num_tokens, stream,
                      kQuantHybrid);
}

kvq_status kvq_append_paged_bf16(const kvq_bf16_cache* cache, const void* k, const void* v,
                                 kvq_dtype dtype, int64_t token_stride,
                                 const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  if (cache == nullptr) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache descriptor is null");
  kvq_status st = check_geometry(cache->num_pages, cache->page_size, cache->num_kv_heads, cache->head_dim);
  if (st != KVQ_OK) return st;
  st = check_append(cache->pool, k, v, dtype, token_stride, slot_mapping, num_tokens,
                    cache->num_kv_heads, cache->head_dim);
  if (st != KVQ_OK || num_tokens == 0) return st;
  AppendArgs a{};
  a.pool = static_cast<uint8_t*>(cache->pool);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.slot_mapping = slot_mapping;
  a.token_stride = token_stride;
  a.num_tokens = num_tokens;
  a.num_pages = cache->num_pages;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.in_bf16 = dtype == KVQ_BF16;
  const hipError_t e = launch_append_bf16(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

kvq_status kvq_decode_attn(const kvq_int4_cache* cache, const void* q, kvq_dtype dtype,
                           int32_t num_q_heads, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                           int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                           void* workspace, size_t workspace_bytes_given, void* stream) {
  return decode_quant(cache, Pool::kInt4, q, dtype, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                      batch, max_seq_len, sm_scale, num_splits, out, workspace,
                      workspace_bytes_given, stream);
}

kvq_status kvq_decode_attn_noalloc(const kvq_int4_cache* cache, const void* q, kvq_dtype dtype,
                                   int32_t num_q_heads, const int32_t* block_table,
                                   int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                   int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                   void* stream) {
  kvq_status st = check_quant_cache(cache, Pool::kInt4);
  if (st != KVQ_OK) return st;
  st = check_decode(cache->pool, q, dtype, num_q_heads, cache->num_kv_heads, block_table,
                    max_pages_per_seq, seq_lens, batch, max_seq_len, sm_scale, num_splits, out);
  if (st != KVQ_OK || batch == 0) return st;
  const size_t need = stream_call(batch, cache->num_kv_heads, max_seq_len, num_splits)
                         ? stream_workspace_bytes(batch, num_q_heads, cache->num_kv_heads, cache->head_dim)
                         : workspace_bytes(batch, num_q_heads, cache->head_dim,
                                           plan_splits(batch, cache->num_kv_heads, max_seq_len, num_splits));
  if (need > KVQ_NOALLOC_SCRATCH_BYTES)
    return fail(KVQ_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of split-K scratch; the static scratch holds %zu "
                "(use kvq_decode_attn with a workspace, or fewer splits)",
                need, static_cast<size_t>(KVQ_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
  }
  return decode_quant(cache, Pool::kInt4, q, dtype, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                      batch, max_seq_len, sm_scale, num_splits, out, ws, need, stream);
}

kvq_status kvq_decode_attn_int8(const kvq_int8_cache* cache, const void* q, kvq_dtype dtype,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                void* workspace, size_t workspace_bytes_given, void* stream) {
  return decode_quant(cache, Pool::kInt8, q, dtype, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                      batch, max_seq_len, sm_scale, num_splits, out, workspace,
                      workspace_bytes_given, stream);
}

kvq_status kvq_decode_attn_mxfp4(const kvq_mxfp4_cache* cache, const void* q, kvq_dtype dtype,
                                 int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                 void* workspace, size_t workspace_bytes_given, void* stream) {
  return decode_quant(cache, Pool::kMxfp4, q, dtype, num_q_heads, block_table, max_pages_per_seq,
                      seq_lens, batch, max_seq_len, sm_scale, num_splits, out, workspace,
                      workspace_bytes_given, stream);
}

kvq_status kvq_decode_attn_int4g(const kvq_int4g_cache* cache, const void* q, kvq_dtype dtype,
                                 int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                 void* workspace, size_t workspace_bytes_given, void* stream) {
  return decode_quant(cache, Pool::kInt4g, q, dtype, num_q_heads, block_table, max_pages_per_seq,
                      seq_lens, batch, max_seq_len, sm_scale, num_splits, out, workspace,
                      workspace_bytes_given, stream);
}

kvq_status kvq_decode_attn_bf16(const kvq_bf16_cache* cache, const void* q, kvq_dtype dtype,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, float sm_scale, int32_t num_splits, float* out,
                                void* workspace, size_t workspace_bytes_given, void* stream) {
  if (cache == nullptr) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache descriptor is null");
  kvq_status st = check_geometry(cache->num_pages, cache->page_size, cache->num_kv_heads, cache->head_dim);
  if (st != KVQ_OK) return st;
  return launch_decode(Pool::kBf16, cache->pool, cache->num_pages, cache->num_kv_heads, cache->head_dim, 0, 0,
                       q, dtype, num_q_heads, block_table, max_pages_per_seq, seq_lens, batch,
                       max_seq_len, sm_scale, num_splits, out, workspace, workspace_bytes_given,
                       stream);
}

kvq_status kvq_decode_attn_windowed(const kvq_int4_cache* cache, const kvq_bf16_cache* window,
                                    const void* q, kvq_dtype dtype, int32_t num_q_heads,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    const int32_t* window_table, int32_t max_window_pages,
                                    const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                    int32_t w_sink, int32_t w_recent, float sm_scale,
                                    int32_t num_splits, float* out, void* workspace,
                                    size_t workspace_bytes_given, void* stream) {
  if (cache == nullptr || window == nullptr) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache descriptor is null");
  kvq_status st = check_geometry(cache->num_pages, cache->page_size, cache->num_kv_heads, cache->head_dim);
  if (st != KVQ_OK) return st;
  st = check_geometry(window->num_pages, window->page_size, window->num_kv_heads, window->head_dim);
  if (st != KVQ_OK) return st;
  if (window->num_kv_heads != cache->num_kv_heads || window->head_dim != cache->head_dim)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "window pool geometry differs from the INT4 cache");
  const int blk = cache->hadamard_block;
  st = check_block(blk, cache->head_dim);
  if (st != KVQ_OK) return st;
  const int32_t hkv = cache->num_kv_heads, d = cache->head_dim, hq = num_q_heads;
  st = check_decode(cache->pool, q, dtype, hq, hkv, block_table, max_pages_per_seq, seq_lens, batch,
                    max_seq_len, sm_scale, num_splits, out);
  if (st != KVQ_OK) return st;
  if (w_sink < 0 || w_recent < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "window sizes must be >= 0");
  const int64_t wlen = static_cast<int64_t>(w_sink) + w_recent;
  if (wlen > INT32_MAX / 2) return fail(KVQ_ERR_INVALID_ARGUMENT, "window sizes too large");
  if (wlen > 0) {
    if (window->pool == nullptr || !aligned16(window->pool))
      return fail(KVQ_ERR_INVALID_ARGUMENT, "window pool null or not 16-byte aligned");
    if (batch > 0 && (window_table == nullptr || !aligned4(window_table)))
      return fail(KVQ_ERR_INVALID_ARGUMENT, "window_table null or misaligned");
    if (static_cast<int64_t>(max_window_pages) * 16 < wlen)
      return fail(KVQ_ERR_INVALID_ARGUMENT, "max_window_pages*16 < w_sink + w_recent");
  }
  if (batch == 0) return KVQ_OK;
  const SplitPlan plan = plan_splits(batch, hkv, max_seq_len, num_splits);
  // one partial per INT4 split, and one for the window pass
  const int32_t stride = plan.nsplit + (wlen > 0 ? 1 : 0);
  if (static_cast<int64_t>(plan.nsplit + 1) * hkv * batch > INT32_MAX)
    return fail(KVQ_ERR_UNSUPPORTED, "batch * num_kv_heads * splits above 2^31 workgroups");
  const size_t need = static_cast<size_t>(batch) * hq * stride * (d + 2) * sizeof(float);
  if (workspace_bytes_given < need)
    return fail(KVQ_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes_given, need);
  if (workspace == nullptr || !aligned16(workspace))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "workspace null or not 16-byte aligned");

  DecodeArgs a{};   // the INT4 pass over the tokens between the windows
  a.pool = static_cast<const uint8_t*>(cache->pool);
  a.q = static_cast<const uint16_t*>(q);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.part_acc = static_cast<float*>(workspace);
  a.part_ml = static_cast<float*>(workspace) + static_cast<size_t>(batch) * hq * stride * d;
  a.num_pages = cache->num_pages;
  a.num_kv_heads = hkv;
  a.num_q_heads = hq;
  a.head_dim = d;
  a.block = blk;
  a.bt_stride = max_pages_per_seq;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.split_pages = plan.split_pages;
  a.nsplit = plan.nsplit;
  a.sm_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  a.in_bf16 = dtype == KVQ_BF16;
  a.skip_first = w_sink;
  a.skip_last = w_recent;
  a.part_stride = stride;
  a.force_partial = 1;
  a.balance = may_balance(batch, hkv, max_seq_len, plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (wlen > 0) {
    // the bf16 pass over each sequence's window, in the same grid as the
    // INT4 pass, into the last slot of each row
    DecodeArgs w = a;
    w.pool = static_cast<const uint8_t*>(window->pool);
    w.block_table = window_table;
    w.bt_stride = max_window_pages;
    w.num_pages = window->num_pages;
    w.block = 0;
    w.skip_first = w.skip_last = 0;
    w.len_cap = static_cast<int32_t>(wlen);
    w.split_pages = static_cast<int32_t>((wlen + 15) / 16 + 3) / 4 * 4;
    w.nsplit = 1;
    w.balance = 0;
    w.part_slot0 = plan.nsplit;
    e = launch_decode_windowed(a, w, s);
    a.has_window = 1;
    a.win_len = static_cast<int32_t>(wlen);
  } else {
    e = launch_decode_int4(a, s);
  }
  if (e == hipSuccess) e = launch_reduce(a, s);   // merge and normalise
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

size_t kvq_decode_windowed_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_seq_len, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      num_splits < 0)
    return 0;
  const SplitPlan plan = plan_splits(batch, num_kv_heads, max_seq_len, num_splits);
  return static_cast<size_t>(batch) * num_q_heads * (plan.nsplit + 1) * (head_dim + 2) * sizeof(float);
}

size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      num_splits < 0)
    return 0;
  // the larger of the two plans' needs: the same size serves every decode
  const size_t planned = workspace_bytes(batch, num_q_heads, head_dim,
                                         plan_splits(batch, num_kv_heads, max_seq_len, num_splits));
  if (!stream_call(batch, num_kv_heads, max_seq_len, num_splits) || num_q_heads % num_kv_heads != 0)
    return planned;
  return std::max(planned, stream_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim));
}

const char* kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARGUMENT: return "KVQ_ERR_INVALID_ARGUMENT";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "KVQ_ERR_WORKSPACE_TOO_SMALL";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
  }
  return "KVQ_ERR_UNKNOWN";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

}  // extern "C"

// Internal host-side interface between the C ABI (api.cpp) and the kernel
// launchers (*.hip).  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

// Decode calls of at most this many sequences may grow their splits on the
// device from the batch's whole work (DecodeArgs::balance; one wave reads the
// lengths, so at most 64).
constexpr int kBalanceMaxBatch = 32;

struct AppendArgs {
  uint8_t* pool;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* slot_mapping;
  int64_t token_stride;      // elements
  int32_t num_tokens;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block;             // Hadamard block (0 = none); unused by the bf16 pool
  int32_t in_bf16;           // 1: inputs are bf16, 0: fp16
  int32_t group;             // channels per scale/zero pair (grouped INT4 pool only)
  int32_t mode;              // quantizer: kQuantPlain, kQuantKeySearch or kQuantHybrid
};

// Quantizer modes of the 4-bit appends: the plain token-wise (or per-group)
// asymmetric quantizer; the scale search for keys (token-wise pool); the
// hybrid symmetric/asymmetric choice per group (grouped pool).
constexpr int kQuantPlain = 0;
constexpr int kQuantKeySearch = 1;
constexpr int kQuantHybrid = 2;

struct DecodeArgs {
  const uint8_t* pool;
  const uint16_t* q;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* out;
  float* part_acc;           // [batch][hq][nsplit][head_dim]
  float* part_ml;            // [batch][hq][nsplit][2]
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t block;             // Hadamard block (0 = none)
  int32_t bt_stride;         // max_pages_per_seq
  int32_t batch;
  int32_t max_seq_len;
  int32_t split_pages;       // pages per split-K partition (multiple of 4)
  int32_t nsplit;            // partitions of the longest sequence
  float sm_log2;             // sm_scale * log2(e)
  int32_t in_bf16;
  // High-precision windows (zero for plain decode): the INT4 pass skips the
  // first skip_first and the last skip_last tokens of each sequence; the bf16
  // window pass attends at most len_cap tokens.
  int32_t skip_first;
  int32_t skip_last;
  int32_t len_cap;
  // Partials of (sequence b, query head h, split s) go to slot
  // (b * hq + h) * part_stride + part_slot0 + s; force_partial stores them
  // even with one split.
  int32_t part_stride;
  int32_t part_slot0;
  int32_t force_partial;
  int32_t group;             // channels per scale/zero pair (grouped INT4 pool only)
  // Split merge of a windowed call (has_window = 1): the last slot of each
  // row holds the bf16 window pass's partial, which exists when the sequence
  // has a token among its first win_len positions.
  int32_t has_window;
  int32_t win_len;
  // The splits may grow with the batch's whole work (balanced_split_pages).
  int32_t balance;
  // Stream-K mapping of the plain INT4-family decode (sk_ranges > 0): the
  // batch's pages, one sequence after another, cut per KV head into
  // sk_ranges ranges (stream_range), one workgroup each.  The partial of
  // (KV head, range, slot, head of the group) is at
  // ((kvh * sk_ranges + range) * 2 + slot) * G + head; sk_rec[2b] is the
  // first range sequence b meets, sk_rec[2b + 1] twice the number of ranges
  // it meets plus 1 if its piece in the first one is in slot 1 (written by
  // the decode for every sequence with pages, read by the merge).
  int32_t sk_ranges;
  // ranges per dispatch slot (the workgroups a CU holds at once take slots
  // 0, 1, ... of it in launch order: sk_ranges / sk_per_slot of them)
  int32_t sk_per_slot;
  int32_t* sk_rec;
};

// How a decode workgroup finds its work: the host's split plan, the plan's
// splits grown on the device (balanced_split_pages), or stream-K ranges.
constexpr int kMapPlanned = 0;
constexpr int kMapBalanced = 1;
constexpr int kMapStream = 2;
// Stream-K: at most this many workgroups (ranges times KV heads, rounded up
// to whole KV heads) -- the workspace is sized for it.
constexpr int kStreamMaxWorkgroups = 2048;
// What a stream-K workgroup spends on a sequence whatever its length (query
// prologue, merge, the unused page slots of its last step), in pages of
// work, for the one-set and the two-set builds: the run's cost of a sequence
// beside its pages.
constexpr int kStreamItemCost1 = 16;
constexpr int kStreamItemCost2 = 20;
// How much more range each earlier dispatch slot of a CU takes than the next
// (64ths), one-set and two-set builds.
constexpr int kStreamSkew1 = 24;
constexpr int kStreamSkew2 = 24;

// Split-K plan shared by the launch and the workspace query.
struct SplitPlan {
  int32_t split_pages;
  int32_t nsplit;
};
SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len, int32_t num_splits);
size_t workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim, const SplitPlan& p);
bool may_balance(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len, const SplitPlan& p);

hipError_t launch_append_int4(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_int8(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_int4g(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_mxfp4(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode_int4(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_int4g(const DecodeArgs& a, hipStream_t s);
// The balanced build (a.balance set) of the three above: codes of `bits` bits
// with one scale and zero per `gs` channels (0: per token).
hipError_t launch_decode_quant_balanced(const DecodeArgs& a, int bits, int gs, hipStream_t s);
// The stream-K build of the three (a.sk_ranges set by stream_ranges of the
// same format): a grid of num_kv_heads * sk_ranges workgroups.
hipError_t launch_decode_quant_stream(const DecodeArgs& a, int bits, int gs, hipStream_t s);
// Ranges per KV head for the stream-K build of a format on the current
// device: as many workgroups as the device holds at once, at most
// kStreamMaxWorkgroups (rounded up to whole KV heads); per_slot: the ranges
// of one dispatch slot (ranges / workgroups per CU, rounded up).
hipError_t stream_ranges(const DecodeArgs& a, int bits, int gs, int32_t* ranges, int32_t* per_slot);
hipError_t launch_decode_mxfp4(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t s);
// One grid of the bf16 window workgroups (aw, one split) and the INT4
// workgroups (a4), both storing partials.
hipError_t launch_decode_windowed(const DecodeArgs& a4, const DecodeArgs& aw, hipStream_t s);

}  // namespace kvq

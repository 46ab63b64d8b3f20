// Split-K merge: for each (sequence, query head) combine the partials (max,
// sum, unnormalised output) of its splits with the log-sum-exp rule and
// normalise.  The decode kernels store each partial already rotated back to
// the original basis (the rotation is linear and the merge is a weighted
// sum), so nothing is rotated here.
//
// A wave merges four (sequence, query head) rows, one per row of 16 lanes;
// lane n of a row owns channels [C n, C n + C) with C = D / 16, read as
// 16-byte vectors from every split.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int kReduceThreads = 256;   // 16 (sequence, query head) rows per workgroup

template <int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(DecodeArgs a) {
  constexpr int kC = D / 16;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int64_t rows = static_cast<int64_t>(a.batch) * a.num_q_heads;
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * (kReduceThreads / 16) + (threadIdx.x >> 4);
  if (bh >= rows) return;
  const int b = static_cast<int>(bh / a.num_q_heads);
  float* dst = a.out + bh * D + kC * n;

  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  // the splits that held pages of this sequence
  int lo, hi;
  int4_token_range(len, a.skip_first, a.skip_last, lo, hi);
  const int npg = (hi + kPage - 1) / kPage, pfirst = lo / kPage;
  auto valid = [&](int slot) {
    const int q0 = max(slot * a.split_pages, pfirst);
    return hi > lo && q0 < min(npg, (slot + 1) * a.split_pages);
  };
  const float* ml = a.part_ml + bh * a.part_stride * 2;
  const float* pa = a.part_acc + bh * a.part_stride * D + kC * n;

  // Every slot's loads are issued (the workspace holds part_stride slots per
  // row) and only the valid slots are taken, by selection rather than by a
  // zero weight, so the stale bytes of unused slots never enter the sums; the
  // unrolled loops keep several slots' loads in flight instead of one round
  // trip per split.
  float mstar = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < a.part_stride; ++s) {
    const float m = ml[2 * s];
    mstar = valid(s) ? fmaxf(mstar, m) : mstar;
  }
  const float muse = mstar == -__builtin_inff() ? 0.0f : mstar;
  float lsum = 0.0f;
  float o[kC];
#pragma unroll
  for (int k = 0; k < kC; ++k) o[k] = 0.0f;
#pragma unroll 4
  for (int s = 0; s < a.part_stride; ++s) {
    const float m = ml[2 * s], l = ml[2 * s + 1];
    v4f x[kC / 4];
#pragma unroll
    for (int k = 0; k < kC / 4; ++k) x[k] = *reinterpret_cast<const v4f*>(pa + static_cast<int64_t>(s) * D + 4 * k);
    if (valid(s)) {
      const float w = exp2f(m - muse);
      lsum = __builtin_fmaf(l, w, lsum);
#pragma unroll
      for (int k = 0; k < kC / 4; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 * k + i] = __builtin_fmaf(x[k][i], w, o[4 * k + i]);
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;   // an empty sequence stores zeros
#pragma unroll
  for (int k = 0; k < kC; k += 4)
    *reinterpret_cast<v4f*>(dst + k) = v4f{o[k] * inv, o[k + 1] * inv, o[k + 2] * inv, o[k + 3] * inv};
}

}  // namespace

hipError_t launch_reduce(const DecodeArgs& a, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.batch) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>((rows + kReduceThreads / 16 - 1) / (kReduceThreads / 16)));
  if (a.head_dim == 128)
    reduce_kernel<128><<<grid, kReduceThreads, 0, s>>>(a);
  else
    reduce_kernel<64><<<grid, kReduceThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq

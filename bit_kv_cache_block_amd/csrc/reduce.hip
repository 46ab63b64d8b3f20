// Split-K merge: for each (sequence, query head) combine the partials (max,
// sum, unnormalised output) of its splits with the log-sum-exp rule and
// normalise.  In a windowed call the last slot of each row is the bf16 window
// pass's partial.  The decode kernels store each partial already rotated back to
// the original basis (the rotation is linear and the merge is a weighted
// sum), so nothing is rotated here.
//
// A row's splits are dealt round-robin to G groups of D/4 lanes; lane c of a
// group owns channels [4c, 4c + 4), read as one 16-byte vector per split.
// Each group folds its splits in with the online form of the rule (running
// maximum, rescaled sum and output), so the loads of all its splits can be in
// flight at once and no separate pass over the maxima is needed; the G group
// results of a row then meet in LDS.  The host picks G so that a lane reads
// at most about four splits: a merge of few rows and many splits (small
// batches cut finely) is a couple of memory round trips rather than one per
// split.
//
// After a stream-K decode (SK) a row's partials are those of the ranges its
// sequence met, found from the decode's record of the sequence; a sequence
// inside one range was finished by the decode, one with no pages gets zeros
// here.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int kReduceThreads = 256;

template <int D, int G, bool SK>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(DecodeArgs a) {
  constexpr int kL = D / 4;                          // lanes per split group
  constexpr int kRows = kReduceThreads / (kL * G);   // rows per workgroup
  static_assert(kRows >= 1 && kRows * kL * G == kReduceThreads, "group shape");
  __shared__ float sm_o[kRows][G][D];
  __shared__ float sm_m[kRows][G];
  __shared__ float sm_l[kRows][G];

  const int t = threadIdx.x;
  const int r = t / (kL * G);
  const int g = (t / kL) % G;
  const int c = t % kL;
  const int64_t rows = static_cast<int64_t>(a.batch) * a.num_q_heads;
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * kRows + r;
  const bool live = bh < rows;

  float m = -__builtin_inff(), l = 0.0f;
  v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
  bool done = false;   // the decode already wrote this row
  if constexpr (SK) {
    if (live) {
      const int b = static_cast<int>(bh / a.num_q_heads);
      const int h = static_cast<int>(bh % a.num_q_heads);
      const int gq = a.num_q_heads / a.num_kv_heads;
      const int kvh = h / gq, j = h % gq;
      int cnt = 0, rf = 0, fs = 0;
      if (stream_pages_of(a.seq_lens, b, a.batch, a.max_seq_len) > 0) {
        rf = a.sk_rec[2 * b];
        cnt = a.sk_rec[2 * b + 1] >> 1;
        fs = a.sk_rec[2 * b + 1] & 1;
      }
      done = cnt == 1;
      if (!done) {
#pragma unroll 4
        for (int k = g; k < cnt; k += G) {
          const int64_t idx = ((static_cast<int64_t>(kvh) * a.sk_ranges + rf + k) * 2 + (k == 0 ? fs : 0)) * gq + j;
          const float ms = a.part_ml[2 * idx], ls = a.part_ml[2 * idx + 1];
          const v4f x = *reinterpret_cast<const v4f*>(a.part_acc + idx * D + 4 * c);
          const float mn = fmaxf(m, ms);
          const float mu = mn == -__builtin_inff() ? 0.0f : mn;
          const float fo = fast_exp2(m - mu), fs2 = fast_exp2(ms - mu);
          l = __builtin_fmaf(l, fo, ls * fs2);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = __builtin_fmaf(o[i], fo, x[i] * fs2);
          m = mn;
        }
      }
    }
  } else {
    // (every lane of the wave takes part in reading the lengths)
    const int sp = a.balance ? balanced_split_pages(a.split_pages, a.seq_lens, a.batch, a.max_seq_len,
                                                    a.num_kv_heads)
                             : a.split_pages;
    if (live) {
      const int b = static_cast<int>(bh / a.num_q_heads);
      int len = a.seq_lens[b];
      len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
      // the splits that held pages of this sequence
      int lo, hi;
      int4_token_range(len, a.skip_first, a.skip_last, lo, hi);
      const int npg = (hi + kPage - 1) / kPage, pfirst = lo / kPage;
      // a sequence whose pages lie in one split was finished by the decode,
      // unless the decode was told to store partials only (windowed calls)
      done = !a.force_partial && hi > lo && (npg - 1) / sp == pfirst / sp;
    }
    if (live && !done) {
      const int b = static_cast<int>(bh / a.num_q_heads);
      int len = a.seq_lens[b];
      len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
      int lo, hi;
      int4_token_range(len, a.skip_first, a.skip_last, lo, hi);
      const int npg = (hi + kPage - 1) / kPage, pfirst = lo / kPage;
      const float* ml = a.part_ml + bh * a.part_stride * 2;
      const float* pa = a.part_acc + bh * a.part_stride * D + 4 * c;
      // Every slot's loads are issued (the workspace holds part_stride slots
      // per row) and only valid slots are folded in, by selection rather than
      // a zero weight, so stale bytes never enter the sums; without a branch in
      // the loop the unrolled iterations' loads are all in flight together.
#pragma unroll 4
      for (int s = g; s < a.part_stride; s += G) {
        const float ms = ml[2 * s], ls = ml[2 * s + 1];
        const v4f x = *reinterpret_cast<const v4f*>(pa + static_cast<int64_t>(s) * D);
        // INT4 split s, or (windowed calls) the window pass's slot, the last
        const bool ok = (a.has_window && s == a.part_stride - 1)
                            ? min(len, a.win_len) > 0
                            : hi > lo && max(s * sp, pfirst) < min(npg, (s + 1) * sp);
        const float mn = ok ? fmaxf(m, ms) : m;
        const float mu = mn == -__builtin_inff() ? 0.0f : mn;
        const float fo = fast_exp2(m - mu), fs = fast_exp2(ms - mu);
        l = ok ? __builtin_fmaf(l, fo, ls * fs) : l;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = ok ? __builtin_fmaf(o[i], fo, x[i] * fs) : o[i];
        m = mn;
      }
    }
  }
  float* dst = a.out + bh * D + 4 * c;
  if constexpr (G == 1) {
    if (!live || done) return;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;   // an empty sequence stores zeros
    *reinterpret_cast<v4f*>(dst) = v4f{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  } else {
    *reinterpret_cast<v4f*>(&sm_o[r][g][4 * c]) = o;
    if (c == 0) {
      sm_m[r][g] = m;
      sm_l[r][g] = l;
    }
    __syncthreads();
    if (!live || done || g != 0) return;
    float mstar = sm_m[r][0];
#pragma unroll
    for (int k = 1; k < G; ++k) mstar = fmaxf(mstar, sm_m[r][k]);
    const float mu = mstar == -__builtin_inff() ? 0.0f : mstar;
    float lsum = 0.0f;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float f = fast_exp2(sm_m[r][k] - mu);
      lsum = __builtin_fmaf(sm_l[r][k], f, lsum);
      const v4f y = *reinterpret_cast<const v4f*>(&sm_o[r][k][4 * c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(y[i], f, acc[i]);
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    *reinterpret_cast<v4f*>(dst) = v4f{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  }
}

template <int D, int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  constexpr int kRows = kReduceThreads / (D / 4 * G);
  const int64_t rows = static_cast<int64_t>(a.batch) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>((rows + kRows - 1) / kRows));
  if (a.sk_ranges > 0)
    reduce_kernel<D, G, true><<<grid, kReduceThreads, 0, s>>>(a);
  else
    reduce_kernel<D, G, false><<<grid, kReduceThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const DecodeArgs& a, hipStream_t s) {
  // about four splits per lane: G = the power of two >= part_stride / 4,
  // at most one row per workgroup
  constexpr int kMaxG = kReduceThreads / (D / 4);
  int g = 1;
  while (g < kMaxG && 4 * g < a.part_stride) g *= 2;
  switch (g) {
    case 1: return launch_g<D, 1>(a, s);
    case 2: return launch_g<D, 2>(a, s);
    case 4: return launch_g<D, 4>(a, s);
    case 8: return launch_g<D, 8>(a, s);
    default:
      if constexpr (kMaxG >= 16) return launch_g<D, 16>(a, s);
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_reduce(const DecodeArgs& a, hipStream_t s) {
  if (a.head_dim == 128) return launch_dim<128>(a, s);
  return launch_dim<64>(a, s);
}

}  // namespace kvq

// Split-K merge: for each (sequence, query head) combine the partial
// (max, sum, unnormalised output) of every split with the log-sum-exp rule,
// normalise, and rotate the output back to the original basis with the same
// block Hadamard (it is symmetric, so it is its own inverse up to the 1/sqrt(b)
// normalisation already folded into each factor).
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

__global__ __launch_bounds__(64) void reduce_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.num_q_heads;
  const int d = a.head_dim;
  const int lane = threadIdx.x;
  __shared__ float o[128];
  __shared__ float wsplit[64];
  float* dst = a.out + static_cast<int64_t>(bh) * d;

  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int npg = (len + kPage - 1) / kPage;
  const int nsp = (npg + a.split_pages - 1) / a.split_pages;
  const float* ml = a.part_ml + static_cast<int64_t>(bh) * a.nsplit * 2;
  const float* pa = a.part_acc + static_cast<int64_t>(bh) * a.nsplit * d;

  float mstar = -__builtin_inff();
  for (int s = lane; s < nsp; s += 64) mstar = fmaxf(mstar, ml[2 * s]);
  for (int off = 32; off > 0; off >>= 1) mstar = fmaxf(mstar, __shfl_xor(mstar, off));
  float lsum = 0.0f;
  for (int s = lane; s < nsp; s += 64) lsum += ml[2 * s + 1] * exp2f(ml[2 * s] - mstar);
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);

  if (nsp == 0 || !(lsum > 0.0f)) {
    for (int c = lane; c < d; c += 64) dst[c] = 0.0f;
    return;
  }
  const float inv_l = 1.0f / lsum;
  float accv[2] = {0.0f, 0.0f};
  for (int s0 = 0; s0 < nsp; s0 += 64) {
    const int cnt = min(64, nsp - s0);
    __syncthreads();
    if (lane < cnt) wsplit[lane] = exp2f(ml[2 * (s0 + lane)] - mstar);
    __syncthreads();
    for (int s = 0; s < cnt; ++s) {
      const float w = wsplit[s];
      const float* row = pa + static_cast<int64_t>(s0 + s) * d;
      for (int k = 0, c = lane; c < d; ++k, c += 64) accv[k] = __builtin_fmaf(row[c], w, accv[k]);
    }
  }
  for (int k = 0, c = lane; c < d; ++k, c += 64) o[c] = accv[k] * inv_l;
  __syncthreads();
  if (a.block > 0) {
    for (int hh = 1; hh < a.block; hh *= 2) {
      for (int q = lane; q < d / 2; q += 64) {
        const int i = (q / hh) * (2 * hh) + (q % hh);
        const float u = o[i], w = o[i + hh];
        o[i] = u + w;
        o[i + hh] = u - w;
      }
      __syncthreads();
    }
    const float sb = block_norm(a.block);
    for (int c = lane; c < d; c += 64) dst[c] = o[c] * sb;
  } else {
    for (int c = lane; c < d; c += 64) dst[c] = o[c];
  }
}

}  // namespace

hipError_t launch_reduce(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch * a.num_q_heads));
  reduce_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq

// Windowed decode in one grid: the bf16 workgroups over each sequence's
// high-precision window (sink and recent tokens, "InnerQ", Abstract and
// Figure 2) and the INT4 workgroups over the tokens between the windows run
// side by side, each storing a partial (max, sum, unnormalised output); the
// split merge then finishes the call.  The INT4 workgroups come first in the
// grid, so that all of them start at once, and the short, latency-bound
// window workgroups take the slots that are left (and those that free up)
// while the INT4 workgroups stream the cache, instead of running after them.
#include "decode_bf16_body.hpp"
#include "decode_int4_body.hpp"

namespace kvq {
namespace {

static_assert(b16::kWaves == q4::kWaves, "one workgroup shape");

// BAL: the INT4 pass is a balanced call (balanced_split_pages; the window
// pass never is)
template <int D, int NS, bool QBF16, bool BAL>
__global__ __launch_bounds__(64 * q4::kWaves) void decode_windowed_kernel(DecodeArgs a4, DecodeArgs aw,
                                                                         uint32_t n4) {
  if (blockIdx.x < n4)
    q4::decode_quant_body<D, NS, QBF16, 4, 0, 1, BAL>(a4, blockIdx.x);
  else
    b16::decode_bf16_body<D, NS, QBF16, false>(aw, blockIdx.x - n4);
}

template <int D, int NS, bool BAL>
hipError_t launch_b(const DecodeArgs& a4, const DecodeArgs& aw, hipStream_t s) {
  const uint32_t n_win = static_cast<uint32_t>(aw.nsplit) * aw.num_kv_heads * aw.batch;
  const uint32_t n4 = static_cast<uint32_t>(a4.nsplit) * a4.num_kv_heads * a4.batch;
  const dim3 grid(n_win + n4);
  if (a4.in_bf16)
    decode_windowed_kernel<D, NS, true, BAL><<<grid, 64 * q4::kWaves, 0, s>>>(a4, aw, n4);
  else
    decode_windowed_kernel<D, NS, false, BAL><<<grid, 64 * q4::kWaves, 0, s>>>(a4, aw, n4);
  return hipGetLastError();
}

template <int D, int NS>
hipError_t launch_d(const DecodeArgs& a4, const DecodeArgs& aw, hipStream_t s) {
  return a4.balance ? launch_b<D, NS, true>(a4, aw, s) : launch_b<D, NS, false>(a4, aw, s);
}

template <int D>
hipError_t launch_ns(const DecodeArgs& a4, const DecodeArgs& aw, hipStream_t s) {
  const int g = a4.num_q_heads / a4.num_kv_heads;
  if (g <= 4) return launch_d<D, 1>(a4, aw, s);
  if (g <= 8) return launch_d<D, 2>(a4, aw, s);
  return launch_d<D, 4>(a4, aw, s);
}

}  // namespace

hipError_t launch_decode_windowed(const DecodeArgs& a4, const DecodeArgs& aw, hipStream_t s) {
  return a4.head_dim == 128 ? launch_ns<128>(a4, aw, s) : launch_ns<64>(a4, aw, s);
}

}  // namespace kvq

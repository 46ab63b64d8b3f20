// bf16-KV baseline of the split-K paged decode attention: the same workgroup
// organisation (four waves, LDS merge, direct output without a global split)
// and online softmax as the INT4 kernel, with bf16 MFMA.  The query and the
// probabilities are each carried as three bf16 limbs (hi, mid, lo: 24
// significant bits) in the rows of the GQA group's tile, so the products keep
// fp32 accuracy against the exact bf16 cache values.
#include "decode_bf16_body.hpp"

namespace kvq {
namespace {

using b16::kWaves;

template <int D, int NS, bool QBF16, bool BAL>
__global__ __launch_bounds__(64 * kWaves) void decode_bf16_kernel(DecodeArgs a) {
  b16::decode_bf16_body<D, NS, QBF16, BAL>(a, blockIdx.x);
}

template <int D, int NS, bool BAL>
hipError_t launch_b(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.nsplit) * a.num_kv_heads * a.batch);
  if (a.in_bf16)
    decode_bf16_kernel<D, NS, true, BAL><<<grid, 64 * kWaves, 0, s>>>(a);
  else
    decode_bf16_kernel<D, NS, false, BAL><<<grid, 64 * kWaves, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, int NS>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  return a.balance ? launch_b<D, NS, true>(a, s) : launch_b<D, NS, false>(a, s);
}

template <int D>
hipError_t launch_ns(const DecodeArgs& a, hipStream_t s) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 4) return launch_d<D, 1>(a, s);
  if (g <= 8) return launch_d<D, 2>(a, s);
  return launch_d<D, 4>(a, s);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_ns<128>(a, s) : launch_ns<64>(a, s);
}

}  // namespace kvq

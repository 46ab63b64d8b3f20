// Launch of the INT4-family decode kernel (token-wise INT4, INT8 and grouped
// INT4 codes; the kernel itself is decode_quant_body): the number of query
// heads per KV head picks the sets of four heads a workgroup carries, the
// grid size the register budget.  The planned and balanced builds
// (decode_int4.hip) and the stream-K build (decode_int4_sk.hip) each
// instantiate it with their own MAP, in two translation units that compile
// side by side.
#pragma once
#include "decode_int4_body.hpp"

namespace kvq {
namespace {

using q4::kWaves;

template <int D, int NS, bool QBF16, int BITS, int GS, int WPE, int MAP>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(WPE)))
void decode_quant_kernel(DecodeArgs a) {
  q4::decode_quant_body<D, NS, QBF16, BITS, GS, WPE, MAP>(a, blockIdx.x);
}

template <int MAP, int D, int NS, int BITS, int GS, int WPE>
hipError_t launch_w(const DecodeArgs& a, hipStream_t s, unsigned wgs) {
  if (a.in_bf16)
    decode_quant_kernel<D, NS, true, BITS, GS, WPE, MAP><<<dim3(wgs), 64 * kWaves, 0, s>>>(a);
  else
    decode_quant_kernel<D, NS, false, BITS, GS, WPE, MAP><<<dim3(wgs), 64 * kWaves, 0, s>>>(a);
  return hipGetLastError();
}

// The stream-K build of each format: the one that keeps most waves
// resident (its grid is what the device holds at once) -- for the
// one-set INT4 kernel 128 VGPRs (4 waves per SIMD), for the two-set one at
// head_dim 128 the LDS-staged build (3 waves per SIMD).
template <int D, int NS, int BITS, int GS>
constexpr int stream_wpe() {
  if (NS == 1 && BITS == 4 && GS == 0) return 4;
  if (D == 128 && NS == 2 && BITS == 4 && GS == 0) return 3;
  return 1;
}

template <int MAP, int D, int NS, int BITS, int GS>
hipError_t launch_planned(const DecodeArgs& a, hipStream_t s) {
  const unsigned wgs = static_cast<unsigned>(a.nsplit) * a.num_kv_heads * a.batch;
  // The 4-byte-sidecar INT4 kernel for one set of heads needs a few VGPRs more
  // than 128.  When the grid is larger than 512 workgroups (two per CU), a
  // build held to 128 VGPRs (4 waves per SIMD) keeps more of it resident:
  // measured 7% faster at 1024 workgroups, 2% slower at 512.
  if constexpr (NS == 1 && BITS == 4 && GS == 0) {
    if (wgs > 512) return launch_w<MAP, D, NS, BITS, GS, 4>(a, s, wgs);
  }
  // The two-set INT4 kernel at head_dim 128: on large grids the build for 3
  // waves per SIMD (at most 168 VGPRs), which keeps its next step in flight
  // in an LDS stage rather than in a second register buffer; on smaller ones
  // (a few long chains of steps set the time) the build with two register
  // buffers (about 200 VGPRs, 2 waves per SIMD), which holds two steps in
  // flight while it waits for one.  (Head_dim 64 fits 3 waves with both
  // register buffers.)
  if constexpr (D == 128 && NS == 2 && BITS == 4 && GS == 0) {
    if (wgs > 4096) return launch_w<MAP, D, NS, BITS, GS, 3>(a, s, wgs);
  }
  return launch_w<MAP, D, NS, BITS, GS, 1>(a, s, wgs);
}

template <int MAP, int D, int NS, int BITS, int GS>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  if constexpr (MAP == kMapStream) {
    const unsigned wgs = static_cast<unsigned>(a.sk_ranges) * a.num_kv_heads;
    return launch_w<MAP, D, NS, BITS, GS, stream_wpe<D, NS, BITS, GS>()>(a, s, wgs);
  } else {
    return launch_planned<MAP, D, NS, BITS, GS>(a, s);
  }
}

template <int MAP, int D, int BITS, int GS>
hipError_t launch_ns(const DecodeArgs& a, hipStream_t s) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 4) return launch_d<MAP, D, 1, BITS, GS>(a, s);
  if (g <= 8) return launch_d<MAP, D, 2, BITS, GS>(a, s);
  return launch_d<MAP, D, 4, BITS, GS>(a, s);
}

// codes of `bits` bits (4 or 8) with one scale and zero per `gs` channels (0:
// per token; 32 or 64 with 4-bit codes)
template <int MAP>
hipError_t launch_format(const DecodeArgs& a, int bits, int gs, hipStream_t s) {
  const bool d128 = a.head_dim == 128;
  if (bits == 8) return d128 ? launch_ns<MAP, 128, 8, 0>(a, s) : launch_ns<MAP, 64, 8, 0>(a, s);
  if (gs == 32) return d128 ? launch_ns<MAP, 128, 4, 32>(a, s) : launch_ns<MAP, 64, 4, 32>(a, s);
  if (gs == 64) return d128 ? launch_ns<MAP, 128, 4, 64>(a, s) : launch_ns<MAP, 64, 4, 64>(a, s);
  return d128 ? launch_ns<MAP, 128, 4, 0>(a, s) : launch_ns<MAP, 64, 4, 0>(a, s);
}

}  // namespace
}  // namespace kvq

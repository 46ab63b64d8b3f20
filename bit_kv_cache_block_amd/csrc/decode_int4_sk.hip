// The stream-K build of the INT4-family decode: the same kernels compiled to
// take equal ranges of the batch's pages (stream_range) in a grid of as many
// workgroups as the device holds at once.  Apart from the planned and
// balanced builds so that their calls carry none of its code.
#include <atomic>

#include "decode_int4_launch.hpp"

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;

// Workgroups of one build that the current device holds at once, looked up
// once per device and query type.
template <int D, int NS, int BITS, int GS>
hipError_t resident(const DecodeArgs& a, int* wgs) {
  constexpr int WPE = stream_wpe<D, NS, BITS, GS>();
  static std::atomic<int> held[kMaxDevices][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int qt = a.in_bf16 ? 1 : 0;
  int n = dev >= 0 && dev < kMaxDevices ? held[dev][qt].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    int per_cu = 0, cus = 0;
    const void* k = a.in_bf16 ? reinterpret_cast<const void*>(&decode_quant_kernel<D, NS, true, BITS, GS, WPE, kMapStream>)
                              : reinterpret_cast<const void*>(&decode_quant_kernel<D, NS, false, BITS, GS, WPE, kMapStream>);
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * kWaves, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    n = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (dev >= 0 && dev < kMaxDevices) held[dev][qt].store(n, std::memory_order_relaxed);
  }
  *wgs = n;
  return hipSuccess;
}

template <int D, int BITS, int GS>
hipError_t resident_ns(const DecodeArgs& a, int* wgs) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 4) return resident<D, 1, BITS, GS>(a, wgs);
  if (g <= 8) return resident<D, 2, BITS, GS>(a, wgs);
  return resident<D, 4, BITS, GS>(a, wgs);
}

}  // namespace

hipError_t launch_decode_quant_stream(const DecodeArgs& a, int bits, int gs, hipStream_t s) {
  return launch_format<kMapStream>(a, bits, gs, s);
}

hipError_t stream_ranges(const DecodeArgs& a, int bits, int gs, int32_t* ranges) {
  const bool d128 = a.head_dim == 128;
  int wgs = 0;
  hipError_t e;
  if (bits == 8) e = d128 ? resident_ns<128, 8, 0>(a, &wgs) : resident_ns<64, 8, 0>(a, &wgs);
  else if (gs == 32) e = d128 ? resident_ns<128, 4, 32>(a, &wgs) : resident_ns<64, 4, 32>(a, &wgs);
  else if (gs == 64) e = d128 ? resident_ns<128, 4, 64>(a, &wgs) : resident_ns<64, 4, 64>(a, &wgs);
  else e = d128 ? resident_ns<128, 4, 0>(a, &wgs) : resident_ns<64, 4, 0>(a, &wgs);
  if (e != hipSuccess) return e;
  if (wgs > kStreamMaxWorkgroups) wgs = kStreamMaxWorkgroups;
  *ranges = (wgs + a.num_kv_heads - 1) / a.num_kv_heads;
  return hipSuccess;
}

}  // namespace kvq

// The stream-K build of the INT4-family decode: the same kernels compiled to
// take ranges of the batch's pages (stream_range) in a grid of as many
// workgroups as the device holds at once.  Apart from the planned and
// balanced builds so that their calls carry none of its code.
#include <atomic>

#include "decode_int4_launch.hpp"

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;

// Workgroups of one build that the current device holds at once (in all,
// and per CU), looked up once per device and query type.
template <int D, int NS, int BITS, int GS>
hipError_t resident(const DecodeArgs& a, int* wgs, int* per_cu_out) {
  constexpr int WPE = stream_wpe<D, NS, BITS, GS>();
  static std::atomic<int> held[kMaxDevices][2][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int qt = a.in_bf16 ? 1 : 0;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int n = cached ? held[dev][qt][0].load(std::memory_order_relaxed) : 0;
  int pc = cached ? held[dev][qt][1].load(std::memory_order_relaxed) : 0;
  if (n == 0 || pc == 0) {
    int per_cu = 0, cus = 0;
    const void* k = a.in_bf16 ? reinterpret_cast<const void*>(&decode_quant_kernel<D, NS, true, BITS, GS, WPE, kMapStream>)
                              : reinterpret_cast<const void*>(&decode_quant_kernel<D, NS, false, BITS, GS, WPE, kMapStream>);
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * kWaves, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    pc = per_cu > 0 ? per_cu : 1;
    n = pc * (cus > 0 ? cus : 1);
    if (cached) {
      held[dev][qt][1].store(pc, std::memory_order_relaxed);
      held[dev][qt][0].store(n, std::memory_order_relaxed);
    }
  }
  *wgs = n;
  *per_cu_out = pc;
  return hipSuccess;
}

template <int D, int BITS, int GS>
hipError_t resident_ns(const DecodeArgs& a, int* wgs, int* per_cu) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 4) return resident<D, 1, BITS, GS>(a, wgs, per_cu);
  if (g <= 8) return resident<D, 2, BITS, GS>(a, wgs, per_cu);
  return resident<D, 4, BITS, GS>(a, wgs, per_cu);
}

}  // namespace

hipError_t launch_decode_quant_stream(const DecodeArgs& a, int bits, int gs, hipStream_t s) {
  return launch_format<kMapStream>(a, bits, gs, s);
}

hipError_t stream_ranges(const DecodeArgs& a, int bits, int gs, int32_t* ranges, int32_t* per_slot) {
  const bool d128 = a.head_dim == 128;
  int wgs = 0, per_cu = 1;
  hipError_t e;
  if (bits == 8) e = d128 ? resident_ns<128, 8, 0>(a, &wgs, &per_cu) : resident_ns<64, 8, 0>(a, &wgs, &per_cu);
  else if (gs == 32) e = d128 ? resident_ns<128, 4, 32>(a, &wgs, &per_cu) : resident_ns<64, 4, 32>(a, &wgs, &per_cu);
  else if (gs == 64) e = d128 ? resident_ns<128, 4, 64>(a, &wgs, &per_cu) : resident_ns<64, 4, 64>(a, &wgs, &per_cu);
  else e = d128 ? resident_ns<128, 4, 0>(a, &wgs, &per_cu) : resident_ns<64, 4, 0>(a, &wgs, &per_cu);
  if (e != hipSuccess) return e;
  if (wgs > kStreamMaxWorkgroups) wgs = kStreamMaxWorkgroups;
  *ranges = (wgs + a.num_kv_heads - 1) / a.num_kv_heads;
  *per_slot = (*ranges + per_cu - 1) / per_cu;
  return hipSuccess;
}

}  // namespace kvq

// Memory-system ceilings for the two access patterns of the hot path, built
// into libkvq_probe.so (not part of the C ABI of libkvq.so; the benchmark's
// ceiling mode calls them):
//   - gather: the decode's pattern, a read of page slabs in a permuted order,
//     four slabs per wave step, non-temporal buffer loads;
//   - stream: a streaming read with a fixed read:write ratio (4:1 for 2-byte
//     inputs against 4-bit codes), or a pure read, the pieces in flight
//     spread over the grid;
//   - stream_block: the same mix with each workgroup on its own contiguous
//     stretch, stores plain or non-temporal, the output contiguous or in
//     1 KiB pieces at permuted places (the append writes page slabs of a
//     permuted page table).
// Each probe reduces what it reads with xor so that no load is dead code, and
// stores one word per thread (gather, pure stream) or its write share.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dev_common.hpp"

namespace {

using kvq::u32x4;

// Slab i of the work list is ids[i] of the pool (slab_bytes each, a multiple
// of 16, at most R KiB); a wave reads four slabs per step, its lanes taking
// consecutive 16-byte pieces (loads past a slab's end return zeros without
// touching memory).
template <int R>
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* pool, int32_t slab_bytes,
                                                     const int32_t* ids, int32_t n, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int waves = (gridDim.x * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (int i0 = 4 * wave; i0 < n; i0 += 4 * waves) {
    u32x4 v[4][R];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j < n ? i0 + j : n - 1;
      const __amdgpu_buffer_rsrc_t rs =
          kvq::make_rsrc(pool + static_cast<int64_t>(ids[i]) * slab_bytes, i0 + j < n ? slab_bytes : 0);
#pragma unroll
      for (int r = 0; r < R; ++r)
        v[j][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rs, static_cast<uint32_t>(16 * (lane + 64 * r)), 0,
                                                kvq::kStreamOnce));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc ^= v[j][r][0] ^ v[j][r][1] ^ v[j][r][2] ^ v[j][r][3];
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Work item j reads piece j of each of the `ratio` consecutive stretches of
// `items` 16-byte pieces of src (so every load of a wave is 1 KiB contiguous)
// and writes their xor to piece j of dst; with dst null the xor of all a
// thread read goes to sink instead (a pure read).
template <int RATIO>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* src, int64_t items, u32x4* dst,
                                                     uint32_t* sink) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * blockDim.x;
  u32x4 all = {0u, 0u, 0u, 0u};
  for (int64_t j = tid; j < items; j += nth) {
    u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RATIO; ++r) x ^= __builtin_nontemporal_load(&src[r * items + j]);
    if (dst) dst[j] = x;
    else all ^= x;
  }
  if (!dst) sink[tid] = all[0] ^ all[1] ^ all[2] ^ all[3];
}

// Workgroup b reads pieces [b * per_block, (b + 1) * per_block) of each of
// the RATIO stretches (four pieces per thread in flight) and writes their
// xor to the same piece of dst, or with perm to piece perm[j / 64] * 64 +
// j % 64 (1 KiB pieces at permuted places; perm holds items / 64 entries).
template <int RATIO, bool NT>
__global__ __launch_bounds__(256) void stream_block_kernel(const u32x4* src, int64_t items, u32x4* dst,
                                                           int64_t per_block, const int32_t* perm) {
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t b1 = b0 + per_block < items ? b0 + per_block : items;
  for (int64_t j0 = b0 + threadIdx.x; j0 < b1; j0 += 4 * 256) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = j0 + u * 256;
      x[u] = u32x4{0u, 0u, 0u, 0u};
      if (j < b1) {
#pragma unroll
        for (int r = 0; r < RATIO; ++r) x[u] ^= __builtin_nontemporal_load(&src[r * items + j]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = j0 + u * 256;
      if (j < b1) {
        const int64_t d = perm ? static_cast<int64_t>(perm[j >> 6]) * 64 + (j & 63) : j;
        if constexpr (NT) __builtin_nontemporal_store(x[u], &dst[d]);
        else dst[d] = x[u];
      }
    }
  }
}

}  // namespace

extern "C" {

// Slab reads in the order of ids[0 .. n) (each id < the pool's slab count,
// slab_bytes a multiple of 16 and at most 4096); sink holds grid * 256 words.
int kvq_probe_gather(const void* pool, int32_t slab_bytes, const int32_t* ids, int32_t n, int32_t grid,
                     void* sink, void* stream) {
  if (!pool || !ids || !sink || n <= 0 || grid <= 0 || slab_bytes <= 0 || slab_bytes % 16 != 0 ||
      slab_bytes > 4096)
    return 1;
  const auto* p = static_cast<const uint8_t*>(pool);
  auto* k = static_cast<uint32_t*>(sink);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch ((slab_bytes + 1023) / 1024) {   // 1 KiB per 64 lanes and load
    case 1: gather_kernel<1><<<grid, 256, 0, s>>>(p, slab_bytes, ids, n, k); break;
    case 2: gather_kernel<2><<<grid, 256, 0, s>>>(p, slab_bytes, ids, n, k); break;
    case 3: gather_kernel<3><<<grid, 256, 0, s>>>(p, slab_bytes, ids, n, k); break;
    default: gather_kernel<4><<<grid, 256, 0, s>>>(p, slab_bytes, ids, n, k); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// A read of items * ratio 16-byte pieces of src (ratio 1, 2 or 4); with dst,
// items pieces are written (read:write = ratio:1); without, sink holds
// grid * 256 words.
int kvq_probe_stream(const void* src, int64_t items, int32_t ratio, void* dst, int32_t grid, void* sink,
                     void* stream) {
  if (!src || items <= 0 || grid <= 0 || (!dst && !sink)) return 1;
  const auto* in = static_cast<const u32x4*>(src);
  auto* out = static_cast<u32x4*>(dst);
  auto* k = static_cast<uint32_t*>(sink);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (ratio) {
    case 1: stream_kernel<1><<<grid, 256, 0, s>>>(in, items, out, k); break;
    case 2: stream_kernel<2><<<grid, 256, 0, s>>>(in, items, out, k); break;
    case 4: stream_kernel<4><<<grid, 256, 0, s>>>(in, items, out, k); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The 4:1 mix with one contiguous stretch per workgroup (items a multiple
// of 64): nt selects non-temporal stores; perm (items / 64 entries, a
// permutation of 0 .. items / 64 - 1) scatters the output in 1 KiB pieces,
// null keeps it contiguous.
int kvq_probe_stream_block(const void* src, int64_t items, void* dst, int32_t grid, int32_t nt,
                           const int32_t* perm, void* stream) {
  if (!src || !dst || items <= 0 || items % 64 != 0 || grid <= 0) return 1;
  const auto* in = static_cast<const u32x4*>(src);
  auto* out = static_cast<u32x4*>(dst);
  const int64_t per_block = ((items + grid - 1) / grid + 63) / 64 * 64;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (nt) stream_block_kernel<4, true><<<grid, 256, 0, s>>>(in, items, out, per_block, perm);
  else stream_block_kernel<4, false><<<grid, 256, 0, s>>>(in, items, out, per_block, perm);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"

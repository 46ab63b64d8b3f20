// Device helpers for gfx950 (CDNA4, wave64): cross-lane moves, MFMA wrappers,
// nibble packing.  Host code never includes this header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// ---- DPP within groups of four lanes (quad_perm) ---------------------------
// quad_perm [1,0,3,2] (lane ^ 1) and [2,3,0,1] (lane ^ 2).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppBcast0 = 0x00;   // quad_perm [0,0,0,0]
constexpr int kDppXor3 = 0x1B;            // quad_perm [3,2,1,0] (lane ^ 3)
constexpr int kDppRowRor8 = 0x128;        // rotate a row of 16 by 8: lane i <- i ^ 8
constexpr int kDppRowMirror = 0x140;      // lane i <- 15 - i within a row of 16
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- 7 - i within each half row

// Every pattern used reads an existing lane of the same row, so bound_ctrl
// is irrelevant; setting it lets the compiler fold the move into its user.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return u2f(__builtin_amdgcn_mov_dpp(f2u(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}

// ---- row-crossing exchanges with the gfx950 permlane swaps ------------------
// After swapping a copy of x with itself, the two results hold, in every lane,
// the lane's own value and its partner's (lane ^ 16, resp. lane ^ 32) in some
// order; a symmetric op over them is the same in both partners.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  return u2f(r[0]) + u2f(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(r[0]) + u2f(r[1]);
}
// max over the four rows of 16 lanes (same lane position in each row)
__device__ __forceinline__ float max_rows(float x) { return max_xor32(max_xor16(x)); }
__device__ __forceinline__ float sum_rows(float x) { return sum_xor32(sum_xor16(x)); }

// value of lane `src` (wave-wide gather through the LDS crossbar)
__device__ __forceinline__ float lane_read(float x, int src) {
  return u2f(__builtin_amdgcn_ds_bpermute(src << 2, f2u(x)));
}

// ---- MFMA ------------------------------------------------------------------
// 16x16x64 int8 -> int32.  Lane l supplies row (A) / column (B) l % 16 and 16
// k-slots of group l / 16; C[4*(l/16) + i][l % 16] lands in lane l, element i.
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 -> fp32, same lane mapping with 8 k-slots per lane.
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- nibbles -----------------------------------------------------------------
constexpr uint32_t kLowNibbles = 0x0F0F0F0Fu;

// 4x4 byte transpose: out[j] = (x0.byte j, x1.byte j, x2.byte j, x3.byte j).
__device__ __forceinline__ void transpose_bytes4(uint32_t x0, uint32_t x1, uint32_t x2,
                                                 uint32_t x3, uint32_t out[4]) {
  // v_perm_b32(s0, s1, sel): selector bytes 0..3 pick bytes of s1, 4..7 of s0.
  uint32_t a = __builtin_amdgcn_perm(x1, x0, 0x06020400u);  // x0.b0 x1.b0 x0.b2 x1.b2
  uint32_t b = __builtin_amdgcn_perm(x1, x0, 0x07030501u);  // x0.b1 x1.b1 x0.b3 x1.b3
  uint32_t c = __builtin_amdgcn_perm(x3, x2, 0x06020400u);  // x2.b0 x3.b0 x2.b2 x3.b2
  uint32_t d = __builtin_amdgcn_perm(x3, x2, 0x07030501u);  // x2.b1 x3.b1 x2.b3 x3.b3
  out[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);        // a.lo16 | c.lo16 << 16
  out[2] = __builtin_amdgcn_perm(c, a, 0x07060302u);        // a.hi16 | c.hi16 << 16
  out[1] = __builtin_amdgcn_perm(d, b, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
}

// Packs eight 4-bit codes held in bits 0..3 of eight words (higher bits are
// ignored as long as bits 4..7 of c[2j] are zero) into one word: byte j =
// c[2j] | c[2j+1] << 4.
__device__ __forceinline__ uint32_t pack8_nibbles(const uint32_t c[8]) {
  uint32_t b0 = (c[1] << 4) | c[0];
  uint32_t b1 = (c[3] << 4) | c[2];
  uint32_t b2 = (c[5] << 4) | c[4];
  uint32_t b3 = (c[7] << 4) | c[6];
  uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // b0.byte0, b1.byte0
  uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return lo | (hi << 16);
}

// Value of lane i ^ M within a row of 16 lanes (M = 1, 2, 4, 8), all by DPP;
// lane ^ 4 is lane ^ 3 followed by the half-row mirror (lane ^ 7).
template <int M>
__device__ __forceinline__ float dpp_xor(float x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "row xor");
  if constexpr (M == 1) return dpp_f<kDppXor1>(x);
  else if constexpr (M == 2) return dpp_f<kDppXor2>(x);
  else if constexpr (M == 4) return dpp_f<kDppRowHalfMirror>(dpp_f<kDppXor3>(x));
  else return dpp_f<kDppRowRor8>(x);
}

// Block Walsh-Hadamard butterfly over one vector held by a row of 16 lanes:
// lane n holds channels [C n, C n + C) in v[0 .. C).  Stages h = 1, 2, ...,
// block/2 in ascending order, inside the lane while h < C, then with lane
// n ^ (h / C) through DPP.  The lower element of each pair becomes x + y, the
// upper x - y (the upper lane computes partner - own as an fma by -1, which
// rounds once).  Unnormalised; block is a power of two up to 16 C.
template <int C>
__device__ __forceinline__ void fwht_row(float* v, int block, int n) {
#pragma unroll
  for (int h = 1; h < C; h *= 2) {
    if (h < block) {
#pragma unroll
      for (int i = 0; i < C; i += 2 * h)
#pragma unroll
        for (int k = i; k < i + h; ++k) {
          const float x = v[k], y = v[k + h];
          v[k] = x + y;
          v[k + h] = x - y;
        }
    }
  }
  auto cross = [&](auto m_tag) {
    constexpr int M = decltype(m_tag)::value;
    const float sgn = (n & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < C; ++k) v[k] = __builtin_fmaf(sgn, v[k], dpp_xor<M>(v[k]));
  };
  if (C < block) cross(std::integral_constant<int, 1>{});
  if (2 * C < block) cross(std::integral_constant<int, 2>{});
  if (4 * C < block) cross(std::integral_constant<int, 4>{});
  if (8 * C < block) cross(std::integral_constant<int, 8>{});
}

// The same butterfly for a block size known only at run time: one
// straight-line copy per block size (a uniform branch picks it), so that no
// stage is guarded by a run-time test (such guards cost register copies on
// the latency-bound paths that rotate one vector per row).  Block 0: no
// rotation.
template <int C>
__device__ __forceinline__ void fwht_row_any(float* v, int block, int n) {
  switch (block) {
    case 16: fwht_row<C>(v, 16, n); break;
    case 32: fwht_row<C>(v, 32, n); break;
    case 64: fwht_row<C>(v, 64, n); break;
    case 128:
      if constexpr (16 * C >= 128) fwht_row<C>(v, 128, n);
      break;
    default: break;
  }
}

// Pages per split of a decode call.  The host plans splits of at most sp
// pages from the longest length alone (a ragged batch's longest sequence must
// be cut finely).  Balanced calls (the host asks for them only for small
// batches cut into many splits; at most 64 sequences, whose lengths one wave
// reads with one load) grow the split to about total_pages * hkv / 512 pages
// when the batch's whole work is large, so that long uniform contexts run as
// about 512 workgroups of long streams instead of many short ones (the grid
// keeps the planned count; the extra splits are empty).  Every workgroup and
// the merge of a balanced call compute the same value.  All 64 lanes of the
// wave must be active.
__device__ __forceinline__ int balanced_split_pages(int sp, const int32_t* seq_lens, int batch,
                                                    int max_seq_len, int hkv) {
  const int lane = threadIdx.x & 63;
  int len = lane < batch ? seq_lens[lane] : 0;
  len = len < 0 ? 0 : (len > max_seq_len ? max_seq_len : len);
  int total = (len + kPage - 1) / kPage;
#pragma unroll
  for (int m = 1; m < 64; m *= 2) total += __shfl_xor(total, m);
  total = __builtin_amdgcn_readfirstlane(total);
  const int64_t want = (static_cast<int64_t>(total) * hkv + 511) / 512;
  const int64_t even = (want + 3) / 4 * 4;
  return even > sp ? static_cast<int>(even) : sp;
}

// Stream-K cut of a batch (the plain INT4-family decode).  The sequences,
// one after another, each as item_cost units and then its ceil(len / 16)
// pages (len clamped to [0, max_seq_len]; nothing for an empty sequence),
// form a run of `total` units per KV head, cut into `nr` ranges, one per
// workgroup, so that a range's work is its pages plus a fixed cost for each
// sequence that starts in it.
//   The ranges are not equal.  The workgroups of one launch that share a CU
// all start at once (range r's workgroups are dispatched in slot r / rs of
// their CUs), and on equal priority a SIMD issues from its oldest wave
// first: with equal ranges the workgroups of the first slot finished long
// before those of the last, and the kernel waited for these.  So slot k of
// `occ` weighs 64 + skew * (occ - 1 - k) (in 64ths of a range): each slot's
// ranges take the share its workgroups get through in the same time.  A
// small run (under 64 units a range) is cut into equal ranges of
// max(16, ceil(total / nr)) units instead (`unit`), trailing ones empty.
// Every lane of the wave takes part in stream_range; the results are
// wave-uniform.
struct StreamRange {
  int first, end;     // this range: units [first, end) (first >= end: empty)
  int b, start_b;     // the first sequence meeting it, and where that sequence starts
  int total, nr, rs, occ, skew, unit;
};
__device__ __forceinline__ int stream_pages_of(const int32_t* seq_lens, int b, int batch, int max_seq_len) {
  int len = b < batch ? seq_lens[b] : 0;
  len = len < 0 ? 0 : (len > max_seq_len ? max_seq_len : len);
  return (len + kPage - 1) / kPage;
}
__device__ __forceinline__ int stream_cost_of(const int32_t* seq_lens, int b, int batch, int max_seq_len,
                                              int item_cost) {
  const int np = stream_pages_of(seq_lens, b, batch, max_seq_len);
  return np > 0 ? np + item_cost : 0;
}
// the weight of ranges [0, r), 0 <= r <= nr
__device__ __forceinline__ int64_t stream_weight_before(const StreamRange& g, int r) {
  const int k = min(r / g.rs, g.occ - 1);
  const int64_t full = 64 * static_cast<int64_t>(k) +
                       static_cast<int64_t>(g.skew) * (static_cast<int64_t>(k) * (g.occ - 1) - k * (k - 1) / 2);
  return g.rs * full + static_cast<int64_t>(r - k * g.rs) * (64 + g.skew * (g.occ - 1 - k));
}
// the first unit of range r, 0 <= r <= nr (range nr: the run's end)
__device__ __forceinline__ int stream_first(const StreamRange& g, int r) {
  if (g.unit > 0) return min(r * g.unit, g.total);
  return static_cast<int>(static_cast<int64_t>(g.total) * stream_weight_before(g, r) /
                          stream_weight_before(g, g.nr));
}
// the range holding unit x, 0 <= x < total
__device__ __forceinline__ int stream_range_of(const StreamRange& g, int x) {
  if (g.unit > 0) return x / g.unit;
  const int64_t wt = stream_weight_before(g, g.nr);
  const int64_t y = static_cast<int64_t>(x) * wt / g.total;   // x's weight coordinate (rounded down)
  int k = 0;
  while (k + 1 < g.occ && stream_weight_before(g, (k + 1) * g.rs) <= y) ++k;
  int r = k * g.rs + static_cast<int>((y - stream_weight_before(g, k * g.rs)) / (64 + g.skew * (g.occ - 1 - k)));
  r = min(max(r, 0), g.nr - 1);
  while (r > 0 && stream_first(g, r) > x) --r;
  while (r + 1 < g.nr && stream_first(g, r + 1) <= x) ++r;
  return r;
}
__device__ __forceinline__ StreamRange stream_range(const int32_t* seq_lens, int batch, int max_seq_len,
                                                    int ranges, int per_slot, int skew, int r, int item_cost) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int c = 0; c < batch; c += 64) {
    int np = stream_cost_of(seq_lens, c + lane, batch, max_seq_len, item_cost);
#pragma unroll
    for (int m = 1; m < 64; m *= 2) np += __shfl_xor(np, m);
    total += np;
  }
  StreamRange rg;
  rg.total = __builtin_amdgcn_readfirstlane(total);
  rg.nr = ranges;
  rg.rs = max(1, per_slot);
  rg.occ = (ranges + rg.rs - 1) / rg.rs;
  rg.skew = skew;
  rg.unit = rg.total < 64 * ranges ? max(kPage, (rg.total + ranges - 1) / ranges) : 0;
  rg.first = stream_first(rg, r);
  rg.end = stream_first(rg, r + 1);
  rg.b = 0;
  rg.start_b = 0;
  if (rg.first >= rg.end) return rg;
  // the first sequence whose units end after `first`
  int carry = 0;
  for (int c = 0; c < batch; c += 64) {
    const int np = stream_cost_of(seq_lens, c + lane, batch, max_seq_len, item_cost);
    int incl = np;   // inclusive prefix over the 64 lanes
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int y = __shfl_up(incl, d);
      incl += lane >= d ? y : 0;
    }
    const int chunk = __builtin_amdgcn_readlane(incl, 63);
    if (carry + chunk > rg.first) {
      const uint64_t hit = __ballot(carry + incl > rg.first);
      const int l0 = static_cast<int>(__builtin_ctzll(hit));
      rg.b = c + l0;
      rg.start_b = carry + __builtin_amdgcn_readlane(incl - np, l0);
      break;
    }
    carry += chunk;
  }
  return rg;
}

// Tokens [lo, hi) of a sequence of `len` tokens that an INT4 pass reads
// when the first skip_first and the last skip_last tokens are left to the
// high-precision windows (both zero: all of them).
__device__ __forceinline__ void int4_token_range(int len, int skip_first, int skip_last, int& lo, int& hi) {
  lo = skip_first < len ? skip_first : len;
  hi = len - skip_last > lo ? len - skip_last : lo;
}

// Raw buffer descriptor over [base, base + bytes): loads through it take a
// 32-bit lane offset and return zero beyond `bytes` (word 3 = 32-bit data
// format, the value raw loads expect on CDNA).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}

// Cache-policy operand of the buffer builtins: "nt" (non-temporal) marks data
// that is read once.  On gfx950 a random gather of 2 KiB page slabs streams
// about 12% faster from HBM with it than with the default policy.
constexpr int kStreamOnce = 2;

// fp32 constant 1/sqrt(b) of a Hadamard block (the correctly rounded values
// 0x3E800000, 0x3E3504F3, 0x3E000000, 0x3DB504F3 for b = 16, 32, 64, 128).
__device__ __forceinline__ float block_norm(int b) {
  uint32_t bits = b == 16 ? 0x3E800000u : b == 32 ? 0x3E3504F3u : b == 64 ? 0x3E000000u
                : b == 128 ? 0x3DB504F3u : 0x3F800000u;
  return u2f(bits);
}

// ---- helpers shared by the decode kernels ---------------------------------

__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Limbs of the balanced base-256 split v = l0*2^16 + l1*2^8 + l2 with l1, l2
// in [-128, 127] (|v| <= 2^22): with y = v + 0x8080, limb 0 is byte 2 of y,
// limbs 1 and 2 are bytes 1 and 0 of y with the top bit flipped.  A lane
// extracts its own limb `lam` (3 = the zero pad row) branch-free with the
// per-lane shift / flip / keep constants below.
struct LimbSel {
  uint32_t shift, flip, keep;
  __device__ explicit LimbSel(int lam)
      : shift(lam < 3 ? 16u - 8u * lam : 0u), flip(lam == 1 || lam == 2 ? 0x80u : 0u),
        keep(lam < 3 ? 0xFFu : 0u) {}
  __device__ __forceinline__ uint32_t byte(int32_t v) const {
    return ((static_cast<uint32_t>(v + 0x8080) >> shift) ^ flip) & keep;
  }
};

// 2^x with the hardware's v_exp_f32 alone.  exp2f adds a rescaling around it
// so that results below 2^-126 come out as denormals; the softmax weights and
// rescale factors here are relative to a running maximum, so such values are
// below 2^-126 of the weights that matter, and flushing them changes nothing
// at the accuracy the decode keeps.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the 16 lanes of a row, result in every lane of the row.
// The maximum of any values but NaN is taken on keys that order as the
// values do when read as signed integers (a negative value's magnitude bits
// flipped; the map is its own inverse), so that each stage is an integer
// maximum with the lane move folded in, where a float maximum of a moved
// value also quiets possible NaNs (one more instruction per stage).  -0
// orders below +0, a difference no caller can see (the maximum is subtracted
// from logits or compared with -inf).
__device__ __forceinline__ float row_max16_ordered(float x) {
  const int32_t u = static_cast<int32_t>(f2u(x));
  int32_t k = u ^ ((u >> 31) & 0x7FFFFFFF);
  k = max(k, static_cast<int32_t>(dpp_u<kDppXor1>(static_cast<uint32_t>(k))));
  k = max(k, static_cast<int32_t>(dpp_u<kDppXor2>(static_cast<uint32_t>(k))));
  k = max(k, static_cast<int32_t>(dpp_u<kDppRowHalfMirror>(static_cast<uint32_t>(k))));
  k = max(k, static_cast<int32_t>(dpp_u<kDppRowMirror>(static_cast<uint32_t>(k))));
  return u2f(static_cast<uint32_t>(k ^ ((k >> 31) & 0x7FFFFFFF)));
}
// The same of values known to be >= 0 (no NaN): for those the order of
// the bit patterns as unsigned integers is the order of the values, so the
// maximum is taken on the bits, where the lane moves need none of the
// quieting of possible NaNs that a float maximum of a moved value costs
// (one instruction per stage).  Bit-identical to a float maximum on such values.
__device__ __forceinline__ float row_max16_nonneg(float x) {
  uint32_t u = f2u(x);
  u = max(u, dpp_u<kDppXor1>(u));
  u = max(u, dpp_u<kDppXor2>(u));
  u = max(u, dpp_u<kDppRowHalfMirror>(u));
  return u2f(max(u, dpp_u<kDppRowMirror>(u)));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppRowHalfMirror>(x);
  return x + dpp_f<kDppRowMirror>(x);
}
__device__ __forceinline__ int32_t row_sum16_i(int32_t x) {
  uint32_t u = static_cast<uint32_t>(x);
  u += dpp_u<kDppXor1>(u);
  u += dpp_u<kDppXor2>(u);
  u += dpp_u<kDppRowHalfMirror>(u);
  return static_cast<int32_t>(u + dpp_u<kDppRowMirror>(u));
}

}  // namespace kvq

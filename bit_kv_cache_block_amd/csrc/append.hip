// Write path: fused block-Hadamard rotation + token-wise asymmetric INT4
// quantization + paged scatter ("SAW-INT4: System-Aware 4-Bit KV-Cache
// Quantization for Real-World LLM Serving", summary page, Research Findings:
// token-wise INT4 after a block-diagonal Hadamard rotation, with a fused
// rotation-quantization kernel writing into the paged KV-cache layout; scale
// and zero point kept as FP16 as in "InnerQ", Table 3).  The same kernel with
// 8-bit codes (255 levels) writes the INT8 variant ("GPU-Accelerated INT8
// Quantization for KV Cache Compression in Large Language Models",
// Abstract), and with one scale and zero per group of channels the grouped
// INT4 variant (grouping along the inner dimension as in "InnerQ", Abstract
// and Figure 1), and with E2M1 codes under one E8M0 power-of-two scale per 32
// channels the MXFP4 variant ("BitDecoding-FP4", Abstract: an FP4 KV cache
// with Hadamard rotation under token-wise scaling).  Also the bf16-cache
// baseline copy.
//
// Bit-exactness: the quantizer's fp32 steps are done one rounding at a time
// in the order the header of kvq.h states (this file is built with
// -ffp-contract=off; division and reciprocal are the correctly rounded HIP
// defaults), so codes and sidecars equal those of any implementation that
// follows the same steps.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int kAppendThreads = 256;  // 4 independent waves
constexpr int kLaneElems = 64;       // elements of one vector owned by one lane
// Waves stay resident and loop over work units: 1024 workgroups of 4 waves
// are 4 waves per SIMD on the 256 CUs of an MI355X (the kernel is held to
// 128 VGPRs and 32 KiB of LDS per workgroup so that they all fit).
constexpr int kResidentBlocks = 1024;

template <bool BF16>
__device__ __forceinline__ void widen8(u32x4 w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = w[i];
    if constexpr (BF16) {
      x[2 * i] = u2f(u << 16);
      x[2 * i + 1] = u2f(u & 0xFFFF0000u);
    } else {
      x[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xFFFFu)));
      x[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
    }
  }
}

// A work unit is (tile of kTok consecutive tokens, KV head, K or V) and
// belongs to one wave.  The unit's rows go straight from HBM into a
// wave-private LDS image with direct-to-LDS buffer loads (16 bytes per lane,
// 1 KiB of whole rows per instruction; no VGPRs held), from which lane
// (r, hf) takes channels [64 hf, 64 hf + 64) of token t0 + r (two lanes per
// vector at D = 128, one at D = 64).  The next unit's rows are requested as
// soon as the current ones are in registers, so they stream in while the
// current unit is computed.  Lanes of consecutive tokens write consecutive
// words of a page slab, so tokens that fill a page in order are stored as
// contiguous runs.
// E2M1 code of v (nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 by magnitude; a tie
// goes to the code with mantissa bit 0; 6 and above saturate; the sign bit
// only on nonzero codes).  Each comparison is exact, and the strict / non-
// strict choice at each midpoint is the tie rule.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.0f);
  return m | ((v < 0.0f && m != 0u) ? 8u : 0u);
}

// E2M1 codes of y0 / s and y1 / s in byte SEL of `old` (y0 in the low
// nibble) by gfx950's conversion instruction, whose rounding is the rule
// above (nearest, ties to mantissa bit 0, saturating at 6; checked on the
// device against it at every tie) except that it keeps the sign of a zero,
// which clear_negative_zeros then drops.  s = 2^X must be a normal float.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, float y0, float y1, float s) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, s, SEL);
}
// Eight E2M1 codes of a word with a zero magnitude (-0, code 8) made +0.
__device__ __forceinline__ uint32_t clear_negative_zeros(uint32_t w) {
  const uint32_t keep = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;   // bit 3 of nonzero codes
  return (w & 0x77777777u) | (w & keep);
}

// The asymmetric quantizer of one vector (or group), shared by both append
// kernels so that their codes and sidecars agree bit for bit.  From the range
// [mn, mx] of the (normalised) elements: zero point mn and scale
// (mx - mn) / top, both rounded to fp16, and the reciprocal of the rounded
// scale (0 for a zero scale).  meta packs the fp16 scale (low half) and zero
// point (high half).
struct QParams {
  float zf, inv;
  uint32_t meta;
};
template <int BITS>
__device__ __forceinline__ QParams tok_params(float mn, float mx) {
  constexpr float kTop = BITS == 4 ? 15.0f : 255.0f;
  const float zero_f = mn + 0.0f;
  const float range = (mx - mn) + 0.0f;
  const float step = range / kTop;
  const _Float16 sh = static_cast<_Float16>(step);
  const _Float16 zh = static_cast<_Float16>(zero_f);
  const float sf = static_cast<float>(sh);
  QParams q;
  q.zf = static_cast<float>(zh);
  q.inv = (sf == 0.0f) ? 0.0f : 1.0f / sf;
  q.meta = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, sh)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, zh)) << 16);
  return q;
}

// Code of one element: (y - zero) * inv, then round-half-even and clamp to
// [0, top].  Adding 2^23 rounds to an integer in the current (nearest-even)
// mode for any value in [0, 2^23); the clamp in that biased domain equals
// clamping the rounded value; the code is then the low 4 (8) bits of the
// float.  A power-of-two normalisation (b = 16, 64) is exact, so it is folded
// into the subtraction: fma(x, s, -zero) rounds x*s - zero once, which is the
// rounding of (x*s) - zero.  (Only a product below 2^-126 can lose bits; that
// is far below half an ulp of any nonzero fp16 zero point, and with a zero
// zero point both forms are the rounded product.)  Otherwise x is already the
// normalised y.
template <bool EXACT_NORM>
__device__ __forceinline__ float tok_scaled(float x, float sb, float zf, float inv) {
  const float d = EXACT_NORM ? __builtin_fmaf(x, sb, -zf) : x - zf;
  return d * inv;
}
template <int BITS, bool EXACT_NORM>
__device__ __forceinline__ uint32_t tok_code(float x, float sb, float zf, float inv) {
  constexpr float kTop = BITS == 4 ? 15.0f : 255.0f;
  const float q = tok_scaled<EXACT_NORM>(x, sb, zf, inv);
  return f2u(__builtin_amdgcn_fmed3f(q + 8388608.0f, 8388608.0f, 8388608.0f + kTop));
}

// Squared reconstruction error of elements x[k0 .. k0 + n) under the 4-bit
// quantizer (zf, inv) with scale sf (as a positive fp32), measured on the
// integer grid 2^-ks: the code of tok_code, decoded as code * sf + zf (the
// product is exact, so one fma rounds like the add), the error y - decoded
// rounded once (with a power-of-two normalisation folded in, fma(x, sb, -dec)
// is exact(x * sb) - dec rounded once: equal to rounding y - dec, since a
// nonzero decoded value is a multiple of 2^-24 and a product that could lose
// bits is below 2^-126), scaled by 2^ks, rounded to an integer and squared;
// the squares are summed exactly in 64 bits, so the lanes' partial sums
// combine in any order.  The criterion of the scale search and of the hybrid
// mode.
template <bool EXACT_NORM>
__device__ __forceinline__ int64_t grid_sse(const float* x, int k0, int n, float sb, float zf, float inv,
                                            float sf, int ks) {
  int64_t acc = 0;
  for (int k = k0; k < k0 + n; ++k) {
    const float cf = u2f(tok_code<4, EXACT_NORM>(x[k], sb, zf, inv)) - 8388608.0f;   // the code, exact
    const float dec = __builtin_fmaf(cf, sf, zf);
    const float err = EXACT_NORM ? __builtin_fmaf(x[k], sb, -dec) : x[k] - dec;
    const int32_t e = static_cast<int32_t>(__builtin_rintf(ldexpf(err, ks)));
    acc += static_cast<int64_t>(e) * e;
  }
  return acc;
}

// The grid exponent ks = 20 - ex with amax < 2^ex: every error stays below
// 2^21 grid steps.
__device__ __forceinline__ int grid_exponent(float amax) {
  int ex = 0;
  frexpf(amax, &ex);
  return 20 - ex;
}

// QM: the quantizer mode (kQuantPlain, kQuantKeySearch: the key vectors of
// the token-wise INT4 pool take the scale search; kQuantHybrid: every group
// of the grouped INT4 pool picks its symmetric or asymmetric form).  The two
// searching modes hold their candidates' error sums beside the unit's 64
// elements per lane, so they are built for 2 waves per SIMD (256 VGPRs)
// rather than 4.
template <int D, int BLK, bool BF16, int BITS, int GS, bool MX, int QM = kQuantPlain>
__global__ __launch_bounds__(kAppendThreads) __attribute__((amdgpu_waves_per_eu(QM == kQuantPlain ? 4 : 2)))
void append_quant_kernel(AppendArgs a) {
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit codes");
  static_assert(GS == 0 || (BITS == 4 && (GS == 32 || GS == 64) && GS <= D), "groups of 32 or 64 channels, 4-bit");
  static_assert(!MX || (BITS == 4 && GS == 32), "MXFP4: 4-bit codes in blocks of 32");
  static_assert(QM == kQuantPlain || (QM == kQuantKeySearch && BITS == 4 && GS == 0 && !MX) ||
                    (QM == kQuantHybrid && BITS == 4 && GS != 0 && !MX),
                "scale search: token-wise INT4; hybrid: grouped INT4");
  constexpr int kLPV = D / kLaneElems;   // lanes per vector
  constexpr int kTok = 64 / kLPV;        // tokens per unit
  constexpr int kChunks = D / 8;         // 16-byte pieces per row
  constexpr int kRowBytes = 2 * D;
  constexpr int kCodeBytes = D * BITS / 8;             // one vector's codes
  constexpr int kNG = GS ? D / GS : 1;                 // scale/zero pairs per vector
  constexpr int kGL = GS ? kLaneElems / GS : 1;        // of them held by one lane
  constexpr int kGE = kLaneElems / kGL;                // elements of a lane's group
  constexpr int kSideBytes = MX ? kNG : 4 * kNG;       // sidecar bytes per vector
  constexpr int kSlab = kPage * (2 * kCodeBytes + 2 * kSideBytes);
  constexpr int kWords = kLaneElems * BITS / 32;       // code words per lane
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[kAppendThreads / 64][kTok * kRowBytes];
  uint8_t* lds = lds_all[threadIdx.x >> 6];
  const int lane = threadIdx.x & 63;
  const int r = lane / kLPV, hf = lane % kLPV;
  const uint32_t hkv = static_cast<uint32_t>(a.num_kv_heads);
  const uint32_t tiles = (static_cast<uint32_t>(a.num_tokens) + kTok - 1) / kTok;
  // Unit u = (tile * hkv + head) * 2 + kind; wave w takes u = w, w + S, ...
  // with S = 4 * gridDim.x even, so its kind never changes and (tile, head)
  // advance by a fixed step (all wave-uniform scalar arithmetic).
  const uint32_t w0 = blockIdx.x * (kAppendThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kind = static_cast<int>(w0 & 1u);
  const uint16_t* in = kind ? a.v : a.k;
  const uint32_t half_stride = gridDim.x * (kAppendThreads / 128);
  const uint32_t st_t = half_stride / hkv, st_h = half_stride - st_t * hkv;
  struct Unit { uint32_t tile, h; };
  Unit cur{(w0 >> 1) / hkv, (w0 >> 1) % hkv};
  auto advance = [&](Unit x) {
    x.h += st_h;
    x.tile += st_t;
    if (x.h >= hkv) {
      x.h -= hkv;
      ++x.tile;
    }
    return x;
  };

  // LDS image of a unit: row rr holds kChunks 16-byte slots; chunk c of the
  // row sits in slot swz(rr, c), a permutation of the row chosen so that the
  // reads below (any 16 consecutive lanes) fall in distinct banks.
  auto swz = [](int rr, int c) {
    if constexpr (kChunks == 16) return c ^ ((2 * rr) & 15) ^ (c >> 3);
    else return c ^ ((rr ^ (rr >> 3)) & 7);
  };
  auto unswz = [](int rr, int sl) {   // the chunk held by slot sl of row rr
    if constexpr (kChunks == 16) {
      const int u = sl ^ ((2 * rr) & 15);
      return u ^ (u >> 3);
    } else {
      return sl ^ ((rr ^ (rr >> 3)) & 7);
    }
  };
  // Load m of lane L fills LDS bytes [1024 m + 16 L, +16): row
  // rr = m * kRowsPerLoad + L / kChunks, slot L % kChunks.  One buffer
  // descriptor spans the unit's rows that exist: rows past the last token
  // read as zeros.
  constexpr int kRowsPerLoad = 64 / kChunks;
  const uint32_t row_bytes = static_cast<uint32_t>(a.token_stride) * 2u;
  uint32_t voff[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int rr = m * kRowsPerLoad + lane / kChunks;
    voff[m] = static_cast<uint32_t>(lane / kChunks) * row_bytes + unswz(rr, lane % kChunks) * 16u;
  }
  auto request = [&](Unit w) {
    const int t0 = static_cast<int>(w.tile) * kTok;
    const uint16_t* src = in + static_cast<int64_t>(t0) * a.token_stride + w.h * D;
    const int rows = min(kTok, a.num_tokens - t0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, static_cast<int>(static_cast<uint32_t>(rows) * row_bytes));
#pragma unroll
    for (int m = 0; m < 8; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + 1024 * m), 16, voff[m],
          static_cast<int>(m * kRowsPerLoad * row_bytes), 0, kStreamOnce);
    return t0 + r < a.num_tokens ? a.slot_mapping[t0 + r] : -1;
  };

  // Codes and sidecar of one unit, written into the slot's page (tokens past
  // the end have slot -1).  A unit is stored one iteration after it is
  // computed, so that the wait for the next rows never waits for fresh stores.
  struct Pending { uint32_t words[kWords]; uint32_t meta[kGL]; int32_t slot; uint32_t h; };
  auto store = [&](const Pending& q) {
    if (q.slot < 0 || static_cast<int64_t>(q.slot) >= static_cast<int64_t>(a.num_pages) * kPage) return;
    const int page = q.slot / kPage, off = q.slot % kPage;
    uint8_t* slab = a.pool + (static_cast<int64_t>(page) * hkv + q.h) * kSlab;
    if (kind == 0) {   // K: token-major, the lane's 64 channels contiguous
      u32x4* dst = reinterpret_cast<u32x4*>(slab + off * kCodeBytes + hf * (kWords * 4));
#pragma unroll
      for (int i = 0; i < kWords / 4; ++i)
        dst[i] = u32x4{q.words[4 * i], q.words[4 * i + 1], q.words[4 * i + 2], q.words[4 * i + 3]};
    } else if constexpr (BITS == 4) {   // V: word n*P + t of token t (8 channels)
      uint32_t* vw = reinterpret_cast<uint32_t*>(slab + kPage * kCodeBytes);
#pragma unroll
      for (int m = 0; m < 8; ++m) vw[(hf * 8 + m) * kPage + off] = q.words[m];
    } else {           // V: words (n*P + t)*2 + {0, 1} = channels 8n..8n+7 of token t
      u32x2* vw = reinterpret_cast<u32x2*>(slab + kPage * kCodeBytes);
#pragma unroll
      for (int m = 0; m < 8; ++m) vw[(hf * 8 + m) * kPage + off] = u32x2{q.words[2 * m], q.words[2 * m + 1]};
    }
    uint8_t* meta = slab + 2 * kPage * kCodeBytes + kind * kPage * kSideBytes;
    if constexpr (MX) {   // E8M0 bytes of this lane's blocks (2hf, 2hf+1)
      *reinterpret_cast<uint16_t*>(meta + off * kSideBytes + hf * kGL) =
          static_cast<uint16_t>(q.meta[0] | (q.meta[1] << 8));
    } else if constexpr (GS == 0) {
      if (hf == 0) *reinterpret_cast<uint32_t*>(meta + off * 4) = q.meta[0];
    } else if constexpr (kGL == 1) {   // group hf of token off
      *reinterpret_cast<uint32_t*>(meta + (off * kNG + hf) * 4) = q.meta[0];
    } else {                           // groups 2hf, 2hf+1
      *reinterpret_cast<u32x2*>(meta + (off * kNG + hf * kGL) * 4) = u32x2{q.meta[0], q.meta[1]};
    }
  };

  int32_t slot_nxt = -1;
  if (cur.tile < tiles) slot_nxt = request(cur);
  Pending pend;
  bool have_pend = false;
  for (; cur.tile < tiles; cur = advance(cur)) {
    const int32_t slot = slot_nxt;
    // the unit's rows have landed in LDS (the direct loads count in vmcnt,
    // which the compiler does not track for them); the stores waited for
    // here were issued one whole unit earlier
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (have_pend) store(pend);
    float x[kLaneElems];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int c = hf * 8 + m;
      widen8<BF16>(*reinterpret_cast<const u32x4*>(lds + r * kRowBytes + swz(r, c) * 16), x + 8 * m);
    }
    // the reads above are complete before the next unit's rows overwrite them
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const Unit nxt = advance(cur);
    if (nxt.tile < tiles) slot_nxt = request(nxt);

    // block Hadamard butterfly, stages h = 1, 2, ..., BLK/2 ascending
    if constexpr (BLK > 0) {
      constexpr int kIn = BLK < kLaneElems ? BLK : kLaneElems;
#pragma unroll
      for (int hh = 1; hh < kIn; hh *= 2)
#pragma unroll
        for (int i = 0; i < kLaneElems; i += 2 * hh)
#pragma unroll
          for (int k = i; k < i + hh; ++k) {
            const float p = x[k], q = x[k + hh];
            x[k] = p + q;
            x[k + hh] = p - q;
          }
      if constexpr (BLK == 128) {
        // last stage h = 64 pairs channel k (lane hf = 0) with k + 64 (hf = 1):
        // lower half keeps own + partner, upper half partner - own; the
        // product by +-1 is exact, so the fma rounds once like an add/sub.
        const float sgn = hf ? -1.0f : 1.0f;
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) {
          const float p = dpp_f<kDppXor1>(x[k]);
          x[k] = __builtin_fmaf(sgn, x[k], p);
        }
      }
    }

    // range of each group (the whole vector when GS = 0).  Rounding is
    // monotone, so min/max of the unscaled butterfly output, scaled once,
    // equal min/max of the scaled elements.
    float mn[kGL], mx[kGL];
#pragma unroll
    for (int gl = 0; gl < kGL; ++gl) {
      mn[gl] = mx[gl] = x[gl * kGE];
#pragma unroll
      for (int k = gl * kGE + 1; k < (gl + 1) * kGE; ++k) {
        mn[gl] = fminf(mn[gl], x[k]);
        mx[gl] = fmaxf(mx[gl], x[k]);
      }
    }
    if constexpr (GS == 0 && kLPV == 2) {
      mn[0] = fminf(mn[0], dpp_f<kDppXor1>(mn[0]));
      mx[0] = fmaxf(mx[0], dpp_f<kDppXor1>(mx[0]));
    }
    // A power-of-two normalisation (b = 16, 64) is exact and folded into the
    // code's subtraction (tok_code); b = 32, 128 scale the elements here.
    constexpr bool kExactNorm = BLK == 16 || BLK == 64;
    const float sb = BLK > 0 ? block_norm(BLK) : 1.0f;
    if constexpr (BLK > 0) {
#pragma unroll
      for (int gl = 0; gl < kGL; ++gl) {
        mn[gl] = mn[gl] * sb;
        mx[gl] = mx[gl] * sb;
      }
      if constexpr (!kExactNorm) {
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) x[k] = x[k] * sb;
      }
    }

    // fp16 zero and scale, reciprocal (0 for a zero scale), per group; for
    // MXFP4 the shared exponent X = floor(log2 max|y|) - 2 of each block
    float zf[kGL], inv[kGL];
    int xe[kGL];
#pragma unroll
    for (int gl = 0; gl < kGL; ++gl) {
      if constexpr (MX) {
        const float amax = fmaxf(fabsf(mn[gl]), fabsf(mx[gl]));
        int e = 0;
        frexpf(amax, &e);                      // amax in [2^(e-1), 2^e)
        int x = amax > 0.0f ? e - 3 : -127;
        x = x < -127 ? -127 : (x > 127 ? 127 : x);
        xe[gl] = x;
        pend.meta[gl] = static_cast<uint32_t>(x + 127);
        zf[gl] = inv[gl] = 0.0f;
        continue;
      }
      const QParams qp = tok_params<BITS>(mn[gl], mx[gl]);
      zf[gl] = qp.zf;
      inv[gl] = qp.inv;
      pend.meta[gl] = qp.meta;
      if constexpr (QM == kQuantHybrid) {
        // The symmetric candidate: scale fp16(amax / 7), zero -8 * scale
        // (exact in fp16), so that 0 is the level of code 8; it is kept when
        // its grid error is not larger than the asymmetric one's (a group of
        // zeros, a zero symmetric scale or a zero point beyond fp16 stay
        // asymmetric), and marked by the sign bit of the stored scale.
        const float amax = fmaxf(fabsf(mn[gl]), fabsf(mx[gl]));
        const _Float16 ss = static_cast<_Float16>(amax / 7.0f);
        const float sfs = static_cast<float>(ss);
        const float zs = -8.0f * sfs;
        if (amax > 0.0f && sfs != 0.0f && fabsf(zs) <= 65504.0f) {
          const float inv_s = 1.0f / sfs;
          const int ks = grid_exponent(amax);
          const float sf_a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qp.meta & 0xFFFFu)));
          const int64_t e_s = grid_sse<kExactNorm>(x, gl * kGE, kGE, sb, zs, inv_s, sfs, ks);
          const int64_t e_a = grid_sse<kExactNorm>(x, gl * kGE, kGE, sb, qp.zf, qp.inv, sf_a, ks);
          if (e_s <= e_a) {
            zf[gl] = zs;
            inv[gl] = inv_s;
            pend.meta[gl] = (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ss)) | 0x8000u) |
                            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(zs))) << 16);
          }
        }
      }
    }
    if constexpr (QM == kQuantKeySearch) {
      if (kind == 0) {
        // Keys: the range [mn, mx] shrunk toward zero by alpha_j = (16 - j)
        // / 16, j = 0 .. 7; the candidate with the smallest grid error over
        // the whole vector (the two lanes' partial sums added) wins, the
        // smaller j on a tie.  Candidate 0 is the plain quantizer.
        const float amax = fmaxf(fabsf(mn[0]), fabsf(mx[0]));
        const int ks = grid_exponent(amax);
        int64_t best = 0;
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
          const float alpha = static_cast<float>(16 - j) / 16.0f;
          const QParams qc = tok_params<4>(mn[0] * alpha, mx[0] * alpha);
          const float sfc = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qc.meta & 0xFFFFu)));
          int64_t e = grid_sse<kExactNorm>(x, 0, kLaneElems, sb, qc.zf, qc.inv, sfc, ks);
          if constexpr (kLPV == 2) {
            const uint32_t lo = static_cast<uint32_t>(e), hi = static_cast<uint32_t>(e >> 32);
            e += static_cast<int64_t>((static_cast<uint64_t>(dpp_u<kDppXor1>(hi)) << 32) | dpp_u<kDppXor1>(lo));
          }
          if (j == 0 || e < best) {
            best = e;
            zf[0] = qc.zf;
            inv[0] = qc.inv;
            pend.meta[0] = qc.meta;
          }
        }
      }
    }

    // codes (tok_code; MXFP4: E2M1 of y / 2^X)
    constexpr int kPer = 32 / BITS;   // codes per word
    auto code = [&](int k) -> uint32_t {
      constexpr int gl_div = kGE;
      const int gl = k / gl_div;
      if constexpr (MX) {   // y / 2^X (exact scaling), then E2M1
        // (b = 32, 128 scaled x in place above; b = 16, 64 scale exactly here)
        const float y = kExactNorm ? x[k] * sb : x[k];
        return e2m1_code(ldexpf(y, -xe[gl]));
      }
      return tok_code<BITS, kExactNorm>(x[k], sb, zf[gl], inv[gl]);
    };
    // MXFP4 codes through the conversion instruction, two per instruction,
    // when every block of the lane has X > -124: then a code that is not
    // zero comes from an element of at least 2^-125 (a normal float), and the
    // scale 2^X is normal.  (Blocks of smaller elements, all-zero ones
    // included, keep the comparisons: the instruction's handling of subnormal
    // inputs is not relied on.)
    [[maybe_unused]] bool mx_hw = false;
    [[maybe_unused]] float mx_s[kGL];
    if constexpr (MX) {
      mx_hw = true;
#pragma unroll
      for (int gl = 0; gl < kGL; ++gl) {
        mx_hw = mx_hw && xe[gl] > -124;
        mx_s[gl] = ldexpf(1.0f, xe[gl] > -124 ? xe[gl] : 0);
      }
    }
    auto mx_y = [&](int k) { return kExactNorm ? x[k] * sb : x[k]; };
    // the unit's results are stored at the start of the next iteration
    if (MX && mx_hw && kind == 0) {   // K: word m holds elements 8m .. 8m+7 of one block
#pragma unroll
      for (int m = 0; m < kWords; ++m) {
        const float sc = mx_s[(8 * m) / kGE];
        uint32_t w = e2m1_pair<0>(0u, mx_y(8 * m), mx_y(8 * m + 1), sc);
        w = e2m1_pair<1>(w, mx_y(8 * m + 2), mx_y(8 * m + 3), sc);
        w = e2m1_pair<2>(w, mx_y(8 * m + 4), mx_y(8 * m + 5), sc);
        w = e2m1_pair<3>(w, mx_y(8 * m + 6), mx_y(8 * m + 7), sc);
        pend.words[m] = clear_negative_zeros(w);
      }
    } else if (MX && (GS == 0 || kind == 0)) {   // MXFP4 K without the conversion instruction
#pragma unroll
      for (int m = 0; m < kWords; ++m) {
        uint32_t c[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) c[i] = code(kPer * m + i);
        pend.words[m] = pack8_nibbles(c);
      }
    } else if (GS == 0 || kind == 0) {   // consecutive channels: K, or V of the token-wise pools
      // tok_code's codes, rounded by v_cvt_pk_u8_f32 instead: it rounds to
      // nearest even, clamps to [0, 255] and writes one byte of a word.
      // 4-bit values are clamped to [0, 15] first (on that range clamping
      // before rounding gives what clamping after does); the even-numbered
      // codes fill the bytes of one word, the odd ones another, and the two
      // words are joined as nibbles.
      auto qv = [&](int k) {
        const int gl = k / kGE;
        const float q = tok_scaled<kExactNorm>(x[k], sb, zf[gl], inv[gl]);
        return BITS == 4 ? __builtin_amdgcn_fmed3f(q, 0.0f, 15.0f) : q;
      };
#pragma unroll
      for (int m = 0; m < kWords; ++m) {
        const int k0 = kPer * m;
        if constexpr (BITS == 4) {
          uint32_t ev = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0), 0, 0u);
          ev = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 2), 1, ev);
          ev = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 4), 2, ev);
          ev = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 6), 3, ev);
          uint32_t od = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 1), 0, 0u);
          od = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 3), 1, od);
          od = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 5), 2, od);
          od = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 7), 3, od);
          pend.words[m] = ev | (od << 4);
        } else {
          uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0), 0, 0u);
          w = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 1), 1, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 2), 2, w);
          pend.words[m] = __builtin_amdgcn_cvt_pk_u8_f32(qv(k0 + 3), 3, w);
        }
      }
    } else if constexpr (GS != 0 && kLPV == 1) {
      // grouped V, D = 64: word n holds channels n + 8j, j = 0..7
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = code(m + 8 * j);
        pend.words[m] = pack8_nibbles(c);
      }
    } else if constexpr (GS != 0) {
      // grouped V, D = 128: word n holds channels n + 16j, j = 0..7; this
      // lane has j = 4hf .. 4hf+3 (its channels n + 16j'), i.e. 16 bits of
      // every word, and stores words 8hf .. 8hf+7 after swapping the other
      // half-words with its partner lane
      uint32_t hw[16];
      if (MX && mx_hw) {   // (channels n2, n2 + 16 in block 0 of the lane, n2 + 32, n2 + 48 in block 1)
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) {
          const uint32_t w = e2m1_pair<0>(0u, mx_y(n2), mx_y(n2 + 16), mx_s[0]);
          hw[n2] = clear_negative_zeros(e2m1_pair<1>(w, mx_y(n2 + 32), mx_y(n2 + 48), mx_s[kGL - 1]));
        }
      } else {
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) {
          const uint32_t t0 = __builtin_amdgcn_perm(code(n2 + 16), code(n2), 0x0c0c0400u);        // c0 | c1 << 8
          const uint32_t t1 = __builtin_amdgcn_perm(code(n2 + 48), code(n2 + 32), 0x0c0c0400u);
          const uint32_t b0 = (t0 | (t0 >> 4)) & 0xFFu;                                           // c0 | c1 << 4
          const uint32_t b1 = (t1 | (t1 >> 4)) & 0xFFu;
          hw[n2] = b0 | (b1 << 8);
        }
      }
      uint32_t send[4], recv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        send[i] = hf ? (hw[2 * i] | (hw[2 * i + 1] << 16)) : (hw[8 + 2 * i] | (hw[9 + 2 * i] << 16));
        recv[i] = dpp_u<kDppXor1>(send[i]);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t other = (m & 1) ? (recv[m >> 1] >> 16) : (recv[m >> 1] & 0xFFFFu);
        pend.words[m] = hf ? (other | (hw[8 + m] << 16)) : (hw[m] | (other << 16));
      }
    }
    pend.slot = slot;
    pend.h = cur.h;
    have_pend = true;
  }
  if (have_pend) store(pend);
}

// Few tokens (appends of one token per sequence at decode time): a vector
// is spread over D/8 lanes, eight consecutive channels per lane, loaded
// straight from memory.  The butterfly's first three stages run inside the
// lane and the rest across lanes (DPP), and the range is a reduction across
// the vector's lanes, so each lane's serial work is that of 8 elements
// instead of 64: such an append is bound by that latency, not by memory.
// The butterfly order and the quantizer steps are the tile kernel's, so the
// codes and sidecars are the same bit for bit.  Token-wise INT4 and INT8.
template <int D, int BLK, bool BF16, int BITS>
__global__ __launch_bounds__(256) void append_small_kernel(AppendArgs a) {
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit codes");
  constexpr int kLPV = D / 8;          // lanes per vector
  constexpr int kVPW = 64 / kLPV;      // vectors per wave
  constexpr int kCodeBytes = D * BITS / 8;
  constexpr int kSlab = kPage * (2 * kCodeBytes + 8);
  const int lane = threadIdx.x & 63;
  const int c = lane % kLPV;           // channels [8c, 8c + 8)
  // vector (token, KV head, K or V), K/V fastest; the kLPV lanes of a vector
  // are all live or all not, so the cross-lane steps read live lanes only
  const int64_t vec = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kVPW + lane / kLPV;
  if (vec >= static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * 2) return;
  const int kind = static_cast<int>(vec & 1);
  const int64_t th = vec >> 1;
  const int h = static_cast<int>(th % a.num_kv_heads);
  const int64_t t = th / a.num_kv_heads;
  const uint16_t* src = (kind ? a.v : a.k) + t * a.token_stride + static_cast<int64_t>(h) * D + 8 * c;
  const int32_t slot = a.slot_mapping[t];
  float x[8];
  widen8<BF16>(*reinterpret_cast<const u32x4*>(src), x);
  if constexpr (BLK > 0) fwht_row<8>(x, BLK, c);   // stages 1, 2, ..., BLK/2
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    mn = fminf(mn, x[k]);
    mx = fmaxf(mx, x[k]);
  }
  mn = fminf(mn, dpp_xor<1>(mn));
  mx = fmaxf(mx, dpp_xor<1>(mx));
  mn = fminf(mn, dpp_xor<2>(mn));
  mx = fmaxf(mx, dpp_xor<2>(mx));
  mn = fminf(mn, dpp_xor<4>(mn));
  mx = fmaxf(mx, dpp_xor<4>(mx));
  if constexpr (kLPV == 16) {
    mn = fminf(mn, dpp_xor<8>(mn));
    mx = fmaxf(mx, dpp_xor<8>(mx));
  }
  constexpr bool kExactNorm = BLK == 16 || BLK == 64;
  const float sb = BLK > 0 ? block_norm(BLK) : 1.0f;
  if constexpr (BLK > 0) {
    mn = mn * sb;
    mx = mx * sb;
    if constexpr (!kExactNorm) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = x[k] * sb;
    }
  }
  const QParams qp = tok_params<BITS>(mn, mx);
  uint32_t cd[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) cd[k] = tok_code<BITS, kExactNorm>(x[k], sb, qp.zf, qp.inv);

  if (slot < 0 || static_cast<int64_t>(slot) >= static_cast<int64_t>(a.num_pages) * kPage) return;
  const int page = slot / kPage, off = slot % kPage;
  uint8_t* slab = a.pool + (static_cast<int64_t>(page) * a.num_kv_heads + h) * kSlab;
  if constexpr (BITS == 4) {   // K: token-major; V: word c*P + t holds channels 8c .. 8c+7
    const uint32_t w = pack8_nibbles(cd);
    if (kind == 0) *reinterpret_cast<uint32_t*>(slab + off * kCodeBytes + 4 * c) = w;
    else reinterpret_cast<uint32_t*>(slab + kPage * kCodeBytes)[c * kPage + off] = w;
  } else {                     // the same with two words (8 bytes) per 8 channels
    const uint32_t w0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(cd[3], cd[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(cd[1], cd[0], 0x0c0c0400u), 0x05040100u);
    const uint32_t w1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(cd[7], cd[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(cd[5], cd[4], 0x0c0c0400u), 0x05040100u);
    if (kind == 0) *reinterpret_cast<u32x2*>(slab + off * kCodeBytes + 8 * c) = u32x2{w0, w1};
    else reinterpret_cast<u32x2*>(slab + kPage * kCodeBytes)[c * kPage + off] = u32x2{w0, w1};
  }
  if (c == 0) *reinterpret_cast<uint32_t*>(slab + 2 * kPage * kCodeBytes + kind * kPage * 4 + off * 4) = qp.meta;
}

// bf16 baseline: one thread per (token, head, 8-channel group).
template <bool BF16>
__global__ __launch_bounds__(256) void append_bf16_kernel(AppendArgs a) {
  const int d = a.head_dim, groups = d / 8, hkv = a.num_kv_heads;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * hkv * groups;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % groups);
  const int64_t r = idx / groups;
  const int64_t t = r / hkv;
  const int h = static_cast<int>(r - t * hkv);
  const int32_t slot = a.slot_mapping[t];
  if (slot < 0 || static_cast<int64_t>(slot) >= static_cast<int64_t>(a.num_pages) * kPage) return;
  const int page = slot / kPage, off = slot % kPage;
  const int64_t in_off = t * a.token_stride + static_cast<int64_t>(h) * d + n * 8;
  u32x4 kw = *reinterpret_cast<const u32x4*>(a.k + in_off);
  u32x4 vw = *reinterpret_cast<const u32x4*>(a.v + in_off);
  if constexpr (!BF16) {
    auto cvt = [](u32x4 w) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xFFFFu)));
        const float hi = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
        const uint16_t blo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
        const uint16_t bhi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
        o[i] = static_cast<uint32_t>(blo) | (static_cast<uint32_t>(bhi) << 16);
      }
      return o;
    };
    kw = cvt(kw);
    vw = cvt(vw);
  }
  uint16_t* slab = reinterpret_cast<uint16_t*>(a.pool + (static_cast<int64_t>(page) * hkv + h) * (4 * kPage * d));
  *reinterpret_cast<u32x4*>(slab + off * d + n * 8) = kw;
  const int g = off / 4, i = off % 4;
  uint16_t* vb = slab + kPage * d + ((n * (kPage / 4) + g) * 8) * 4 + i;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const uint32_t w = vw[jj / 2];
    vb[jj * 4] = static_cast<uint16_t>((jj & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
}

// Appends of at most this many tokens (decode steps) use the few-token kernel.
constexpr int kSmallTokens = 1024;

template <int D, int BLK, int BITS, int GS, bool MX = false, int QM = kQuantPlain>
hipError_t launch_quant_d(const AppendArgs& a, hipStream_t s) {
  if constexpr (GS == 0 && !MX && QM == kQuantPlain) {
    if (a.num_tokens <= kSmallTokens) {
      constexpr int kVecPerBlock = 4 * (64 / (D / 8));
      const int64_t nvec = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * 2;
      const dim3 grid(static_cast<unsigned>((nvec + kVecPerBlock - 1) / kVecPerBlock));
      if (a.in_bf16)
        append_small_kernel<D, BLK, true, BITS><<<grid, 256, 0, s>>>(a);
      else
        append_small_kernel<D, BLK, false, BITS><<<grid, 256, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  constexpr int kTok = D == 128 ? 32 : 64;
  const int64_t units = (static_cast<int64_t>(a.num_tokens) + kTok - 1) / kTok * a.num_kv_heads * 2;
  const int64_t blocks = (units + kAppendThreads / 64 - 1) / (kAppendThreads / 64);
  const dim3 grid(static_cast<unsigned>(blocks < kResidentBlocks ? blocks : kResidentBlocks));
  if (a.in_bf16)
    append_quant_kernel<D, BLK, true, BITS, GS, MX, QM><<<grid, kAppendThreads, 0, s>>>(a);
  else
    append_quant_kernel<D, BLK, false, BITS, GS, MX, QM><<<grid, kAppendThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, int BITS, int GS, bool MX = false, int QM = kQuantPlain>
hipError_t launch_quant_block(const AppendArgs& a, hipStream_t s) {
  switch (a.block) {
    case 0: return launch_quant_d<D, 0, BITS, GS, MX, QM>(a, s);
    case 16: return launch_quant_d<D, 16, BITS, GS, MX, QM>(a, s);
    case 32: return launch_quant_d<D, 32, BITS, GS, MX, QM>(a, s);
    case 64: return launch_quant_d<D, 64, BITS, GS, MX, QM>(a, s);
    case 128:
      if constexpr (D == 128) return launch_quant_d<D, 128, BITS, GS, MX, QM>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append_int4(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.mode == kQuantKeySearch)
    return a.head_dim == 128 ? launch_quant_block<128, 4, 0, false, kQuantKeySearch>(a, s)
                             : launch_quant_block<64, 4, 0, false, kQuantKeySearch>(a, s);
  return a.head_dim == 128 ? launch_quant_block<128, 4, 0>(a, s) : launch_quant_block<64, 4, 0>(a, s);
}

hipError_t launch_append_int4g(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.mode == kQuantHybrid) {
    if (a.head_dim == 128)
      return a.group == 32 ? launch_quant_block<128, 4, 32, false, kQuantHybrid>(a, s)
                           : launch_quant_block<128, 4, 64, false, kQuantHybrid>(a, s);
    return a.group == 32 ? launch_quant_block<64, 4, 32, false, kQuantHybrid>(a, s)
                         : launch_quant_block<64, 4, 64, false, kQuantHybrid>(a, s);
  }
  if (a.head_dim == 128)
    return a.group == 32 ? launch_quant_block<128, 4, 32>(a, s) : launch_quant_block<128, 4, 64>(a, s);
  return a.group == 32 ? launch_quant_block<64, 4, 32>(a, s) : launch_quant_block<64, 4, 64>(a, s);
}

hipError_t launch_append_mxfp4(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  return a.head_dim == 128 ? launch_quant_block<128, 4, 32, true>(a, s) : launch_quant_block<64, 4, 32, true>(a, s);
}

hipError_t launch_append_int8(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  return a.head_dim == 128 ? launch_quant_block<128, 8, 0>(a, s) : launch_quant_block<64, 8, 0>(a, s);
}

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * (a.head_dim / 8);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (a.in_bf16)
    append_bf16_kernel<true><<<grid, 256, 0, s>>>(a);
  else
    append_bf16_kernel<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq

// Read path over the MXFP4 cache: split-K paged decode attention whose QK
// product runs on gfx950's block-scaled FP4 matrix instruction
// ("BitDecoding-FP4", Abstract: native FP4 KV decoding, the query heads of a
// GQA group stacked into one product per page; the cache holds E2M1 codes
// with one E8M0 power-of-two scale per 32 channels, the OCP microscaling
// block format).
//
// Work split, page streaming, online softmax and merge follow the INT4
// decode kernel.  Per page and per group of four query heads:
//   QK:  v_mfma_scale_f32_16x16x128_f8f6f4 with B = the page's K codes as
//        they are stored (E2M1, 32 channels per lane) and their E8M0 block
//        scales applied by the hardware, and A = the rotated query as eight
//        FP8 (E4M3) limbs: limb L of each element is the E4M3 rounding of
//        what limbs 0..L-1 left, at 2^-4L of the block's scale, so the eight
//        rows of a head sum to the query within 2^-32 of its block maximum.
//        Limbs 0-3 and 4-7 are the rows of two products that accumulate into
//        the same tile; each lane then adds its head's four rows.
//   PV:  the V scales run along channels (one per token and 32 channels), a
//        direction the instruction's per-column scales cannot carry, so PV
//        runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16): the weights
//        w = p * 2^(E-128) of each 32-channel block go through LDS as three
//        bf16 limbs (hi = bf16(w), then what it left, twice: 24 bits), rows
//        of the A operand; the V codes, two pages' nibbles of one channel
//        paired in a byte, become exact bf16 (twice the E2M1 value) by the
//        FP4 conversion instruction.  The V codes are laid out so that each 16-channel output
//        tile lies in one block.
#include "dev_common.hpp"
#include "kvq_internal.hpp"

#include <type_traits>

namespace kvq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = 4;
constexpr int kStep = 4;       // pages per step
constexpr int kD = 128;        // head_dim
constexpr int kBlocks = kD / 32;
constexpr int kLimbs = 8;      // FP8 limbs of the query

template <int NS>
struct alignas(16) MxSmem {
  static constexpr int kGP = 4 * NS;
  union {
    uint8_t qb[kGP][kLimbs][kD];   // FP8 limbs of the rotated query, by channel (prologue)
    // the PV weights of a step (A operand): [wave][set][block][page pair m]
    // [limb][head][token], a dword holding the bf16 limb of pages 2m, 2m+1
    uint32_t wb[kWaves][NS][kBlocks][2][4][4][16];
    struct {
      float acc[kWaves][kGP][kD];
      float m[kWaves][kGP];
      float l[kWaves][kGP];
    } merge;
  } u;
  int32_t qexp[kGP][kBlocks];       // block exponent s0 of limb 0
};

struct MxStep {
  u32x4 kx[kStep];
  u32x4 vx[kStep];
  uint32_t ks[kStep], vs[kStep];   // E8M0 bytes of the token's four blocks
  bool pv[kStep];
  bool all_ok;
};

// Two packed floats as bf16, rounded to nearest even (v_cvt_pk_bf16_f32),
// and back.
__device__ __forceinline__ uint32_t bf16_pair(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{x, y}, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t h) { return u2f(h << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t h) { return u2f(h & 0xFFFF0000u); }

// Twice the two E2M1 codes of byte `sel` of w as bf16 (exact; low nibble
// first), by v_cvt_scalef32_pk_bf16_fp4 at scale 2 (the byte is an immediate
// of the instruction: sel must fold to a constant).
__device__ __forceinline__ bf16x2 e2m1_pair_bf16(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, 3);
  }
}

// BAL: a balanced call (balanced_split_pages), built apart so that the
// planned calls carry none of its code
template <int NS, bool QBF16, bool BAL>
__global__ __launch_bounds__(64 * kWaves) void decode_mxfp4_kernel(DecodeArgs a) {
  constexpr int D = kD;
  constexpr int kSlab = kPage * (D + D / 16);
  constexpr int kNT = D / 16;          // PV tiles
  constexpr int kC = D / 16;           // channels per lane in a row of 16 lanes
  __shared__ MxSmem<NS> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, n = lane & 15, hs = n >> 2, lam = n & 3;
  // work item (split s, sequence b, KV head): KV head fastest, split slowest,
  // last split first (as the INT4 decode)
  const uint32_t wid = blockIdx.x;
  const int kvh = static_cast<int>(wid % a.num_kv_heads);
  const int b = static_cast<int>((wid / a.num_kv_heads) % a.batch);
  // pages per split, and the split: last first, unless the device grew the
  // splits (then the later ones are empty, and first-split-first keeps them
  // from holding the machine before the work starts)
  const int sp = BAL ? balanced_split_pages(a.split_pages, a.seq_lens, a.batch, a.max_seq_len,
                                            a.num_kv_heads)
                     : a.split_pages;
  const int s = BAL && sp != a.split_pages
                    ? static_cast<int>(wid / a.num_kv_heads / a.batch)
                    : a.nsplit - 1 - static_cast<int>(wid / a.num_kv_heads / a.batch);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t hq0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * G;

  // ---- query: wave w < NS rotates heads 4w..4w+3, one per row of 16 lanes ----
  const bool qwave = wave < NS;
  const int qhead = 4 * wave + g;
  uint32_t qraw[kC / 2];
  if (qwave) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(a.q + (hq0 + min(qhead, G - 1)) * D + kC * n);
#pragma unroll
    for (int i = 0; i < 4; ++i) qraw[i] = t[i];
  }
  const int p0 = s * sp;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int npg = (len + kPage - 1) / kPage;
  const int p1 = min(npg, p0 + sp);
  if (p0 >= p1) {
    if (a.nsplit == 1) {
      for (int e = tid; e < G * D; e += 64 * kWaves) a.out[hq0 * D + e] = 0.0f;
    }
    return;
  }
  // a sequence whose pages all lie in one split is finished here (the split
  // merge skips its rows)
  const bool direct = a.nsplit == 1 || (npg - 1) / sp == 0;
  const int span = p1 - p0;
  const int per_wave = ((span + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
  const int pw0 = p0 + wave * per_wave;
  const int pw1 = min(p1, pw0 + per_wave);
  const uint8_t* pool_h = a.pool + static_cast<int64_t>(kvh) * kSlab;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * kSlab;
  // lane offsets in a page slab: K codes of token n, channels [32g, 32g+32);
  // V codes of tokens 4g..4g+3, word n; the token's E8M0 bytes
  const uint32_t k_off = n * (D / 2) + g * 16;
  const uint32_t v_off = kPage * D / 2 + (n * kPage + 4 * g) * 4;
  const uint32_t ks_off = kPage * D + n * kBlocks;
  const uint32_t vs_off = ks_off + kPage * kBlocks;
  // page ids by scalar loads (wave-uniform, inside the row; pages at or past
  // pw1 are dropped where the ids are used), a step ahead of their loads
  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  ConstI32* bt_s = (ConstI32*)bt;   // generic to constant address space
  auto ids4 = [&](int p, int32_t (&id)[kStep]) {
#pragma unroll
    for (int i = 0; i < kStep; ++i) id[i] = bt_s[min(p + i, pw1 - 1)];
  };
  int32_t idA[kStep], idB[kStep];
  ids4(pw0, idA);
  auto load = [&](MxStep& sb, int p, const int32_t (&ids)[kStep]) {
    sb.all_ok = true;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const int id = p + i < pw1 ? ids[i] : -1;
      sb.pv[i] = id >= 0 && id < a.num_pages;
      sb.all_ok = sb.all_ok && sb.pv[i];
      // a page that is not there gets an empty descriptor (its loads return
      // zeros without touching memory)
      const uint8_t* sl = pool_h + static_cast<int64_t>(sb.pv[i] ? id : 0) * page_stride;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(sl, sb.pv[i] ? kSlab : 0);
      sb.kx[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, k_off, 0, kStreamOnce));
      sb.vx[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, v_off, 0, kStreamOnce));
      sb.ks[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, ks_off, 0, kStreamOnce);
      sb.vs[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs_off, 0, kStreamOnce);
    }
  };
  // the first step's page loads go out before the query is waited for (the
  // query was requested first, so its wait leaves them in flight)
  MxStep buf0;
  load(buf0, pw0, idA);
  ids4(pw0 + kStep, idB);
  __builtin_amdgcn_sched_barrier(0);
  float qv[kC];
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    const uint16_t u = qwave ? static_cast<uint16_t>(qraw[k / 2] >> (16 * (k & 1))) : 0;
    const float x = QBF16 ? u2f(static_cast<uint32_t>(u) << 16) : static_cast<float>(__builtin_bit_cast(_Float16, u));
    qv[k] = (qwave && qhead < G) ? x : 0.0f;
  }

  if (qwave) {
    float v[kC];
#pragma unroll
    for (int k = 0; k < kC; ++k) v[k] = qv[k];
    if (a.block > 0) {
      fwht_row_any<kC>(v, a.block, n);
      const float sbn = block_norm(a.block);
#pragma unroll
      for (int k = 0; k < kC; ++k) v[k] *= sbn;
    }
    // block exponent: lanes 4i..4i+3 hold the 32 channels of block i
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < kC; ++k) am = fmaxf(am, fabsf(v[k]));
    am = u2f(max(f2u(am), dpp_u<kDppXor1>(f2u(am))));   // (|q| >= 0: its bits order like its values)
    am = u2f(max(f2u(am), dpp_u<kDppXor2>(f2u(am))));
    int ex = 0;
    frexpf(am, &ex);                                  // am < 2^ex
    int s0 = am > 0.0f ? ex - 8 : -99;                // limb 0 below 2^8 (E4M3 max 448)
    s0 = s0 < -99 ? -99 : (s0 > 120 ? 120 : s0);      // limb 7's scale stays a valid E8M0
    if ((n & 3) == 0) sm.qexp[qhead][n >> 2] = s0;
    // FP8 limbs: t = q * 2^-s0; limb L = E4M3(t), t <- (t - limb L) * 16
    float t[kC];
#pragma unroll
    for (int k = 0; k < kC; ++k) t[k] = ldexpf(v[k], -s0);
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) {
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], hi, true);
      *reinterpret_cast<u32x2*>(&sm.u.qb[qhead][L][kC * n]) = u32x2{static_cast<uint32_t>(lo), static_cast<uint32_t>(hi)};
      const float back[kC] = {__builtin_amdgcn_cvt_f32_fp8(lo, 0), __builtin_amdgcn_cvt_f32_fp8(lo, 1),
                              __builtin_amdgcn_cvt_f32_fp8(lo, 2), __builtin_amdgcn_cvt_f32_fp8(lo, 3),
                              __builtin_amdgcn_cvt_f32_fp8(hi, 0), __builtin_amdgcn_cvt_f32_fp8(hi, 1),
                              __builtin_amdgcn_cvt_f32_fp8(hi, 2), __builtin_amdgcn_cvt_f32_fp8(hi, 3)};
#pragma unroll
      for (int k = 0; k < kC; ++k) t[k] = (t[k] - back[k]) * 16.0f;
    }
  }
  __syncthreads();

  // A operands of QK: lane (g, r) is row r = (head r/4, limb 4ls + r%4) and
  // holds channels 16g..16g+15 and 64+16g..64+16g+15; its scale byte is that
  // row's E8M0 for channel block g
  v8i aq[NS][2];
  int sa[NS][2];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int ls = 0; ls < 2; ++ls) {
      const int head = 4 * st + hs, L = 4 * ls + lam;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(&sm.u.qb[head][L][16 * g]);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(&sm.u.qb[head][L][64 + 16 * g]);
      aq[st][ls] = v8i{static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]), static_cast<int>(x0[3]),
                       static_cast<int>(x1[0]), static_cast<int>(x1[1]), static_cast<int>(x1[2]), static_cast<int>(x1[3])};
      sa[st][ls] = sm.qexp[head][g] - 4 * L + 127;
    }
  // the PV weight tiles share the query limbs' LDS: once every wave has read
  // its QK operands, each wave zeroes the limb-3 rows of its own tiles (the
  // fourth row of each head, never written)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int t = 0; t < kBlocks * 2; ++t) sm.u.wb[wave][st][t >> 1][t & 1][3][g][n] = 0u;

  float m_run[NS], l_run[NS], acc[NS][kNT];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    m_run[st] = kNegInf;
    l_run[st] = 0.0f;
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[st][t] = 0.0f;
  }
  const v4f zero4f = {0.0f, 0.0f, 0.0f, 0.0f};
  // PV A operand: lane (g, r) is row r = (head r/4, limb r%4), tokens 4g..4g+3
  // of the two pages of a pair
  const int wb_row = (lam * 4 + hs) * 16 + 4 * g;

  auto compute = [&](const MxStep& sb, int p, auto mask_tag) {
    constexpr bool tail = decltype(mask_tag)::value;
    float lg[NS][kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const v8i bk = v8i{static_cast<int>(sb.kx[i][0]), static_cast<int>(sb.kx[i][1]),
                         static_cast<int>(sb.kx[i][2]), static_cast<int>(sb.kx[i][3]), 0, 0, 0, 0};
      const int sbk = static_cast<int>((sb.ks[i] >> (8 * g)) & 0xFFu);   // token n, block g
      const int tok = (p + i) * kPage + n;
      const bool ok = !tail || (sb.pv[i] && tok < len);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[st][0], bk, zero4f, 0, 4, 0, sa[st][0], 0, sbk);
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[st][1], bk, c, 0, 4, 0, sa[st][1], 0, sbk);
        const float dot = (c[0] + c[1]) + (c[2] + c[3]);
        lg[st][i] = ok ? a.sm_log2 * dot : kNegInf;
      }
    }

    float alpha[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float mc = lg[st][0];
#pragma unroll
      for (int i = 1; i < kStep; ++i) mc = fmaxf(mc, lg[st][i]);
      mc = row_max16_ordered(mc);
      const float mnew = fmaxf(m_run[st], mc);
      const float muse = mnew == kNegInf ? 0.0f : mnew;
      alpha[st] = fast_exp2(m_run[st] - muse);
      m_run[st] = mnew;
      float pp[kStep], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        pp[i] = tail && lg[st][i] == kNegInf ? 0.0f : fast_exp2(lg[st][i] - muse);
        psum += pp[i];
      }
      l_run[st] = __builtin_fmaf(l_run[st], alpha[st], psum);
      // w = p * 2^(E - 128) of each block (E - 128 is the E8M0 byte with its
      // top bit flipped, as a signed byte; the V operand is twice the E2M1
      // value) as three bf16 limbs (each limb the rounding of what the ones
      // before left: exact differences), two pages to a dword, into the
      // wave's weight tiles
#pragma unroll
      for (int gi = 0; gi < kBlocks; ++gi) {
        float w[kStep];
#pragma unroll
        for (int i = 0; i < kStep; ++i) {
          const int e = static_cast<int8_t>(((sb.vs[i] ^ 0x80808080u) >> (8 * gi)) & 0xFFu);
          w[i] = ldexpf(pp[i], e);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t h0 = bf16_pair(w[2 * m], w[2 * m + 1]);
          const float r0 = w[2 * m] - bf16_lo(h0), r1 = w[2 * m + 1] - bf16_hi(h0);
          const uint32_t h1 = bf16_pair(r0, r1);
          const uint32_t h2 = bf16_pair(r0 - bf16_lo(h1), r1 - bf16_hi(h1));
          uint32_t* wt = &sm.u.wb[wave][st][gi][m][0][0][0];
          wt[(0 * 4 + g) * 16 + n] = h0;
          wt[(1 * 4 + g) * 16 + n] = h1;
          wt[(2 * 4 + g) * 16 + n] = h2;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    bf16x8 apv[NS][kBlocks][2];
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int gi = 0; gi < kBlocks; ++gi)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          apv[st][gi][m] = *reinterpret_cast<const bf16x8*>(&sm.u.wb[wave][st][gi][m][0][0][0] + wb_row);

    // V: for token r of the lane group and page pair m, the bytes of vp[m][r]
    // hold one channel's codes of pages 2m (low nibble) and 2m+1 (high):
    // channel pairs 2j (word 0) and 2j+1 (word 1) of byte j, nibble tau of a
    // page's word being channel n + 16 tau
    uint32_t vp[2][4][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t x = sb.vx[2 * m][r], y = sb.vx[2 * m + 1][r];
        vp[m][r][0] = (x & kLowNibbles) | ((y << 4) & ~kLowNibbles);
        vp[m][r][1] = ((x >> 4) & kLowNibbles) | (y & ~kLowNibbles);
      }
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) {
      // B operand of pair m: k = 8g + 2r + (page - 2m), column n (channel n + 16 tau)
      bf16x8 bv[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bf16x2 two = e2m1_pair_bf16(vp[m][r][tau & 1], tau >> 1);
          bv[m][2 * r] = two[0];
          bv[m][2 * r + 1] = two[1];
        }
      const int gi = tau >> 1;   // channels n + 16 tau lie in block tau / 2
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v4f c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apv[st][gi][0], bv[0], zero4f, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apv[st][gi][1], bv[1], c, 0, 0, 0);
        acc[st][tau] = __builtin_fmaf(acc[st][tau], alpha[st], (c[0] + c[1]) + c[2]);
      }
    }
  };

  auto step = [&](const MxStep& sb, int p) {
    if (!sb.all_ok || (p + kStep) * kPage > len)
      compute(sb, p, std::true_type{});
    else
      compute(sb, p, std::false_type{});
  };
  if constexpr (NS == 1) {
    // Two step buffers: the next step's loads go out before this step is
    // computed, so the two waves per SIMD (all the 512-workgroup grid of a
    // one-set decode fills; the registers still allow two) keep loads in
    // flight while they compute.  Loads of a step past the range have empty
    // descriptors, so each wait leaves the next step in flight.  (One
    // buffer measured 55.3 against 53.2 us, a third one two steps ahead
    // slower too.)
    MxStep buf1;
    for (int p = pw0; p < pw1; p += 2 * kStep) {
      load(buf1, p + kStep, idB);
      ids4(p + 2 * kStep, idA);
      step(buf0, p);
      if (p + kStep >= pw1) break;
      load(buf0, p + 2 * kStep, idA);
      ids4(p + 3 * kStep, idB);
      step(buf1, p + kStep);
    }
  } else {
    for (int p = pw0; p < pw1; p += kStep) {
      step(buf0, p);
      if (p + kStep >= pw1) break;
      load(buf0, p + kStep, idB);
      ids4(p + 2 * kStep, idB);
    }
  }

  // ---- merge the four waves, rotate back, store ------------------------------
  __syncthreads();   // the query limbs are reused below
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float lt = row_sum16(l_run[st]);
    const int j = 4 * st + g;
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) sm.u.merge.acc[wave][j][n + 16 * tau] = acc[st][tau];
    if (n == 0) {
      sm.u.merge.m[wave][j] = m_run[st];
      sm.u.merge.l[wave][j] = lt;
    }
  }
  __syncthreads();
  if (qwave) {
    const int j = qhead;
    float mstar = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm.u.merge.m[w][j]);
    const float muse = mstar == kNegInf ? 0.0f : mstar;
    float f[kWaves], lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f[w] = fast_exp2(sm.u.merge.m[w][j] - muse);
      lsum = __builtin_fmaf(sm.u.merge.l[w][j], f[w], lsum);
    }
    float o[kC];
#pragma unroll
    for (int k = 0; k < kC; ++k) o[k] = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int k = 0; k < kC; k += 4) {
        const v4f x = *reinterpret_cast<const v4f*>(&sm.u.merge.acc[w][j][kC * n + k]);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[k + i] = __builtin_fmaf(x[i], f[w], o[k + i]);
      }
    float scale = 1.0f;
    if (a.block > 0) {
      fwht_row_any<kC>(o, a.block, n);
      scale = block_norm(a.block);
    }
    if (direct) {
      scale *= lsum > 0.0f ? 1.0f / lsum : 0.0f;
      if (j < G) {
        float* dst = a.out + (hq0 + j) * D + kC * n;
#pragma unroll
        for (int k = 0; k < kC; k += 4)
          *reinterpret_cast<v4f*>(dst + k) = v4f{o[k] * scale, o[k + 1] * scale, o[k + 2] * scale, o[k + 3] * scale};
      }
    } else if (j < G) {
      const int64_t idx = (hq0 + j) * a.part_stride + a.part_slot0 + s;
      float* dst = a.part_acc + idx * D + kC * n;
#pragma unroll
      for (int k = 0; k < kC; k += 4)
        *reinterpret_cast<v4f*>(dst + k) = v4f{o[k] * scale, o[k + 1] * scale, o[k + 2] * scale, o[k + 3] * scale};
      if (n == 0) {
        a.part_ml[idx * 2 + 0] = mstar;
        a.part_ml[idx * 2 + 1] = lsum;
      }
    }
  }
}

template <int NS, bool BAL>
hipError_t launch_b(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.nsplit) * a.num_kv_heads * a.batch);
  if (a.in_bf16)
    decode_mxfp4_kernel<NS, true, BAL><<<grid, 64 * kWaves, 0, s>>>(a);
  else
    decode_mxfp4_kernel<NS, false, BAL><<<grid, 64 * kWaves, 0, s>>>(a);
  return hipGetLastError();
}

template <int NS>
hipError_t launch_mx(const DecodeArgs& a, hipStream_t s) {
  return a.balance ? launch_b<NS, true>(a, s) : launch_b<NS, false>(a, s);
}

}  // namespace

hipError_t launch_decode_mxfp4(const DecodeArgs& a, hipStream_t s) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 4) return launch_mx<1>(a, s);
  if (g <= 8) return launch_mx<2>(a, s);
  return launch_mx<4>(a, s);
}

}  // namespace kvq

// Body of the INT4 / INT8 / grouped-INT4 decode workgroup (the kernels that
// run it alone are launched from decode_int4.hip and decode_int4_sk.hip, the
// windowed decode runs it beside the bf16 window workgroups).
//
// Read path: split-K paged decode attention over the INT4 cache with the
// dequantization folded into the products ("SAW-INT4", summary page: fused
// attention execution over paged quantized KV; "BitDecoding-FP4", Abstract:
// the query heads of a GQA group stacked into one matrix product per KV page;
// factoring the per-token scale out of the dot product follows the grouping
// idea of "InnerQ", Figure 1).
//
// A workgroup of four waves owns one (sequence b, KV head, split s), or in
// the stream-K mapping a range of the batch's pages, and each wave streams a
// quarter of a sequence's pages, four pages per step, with non-temporal
// buffer loads (the cache is read once per call).  Per page and
// per group of four query heads:
//   QK:  C[(head, limb)][token] = sum_c qlimb[c] * code[token][c]   (int8 MFMA)
//        The rotated query is a 23-bit fixed-point integer split into three
//        signed 8-bit limbs (rows of the tile); codes are exact int8; products
//        and sums are exact in int32.  Each lane ends with the four limb rows
//        of one (head, token) and combines them in-lane:
//        logit = sm * 2^(e-22) * (k_scale * sum_c code*qfix + k_zero * sum_c qfix).
//   softmax: online, base 2; one row of 16 lanes = one head.
//   PV:  acc[(head, limb)][c] = sum_t wlimb[t] * code_v[t][c]        (int8 MFMA)
//        w = p * v_scale as a 23-bit fixed-point integer relative to the
//        step's largest w of the head (power-of-two scale), its limbs moved to
//        the operand layout through a 1 KiB LDS tile; sum_t p * v_zero is added
//        to every channel at the end.
// The four waves merge in LDS.  With one split each wave finishes heads of the
// group (normalise, rotate back, store); otherwise it stores a partial (max,
// sum, unnormalised output) for the reduce kernel.
//
// The same kernel reads the token-wise INT8 variant ("GPU-Accelerated INT8
// Quantization for KV Cache Compression in Large Language Models",
// Abstract): codes 0..255 enter the int8 MFMA as code - 128 (one xor per
// byte) and the 128 * scale they lose is added to the zero point.
//
// And the grouped INT4 variant (one scale and zero per group of GS channels,
// grouping along the inner dimension as "InnerQ", Abstract and Figure 1): QK
// runs one product per group with the query operand masked to the group's
// channels; V is stored so that each PV tile of 16 output channels lies in
// one group, so PV keeps one product per tile, with the softmax weights of
// that group (w = p * v_scale of the group) as its operand.
#pragma once
#include "dev_common.hpp"
#include "kvq_internal.hpp"
#include <type_traits>

namespace kvq {
namespace q4 {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = 4;
constexpr int kStep = 4;   // pages per step

// channel of k-slot (dword i, byte k) of the QK operand `op` for lane group g:
// 4-bit codes split into low and high nibbles, 8-bit codes in byte order
template <int D, int BITS>
__device__ __forceinline__ int qk_channel(int g, int op, int i, int k) {
  if constexpr (BITS == 8) return (D / 4) * g + 16 * op + 4 * i + k;
  else if constexpr (D == 128) return 32 * g + 8 * i + 2 * k + op;
  else return 16 * g + 8 * (i & 1) + 2 * k + (i >> 1);
}

// output channel of PV tile tau for lane column n (the V layout of the
// token-wise pools puts 8 consecutive channels in a word, the grouped pool
// channels n + (D/8) j)
template <int D, int GS>
__device__ __forceinline__ int pv_channel(int n, int tau) {
  if constexpr (GS != 0) {
    if constexpr (D == 128) return n + 16 * tau;
    else return (n & 7) + 8 * (2 * tau + (n >> 3));
  } else {
    if constexpr (D == 128) return 8 * n + tau;
    else return 8 * (n & 7) + 2 * tau + (n >> 3);
  }
}

// Scale of a sidecar word (the low fp16).  In the grouped pool the sign bit
// marks a group of the hybrid quantizer's symmetric form, so the magnitude is
// taken there (for free: an input modifier of the instruction that uses it).
template <int GS>
__device__ __forceinline__ float side_scale(uint32_t w) {
  return GS ? fabsf(half_lo(w)) : half_lo(w);
}

// Bytes of one page in a wave's LDS stage (staged builds): K codes and V
// codes (16 bytes per lane each, where the lane's own loads would put them)
// and one 4-byte-per-lane load of the sidecars.
template <int D>
constexpr int stage_page_bytes() { return 2 * kPage * (D / 2) + 256; }

// STAGE: the staged build, whose page stage (in flight during the query's
// prologue) shares its LDS with the merge only, not with the query scratch.
template <int D, int NS, int NG, bool STAGE>
struct alignas(16) Smem {
  static constexpr int kGP = 4 * NS;
  struct Merge {
    float acc[kWaves][kGP][D];
    float m[kWaves][kGP];
    float l[kWaves][kGP];
  };
  union {
    int32_t qi[STAGE ? 1 : kGP][D];
    Merge merge;
    uint8_t stage[STAGE ? kWaves : 1][4][stage_page_bytes<D>()];   // [wave][page of the step]
  } u;
  int32_t qi_own[STAGE ? kGP : 1][D];
  uint8_t qstage[STAGE ? NS : 1][64 * 16];   // the query waves' query rows (staged build)
  float hA[kGP], hS[kGP][NG];
  uint32_t wl[kWaves][NS][NG][4][4][16];   // [wave][set][group][limb][head][token] = 4 pages' bytes
};

// one step's loads: four pages of one KV head, KX (VX) 16-byte pieces of
// K (V) codes per lane and page
template <int KX, int VX, int NG>
struct StepBuf {
  u32x4 kx[kStep][KX];
  u32x4 vx[kStep][VX];
  uint32_t km[kStep][NG], vm[kStep][NG];   // (scale, zero) per group
  bool pv[kStep];
  bool all_ok;
};

// WPE: waves per SIMD the register allocation must allow (1 = no limit);
// MAP: how workgroup `wid` finds its work (kMapPlanned, kMapBalanced,
// kMapStream), each built apart so that a call carries no other's code
template <int D, int NS, bool QBF16, int BITS, int GS, int WPE, int MAP>
__device__ __forceinline__ void decode_quant_body(const DecodeArgs& a, uint32_t wid) {
  constexpr bool BAL = MAP == kMapBalanced;
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit codes");
  static_assert(GS == 0 || (BITS == 4 && (GS == 32 || GS == 64) && GS <= D), "groups of 32 or 64 channels, 4-bit");
  constexpr int kCodeBytes = D * BITS / 8;           // one vector's codes
  constexpr int kNG = GS ? D / GS : 1;               // (scale, zero) pairs per vector
  constexpr int kSlab = kPage * (2 * kCodeBytes + 8 * kNG);
  constexpr int kKX = BITS == 8 && D == 128 ? 2 : 1;  // 16-byte K pieces per lane and page
  constexpr int kVX = BITS == 8 ? 2 : 1;              // 16-byte V pieces per lane and page
  using Buf = StepBuf<kKX, kVX, kNG>;
  // one scale/zero per vector and no register cap: the single-pass form of
  // the step (fewest instructions); otherwise the per-group form, whose
  // shorter live ranges also fit the 128-VGPR build
  constexpr bool kOnePass = kNG == 1 && WPE == 1;
  // two step buffers (see the streaming loop): the two-set INT4 kernel, whose
  // registers allow two waves per SIMD with or without the second buffer
  // (the build held to three waves per SIMD keeps one)
  constexpr bool kPrefetch = NS == 2 && BITS == 4 && GS == 0 && WPE == 1;
  // The two-set INT4 build held to three waves per SIMD stages the next
  // step's pages in LDS (direct-to-LDS buffer loads hold no VGPRs while they
  // fly), so it keeps a step in flight while it computes without the second
  // register buffer that would cost it the third wave.
  constexpr bool kStage = NS == 2 && BITS == 4 && GS == 0 && D == 128 && WPE == 3;
  static_assert(!kStage || kStep == 4, "stage of four pages");
  constexpr int kNT = D / 16;          // PV tiles = output channels per lane
  constexpr int kOps = D / 64;         // QK MFMAs per page and head group
  constexpr int kC = D / 16;           // channels per lane when a row of 16 lanes holds a vector
  // head_dim 128: the QK operand is built once, by the query waves, into an
  // LDS image of NS * kOps * 64 lanes * 16 bytes (the size of the query
  // scratch it replaces) that every wave then reads
  constexpr bool kOpImage = D == 128;
  static_assert(!kOpImage || NS * kOps * 64 * 16 == sizeof(int32_t) * 4 * NS * D, "operand image size");
  __shared__ Smem<D, NS, kNG, kStage> sm;
  // the query scratch (fixed-point query, or the operand image)
  int32_t (*const qscr)[D] = kStage ? sm.qi_own : sm.u.qi;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;
  const bool qwave = wave < NS;
  const int qhead = 4 * wave + g;
  const int G = a.num_q_heads / a.num_kv_heads;
  // query: wave w < NS takes heads 4w .. 4w+3 of the group, one per row of 16
  // lanes; lane (g, n) holds channels [kC n, kC n + kC) of head 4w + g.
  // Padding heads read head G-1 and are zeroed below.  (The staged build
  // brings it in through LDS once the workgroup is known to have work.)
  auto load_query = [&](int64_t hq0, uint32_t (&qraw)[kC / 2]) {
    if constexpr (kStage) {
#pragma unroll
      for (int i = 0; i < kC / 2; ++i) qraw[i] = 0u;
    } else if (qwave) {
      const uint16_t* qp = a.q + (hq0 + min(qhead, G - 1)) * D + kC * n;
      if constexpr (kC == 8) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(qp);
#pragma unroll
        for (int i = 0; i < 4; ++i) qraw[i] = t[i];
      } else {
        const u32x2 t = *reinterpret_cast<const u32x2*>(qp);
        qraw[0] = t[0];
        qraw[1] = t[1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kC / 2; ++i) qraw[i] = 0u;
    }
  };

  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  // raw entries of pages p .. p+3 of a block-table row, indexes clamped below
  // lim (pages at or past the range are dropped where the ids are used);
  // page ids come by scalar loads (wave-uniform addresses, always inside the
  // row)
  auto ids4_of = [&](ConstI32* row, int p, int lim, int32_t (&id)[kStep]) {
#pragma unroll
    for (int i = 0; i < kStep; ++i) id[i] = row[min(p + i, lim - 1)];
  };

  // One work item: pages [q0, p1) of sequence b (tokens [lo, hi) of it
  // count) for KV head kvh, its result stored normalised in the output rows
  // (direct) or as a partial at part_base + head * part_mul.  qraw holds the
  // query row already loaded (not in the staged build), idA the ids of pages
  // cb .. cb+3.
  // tid_r and wave_r are the thread and wave ids, passed in so that a caller
  // running several items can keep what depends on them inside its loop.
  auto run = [&](const int kvh, const int64_t hq0, ConstI32* const bt_s, const int q0, const int p1,
                 const int lo, const int hi, const bool direct, const int64_t part_base, const int part_mul,
                 uint32_t (&qraw)[kC / 2], int32_t (&idA)[kStep], const int cb, const bool grown,
                 const int tid_r, const int wave_r) {
  const int tid = tid_r;
  const int wave = wave_r;
  const int lane = tid & 63;
  const int g = lane >> 4, n = lane & 15, hs = n >> 2, lam = n & 3;
  const bool qwave = wave < NS;
  const int qhead = 4 * wave + g;
  auto ids4 = [&](int p, int lim, int32_t (&id)[kStep]) { ids4_of(bt_s, p, lim, id); };
  int32_t idB[kStep];
  // The staged build's query goes out only now (no stage or query load may
  // be in flight when a workgroup with no work exits): through LDS, so that
  // its wait below leaves the first step's stage loads in flight.
  if constexpr (kStage) {
    if (qwave) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + hq0 * D, G * D * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (__attribute__((address_space(3))) void*)(&sm.qstage[wave][0]), 16,
          static_cast<uint32_t>((min(qhead, G - 1) * D + kC * n) * 2), 0, 0, 0);
    }
  }

  // ---- this wave's share of the split's pages ---------------------------------
  const int span = p1 - q0;
  const int per_wave = ((span + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
  const int pw0 = q0 + wave * per_wave;
  const int pw1 = min(p1, pw0 + per_wave);
  const uint8_t* pool_h = a.pool + static_cast<int64_t>(kvh) * kSlab;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * kSlab;
  const int vn = n & (D / 8 - 1);
  // lane offsets within a page slab, unsigned so that each load is a uniform
  // 64-bit base plus a 32-bit lane offset: lane (g, n) reads K codes of token
  // n (channels [D/4 g, D/4 (g+1))) and V codes of tokens 4g..4g+3 (channel
  // group vn)
  const uint32_t k_off = n * kCodeBytes + g * (kCodeBytes / 4);
  const uint32_t v_off = kPage * kCodeBytes + (vn * kPage + 4 * g) * (BITS == 8 ? 8 : 4);
  const uint32_t km_off = 2 * kPage * kCodeBytes + 4 * kNG * n;
  if (cb != pw0 || grown) ids4(pw0, pw1, idA);   // the range starts elsewhere
  // id_of(i) is the id of page p + i (-1 when the page is past the range)
  auto load_with = [&](Buf& sb, int p, auto id_of) {
    sb.all_ok = true;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const int id = id_of(i);
      sb.pv[i] = id >= 0 && id < a.num_pages;
      sb.all_ok = sb.all_ok && sb.pv[i];
      // one buffer descriptor per page slab (scalar registers): each load is
      // that base plus the lane's 32-bit offset; nothing can reach past the
      // slab, and a page that is not there gets an empty descriptor, whose
      // loads return zeros without touching memory
      const uint8_t* sl = pool_h + static_cast<int64_t>(sb.pv[i] ? id : 0) * page_stride;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(sl, sb.pv[i] ? kSlab : 0);
      if constexpr (kCodeBytes / 4 >= 16) {
#pragma unroll
        for (int j = 0; j < kKX; ++j)
          sb.kx[i][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, k_off + 16 * j, 0, kStreamOnce));
      } else {
        const u32x2 t2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, k_off, 0, kStreamOnce));
        sb.kx[i][0] = u32x4{t2[0], t2[1], 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kVX; ++j)
        sb.vx[i][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, v_off + 16 * j, 0, kStreamOnce));
      if constexpr (kNG == 1) {
        sb.km[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, km_off, 0, kStreamOnce);
        sb.vm[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, km_off + 4 * kPage, 0, kStreamOnce);
      } else if constexpr (kNG == 2) {
        const u32x2 k2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, km_off, 0, kStreamOnce));
        const u32x2 v2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, km_off + 8 * kPage, 0, kStreamOnce));
        sb.km[i][0] = k2[0];
        sb.km[i][1] = k2[1];
        sb.vm[i][0] = v2[0];
        sb.vm[i][1] = v2[1];
      } else {
        const u32x4 k4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, km_off, 0, kStreamOnce));
        const u32x4 v4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, km_off + 16 * kPage, 0, kStreamOnce));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sb.km[i][j] = k4[j];
          sb.vm[i][j] = v4[j];
        }
      }
    }
  };
  // Staged build: every step's pages go through this wave's LDS stage.
  struct StageMeta { bool pv[kStep]; bool all_ok; };
  uint8_t* const stage = kStage ? &sm.u.stage[wave][0][0] : nullptr;
  constexpr int kSP = stage_page_bytes<D>();
  const uint32_t side_off = lane < 32 ? static_cast<uint32_t>(2 * kPage * kCodeBytes + 4 * lane)
                                      : static_cast<uint32_t>(kSlab);
  auto stage_issue = [&](int p, auto id_of, StageMeta& mt) {
    mt.all_ok = true;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const int id = id_of(i);
      mt.pv[i] = id >= 0 && id < a.num_pages;
      mt.all_ok = mt.all_ok && mt.pv[i];
      const uint8_t* sl = pool_h + static_cast<int64_t>(mt.pv[i] ? id : 0) * page_stride;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(sl, mt.pv[i] ? kSlab : 0);
      uint8_t* dst = stage + i * kSP;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst), 16, k_off,
                                               0, 0, kStreamOnce);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 1024), 16,
                                               v_off, 0, 0, kStreamOnce);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 2048), 4,
                                               side_off, 0, 0, kStreamOnce);
    }
  };
  auto stage_read = [&](Buf& sb, const StageMeta& mt) {
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const uint8_t* src = stage + i * kSP;
      sb.kx[i][0] = *reinterpret_cast<const u32x4*>(src + 16 * lane);
      sb.vx[i][0] = *reinterpret_cast<const u32x4*>(src + 1024 + 16 * lane);
      sb.km[i][0] = *reinterpret_cast<const uint32_t*>(src + 2048 + 4 * n);
      sb.vm[i][0] = *reinterpret_cast<const uint32_t*>(src + 2048 + 4 * kPage + 4 * n);
      sb.pv[i] = mt.pv[i];
    }
    sb.all_ok = mt.all_ok;
  };
  // The first step's page loads go out before the query is waited for: the
  // query was requested first, so its wait leaves the pages in flight, and
  // its rotation and limbs are computed while they arrive.  (A staged wave
  // with no pages sends nothing: no stage load may be in flight when the
  // merge reuses the stage's LDS.)
  Buf buf0;
  [[maybe_unused]] StageMeta mt;
  if constexpr (kStage) {
    if (pw0 < pw1) stage_issue(pw0, [&](int i) { return pw0 + i < pw1 ? idA[i] : -1; }, mt);
  } else {
    load_with(buf0, pw0, [&](int i) { return pw0 + i < pw1 ? idA[i] : -1; });
  }
  ids4(pw0 + kStep, pw1, idB);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kStage) {
    if (qwave) {
      // the query's load was issued before the twelve stage loads of the
      // first step (none when the wave has no pages)
      __builtin_amdgcn_sched_barrier(0);
      if (pw0 < pw1) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 t = *reinterpret_cast<const u32x4*>(&sm.qstage[wave][16 * lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i) qraw[i] = t[i];
    }
  }
  float qv[kC];
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    const uint16_t u = static_cast<uint16_t>(qraw[k / 2] >> (16 * (k & 1)));
    const float x = QBF16 ? u2f(static_cast<uint32_t>(u) << 16) : static_cast<float>(__builtin_bit_cast(_Float16, u));
    qv[k] = qhead < G ? x : 0.0f;
  }
  // ---- query: rotate in registers, fixed point, limbs ------------------------
  for (int e = tid; e < kWaves * NS * kNG * 4 * 4 * 16; e += 64 * kWaves)
    (&sm.wl[0][0][0][0][0][0])[e] = 0u;   // the limb-3 rows stay zero
  if (qwave) {
    float v[kC];
#pragma unroll
    for (int k = 0; k < kC; ++k) v[k] = qv[k];
    if (a.block > 0) {
      fwht_row_any<kC>(v, a.block, n);
      const float sb = block_norm(a.block);
#pragma unroll
      for (int k = 0; k < kC; ++k) v[k] *= sb;
    }
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < kC; ++k) am = fmaxf(am, fabsf(v[k]));
    am = row_max16_nonneg(am);   // (a maximum of |q|)
    int ex = 0;
    frexpf(am, &ex);                    // am < 2^ex
    ex = ex < -100 ? -100 : ex;         // keeps 2^(22-ex) finite; smaller q is ~0
    const float sc = ldexpf(1.0f, 22 - ex);
    int32_t qi[kC];
    int32_t sum = 0;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      qi[k] = static_cast<int32_t>(rintf(v[k] * sc));
      sum += qi[k];
    }
    if constexpr (kOpImage) {
      // This lane's words of the QK operand image (see below): limb L of a
      // channel is byte 2 (L = 0), or byte 1 / 0 with the top bit flipped
      // (L = 1, 2), of qi + 0x8080 (the balanced limbs of LimbSel); a word
      // holds one limb of four channels; limb 3 is the zero pad row.
      uint32_t y[kC];
#pragma unroll
      for (int k = 0; k < kC; ++k) y[k] = static_cast<uint32_t>(qi[k] + 0x8080);
      auto word = [&](int c0, int c1, int c2, int c3, int L) -> uint32_t {
        if (L == 3) return 0u;
        const uint32_t sel = L == 0 ? 0x0c0c0602u : (L == 1 ? 0x0c0c0501u : 0x0c0c0400u);
        const uint32_t lo = __builtin_amdgcn_perm(y[c1], y[c0], sel);
        const uint32_t hi = __builtin_amdgcn_perm(y[c3], y[c2], sel);
        return __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ (L == 0 ? 0u : 0x80808080u);
      };
      uint32_t* img = reinterpret_cast<uint32_t*>(&qscr[0][0]);
      const int lane0 = 16 * (n >> 2) + 4 * g;   // reader lanes: row (head g, limb L), group n / 4
#pragma unroll
      for (int L = 0; L < 4; ++L) {
        if constexpr (BITS == 4) {   // op o: channels o, o+2, o+4, o+6 of the lane, dword n % 4
#pragma unroll
          for (int op = 0; op < kOps; ++op)
            img[((wave * kOps + op) * 64 + lane0 + L) * 4 + (n & 3)] = word(op, op + 2, op + 4, op + 6, L);
        } else {                     // op (n/2) % 2: channels 0..3 and 4..7 as dwords 2 (n%2) + {0, 1}
          const int op = (n >> 1) & 1, i0 = 2 * (n & 1);
          img[((wave * kOps + op) * 64 + lane0 + L) * 4 + i0] = word(0, 1, 2, 3, L);
          img[((wave * kOps + op) * 64 + lane0 + L) * 4 + i0 + 1] = word(4, 5, 6, 7, L);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kC; k += 4)
        *reinterpret_cast<v4i*>(&qscr[qhead][kC * n + k]) = v4i{qi[k], qi[k + 1], qi[k + 2], qi[k + 3]};
    }
    // sum of the query over each group (|sum| <= D * 2^22: exact in int32);
    // a lane's kC channels lie in group kC n / GS
    int32_t gsum[kNG];
#pragma unroll
    for (int gi = 0; gi < kNG; ++gi) gsum[gi] = row_sum16_i(kNG == 1 || (kC * n) / (GS ? GS : D) == gi ? sum : 0);
    if (n == 0) {
      sm.hA[qhead] = a.sm_log2 * ldexpf(1.0f, ex - 22);
#pragma unroll
      for (int gi = 0; gi < kNG; ++gi) sm.hS[qhead][gi] = static_cast<float>(gsum[gi]);
    }
  }
  if constexpr (kStage) {
    // the query's results are LDS writes: wait for those alone (a full
    // __syncthreads would also drain the first step's stage loads)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  } else {
    __syncthreads();
  }

  // A operand of QK: row (head hs, limb lam), k-slots of lane group g.  At
  // head_dim 128 the query waves wrote every lane's operand words into an
  // LDS image, so each wave reads one 16-byte vector per set and product;
  // at 64 each wave builds them from the fixed-point query.
  const LimbSel limb(lam);
  v4i aq[NS][kNG][kOps];   // per group: the operand with other groups' channels zeroed
  float qA[NS], qS[NS][kNG];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    qA[st] = sm.hA[4 * st + g];          // C-layout head of this lane: row group g
#pragma unroll
    for (int gi = 0; gi < kNG; ++gi) qS[st][gi] = sm.hS[4 * st + g][gi];
    if constexpr (kOpImage) {
      const v4i* img = reinterpret_cast<const v4i*>(&qscr[0][0]);
#pragma unroll
      for (int op = 0; op < kOps; ++op) {
        const v4i vv = img[(st * kOps + op) * 64 + lane];
#pragma unroll
        for (int gi = 0; gi < kNG; ++gi) aq[st][gi][op] = (kNG == 1 || (D / 4) * g / (GS ? GS : D) == gi) ? vv : v4i{0, 0, 0, 0};
      }
      continue;
    }
    int32_t qc[D / 4];
    const v4i* src = reinterpret_cast<const v4i*>(&qscr[4 * st + hs][(D / 4) * g]);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const v4i x = src[t];
      qc[4 * t] = x[0];
      qc[4 * t + 1] = x[1];
      qc[4 * t + 2] = x[2];
      qc[4 * t + 3] = x[3];
    }
#pragma unroll
    for (int op = 0; op < kOps; ++op) {
      v4i vv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w |= limb.byte(qc[qk_channel<D, BITS>(0, op, i, k)]) << (8 * k);
        vv[i] = static_cast<int32_t>(w);
      }
      // lane group g holds channels [D/4 g, D/4 (g+1)): one group's
#pragma unroll
      for (int gi = 0; gi < kNG; ++gi) aq[st][gi][op] = (kNG == 1 || (D / 4) * g / (GS ? GS : D) == gi) ? vv : v4i{0, 0, 0, 0};
    }
  }

  float m_run[NS], l_run[NS], z_run[NS][kNG], acc[NS][kNT];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    m_run[st] = kNegInf;
    l_run[st] = 0.0f;
#pragma unroll
    for (int gi = 0; gi < kNG; ++gi) z_run[st][gi] = 0.0f;
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[st][t] = 0.0f;
  }
  const v4i zero4 = {0, 0, 0, 0};
  const int wl_row = (lam * 4 + hs) * 16 + 4 * g;   // reader offset within a set, dwords

  auto compute = [&](const Buf& sb, int p, auto mask_tag) {
    constexpr bool tail = decltype(mask_tag)::value;
    // QK: lane (g, n) gets the four limb rows of head g (per set), token n
    float lg[NS][kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      v4i b0, b1;
      if constexpr (BITS == 8) {   // code - 128 as a signed byte
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          b0[w] = static_cast<int32_t>(sb.kx[i][0][w] ^ 0x80808080u);
          if constexpr (kKX == 2) b1[w] = static_cast<int32_t>(sb.kx[i][1][w] ^ 0x80808080u);
        }
      } else if constexpr (D == 128) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          b0[w] = static_cast<int32_t>(sb.kx[i][0][w] & kLowNibbles);
          b1[w] = static_cast<int32_t>((sb.kx[i][0][w] >> 4) & kLowNibbles);
        }
      } else {
        b0 = v4i{static_cast<int32_t>(sb.kx[i][0][0] & kLowNibbles), static_cast<int32_t>(sb.kx[i][0][1] & kLowNibbles),
                 static_cast<int32_t>((sb.kx[i][0][0] >> 4) & kLowNibbles),
                 static_cast<int32_t>((sb.kx[i][0][1] >> 4) & kLowNibbles)};
      }
      const int tok = (p + i) * kPage + n;
      const bool ok = !tail || (sb.pv[i] && tok >= lo && tok < hi);
      if constexpr (kOnePass) {
        // zero point of the codes as the MFMA sees them
        const uint32_t km = sb.km[i][0];
        const float kzero = BITS == 8 ? __builtin_fmaf(128.0f, half_lo(km), half_hi(km)) : half_hi(km);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          v4i c = mfma_i8(aq[st][0][0], b0, zero4);
          if constexpr (kOps == 2) c = mfma_i8(aq[st][0][1], b1, c);
          // limbs: c0 * 2^16 + c1 * 2^8 + c2 (c0 * 2^8 + c1 is exact in int32)
          const float tq = __builtin_fmaf(static_cast<float>((c[0] << 8) + c[1]), 256.0f,
                                          static_cast<float>(c[2]));
          const float l2 = qA[st] * __builtin_fmaf(kzero, qS[st][0], side_scale<GS>(km) * tq);
          lg[st][i] = ok ? l2 : kNegInf;
        }
        continue;
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        float dot = 0.0f;
#pragma unroll
        for (int gi = 0; gi < kNG; ++gi) {
          v4i c = mfma_i8(aq[st][gi][0], b0, zero4);
          if constexpr (kOps == 2) c = mfma_i8(aq[st][gi][1], b1, c);
          // limbs: c0 * 2^16 + c1 * 2^8 + c2 (c0 * 2^8 + c1 is exact in int32)
          const float tq = __builtin_fmaf(static_cast<float>((c[0] << 8) + c[1]), 256.0f,
                                          static_cast<float>(c[2]));
          // zero point of the codes as the MFMA sees them
          const uint32_t km = sb.km[i][gi];
          const float kzero = BITS == 8 ? __builtin_fmaf(128.0f, half_lo(km), half_hi(km)) : half_hi(km);
          dot = gi == 0 ? __builtin_fmaf(kzero, qS[st][0], side_scale<GS>(km) * tq)
                        : dot + __builtin_fmaf(kzero, qS[st][gi], side_scale<GS>(km) * tq);
        }
        lg[st][i] = ok ? qA[st] * dot : kNegInf;
      }
    }

    // online softmax (row = head) and the limbs of w = p * v_scale through LDS
    float alpha[NS], sw[NS][kNG];
    // w = p * v_scale as a 23-bit fixed-point integer relative to the step's
    // largest w of the head (power-of-two scale sw), three int8 limbs of it
    // into the LDS tile of (set st, group gi)
    auto store_limbs = [&](int st, int gi, const float* w, float wmax) {
      wmax = row_max16_nonneg(wmax);   // (w = p * v_scale >= 0)
      int ew = 0;
      frexpf(wmax, &ew);                 // wmax < 2^ew
      ew = ew < -100 ? -100 : ew;        // such a step weighs < 2^-76 of the max
      const float wsc = ldexpf(1.0f, 22 - ew);
      sw[st][gi] = ldexpf(1.0f, ew - 22);
      uint32_t y[kStep];
#pragma unroll
      for (int i = 0; i < kStep; ++i)
        y[i] = static_cast<uint32_t>(static_cast<int32_t>(rintf(w[i] * wsc)) + 0x8080);
      // limb bytes of the four pages, one word per limb: bytes 2 / 1 / 0 of y
      const uint32_t l0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0602u),
                                                __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0602u), 0x05040100u);
      const uint32_t l1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0501u),
                                                __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0501u), 0x05040100u) ^ 0x80808080u;
      const uint32_t l2w = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0400u),
                                                 __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0400u), 0x05040100u) ^ 0x80808080u;
      uint32_t* wl = &sm.wl[wave][st][gi][0][0][0];
      wl[(0 * 4 + g) * 16 + n] = l0;
      wl[(1 * 4 + g) * 16 + n] = l1;
      wl[(2 * 4 + g) * 16 + n] = l2w;
    };
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
      if constexpr (kOnePass) {   // one scale/zero per vector: a single pass over the step
        float psum = 0.0f, zsum = 0.0f, wmax = 0.0f, w[kStep];
#pragma unroll
        for (int i = 0; i < kStep; ++i) {
          const float pp = fast_exp2(lg[st][i] - muse);
          psum += pp;
          const uint32_t vm = sb.vm[i][0];
          const float vzero = BITS == 8 ? __builtin_fmaf(128.0f, half_lo(vm), half_hi(vm)) : half_hi(vm);
          if (tail) {
            const bool ok = lg[st][i] != kNegInf;
            zsum += ok ? pp * vzero : 0.0f;
            w[i] = ok ? pp * side_scale<GS>(vm) : 0.0f;
          } else {
            zsum = __builtin_fmaf(pp, vzero, zsum);
            w[i] = pp * side_scale<GS>(vm);
          }
          wmax = fmaxf(wmax, w[i]);
        }
        l_run[st] = __builtin_fmaf(l_run[st], alpha[st], psum);
        z_run[st][0] = __builtin_fmaf(z_run[st][0], alpha[st], zsum);
        store_limbs(st, 0, w, wmax);
        continue;
      }
      float pp[kStep], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        pp[i] = fast_exp2(lg[st][i] - muse);
        psum += pp[i];
      }
      l_run[st] = __builtin_fmaf(l_run[st], alpha[st], psum);
#pragma unroll
      for (int gi = 0; gi < kNG; ++gi) {
        float zsum = 0.0f, wmax = 0.0f, w[kStep];
#pragma unroll
        for (int i = 0; i < kStep; ++i) {
          const uint32_t vm = sb.vm[i][gi];
          const float vzero = BITS == 8 ? __builtin_fmaf(128.0f, half_lo(vm), half_hi(vm)) : half_hi(vm);
          if (tail) {
            const bool ok = lg[st][i] != kNegInf;
            zsum += ok ? pp[i] * vzero : 0.0f;
            w[i] = ok ? pp[i] * side_scale<GS>(vm) : 0.0f;
          } else {
            zsum = __builtin_fmaf(pp[i], vzero, zsum);
            w[i] = pp[i] * side_scale<GS>(vm);
          }
          wmax = fmaxf(wmax, w[i]);
        }
        z_run[st][gi] = __builtin_fmaf(z_run[st][gi], alpha[st], zsum);
        store_limbs(st, gi, w, wmax);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    v4i apv[NS][kNG];
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int gi = 0; gi < kNG; ++gi)
        apv[st][gi] = *reinterpret_cast<const v4i*>(&sm.wl[wave][st][gi][0][0][0] + wl_row);

    // V: per token r of the lane group, transpose across four pages so a
    // word holds the four pages' codes of one channel pair (4-bit: nibbles
    // split it) or of one channel (8-bit, then made signed).
    uint32_t vt[4][kVX][4];   // [r][half][byte j]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int hh = 0; hh < kVX; ++hh) {
        // 4-bit: dword r of the piece is token 4g+r; 8-bit: dwords
        // 2(r&1)+hh of piece r>>1 are token 4g+r, channels 4hh..4hh+3
        auto src = [&](int pg) {
          return BITS == 8 ? sb.vx[pg][r >> 1][2 * (r & 1) + hh] : sb.vx[pg][0][r];
        };
        transpose_bytes4(src(0), src(1), src(2), src(3), vt[r][hh]);
      }
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau) {
      v4i bv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t yv;
        if constexpr (BITS == 8) {
          if constexpr (D == 128) {   // channel 8n + tau
            yv = vt[r][tau >> 2][tau & 3];
          } else {                    // channel 8(n&7) + 2tau + (n>>3)
            const uint32_t* h4 = vt[r][tau >> 1];
            yv = (n >> 3) ? h4[2 * (tau & 1) + 1] : h4[2 * (tau & 1)];
          }
          yv ^= 0x80808080u;
        } else {   // nibble tau (D = 128) or 2tau + (n>>3) (D = 64) of the word
          if constexpr (D == 128) yv = (tau & 1) ? (vt[r][0][tau >> 1] >> 4) : vt[r][0][tau >> 1];
          else yv = vt[r][0][tau] >> (4 * (n >> 3));
          yv &= kLowNibbles;
        }
        bv[r] = static_cast<int32_t>(yv);
      }
      // the tile's group: its channels n + 16 tau (D = 128) or
      // (n&7) + 16 tau + 8 (n>>3) (D = 64) all lie in group 16 tau / GS
      constexpr int kTileGroupDiv = GS ? GS : 16 * kNT;
      const int gi = 16 * tau / kTileGroupDiv;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const v4i c = mfma_i8(apv[st][gi], bv, zero4);
        const float f = __builtin_fmaf(static_cast<float>((c[0] << 8) + c[1]), 256.0f,
                                       static_cast<float>(c[2]));
        acc[st][tau] = __builtin_fmaf(f, sw[st][gi], acc[st][tau] * alpha[st]);
      }
    }
  };

  // ---- stream the wave's pages ----------------------------------------------
  auto step = [&](const Buf& sb, int p) {
    if (!sb.all_ok || (p + kStep) * kPage > hi || p * kPage < lo)
      compute(sb, p, std::true_type{});
    else
      compute(sb, p, std::false_type{});
  };
  if constexpr (kStage) {
    // Each step's pages land in this wave's LDS stage while the step before
    // it is computed: K and V codes with one 16-byte load per lane each
    // (lane L's bytes at 16 L, the bytes it would load itself), the 128
    // sidecar bytes with one 4-byte load by lanes 0..31 (lanes 32..63 read
    // past the descriptor's end: nothing).  The compiler does not track
    // these loads: vmcnt(0) waits for the staged step (no other vector
    // memory operation is in flight in the loop), lgkmcnt(0) for the reads
    // out of the stage before the next step's loads overwrite it.
    for (int p = pw0; p < pw1; p += kStep) {
      // this step's pages have landed in the stage: into registers, then the
      // next step's loads go to the stage while this one is computed
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      stage_read(buf0, mt);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (p + kStep < pw1)
        stage_issue(p + kStep, [&](int i) { return p + kStep + i < pw1 ? idB[i] : -1; }, mt);
      ids4(p + 2 * kStep, pw1, idB);
      step(buf0, p);
    }
  } else if constexpr (kPrefetch) {
    // The next step's loads go out before this step is computed, so a wave
    // keeps a step in flight while it computes, and the ids of the step after
    // that are fetched meanwhile.  With two sets of heads a step computes long
    // enough that the two waves per SIMD would otherwise leave the SIMD's
    // loads idle much of the time.  The loads are issued whether or not their
    // step exists (its pages then have empty descriptors), so each wait for a
    // step's data leaves the following step's loads in flight.
    Buf buf1;
    for (int p = pw0; p < pw1; p += 2 * kStep) {
      load_with(buf1, p + kStep, [&](int i) { return p + kStep + i < pw1 ? idB[i] : -1; });
      ids4(p + 2 * kStep, pw1, idA);
      step(buf0, p);
      if (p + kStep >= pw1) break;
      load_with(buf0, p + 2 * kStep, [&](int i) { return p + 2 * kStep + i < pw1 ? idA[i] : -1; });
      ids4(p + 3 * kStep, pw1, idB);
      step(buf1, p + kStep);
    }
  } else {
    // One step at a time: its four pages are loaded, then computed.  While a
    // wave computes, the other waves of its SIMD keep loads in flight (with
    // one set of heads an in-register prefetch of the next step measured
    // slower: more VGPRs, fewer waves).
    for (int p = pw0; p < pw1; p += kStep) {
      step(buf0, p);
      if (p + kStep >= pw1) break;
      load_with(buf0, p + kStep, [&](int i) { return p + kStep + i < pw1 ? idB[i] : -1; });
      ids4(p + 2 * kStep, pw1, idB);
    }
  }

  // ---- merge the four waves --------------------------------------------------
  __syncthreads();   // the query scratch is reused below
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const float lt = row_sum16(l_run[st]);
    float zt[kNG];
#pragma unroll
    for (int gi = 0; gi < kNG; ++gi) zt[gi] = row_sum16(z_run[st][gi]);
    const int j = 4 * st + g;            // PV-layout head = row group
#pragma unroll
    for (int tau = 0; tau < kNT; ++tau)
      sm.u.merge.acc[wave][j][pv_channel<D, GS>(n, tau)] = acc[st][tau] + zt[16 * tau / (GS ? GS : 16 * kNT)];
    if (n == 0) {
      sm.u.merge.m[wave][j] = m_run[st];
      sm.u.merge.l[wave][j] = lt;
    }
  }
  __syncthreads();
  if (qwave) {   // wave w < NS finishes heads 4w .. 4w+3, one per row of 16 lanes
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
    // back to the original basis; with several splits each partial is
    // rotated here (the merge is a weighted sum, so it commutes)
    float scale = 1.0f;
    if (a.block > 0) {   // every row takes part: the butterfly reads its neighbours
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
      const int64_t idx = part_base + static_cast<int64_t>(j) * part_mul;
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
  };   // run

  if constexpr (MAP != kMapStream) {
    // Work item (split s, sequence b, KV head), KV head fastest and split
    // slowest, last split first.  Each split is one contiguous run of
    // workgroups that the round-robin dispatch spreads over every XCD and CU
    // (with the split fastest, a period of 2, 4 or 8 left most CUs with the
    // empty splits of short sequences only), and the later splits, busy only
    // for the longest sequences, start first instead of last.
    const int kvh = static_cast<int>(wid % a.num_kv_heads);
    const int b = static_cast<int>((wid / a.num_kv_heads) % a.batch);
    const int s_plan = a.nsplit - 1 - static_cast<int>(wid / a.num_kv_heads / a.batch);
    const int64_t hq0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * G;
    // ---- prologue: loads that do not depend on seq_lens go out first --------
    uint32_t qraw[kC / 2];
    load_query(hq0, qraw);
    // The first step's ids are fetched at once for the range a full-length
    // split of the host's plan gives this wave (a step ahead of the page loads
    // that use them, so they never wait behind vector loads), and again only
    // if the sequence is shorter (its balanced range starts elsewhere) or the
    // split grew.
    const int p0_plan = s_plan * a.split_pages;
    const int per_wave_plan = ((a.split_pages + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
    ConstI32* bt_s = (ConstI32*)(a.block_table + static_cast<int64_t>(b) * a.bt_stride);
    const int cb = p0_plan + wave * per_wave_plan;
    int32_t idA[kStep];
    ids4_of(bt_s, cb, min(p0_plan + a.split_pages, a.bt_stride), idA);
    // pages per split, and the split: last first, unless the device grew the
    // splits (then the later ones are empty, and first-split-first keeps them
    // from holding the machine before the work starts)
    const int sp = BAL ? balanced_split_pages(a.split_pages, a.seq_lens, a.batch, a.max_seq_len,
                                              a.num_kv_heads)
                       : a.split_pages;
    const bool grown = BAL && sp != a.split_pages;
    const int s = grown ? static_cast<int>(wid / a.num_kv_heads / a.batch) : s_plan;
    const int p0 = s * sp;

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    int lo, hi;   // the tokens this pass reads (all of them unless windows take some)
    int4_token_range(len, a.skip_first, a.skip_last, lo, hi);
    const int npg = (hi + kPage - 1) / kPage;
    const int q0 = max(p0, lo / kPage);
    const int p1 = min(npg, p0 + sp);
    if (q0 >= p1 || hi <= lo) {
      if (a.nsplit == 1 && !a.force_partial) {   // empty sequence: zero output rows
        for (int e = tid; e < G * D; e += 64 * kWaves) a.out[hq0 * D + e] = 0.0f;
      }
      return;
    }
    // A sequence whose pages all lie in one split is finished here (normalised
    // output, no partial; the split merge skips its rows): in a ragged batch
    // cut for its longest sequence most rows are such.  Windowed calls always
    // store partials.
    const int busy_splits = (npg - 1) / sp - (lo / kPage) / sp + 1;
    const bool direct = !a.force_partial && (a.nsplit == 1 || busy_splits == 1);
    run(kvh, hq0, bt_s, q0, p1, lo, hi, direct, hq0 * a.part_stride + a.part_slot0 + s, a.part_stride, qraw,
        idA, cb, grown, tid, wave);
  } else {
    // Stream-K: the sequences of the batch, one after another, each as a
    // fixed cost and then its pages, form one run per KV head, cut into
    // sk_ranges ranges; workgroup wid takes range wid / num_kv_heads of KV
    // head wid % num_kv_heads and walks the sequences that meet it.  The
    // ranges are sized for the time the workgroups of each dispatch slot
    // take (stream_range), whatever the lengths: pages, plus what a
    // workgroup spends on each sequence whatever its length (the cost, in
    // pages, of its query prologue, its merge and its last step's unused
    // page slots), so a range of many short sequences holds fewer pages.  A
    // sequence inside one range is finished there; one cut by range ends
    // leaves a partial per range it meets: slot 0 of the range for the piece
    // at the range's start, slot 1 for a piece that starts later (then it
    // runs to the range's end).
    constexpr int kItemCost = NS == 2 ? kStreamItemCost2 : kStreamItemCost1;
    constexpr int kSkew = NS == 1 ? kStreamSkew1 : kStreamSkew2;
    const int kvh = static_cast<int>(wid % a.num_kv_heads);
    const int r = static_cast<int>(wid / a.num_kv_heads);
    const StreamRange rg = stream_range(a.seq_lens, a.batch, a.max_seq_len, a.sk_ranges, a.sk_per_slot, kSkew, r,
                                        kItemCost);
    if (rg.first >= rg.end) return;   // past the batch's work (wave-uniform)
    int b = rg.b, sb = rg.start_b;
    bool later = false;
    int32_t idA[kStep] = {0, 0, 0, 0};
    while (sb < rg.end) {   // sb < total: b < batch
      int len = a.seq_lens[b];
      len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
      const int np = (len + kPage - 1) / kPage;
      const int sp0 = sb + kItemCost;   // the sequence's first page in the run
      const int s0 = max(sp0, rg.first), s1 = min(sp0 + np, rg.end);
      if (np > 0 && s0 < s1) {
        if (kvh == 0 && s0 == sp0) {   // the merge's record of the sequence (its first range is r)
          const int rl = stream_range_of(rg, sp0 + np - 1);
          if (tid == 0) {
            a.sk_rec[2 * b] = r;
            a.sk_rec[2 * b + 1] = 2 * (rl - r + 1) + (sp0 != rg.first ? 1 : 0);
          }
        }
        if (later) __syncthreads();   // the last item's merge is done with the LDS
        later = true;
        const int64_t hq0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * G;
        uint32_t qraw[kC / 2];
        load_query(hq0, qraw);
        ConstI32* bt_s = (ConstI32*)(a.block_table + static_cast<int64_t>(b) * a.bt_stride);
        const bool whole = s0 == sp0 && s1 == sp0 + np;
        const int64_t slot = ((static_cast<int64_t>(kvh) * a.sk_ranges + r) * 2 + (s0 == rg.first ? 0 : 1)) * G;
        // values that depend on the thread alone are computed again for each
        // item rather than held (in registers, or spilled) across the walk
        int tid_l = tid, wave_l = wave;
        asm volatile("" : "+v"(tid_l), "+s"(wave_l));
        run(kvh, hq0, bt_s, s0 - sp0, s1 - sp0, 0, len, whole, slot, 1, qraw, idA, -1, false, tid_l, wave_l);
      }
      sb += np > 0 ? np + kItemCost : 0;
      ++b;
    }
  }
}

}  // namespace q4
}  // namespace kvq

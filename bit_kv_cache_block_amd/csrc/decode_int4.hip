// Read path: split-K paged decode attention over the INT4 cache with the
// dequantization folded into the products ("SAW-INT4", summary page: fused
// attention execution over paged quantized KV; "BitDecoding-FP4", Abstract:
// the query heads of a GQA group stacked into one matrix product per KV page;
// factoring the per-token scale out of the dot product follows the grouping
// idea of "InnerQ", Figure 1).
//
// A workgroup of four waves owns one (sequence b, KV head, split s) and each
// wave streams a quarter of its pages, four pages per step, with
// non-temporal buffer loads (the cache is read once per call).  Per page and
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
#include "decode_int4_launch.hpp"

namespace kvq {

hipError_t launch_decode_int4(const DecodeArgs& a, hipStream_t s) {
  return a.balance ? launch_decode_quant_balanced(a, 4, 0, s) : launch_format<kMapPlanned>(a, 4, 0, s);
}

hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t s) {
  return a.balance ? launch_decode_quant_balanced(a, 8, 0, s) : launch_format<kMapPlanned>(a, 8, 0, s);
}

hipError_t launch_decode_int4g(const DecodeArgs& a, hipStream_t s) {
  return a.balance ? launch_decode_quant_balanced(a, 4, a.group, s) : launch_format<kMapPlanned>(a, 4, a.group, s);
}

}  // namespace kvq

// The INT4, INT8 and grouped INT4 decodes with the host's split plan, and
// with the plan's splits grown on the device from the batch's lengths
// (balanced_split_pages, for small batches cut into many splits).  The two
// mappings are separate kernel instances, so a planned call runs none of the
// balanced code.  The kernel itself is decode_int4_body.hpp.
#include "decode_int4_launch.hpp"

namespace kvq {

hipError_t launch_decode_quant_balanced(const DecodeArgs& a, int bits, int gs, hipStream_t s) {
  return launch_format<kMapBalanced>(a, bits, gs, s);
}

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

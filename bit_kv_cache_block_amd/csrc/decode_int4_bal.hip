// The balanced build of the INT4-family decode: the same kernels compiled to
// size their splits from the batch's lengths on the device
// (balanced_split_pages), for small batches cut into many splits.  Apart from
// the planned build so that the planned calls carry none of its code.
#include "decode_int4_launch.hpp"

namespace kvq {

hipError_t launch_decode_quant_balanced(const DecodeArgs& a, int bits, int gs, hipStream_t s) {
  return launch_format<kMapBalanced>(a, bits, gs, s);
}

}  // namespace kvq

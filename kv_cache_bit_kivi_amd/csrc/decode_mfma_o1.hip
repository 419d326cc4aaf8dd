// Matrix-core decode, lengths uniform across the batch, one key outlier per
// (key group, channel) (the sparse score correction of decode_mfma.hip).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_o1(const DecodeArgs& a, int nw, hipStream_t st) {
  return launch_family<false, false, 1>(a, NoLens{}, nw, st);
}

}  // namespace kivi

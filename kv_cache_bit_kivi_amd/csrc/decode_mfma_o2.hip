// Matrix-core decode, lengths uniform across the batch, two key outliers per
// (key group, channel) (the sparse score correction of decode_mfma.hip).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_o2(const DecodeArgs& a, int nw, hipStream_t st) {
  return launch_family<false, false, 2>(a, NoLens{}, nw, st);
}

}  // namespace kivi

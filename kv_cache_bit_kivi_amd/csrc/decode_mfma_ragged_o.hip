// Matrix-core decode over per-sequence lengths with one or two key outliers
// per (key group, channel) (the sparse score correction of decode_mfma.hip).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_ragged_o(const DecodeArgs& a, const SeqLens& lens, int nw,
                                       hipStream_t st) {
  return a.n_out == 1 ? launch_family<true, false, 1>(a, lens, nw, st)
                      : launch_family<true, false, 2>(a, lens, nw, st);
}

}  // namespace kivi

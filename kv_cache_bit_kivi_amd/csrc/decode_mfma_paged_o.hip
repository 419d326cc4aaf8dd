// Matrix-core decode over a paged store with one or two key outliers per
// (key group, channel); the outlier words of a tile come from the same page
// slice as its codes and metadata.
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_paged_o(const DecodeArgs& a, const SeqLens& lens, int nw,
                                      hipStream_t st) {
  return a.n_out == 1 ? launch_family<true, true, 1>(a, lens, nw, st)
                      : launch_family<true, true, 2>(a, lens, nw, st);
}

}  // namespace kivi

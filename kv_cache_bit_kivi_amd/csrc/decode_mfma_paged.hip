// Matrix-core decode over a paged quantized store: the ragged kernel with
// each tile's codes and metadata read from the page slice that the
// sequence's block table names for it (see PageMap).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_paged(const DecodeArgs& a, const SeqLens& lens, int nw,
                                    hipStream_t st) {
  if (a.rope_theta > 0.f) return launch_decode_mfma_paged_rope(a, lens, nw, st);
  if (a.n_out > 0) return launch_decode_mfma_paged_o(a, lens, nw, st);
  return launch_family<true, true, 0>(a, lens, nw, st);
}

}  // namespace kivi

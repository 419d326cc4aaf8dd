// Matrix-core decode over a paged quantized store: the ragged kernel with
// each tile's codes and metadata read from the page slice that the
// sequence's block table names for it (see PageMap).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_paged(const DecodeArgs& a, const SeqLens& lens, int nw,
                                    hipStream_t st) {
  switch (a.bits) {
    case 1: return launch_bits<1, true, true>(a, lens, nw, st);
    case 2: return launch_bits<2, true, true>(a, lens, nw, st);
    case 3: return launch_bits<3, true, true>(a, lens, nw, st);
    default: return launch_bits<4, true, true>(a, lens, nw, st);
  }
}

}  // namespace kivi

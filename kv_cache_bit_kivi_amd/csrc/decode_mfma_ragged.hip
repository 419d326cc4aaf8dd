// Matrix-core decode over per-sequence lengths (ragged batches): the kernel
// of decode_mfma.hip with each block reading its sequence's quantized and
// residual token counts from the launch's length arrays.
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_ragged(const DecodeArgs& a, const SeqLens& lens, int nw,
                                     hipStream_t st) {
  switch (a.bits) {
    case 1: return launch_bits<1, true, false>(a, lens, nw, st);
    case 2: return launch_bits<2, true, false>(a, lens, nw, st);
    case 3: return launch_bits<3, true, false>(a, lens, nw, st);
    default: return launch_bits<4, true, false>(a, lens, nw, st);
  }
}

}  // namespace kivi

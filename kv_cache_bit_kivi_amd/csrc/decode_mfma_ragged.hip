// Matrix-core decode over per-sequence lengths (ragged batches): the kernel
// of decode_mfma.hip with each block reading its sequence's quantized and
// residual token counts from the launch's length arrays.
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_ragged(const DecodeArgs& a, const SeqLens& lens, int nw,
                                     hipStream_t st) {
  if (a.rope_theta > 0.f) return launch_decode_mfma_ragged_rope(a, lens, nw, st);
  if (a.n_out > 0) return launch_decode_mfma_ragged_o(a, lens, nw, st);
  return launch_family<true, false, 0>(a, lens, nw, st);
}

}  // namespace kivi

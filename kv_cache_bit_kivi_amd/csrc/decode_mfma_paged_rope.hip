// Matrix-core decode over a paged store with pre-RoPE keys (positions are
// logical token indices; pages do not move them).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_paged_rope(const DecodeArgs& a, const SeqLens& lens, int nw,
                                         hipStream_t st) {
  return launch_family<true, true, 0, true>(a, lens, nw, st);
}

}  // namespace kivi

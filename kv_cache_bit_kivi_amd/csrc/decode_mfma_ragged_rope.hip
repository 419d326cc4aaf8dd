// Matrix-core decode over per-sequence lengths with pre-RoPE keys (a key's
// position is its index in its own sequence).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_ragged_rope(const DecodeArgs& a, const SeqLens& lens, int nw,
                                          hipStream_t st) {
  return launch_family<true, false, 0, true>(a, lens, nw, st);
}

}  // namespace kivi

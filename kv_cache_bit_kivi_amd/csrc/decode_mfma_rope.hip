// Matrix-core decode, lengths uniform across the batch, pre-RoPE keys (the
// ROPE variant of decode_mfma_kernel: keys scored on the VALU with the rotary
// embedding applied at each key's position, values on the matrix cores).
#include "decode_mfma_impl.h"

namespace kivi {

hipError_t launch_decode_mfma_rope(const DecodeArgs& a, int nw, hipStream_t st) {
  return launch_family<false, false, 0, true>(a, NoLens{}, nw, st);
}

}  // namespace kivi

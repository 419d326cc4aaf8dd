// Decode attention on the mixed cache with matrix-core (MFMA) contractions,
// for head_dim 128, group 32, 1- to 4-bit codes and GQA ratio r in {1,2,4,8}.
//
// Method (study.space summary of "KIVI: A Tuning-Free Asymmetric 2bit
// Quantization for KV Cache"): the scores of the quantized grouped part are a
// tiled matrix product, and the full-precision residual part is combined with
// them.  With keys k = c*s + z per (channel, 32-token group) and values
// v = c*s + z per (token, 32-channel group), binary32 accumulation:
//   score_t = sum_d q'_d c_td + beta,   q'_d = sc * q_d * s_d,
//                                       beta = sc * sum_d q_d * z_d
//   o_d     = sum_t p'_t c_td + Gamma,  p'_t = p_t * s_t,
//                                       Gamma = sum_t p_t * z_t
// (sc = softmax scale * log2(e): scores live in the log2 domain, p = 2^(s-m)).
//
// Both contractions run on 16x16x32 MFMAs.  Operand B is the codes, converted
// exactly (2-bit codes via the e2m1 convert with scale 2 on nibble planes,
// 1-bit codes likewise on the nibble bit-planes of their words, 3-bit codes as
// their 2-bit plane plus their high-bit plane converted with scale 8, i.e. four
// times the high bit, accumulated with the same factor operand; 4-bit codes
// via the e4m3 convert with scale 2^9).  Operand A is the factor q' (or p'), split
// into hi + lo rows so the products keep at least 16 significant bits:
//   keys (fp16):   A = rows (head, hi|lo) x 32 channels, B = 32 channels x 16
//                  tokens; hi = q' rounded toward zero, lo = the remainder.
//                  The query is normalised per wave by a power of two so that
//                  |q'| < 2^16 and the fp16 hi part never overflows.
//   values (bf16): A = rows (head, hi|lo) x 32 tokens, B = 32 tokens x 16
//                  channels; hi = p' truncated to bf16, lo = the remainder.
//                  bf16 keeps binary32's exponent range, so p' needs no
//                  normalisation however small or large the value scales are.
// The 8 K-slots a lane supplies map to code positions in the order the
// converts produce them (k_pos / v_pos); A is written to LDS in that order.
// The online-softmax reference moves only when a score exceeds it by more
// than 2^8 (p <= 256), so the accumulators are rarely rescaled.
// Residual keys (fp16) feed the MFMA directly; residual values use the VALU.
//
// Work: one block of NW waves per (b*Hkv + h, split).  The waves take the
// split's 64-token value tiles as their loads return (one LDS counter per
// block; fixed contiguous runs for deterministic caches),
// and each owns a slice of the residual.  Per tile a wave computes the key
// scores into LDS, updates the running maximum (online softmax; accumulators
// are rescaled only when the maximum grows) and accumulates P.V.  Codes and metadata arrive through raw buffer loads, 16
// bytes per lane (8 for binary16 metadata, widened to binary32 when the tile
// is computed), one or two tiles ahead of the compute; absent tiles and
// tokens are loaded out of range (zeros, no memory access) instead of being
// branched around, so the completion counter never forces a full drain.
// Codes are staged through LDS and re-read in the MFMA operand layout.  The
// block merges its waves in LDS; one split writes fp16 output, more splits
// write (max, sum, o) partials for the combine kernel.
//
// Key outliers ("KVQuant: Towards 10 Million Context Length LLM Inference
// with KV Cache Quantization", codewithpapers.app paper page, abstract:
// dense-and-sparse keys, outliers isolated per vector): the dense code of an
// outlier is 0, so the MFMA score already counts q_d * z_d for it; the kernel
// adds q_d * (kept value - z_d) per outlier at its token, a sparse correction
// of the score tile, before the tile maximum is taken.
//
// Pre-RoPE keys (same page: keys quantized before the rotary positional
// embedding): the rotation of a key depends on its position, so the key
// product is no longer a shared-operand matrix product.  These variants score
// keys lane-per-token on the VALU in binary32 (dequantize, rotate, dot) while
// values keep the matrix-core path; see the ROPE parameter of
// decode_mfma_kernel.
#include "decode_mfma_impl.h"

namespace kivi {

bool decode_mfma_supported(int D, int G, int r, int n_out, bool rope) {
  return D == kD && G == kG && (r == 1 || r == 2 || r == 4 || r == 8) && n_out >= 0 &&
         n_out <= kMfmaMaxOutliers && !(rope && n_out > 0);
}

namespace {
// (the binary32-metadata variant without outliers; every variant of one
// (bits, r, block) shares its register budget and LDS size, hence its
// occupancy)
template <int BITS, int R, int NW>
int occupancy_of() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&decode_mfma_kernel<BITS, R, NW, false, false, false, 0, false>),
          NW * 64, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}
template <int BITS, int R>
int occupancy_r(int nw) {
  return block_waves<R>(nw) == 8 ? occupancy_of<BITS, R, (R < 8 ? 8 : 4)>()
                                 : occupancy_of<BITS, R, 4>();
}
template <int BITS>
int occupancy_bits(int r, int nw) {
  switch (r) {
    case 1: return occupancy_r<BITS, 1>(nw);
    case 2: return occupancy_r<BITS, 2>(nw);
    case 4: return occupancy_r<BITS, 4>(nw);
    default: return occupancy_r<BITS, 8>(nw);
  }
}
}  // namespace

int decode_mfma_blocks_per_cu(int bits, int r, int nw) {
  // cached per (bits, r, requested waves): queried once per process
  static std::atomic<int> cache[4][4][3];
  const int bi = bits - 1;
  const int ri = r == 1 ? 0 : (r == 2 ? 1 : (r == 4 ? 2 : 3));
  const int wi = nw >= 8 ? 1 : 0;
  int c = cache[bi][ri][wi].load(std::memory_order_relaxed);
  if (c == 0) {
    switch (bits) {
      case 1: c = occupancy_bits<1>(r, nw); break;
      case 2: c = occupancy_bits<2>(r, nw); break;
      case 3: c = occupancy_bits<3>(r, nw); break;
      default: c = occupancy_bits<4>(r, nw); break;
    }
    cache[bi][ri][wi].store(c, std::memory_order_relaxed);
  }
  return c;
}

int decode_mfma_block_waves(int r, int nw) {
  switch (r) {
    case 1: return block_waves<1>(nw);
    case 2: return block_waves<2>(nw);
    case 4: return block_waves<4>(nw);
    default: return block_waves<8>(nw);
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int nw, hipStream_t st) {
  if (a.rope_theta > 0.f) return launch_decode_mfma_rope(a, nw, st);
  if (a.n_out == 1) return launch_decode_mfma_o1(a, nw, st);
  if (a.n_out == 2) return launch_decode_mfma_o2(a, nw, st);
  return launch_family<false, false, 0>(a, NoLens{}, nw, st);
}

}  // namespace kivi

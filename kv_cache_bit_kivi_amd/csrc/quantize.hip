// Quantize kernels: per-channel keys, per-token values, and token copies.
//
// Method: "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
// (mlsanity paper page, Abstract): keys are quantized per channel, values per
// token, with asymmetric low-bit codes; study.space summary: key groups span
// consecutive tokens and new tokens are appended along the token axis.
//
// Codec, per group of G values, b in {1, 2, 3, 4} bits (bit-exact contract,
// IEEE binary32, built with
// -ffp-contract=off and correctly rounded division):
//   mn, mx   : strict-comparison scan in index order (first extremum wins);
//   mx == mn : scale 0, zero mn, codes 0 (the group dequantizes exactly);
//   else     : range = mx - mn; s = range / (2^b - 1); z = mn;
//              code = min(rint((x - z) / s), 2^b - 1), rint = half-to-even.
// Half-width metadata stores s and z rounded to binary16 (nearest even) after
// the codes have been computed from the binary32 values.
// Key outliers ("KVQuant: Towards 10 Million Context Length LLM Inference
// with KV Cache Quantization", codewithpapers.app paper page, abstract:
// outliers are isolated per vector so they do not stretch the quantization
// range), n_out > 0: in each key group (one channel over G tokens) the n_out
// entries of largest |x| (ties: the lower token) are written exactly as
// (i << 16) | fp16 bits, in increasing token i, and left out of mn / mx; their
// codes are 0 (the kernel stores mn in their place before encoding, which
// encodes to 0 exactly).
// Each block stages its fp16 tile in LDS with 16-byte loads, computes the
// group statistics from LDS, then writes whole 32-bit code words, so any
// number of blocks can run concurrently without read-modify-write.
// The LIST variants work on a list of sequences with per-sequence token
// counts and offsets (ragged batches: prefill and per-sequence flushes).
#include <math.h>

#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <int BITS>
__device__ __forceinline__ void group_stats(float mn, float mx, float* s_out) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  if (mx == mn) {
    *s_out = 0.0f;
  } else {
    float range = mx - mn;
    *s_out = range / qmax;
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t encode(float x, float s, float z) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  if (s == 0.0f) return 0u;
  float u = x - z;
  float v = u / s;
  float c = rintf(v);
  if (c > qmax) c = qmax;
  return (uint32_t)c;
}

// metadata store: binary32, or binary16 rounded to nearest even
template <bool MH>
__device__ __forceinline__ void put_meta(void* p, size_t i, float x) {
  if constexpr (MH)
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, (_Float16)x);
  else
    static_cast<float*>(p)[i] = x;
}

// Packed layout of a row of n codes (a key row: one token's D channels; a
// value row: one channel's 64 tokens of a tile), n*BITS/32 words:
//   2, 4 bits: position p at word p/E, bit BITS*(p%E), E = 32/BITS;
//   1 bit    : word p/32, bit beta(p%32);
//   3 bits   : code = lo + 4*hi; lo at word p/16, bits 2*(p%16), then the hi
//              bits at word n/16 + p/32, bit beta(p%32).
// beta keeps the nibble bit-planes of a one-bit word on the code positions
// of a two-bit word's planes (the decode's operand conversion relies on it).
__device__ __forceinline__ int beta(int p) { return 4 * ((p & 15) >> 1) + 2 * (p >> 4) + (p & 1); }

// Word k (0 .. n*BITS/32 - 1) of a row from its codes: code(p) gives the code
// of position p of the row.
template <int BITS, class F>
__device__ __forceinline__ uint32_t pack_word(int n, int k, F code) {
  uint32_t w = 0;
  if constexpr (BITS == 1) {
#pragma unroll
    for (int q = 0; q < 32; q++) w |= code(32 * k + q) << beta(q);
  } else if constexpr (BITS == 3) {
    if (k < n / 16) {
#pragma unroll
      for (int q = 0; q < 16; q++) w |= (code(16 * k + q) & 3u) << (2 * q);
    } else {
      const int kh = k - n / 16;
#pragma unroll
      for (int q = 0; q < 32; q++) w |= (code(32 * kh + q) >> 2) << beta(q);
    }
  } else {
    constexpr int E = 32 / BITS;
#pragma unroll
    for (int e = 0; e < E; e++) w |= code(E * k + e) << (BITS * e);
  }
  return w;
}

struct NoList {};
template <bool LIST>
using ListT = std::conditional_t<LIST, SeqList, NoList>;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 16-byte copy with a non-temporal (read-once) source load
__device__ __forceinline__ void copy16_nt(void* dst, const void* src) {
  *reinterpret_cast<u32x4_t*>(dst) =
      __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
}

// One block per (group of G source tokens, b*H + h), or per (group, item*H +
// h) over a sequence list (blocks past the item's token count exit).  PG: the
// destination is the page slice the block table names for the group's
// tokens (a group never straddles a page; a page outside the pool is skipped).
template <int BITS, bool MH, bool LIST, bool PG>
__global__ void __launch_bounds__(256)
quantize_k_kernel(const uint16_t* __restrict__ k, int D, int G, int cap, int in_stride,
                  int dst_off, uint32_t* __restrict__ codes, void* __restrict__ scale,
                  void* __restrict__ zero, uint32_t* __restrict__ outl, int n_out, int H,
                  ListT<LIST> list, PageMap pm) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);       // [G][D]
  float* s_sc = reinterpret_cast<float*>(tile + G * D);      // [D]
  float* s_zr = s_sc + D;                                    // [D]
  const int g = blockIdx.x;
  size_t bh = blockIdx.y;
  int seq = 0;
  if constexpr (LIST) {
    const int item = blockIdx.y / H;
    if (g * G >= list.a[item]) return;   // the whole block: uniform
    seq = list.seq[item];
    bh = (size_t)seq * H + blockIdx.y % H;
    dst_off = list.b[item];
  }
  // destination: tokens [otok, otok + G) of plane ob, a plane of ocap tokens
  size_t ob = bh;
  int otok = dst_off + g * G, ocap = cap;
  if constexpr (PG) {
    if (!page_slot(pm, seq, (int)(bh % H), H, otok, ob, otok)) return;   // uniform
    ocap = pm.page_tokens;
  }
  const uint4* src = reinterpret_cast<const uint4*>(k + (bh * in_stride + (size_t)g * G) * D);
  for (int i = threadIdx.x; i < G * D / 8; i += blockDim.x)
    copy16_nt(reinterpret_cast<uint4*>(tile) + i, src + i);
  __syncthreads();

  const size_t gg = (size_t)(otok / G);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float mn, mx;
    if (n_out == 0) {
      mn = mx = h2f(tile[d]);
      for (int i = 1; i < G; i++) {
        float x = h2f(tile[i * D + d]);
        if (x < mn) mn = x;
        if (x > mx) mx = x;
      }
    } else {
      // outlier positions as a bit set over the group's G <= 128 tokens; each
      // pass takes the first largest |x| not yet taken
      uint64_t m0 = 0, m1 = 0;
      auto taken = [&](int i) { return ((i < 64 ? m0 >> i : m1 >> (i - 64)) & 1u) != 0; };
      for (int j = 0; j < n_out; j++) {
        int best = 0;
        float bm = -1.0f;
        for (int i = 0; i < G; i++) {
          const float a = fabsf(h2f(tile[i * D + d]));
          if (a > bm && !taken(i)) {
            bm = a;
            best = i;
          }
        }
        if (best < 64) m0 |= 1ull << best; else m1 |= 1ull << (best - 64);
      }
      mn = INFINITY;
      mx = -INFINITY;
      for (int i = 0; i < G; i++) {
        if (taken(i)) continue;
        float x = h2f(tile[i * D + d]);
        if (x < mn) mn = x;
        if (x > mx) mx = x;
      }
      // the sparse row, then mn in the outliers' places (code 0)
      uint32_t* orow = outl + ((ob * (ocap / G) + gg) * n_out) * D + d;
      const uint16_t mn_h = __builtin_bit_cast(uint16_t, (_Float16)mn);   // exact
      int j = 0;
      for (int i = 0; i < G; i++) {
        if (!taken(i)) continue;
        orow[(size_t)j * D] = ((uint32_t)i << 16) | tile[i * D + d];
        tile[i * D + d] = mn_h;
        j++;
      }
    }
    float s;
    group_stats<BITS>(mn, mx, &s);
    s_sc[d] = s;
    s_zr[d] = mn;
    size_t m = (ob * (ocap / G) + gg) * D + d;
    put_meta<MH>(scale, m, s);
    put_meta<MH>(zero, m, mn);
  }
  __syncthreads();

  const int W = D * BITS / 32;   // words per key row
  uint32_t* dst = codes + (ob * ocap + otok) * W;
  for (int it = threadIdx.x; it < G * W; it += blockDim.x) {
    const int i = it / W, w = it % W;
    dst[it] = pack_word<BITS>(D, w, [&](int d) {
      return encode<BITS>(h2f(tile[i * D + d]), s_sc[d], s_zr[d]);
    });
  }
}

// One block per (32 source tokens, b*H + h) (or per item, as above).  Value
// codes are stored in 64-token tiles, channel-major: word ((t/64)*D + d)*(64/E)
// + (t%64)/E.
template <int BITS, bool MH, bool LIST, bool PG>
__global__ void __launch_bounds__(256)
quantize_v_kernel(const uint16_t* __restrict__ v, int D, int G, int cap, int in_stride,
                  int dst_off, uint32_t* __restrict__ codes, void* __restrict__ scale,
                  void* __restrict__ zero, int H, ListT<LIST> list, PageMap pm) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);       // [32][D]
  const int NG = D / G;
  float* s_sc = reinterpret_cast<float*>(tile + 32 * D);     // [32][NG]
  float* s_zr = s_sc + 32 * NG;
  const int blk = blockIdx.x;
  size_t bh = blockIdx.y;
  int seq = 0;
  if constexpr (LIST) {
    const int item = blockIdx.y / H;
    if (blk * 32 >= list.a[item]) return;   // the whole block: uniform
    seq = list.seq[item];
    bh = (size_t)seq * H + blockIdx.y % H;
    dst_off = list.b[item];
  }
  // destination: tokens [t_base, t_base + 32) of plane ob (ocap tokens)
  size_t ob = bh;
  int t_base = dst_off + blk * 32, ocap = cap;
  if constexpr (PG) {
    if (!page_slot(pm, seq, (int)(bh % H), H, t_base, ob, t_base)) return;   // uniform
    ocap = pm.page_tokens;
  }
  const uint4* src = reinterpret_cast<const uint4*>(v + (bh * in_stride + (size_t)blk * 32) * D);
  for (int i = threadIdx.x; i < 32 * D / 8; i += blockDim.x)
    copy16_nt(reinterpret_cast<uint4*>(tile) + i, src + i);
  __syncthreads();

  for (int it = threadIdx.x; it < 32 * NG; it += blockDim.x) {
    const int t = it / NG, j = it % NG;
    const uint16_t* row = tile + t * D + j * G;
    float mn = h2f(row[0]), mx = mn;
    for (int i = 1; i < G; i++) {
      float x = h2f(row[i]);
      if (x < mn) mn = x;
      if (x > mx) mx = x;
    }
    float s;
    group_stats<BITS>(mn, mx, &s);
    s_sc[it] = s;
    s_zr[it] = mn;
    size_t m = (ob * ocap + t_base + t) * NG + j;
    put_meta<MH>(scale, m, s);
    put_meta<MH>(zero, m, mn);
  }
  __syncthreads();

  constexpr int WPC = 2 * BITS;   // words per channel per 64-token tile
  uint32_t* plane = codes + ob * ((size_t)ocap * D * BITS / 32);
  const size_t tile_idx = (size_t)(t_base / 64);
  const int half = (t_base % 64) / 32;   // this block's half of the tile
  // the words of a channel's tile row that hold only this half's tokens: of
  // the 2*BITS words, those whose positions all lie in [32*half, 32*half+32)
  for (int it = threadIdx.x; it < D * BITS; it += blockDim.x) {
    const int d = it / BITS, k = it % BITS;
    const int j = d / G;
    int rw;   // row word index
    if constexpr (BITS == 1) {
      rw = half;
    } else if constexpr (BITS == 3) {
      rw = k < 2 ? 2 * half + k : 4 + half;
    } else {
      rw = half * BITS + k;
    }
    plane[(tile_idx * D + d) * WPC + rw] = pack_word<BITS>(64, rw, [&](int p) {
      const int t = p - 32 * half;   // token of this block
      return encode<BITS>(h2f(tile[t * D + d]), s_sc[t * NG + j], s_zr[t * NG + j]);
    });
  }
}

template <bool LIST>
__global__ void __launch_bounds__(256)
copy_tokens_kernel(const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
                   int src_stride, int t0, uint16_t* __restrict__ k_dst,
                   uint16_t* __restrict__ v_dst, int dst_stride, int slot0, int n, int D, int H,
                   ListT<LIST> list) {
  size_t bh = blockIdx.y;
  if constexpr (LIST) {
    const int item = blockIdx.y / H;
    bh = (size_t)list.seq[item] * H + blockIdx.y % H;
    t0 = list.a[item];
    slot0 = list.b[item];
    n = list.c[item];
  }
  const int per_tok = D / 8;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n * per_tok;
       i += gridDim.x * blockDim.x) {
    const int t = i / per_tok, c = i % per_tok;
    const size_t so = ((bh * src_stride + t0 + t) * D) / 8 + c;
    const size_t dd = ((bh * dst_stride + slot0 + t) * D) / 8 + c;
    copy16_nt(reinterpret_cast<uint4*>(k_dst) + dd, reinterpret_cast<const uint4*>(k_src) + so);
    copy16_nt(reinterpret_cast<uint4*>(v_dst) + dd, reinterpret_cast<const uint4*>(v_src) + so);
  }
}

// f(bits, metadata-half) with both as compile-time constants
template <class F>
void dispatch_bits(int bits, int mh, F f) {
  auto with_mh = [&](auto B) {
    if (mh) f(B, std::true_type{}); else f(B, std::false_type{});
  };
  switch (bits) {
    case 1: with_mh(std::integral_constant<int, 1>{}); break;
    case 2: with_mh(std::integral_constant<int, 2>{}); break;
    case 3: with_mh(std::integral_constant<int, 3>{}); break;
    default: with_mh(std::integral_constant<int, 4>{}); break;
  }
}

}  // namespace

hipError_t launch_quantize_k(const uint16_t* k, int B, int H, int D, int bits, int G, int cap,
                             int in_stride, int ntok, int dst_off, uint32_t* codes,
                             void* scale, void* zero, int mh, uint32_t* outl, int n_out,
                             hipStream_t st) {
  dim3 grid(ntok / G, B * H);
  size_t lds = (size_t)G * D * 2 + 2 * D * sizeof(float);
  auto go = [&](auto kernel) {
    kernel<<<grid, 256, lds, st>>>(k, D, G, cap, in_stride, dst_off, codes, scale, zero, outl,
                                   n_out, H, NoList{}, PageMap{});
  };
  dispatch_bits(bits, mh, [&](auto B, auto M) { go(quantize_k_kernel<B.value, M.value, false, false>); });
  return hipGetLastError();
}

hipError_t launch_quantize_v(const uint16_t* v, int B, int H, int D, int bits, int G, int cap,
                             int in_stride, int ntok, int dst_off, uint32_t* codes,
                             void* scale, void* zero, int mh, hipStream_t st) {
  dim3 grid(ntok / 32, B * H);
  size_t lds = (size_t)32 * D * 2 + 2 * 32 * (D / G) * sizeof(float);
  auto go = [&](auto kernel) {
    kernel<<<grid, 256, lds, st>>>(v, D, G, cap, in_stride, dst_off, codes, scale, zero, H,
                                   NoList{}, PageMap{});
  };
  dispatch_bits(bits, mh, [&](auto B, auto M) { go(quantize_v_kernel<B.value, M.value, false, false>); });
  return hipGetLastError();
}

hipError_t launch_quantize_k_list(const uint16_t* k, const SeqList& list, int H, int D, int bits,
                                  int G, int cap, int in_stride, int ntok_max, uint32_t* codes,
                                  void* scale, void* zero, int mh, uint32_t* outl, int n_out,
                                  hipStream_t st) {
  if (list.n == 0 || ntok_max == 0) return hipSuccess;
  dim3 grid(ntok_max / G, list.n * H);
  size_t lds = (size_t)G * D * 2 + 2 * D * sizeof(float);
  auto go = [&](auto kernel) {
    kernel<<<grid, 256, lds, st>>>(k, D, G, cap, in_stride, 0, codes, scale, zero, outl, n_out,
                                   H, list, PageMap{});
  };
  dispatch_bits(bits, mh, [&](auto B, auto M) { go(quantize_k_kernel<B.value, M.value, true, false>); });
  return hipGetLastError();
}

hipError_t launch_quantize_v_list(const uint16_t* v, const SeqList& list, int H, int D, int bits,
                                  int G, int cap, int in_stride, int ntok_max, uint32_t* codes,
                                  void* scale, void* zero, int mh, hipStream_t st) {
  if (list.n == 0 || ntok_max == 0) return hipSuccess;
  dim3 grid(ntok_max / 32, list.n * H);
  size_t lds = (size_t)32 * D * 2 + 2 * 32 * (D / G) * sizeof(float);
  auto go = [&](auto kernel) {
    kernel<<<grid, 256, lds, st>>>(v, D, G, cap, in_stride, 0, codes, scale, zero, H, list,
                                   PageMap{});
  };
  dispatch_bits(bits, mh, [&](auto B, auto M) { go(quantize_v_kernel<B.value, M.value, true, false>); });
  return hipGetLastError();
}

hipError_t launch_quantize_k_paged(const uint16_t* k, const SeqList& list, const PageMap& pm,
                                   int H, int D, int bits, int G, int in_stride, int ntok_max,
                                   uint32_t* codes, void* scale, void* zero, int mh,
                                   uint32_t* outl, int n_out, hipStream_t st) {
  if (list.n == 0 || ntok_max == 0) return hipSuccess;
  dim3 grid(ntok_max / G, list.n * H);
  size_t lds = (size_t)G * D * 2 + 2 * D * sizeof(float);
  auto go = [&](auto kernel) {
    kernel<<<grid, 256, lds, st>>>(k, D, G, 0, in_stride, 0, codes, scale, zero, outl, n_out, H,
                                   list, pm);
  };
  dispatch_bits(bits, mh, [&](auto B, auto M) { go(quantize_k_kernel<B.value, M.value, true, true>); });
  return hipGetLastError();
}

hipError_t launch_quantize_v_paged(const uint16_t* v, const SeqList& list, const PageMap& pm,
                                   int H, int D, int bits, int G, int in_stride, int ntok_max,
                                   uint32_t* codes, void* scale, void* zero, int mh,
                                   hipStream_t st) {
  if (list.n == 0 || ntok_max == 0) return hipSuccess;
  dim3 grid(ntok_max / 32, list.n * H);
  size_t lds = (size_t)32 * D * 2 + 2 * 32 * (D / G) * sizeof(float);
  auto go = [&](auto kernel) {
    kernel<<<grid, 256, lds, st>>>(v, D, G, 0, in_stride, 0, codes, scale, zero, H, list, pm);
  };
  dispatch_bits(bits, mh, [&](auto B, auto M) { go(quantize_v_kernel<B.value, M.value, true, true>); });
  return hipGetLastError();
}

hipError_t launch_copy_tokens(const uint16_t* k_src, const uint16_t* v_src, int src_stride,
                              int t0, uint16_t* k_dst, uint16_t* v_dst, int dst_stride,
                              int slot0, int n, int B, int H, int D, hipStream_t st) {
  const int items = n * D / 8;
  dim3 grid((items + 255) / 256, B * H);
  copy_tokens_kernel<false><<<grid, 256, 0, st>>>(k_src, v_src, src_stride, t0, k_dst, v_dst,
                                                  dst_stride, slot0, n, D, H, NoList{});
  return hipGetLastError();
}

hipError_t launch_copy_tokens_list(const uint16_t* k_src, const uint16_t* v_src, int src_stride,
                                   uint16_t* k_dst, uint16_t* v_dst, int dst_stride,
                                   const SeqList& list, int n_max, int H, int D, hipStream_t st) {
  if (list.n == 0 || n_max == 0) return hipSuccess;
  const int items = n_max * D / 8;
  dim3 grid((items + 255) / 256, list.n * H);
  copy_tokens_kernel<true><<<grid, 256, 0, st>>>(k_src, v_src, src_stride, 0, k_dst, v_dst,
                                                 dst_stride, 0, 0, D, H, list);
  return hipGetLastError();
}

}  // namespace kivi

// Codec kernels: per-channel keys, per-token values, residual copies.
//
// Method: "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
// (mlsanity paper page, Abstract): keys are quantized per channel, values per
// token, with asymmetric low-bit codes; study.space summary: key groups span
// consecutive tokens and new tokens are appended along the token axis.
//
// Codec, per group of G values, b in {1, 2, 3, 4} bits (bit-exact contract,
// IEEE binary32, built with -ffp-contract=off and correctly rounded division):
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
//
// One launch does a whole prefill or flush: its blocks are key groups (G
// tokens x D channels of one plane), value chunks (32 tokens x D channels)
// and residual-copy chunks, told apart by blockIdx.x.  A quantizing block
// stages its fp16 tile in LDS with 16-byte loads, computes the group
// statistics with several threads per group (partial extremes combined in
// index order), writes every code as a byte into an LDS code tile, and then
// packs whole 32-bit code words from it, so blocks never share a word.
//
// Encoding without a division per element: with r = rcp(s) (v_rcp_f32,
// within one ulp of 1/s) the quotient q = fl(u * r) is within 1.5 * 2^-23 of
// u / s relatively, and the reference's correctly rounded quotient
// v = fl(u / s) within 2^-24; for |u / s| < 16 (at most 2^b - 1 + 2^-20 here)
// |q - v| < 2^-18.  When q lies more than kTieBand = 2^-12 from every
// half-integer, v lies on the same side of the same half-integers, so
// rint(v) = rint(q); otherwise the element takes the reference's own steps
// (the correctly rounded division).  u and s are normal binary32 numbers
// (differences of binary16 values, s >= 2^-24 / 15), so no denormal case
// arises.  The codes are therefore bit-identical to the reference's.
#include <math.h>

#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int kThreads = 256;
// the shape whose launches are compiled with constant sizes (head_dim 128,
// group 32); every other shape takes them at run time
constexpr int kFixD = 128, kFixG = 32;
constexpr float kTieBand = 1.0f / 4096.0f;

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <int BITS>
__device__ __forceinline__ float group_scale(float mn, float mx) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  if (mx == mn) return 0.0f;
  float range = mx - mn;
  return range / qmax;
}

// code = min(rint(fl((x - z) / s)), 2^b - 1) (the reference's steps with a
// correctly rounded division; 0 when s == 0) for four values of one group,
// from the reciprocal r = rcp(s) (0 when s == 0): see the top of this file
// for why the result is the same.  One branch covers the rare case that any
// of the four lies near a half-integer: then all four take the correctly
// rounded division, which the others would agree with anyway.
// The clamp to 2^b - 1 is only needed on the exact path: there q stays below
// (2^b - 1)(1 + 2^-20) (u <= mx - mn and s >= fl(mx - mn) / (2^b - 1) within
// 2^-23), so a q that passes the band test rounds to at most 2^b - 1.
template <int BITS>
__device__ __forceinline__ void encode4(const float (&x)[4], float s, float z, float r,
                                        uint32_t (&c)[4]) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  float u[4], cf[4], dev[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    u[e] = x[e] - z;
    const float q = u[e] * r;
    cf[e] = rintf(q);
    dev[e] = fabsf(q - cf[e]);
  }
  // (one compare for all four: the largest distance from an integer)
  if (fmaxf(fmaxf(dev[0], dev[1]), fmaxf(dev[2], dev[3])) > 0.5f - kTieBand) {
#pragma unroll
    for (int e = 0; e < 4; e++) cf[e] = fminf(rintf(u[e] / s), qmax);   // (s != 0 here)
  }
#pragma unroll
  for (int e = 0; e < 4; e++) c[e] = (uint32_t)cf[e];
}

// metadata store: binary32, or binary16 rounded to nearest even
template <bool MH>
__device__ __forceinline__ void put_meta(void* p, size_t i, float x) {
  if constexpr (MH)
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, (_Float16)x);
  else
    static_cast<float*>(p)[i] = x;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2v as_h2(uint32_t w) { return __builtin_bit_cast(h2v, w); }

// Group extremes.  The reference scans in index order with strict
// comparisons, so of equal values the first one stays; that differs from
// min / max instructions only for +0 / -0, so the kernels take extremes with
// packed binary16 min / max (binary16 comparisons order exactly as binary32
// ones) and replace a zero extreme by the first zero in index order:
// first_zero returns the first of n values p[0], p[stride], ... that is zero.
__device__ __forceinline__ float first_zero(const uint16_t* p, int stride, int n) {
  for (int i = 0; i < n; i++) {
    const float x = h2f(p[i * stride]);
    if (x == 0.0f) return x;
  }
  return 0.0f;
}

// Packed layout of a row of n codes (a key row: one token's D channels; a
// value row: one channel's 64 tokens of a tile), n*BITS/32 words:
//   2, 4 bits: position p at word p/E, bit BITS*(p%E), E = 32/BITS;
//   1 bit    : word p/32, bit beta(p%32);
//   3 bits   : code = lo + 4*hi; lo at word p/16, bits 2*(p%16), then the hi
//              bits at word n/16 + p/32, bit beta(p%32).
// beta keeps the nibble bit-planes of a one-bit word on the code positions
// of a two-bit word's planes (the decode's operand conversion relies on it).
__device__ __forceinline__ constexpr int beta(int p) {
  return 4 * ((p & 15) >> 1) + 2 * (p >> 4) + (p & 1);
}

// n consecutive dwords of LDS from a 4-byte aligned address
template <int N>
__device__ __forceinline__ void ld_dwords(const uint8_t* p, uint32_t* w) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
  for (int i = 0; i < N; i++) w[i] = q[i];
}

// Word k of a row of n codes held one per byte in LDS (row[p] = code of
// position p, the row 4-byte aligned; only the bytes the word covers are
// read).
template <int BITS>
__device__ __forceinline__ uint32_t pack_bytes(const uint8_t* row, int n, int k) {
  auto byte = [](const uint32_t* w, int e) -> uint32_t { return (w[e >> 2] >> (8 * (e & 3))) & 0xFFu; };
  uint32_t wd[8];
  uint32_t w = 0;
  if constexpr (BITS == 2) {
    // four codes (< 4) in the bytes of y -> their 8-bit group: y | y >> 6
    // puts c0 | c1 << 2 in byte 0 and c2 | c3 << 2 in byte 2
    uint32_t x[4];
    ld_dwords<4>(row + 16 * k, x);
    auto sq = [](uint32_t y) -> uint32_t {
      const uint32_t t = y | (y >> 6);
      return (t & 0xFu) | ((t >> 12) & 0xF0u);
    };
    w = sq(x[0]) | (sq(x[1]) << 8) | (sq(x[2]) << 16) | (sq(x[3]) << 24);
  } else if constexpr (BITS == 4) {
    // two codes (< 16) per 16-bit half: y | y >> 4 puts c0 | c1 << 4 in
    // byte 0 and c2 | c3 << 4 in byte 2
    uint32_t x[2];
    ld_dwords<2>(row + 8 * k, x);
    auto sq = [](uint32_t y) -> uint32_t {
      const uint32_t t = y | (y >> 4);
      return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
    };
    w = sq(x[0]) | (sq(x[1]) << 16);
  } else if constexpr (BITS == 1) {
    ld_dwords<8>(row + 32 * k, wd);
#pragma unroll
    for (int q = 0; q < 32; q++) w |= byte(wd, q) << beta(q);
  } else {
    if (k < n / 16) {   // two-bit plane of the low bits
      ld_dwords<4>(row + 16 * k, wd);
#pragma unroll
      for (int e = 0; e < 16; e++) w |= (byte(wd, e) & 3u) << (2 * e);
    } else {            // one-bit plane of the high bit
      const int kh = k - n / 16;
      ld_dwords<8>(row + 32 * kh, wd);
#pragma unroll
      for (int q = 0; q < 32; q++) w |= (byte(wd, q) >> 2) << beta(q);
    }
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

// LDS bytes of a key group block and of a value chunk block
__host__ __device__ constexpr int key_parts(int D) { return kThreads / D; }
__host__ __device__ constexpr int val_pairs(int D, int G) { return 32 * (D / G); }
__host__ __device__ constexpr int val_parts(int D, int G) { return kThreads / val_pairs(D, G); }
size_t key_lds_bytes(int D, int G) {
  return (size_t)G * D * 2 + (size_t)G * D + 3 * (size_t)D * 4 +
         2 * (size_t)(2 * key_parts(D)) * D * 4;
}
// value tiles: rows of D + kVPad binary16 values and code rows of kCRow
// bytes, so that the lanes of one token (and of one channel) spread over the
// LDS banks (unpadded, their rows are multiples of the bank count apart)
constexpr int kVPad = 8, kCRow = 36;
size_t val_lds_bytes(int D, int G) {
  const size_t pr = val_pairs(D, G);
  return 32 * (size_t)(D + kVPad) * 2 + (size_t)kCRow * D + 3 * pr * 4 +
         2 * pr * val_parts(D, G) * 4;
}

// A key group, its G x D fp16 tile already staged at the start of smem ->
// tokens [otok, otok + G) of destination plane ob (capacity ocap).
// Threads: channel d = th % D, part h = th / D (tokens [h*G/P, (h+1)*G/P)).
template <int BITS, bool MH, bool KO, bool FIX>
__device__ void key_group(const QuantJob& j, uint8_t* smem, size_t ob, int otok, int ocap) {
  const int D = FIX ? kFixD : j.D, G = FIX ? kFixG : j.G, W = D * BITS / 32, P = key_parts(D),
            per = G / P;
  const int th = threadIdx.x, d = th % D, h = th / D;
  // statistics: channel pair cp = th % (D/2), part hs of PS = 2P parts
  const int PS = 2 * P, pers = G / PS, cp = th % (D / 2), hs = th / (D / 2);
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);                 // [G][D]
  uint8_t* cb = smem + (size_t)G * D * 2;                              // codes [G][D]
  float* s_sc = reinterpret_cast<float*>(cb + (size_t)G * D);         // [D]
  float* s_zr = s_sc + D;
  float* s_rc = s_zr + D;
  float* p_mn = s_rc + D;                                              // [PS][D]
  float* p_mx = p_mn + PS * D;
  const size_t gg = (size_t)(otok / G);
  const size_t mrow = (ob * (ocap / G) + gg) * D;
  if constexpr (KO) {
    // outlier selection needs the whole group: one thread per channel.  The
    // positions form a bit set over the group's G <= 128 tokens; each pass
    // takes the first largest |x| not yet taken.
    if (h == 0) {
      const int n_out = j.n_out;
      uint64_t m0 = 0, m1 = 0;
      auto taken = [&](int i) { return ((i < 64 ? m0 >> i : m1 >> (i - 64)) & 1u) != 0; };
      for (int q = 0; q < n_out; q++) {
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
      float mn = INFINITY, mx = -INFINITY;
      for (int i = 0; i < G; i++) {
        if (taken(i)) continue;
        const float x = h2f(tile[i * D + d]);
        if (x < mn) mn = x;
        if (x > mx) mx = x;
      }
      // the sparse row, then mn in the outliers' places (code 0)
      uint32_t* orow = j.k_out + ((ob * (ocap / G) + gg) * n_out) * D + d;
      const uint16_t mn_h = __builtin_bit_cast(uint16_t, (_Float16)mn);   // exact
      int q = 0;
      for (int i = 0; i < G; i++) {
        if (!taken(i)) continue;
        orow[(size_t)q * D] = ((uint32_t)i << 16) | tile[i * D + d];
        tile[i * D + d] = mn_h;
        q++;
      }
      const float s = group_scale<BITS>(mn, mx);
      s_sc[d] = s;
      s_zr[d] = mn;
      s_rc[d] = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
      put_meta<MH>(j.k_scale, mrow + d, s);
      put_meta<MH>(j.k_zero, mrow + d, mn);
    }
  } else {
    // channels 2cp, 2cp + 1 over tokens [hs*pers, (hs+1)*pers), packed
    const uint16_t* col = tile + (size_t)hs * pers * D + 2 * cp;
    h2v mn2 = as_h2(*reinterpret_cast<const uint32_t*>(col)), mx2 = mn2;
    for (int i = 1; i < pers; i++) {
      const h2v x = as_h2(*reinterpret_cast<const uint32_t*>(col + (size_t)i * D));
      mn2 = __builtin_elementwise_min(mn2, x);
      mx2 = __builtin_elementwise_max(mx2, x);
    }
    float mn[2] = {(float)mn2.x, (float)mn2.y}, mx[2] = {(float)mx2.x, (float)mx2.y};
#pragma unroll
    for (int e = 0; e < 2; e++) {
      if (mn[e] == 0.0f || mx[e] == 0.0f) {
        const float z0 = first_zero(col + e, D, pers);
        if (mn[e] == 0.0f) mn[e] = z0;
        if (mx[e] == 0.0f) mx[e] = z0;
      }
      p_mn[hs * D + 2 * cp + e] = mn[e];
      p_mx[hs * D + 2 * cp + e] = mx[e];
    }
    __syncthreads();
    if (hs == 0) {
#pragma unroll
      for (int e = 0; e < 2; e++) {
        const int dd = 2 * cp + e;
        // parts in index order, strict comparisons: the earlier part keeps ties
        for (int q = 1; q < PS; q++) {
          const float a = p_mn[q * D + dd], b = p_mx[q * D + dd];
          if (a < mn[e]) mn[e] = a;
          if (b > mx[e]) mx[e] = b;
        }
        const float s = group_scale<BITS>(mn[e], mx[e]);
        s_sc[dd] = s;
        s_zr[dd] = mn[e];
        s_rc[dd] = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
        put_meta<MH>(j.k_scale, mrow + dd, s);
        put_meta<MH>(j.k_zero, mrow + dd, mn[e]);
      }
    }
  }
  __syncthreads();
  {
    // four tokens at a time (per is a multiple of 4): loads, codes, stores
    const float s = s_sc[d], z = s_zr[d], r = s_rc[d];
    for (int i = h * per; i < (h + 1) * per; i += 4) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; e++) x[e] = h2f(tile[(i + e) * D + d]);
      uint32_t c[4];
      encode4<BITS>(x, s, z, r, c);
#pragma unroll
      for (int e = 0; e < 4; e++) cb[(i + e) * D + d] = (uint8_t)c[e];
    }
  }
  __syncthreads();
  uint32_t* dst = j.k_codes + (ob * ocap + otok) * W;
  for (int it = th; it < G * W; it += kThreads) {
    const int i = it / W, w = it % W;
    dst[it] = pack_bytes<BITS>(cb + (size_t)i * D, D, w);
  }
}

// A value chunk, its 32 x D fp16 tile already staged at the start of smem ->
// tokens [t_base, t_base + 32) of destination plane ob (capacity ocap), one
// half of a 64-token tile.  Value
// codes are stored in 64-token tiles, channel-major: word
// ((t/64)*D + d)*(64/E) + (t%64)/E.  Threads: part h = th % P of the
// (token t, channel group jg) pair th / P (channels [jg*G + h*G/P, +G/P)).
template <int BITS, bool MH, bool FIX>
__device__ void value_chunk(const QuantJob& j, uint8_t* smem, size_t ob, int t_base, int ocap) {
  const int D = FIX ? kFixD : j.D, G = FIX ? kFixG : j.G, NG = D / G, NP = val_pairs(D, G),
            P = val_parts(D, G), per = G / P;
  const int th = threadIdx.x, h = th % P, pr = th / P, t = pr / NG, jg = pr % NG;
  const int VT = D + kVPad;                                            // tile row stride
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);                 // [32][VT]
  uint8_t* cbT = smem + 32 * (size_t)VT * 2;                           // codes [D][kCRow]
  float* s_sc = reinterpret_cast<float*>(cbT + (size_t)kCRow * D);    // [pairs]
  float* s_zr = s_sc + NP;
  float* s_rc = s_zr + NP;
  float* p_mn = s_rc + NP;                                             // [pairs][P]
  float* p_mx = p_mn + NP * P;
  const int c0 = jg * G + h * per;
  float mn, mx;
  {
    // channels [c0, c0 + per) of token t, four at a time (per is a multiple
    // of 4), packed
    const uint16_t* row = tile + t * VT + c0;
    const uint2 x0 = *reinterpret_cast<const uint2*>(row);
    h2v mn2 = __builtin_elementwise_min(as_h2(x0.x), as_h2(x0.y));
    h2v mx2 = __builtin_elementwise_max(as_h2(x0.x), as_h2(x0.y));
    for (int c = 4; c < per; c += 4) {
      const uint2 x = *reinterpret_cast<const uint2*>(row + c);
      mn2 = __builtin_elementwise_min(mn2, __builtin_elementwise_min(as_h2(x.x), as_h2(x.y)));
      mx2 = __builtin_elementwise_max(mx2, __builtin_elementwise_max(as_h2(x.x), as_h2(x.y)));
    }
    mn = fminf((float)mn2.x, (float)mn2.y);
    mx = fmaxf((float)mx2.x, (float)mx2.y);
    if (mn == 0.0f || mx == 0.0f) {
      const float z0 = first_zero(row, 1, per);
      if (mn == 0.0f) mn = z0;
      if (mx == 0.0f) mx = z0;
    }
  }
  p_mn[pr * P + h] = mn;
  p_mx[pr * P + h] = mx;
  __syncthreads();
  if (h == 0) {
    for (int q = 1; q < P; q++) {
      const float a = p_mn[pr * P + q], b = p_mx[pr * P + q];
      if (a < mn) mn = a;
      if (b > mx) mx = b;
    }
    const float s = group_scale<BITS>(mn, mx);
    s_sc[pr] = s;
    s_zr[pr] = mn;
    s_rc[pr] = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
    const size_t m = (ob * ocap + t_base + t) * NG + jg;
    put_meta<MH>(j.v_scale, m, s);
    put_meta<MH>(j.v_zero, m, mn);
  }
  __syncthreads();
  {
    // four channels at a time (per is a multiple of 4): one 8-byte load
    const float s = s_sc[pr], z = s_zr[pr], r = s_rc[pr];
    for (int c = c0; c < c0 + per; c += 4) {
      const uint2 x2 = *reinterpret_cast<const uint2*>(tile + t * VT + c);
      const float x[4] = {h2f((uint16_t)(x2.x & 0xFFFFu)), h2f((uint16_t)(x2.x >> 16)),
                          h2f((uint16_t)(x2.y & 0xFFFFu)), h2f((uint16_t)(x2.y >> 16))};
      uint32_t q[4];
      encode4<BITS>(x, s, z, r, q);
#pragma unroll
      for (int e = 0; e < 4; e++) cbT[(c + e) * kCRow + t] = (uint8_t)q[e];
    }
  }
  __syncthreads();

  constexpr int WPC = 2 * BITS;   // words per channel per 64-token tile
  uint32_t* plane = j.v_codes + ob * ((size_t)ocap * D * BITS / 32);
  const size_t tile_idx = (size_t)(t_base / 64);
  const int half = (t_base % 64) / 32;   // this block's half of the tile
  // the words of a channel's tile row that hold only this half's tokens: of
  // the 2*BITS words, those whose positions all lie in [32*half, 32*half+32)
  for (int it = th; it < D * BITS; it += kThreads) {
    const int d = it / BITS, k = it % BITS;
    int rw;   // row word index
    if constexpr (BITS == 1) {
      rw = half;
    } else if constexpr (BITS == 3) {
      rw = k < 2 ? 2 * half + k : 4 + half;
    } else {
      rw = half * BITS + k;
    }
    // (this half's 32 code bytes are positions 32*half .. 32*half + 31 of
    // the channel's tile row: word k of this half reads them from offset 0)
    uint32_t w;
    const uint8_t* row = cbT + (size_t)d * kCRow;
    if constexpr (BITS == 1) {
      w = pack_bytes<1>(row, 32, 0);
    } else if constexpr (BITS == 3) {
      w = k < 2 ? pack_bytes<3>(row, 32, k) : pack_bytes<3>(row, 32, 2);
    } else {
      w = pack_bytes<BITS>(row, 32, k);
    }
    plane[(tile_idx * D + d) * WPC + rw] = w;
  }
}

// Items (key groups or value chunks) per block: a block walks up to kItems
// consecutive items of one plane, holding the next item's tile in registers
// (up to kMaxPf 16-byte units per thread) while it computes the current one
// from LDS, so the tile loads overlap the computation.  Larger tiles are
// loaded at the start of their item instead.  A job too small to give
// kFillBlocks blocks at kItems per block takes fewer items per block (down
// to one), so a short prefill or flush spreads over the compute units
// instead of running a few long chains.
constexpr int kItems = 8;
constexpr long kFillBlocks = 2048;
constexpr int kMaxPf = 4;
struct Prefetch {
  u32x4_t r[kMaxPf];
};
__device__ __forceinline__ void pf_load(Prefetch& p, const uint16_t* src, int n16) {
#pragma unroll
  for (int v = 0; v < kMaxPf; v++) {
    const int i = (int)threadIdx.x + v * kThreads;
    if (i < n16) p.r[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src) + i);
  }
}
// (the tile in LDS has rows of 2^sh 16-byte units plus `pad` units)
__device__ __forceinline__ int padded(int i, int sh, int pad) { return i + (i >> sh) * pad; }
__device__ __forceinline__ void pf_store(const Prefetch& p, uint8_t* smem, int n16, int sh,
                                         int pad) {
#pragma unroll
  for (int v = 0; v < kMaxPf; v++) {
    const int i = (int)threadIdx.x + v * kThreads;
    if (i < n16) reinterpret_cast<u32x4_t*>(smem)[padded(i, sh, pad)] = p.r[v];
  }
}
__device__ __forceinline__ void stage_direct(uint8_t* smem, const uint16_t* src, int n16, int sh,
                                             int pad) {
  for (int i = threadIdx.x; i < n16; i += kThreads)
    copy16_nt(reinterpret_cast<uint4*>(smem) + padded(i, sh, pad),
              reinterpret_cast<const uint4*>(src) + i);
}

// One launch of the codec (blockIdx.y: plane, or list item * H + head):
//   blockIdx.x < nkb           : key groups  (do_k), ipb per block
//   nkb <= blockIdx.x < nkb+nvb: value chunks (do_v), ipb per block
//   above                      : residual copy chunk of 256 x 16 bytes
// Uniform launches quantize source tokens [0, nq) into destination tokens
// [dst_off, dst_off + nq) and copy source tokens [nq, nq + ncopy) into
// residual slots [0, ncopy); list item i does the same with nq = a[i],
// dst_off = b[i], ncopy = c[i] for sequence seq[i] (blocks past an item's
// counts exit).  PG: the destination is the page slice the block table names
// for the group's tokens (a group never straddles a page; a page outside the
// pool is skipped).
template <int BITS, bool MH, bool LIST, bool PG, bool KO, bool FIX>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5, 5)))
quantize_kv_kernel(QuantJob j, ListT<LIST> list, PageMap pm, int ipb) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int H = j.H, D = FIX ? kFixD : j.D, G = FIX ? kFixG : j.G;
  size_t bh = blockIdx.y;
  int seq = 0, nq = j.nq, dst_off = j.dst_off, ncopy = j.ncopy;
  if constexpr (LIST) {
    const int item = blockIdx.y / H;
    seq = list.seq[item];
    bh = (size_t)seq * H + blockIdx.y % H;
    nq = list.a[item];
    dst_off = list.b[item];
    ncopy = list.c[item];
  }
  // (j.nq: the largest item's count)
  const int nkb = j.do_k ? (j.nq / G + ipb - 1) / ipb : 0;
  const int nvb = j.do_v ? (j.nq / 32 + ipb - 1) / ipb : 0;
  int bx = blockIdx.x;
  // items [i0, i1) of `tok` tokens each from source tokens i0*tok, ...: the
  // block loop, `run(i)` computing item i from the staged tile (the branch
  // on the page slot inside it is uniform, so every barrier is reached by
  // the whole block)
  // (row units 2^sh: D / 8 is a power of two)
  const int sh = 31 - __builtin_clz(D / 8);
  auto walk = [&](const uint16_t* src, int tok, int pad, int n_items, auto run) {
    const int i0 = bx * ipb, i1 = min(i0 + ipb, n_items);
    if (i0 >= i1) return;   // the whole block: uniform
    const int n16 = tok * D / 8;
    const bool pf = n16 <= kMaxPf * kThreads;
    auto item_src = [&](int i) { return src + (bh * j.in_stride + (size_t)i * tok) * D; };
    Prefetch p;
    if (pf) pf_load(p, item_src(i0), n16);
    for (int i = i0; i < i1; i++) {
      __syncthreads();   // the previous item's LDS reads are done
      if (pf) {
        pf_store(p, smem, n16, sh, pad);
        if (i + 1 < i1) pf_load(p, item_src(i + 1), n16);
      } else {
        stage_direct(smem, item_src(i), n16, sh, pad);
      }
      __syncthreads();
      run(i);
    }
  };
  if (bx < nkb) {
    walk(j.k, G, 0, nq / G, [&](int g) {
      size_t ob = bh;
      int otok = dst_off + g * G, ocap = j.cap;
      if constexpr (PG) {
        if (!page_slot(pm, seq, (int)(bh % H), H, otok, ob, otok)) return;   // uniform
        ocap = pm.page_tokens;
      }
      key_group<BITS, MH, KO, FIX>(j, smem, ob, otok, ocap);
    });
    return;
  }
  bx -= nkb;
  if (bx < nvb) {
    walk(j.v, 32, kVPad / 8, nq / 32, [&](int c) {
      size_t ob = bh;
      int t_base = dst_off + c * 32, ocap = j.cap;
      if constexpr (PG) {
        if (!page_slot(pm, seq, (int)(bh % H), H, t_base, ob, t_base)) return;   // uniform
        ocap = pm.page_tokens;
      }
      value_chunk<BITS, MH, FIX>(j, smem, ob, t_base, ocap);
    });
    return;
  }
  bx -= nvb;
  // residual copy: source tokens [nq, nq + ncopy) -> slots [0, ncopy)
  const int per_tok = D / 8;
  const int i = bx * kThreads + (int)threadIdx.x;
  if (i >= ncopy * per_tok) return;
  const int t = i / per_tok, c = i % per_tok;
  const size_t so = ((bh * j.in_stride + nq + t) * D) / 8 + c;
  const size_t dd = ((bh * j.R + t) * D) / 8 + c;
  copy16_nt(reinterpret_cast<uint4*>(j.k_res) + dd, reinterpret_cast<const uint4*>(j.k) + so);
  copy16_nt(reinterpret_cast<uint4*>(j.v_res) + dd, reinterpret_cast<const uint4*>(j.v) + so);
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
    if (k_src)
      copy16_nt(reinterpret_cast<uint4*>(k_dst) + dd, reinterpret_cast<const uint4*>(k_src) + so);
    if (v_src)
      copy16_nt(reinterpret_cast<uint4*>(v_dst) + dd, reinterpret_cast<const uint4*>(v_src) + so);
  }
}

// Value quantization of single tokens (the value window): block (b, h) takes
// cache tokens t0 .. t0 + n - 1 in order, one thread per channel; token
// t0 + i comes from source row src_row + i of the plane's [src_stride][D]
// rows.  The steps are the codec's (S1) with the correctly rounded division
// and a strict in-order min / max scan; a token replaces the bits of its
// position in the shared 64-token value rows and keeps the other tokens'
// bits.  Each thread writes only its own channel's rows, in token order.
template <int BITS>
__device__ __forceinline__ void set_code(uint32_t* row, int p, uint32_t c) {
  if constexpr (BITS == 3) {
    row[p >> 4] = (row[p >> 4] & ~(3u << (2 * (p & 15)))) | ((c & 3u) << (2 * (p & 15)));
    const int w = 4 + (p >> 5), b = beta(p & 31);   // (64-position rows: the hi plane at word 4)
    row[w] = (row[w] & ~(1u << b)) | ((c >> 2) << b);
  } else if constexpr (BITS == 1) {
    const int b = beta(p & 31);
    row[p >> 5] = (row[p >> 5] & ~(1u << b)) | (c << b);
  } else {
    constexpr int E = 32 / BITS;
    constexpr uint32_t M = (1u << BITS) - 1u;
    const int sh = BITS * (p % E);
    row[p / E] = (row[p / E] & ~(M << sh)) | (c << sh);
  }
}

// (The window append fuses the new token's copies into the same launch:
// after its token, thread d writes channel d of k_new into key-residual slot
// k_slot and of v_new into window slot v_slot, which it has already read.)
template <int BITS, bool MH>
__global__ void __launch_bounds__(256)
quantize_v_tokens_kernel(QuantJob j, const uint16_t* __restrict__ src, int src_stride,
                         int src_row, int t0, int n, const uint16_t* __restrict__ k_new,
                         int k_slot, const uint16_t* __restrict__ v_new, int v_slot) {
  __shared__ float xs[256];
  __shared__ float gs[8], gz[8];   // (D / G <= 8)
  const int D = j.D, G = j.G, NG = D / G, d = threadIdx.x;
  const size_t bh = blockIdx.x;
  constexpr float qmax = (float)((1 << BITS) - 1);
  uint32_t* plane = j.v_codes + bh * ((size_t)j.cap * D * BITS / 32);
  for (int i = 0; i < n; i++) {
    const int t = t0 + i;
    const float x = h2f(src[(bh * src_stride + src_row + i) * D + d]);
    xs[d] = x;
    __syncthreads();
    if (d < NG) {
      float mn = xs[d * G], mx = mn;
      for (int e = 1; e < G; e++) {
        const float y = xs[d * G + e];
        if (y < mn) mn = y;
        if (y > mx) mx = y;
      }
      const float sc = group_scale<BITS>(mn, mx);
      gs[d] = sc;
      gz[d] = mn;
      put_meta<MH>(j.v_scale, (bh * j.cap + t) * NG + d, sc);
      put_meta<MH>(j.v_zero, (bh * j.cap + t) * NG + d, mn);
    }
    __syncthreads();
    const float sc = gs[d / G], z = gz[d / G];
    const uint32_t c = sc == 0.0f ? 0u : (uint32_t)fminf(rintf((x - z) / sc), qmax);
    set_code<BITS>(plane + ((size_t)(t / 64) * D + d) * (2 * BITS), t % 64, c);
    __syncthreads();   // (xs and gs are rewritten by the next token)
  }
  if (k_new) {
    j.k_res[(bh * j.R + k_slot) * D + d] = k_new[bh * D + d];
    j.v_res[(bh * j.R + v_slot) * D + d] = v_new[bh * D + d];
  }
}

// f(bits, metadata-half, outliers) with all three as compile-time constants
template <class F>
void dispatch(int bits, int mh, bool ko, F f) {
  auto with_ko = [&](auto B, auto M) {
    if (ko) f(B, M, std::true_type{}); else f(B, M, std::false_type{});
  };
  auto with_mh = [&](auto B) {
    if (mh) with_ko(B, std::true_type{}); else with_ko(B, std::false_type{});
  };
  switch (bits) {
    case 1: with_mh(std::integral_constant<int, 1>{}); break;
    case 2: with_mh(std::integral_constant<int, 2>{}); break;
    case 3: with_mh(std::integral_constant<int, 3>{}); break;
    default: with_mh(std::integral_constant<int, 4>{}); break;
  }
}

// item blocks of a job at n items per block
int item_blocks(const QuantJob& j, int n) {
  return (j.do_k ? (j.nq / j.G + n - 1) / n : 0) + (j.do_v ? (j.nq / 32 + n - 1) / n : 0);
}

// items per block, grid x extent and LDS bytes of a job (gy planes or items)
void job_shape(const QuantJob& j, int gy, int ncopy_max, int& ipb, int& gx, size_t& lds) {
  ipb = kItems;
  while (ipb > 1 && (long)item_blocks(j, ipb) * gy < kFillBlocks) ipb /= 2;
  const int nkb = j.do_k ? (j.nq / j.G + ipb - 1) / ipb : 0;
  const int nvb = j.do_v ? (j.nq / 32 + ipb - 1) / ipb : 0;
  const int ncb = (ncopy_max * (j.D / 8) + kThreads - 1) / kThreads;
  gx = nkb + nvb + ncb;
  lds = 0;
  if (nkb) lds = key_lds_bytes(j.D, j.G);
  if (nvb) lds = lds > val_lds_bytes(j.D, j.G) ? lds : val_lds_bytes(j.D, j.G);
}

template <bool LIST, bool PG>
hipError_t launch_job(const QuantJob& j, int bits, int mh, int gy, int ncopy_max,
                      const ListT<LIST>& list, const PageMap& pm, hipStream_t st) {
  int ipb, gx;
  size_t lds;
  job_shape(j, gy, ncopy_max, ipb, gx, lds);
  if (gx == 0 || gy == 0) return hipSuccess;
  const dim3 grid(gx, gy);
  const bool fix = j.D == kFixD && j.G == kFixG;
  dispatch(bits, mh, j.n_out > 0, [&](auto B, auto M, auto K) {
    if (fix)
      quantize_kv_kernel<B.value, M.value, LIST, PG, K.value, true>
          <<<grid, kThreads, lds, st>>>(j, list, pm, ipb);
    else
      quantize_kv_kernel<B.value, M.value, LIST, PG, K.value, false>
          <<<grid, kThreads, lds, st>>>(j, list, pm, ipb);
  });
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_kv(const QuantJob& j, int bits, int mh, int B, hipStream_t st) {
  return launch_job<false, false>(j, bits, mh, B * j.H, j.ncopy, NoList{}, PageMap{}, st);
}

hipError_t launch_quantize_kv_list(const QuantJob& j, const SeqList& list, int bits, int mh,
                                   int ncopy_max, hipStream_t st) {
  if (list.n == 0) return hipSuccess;
  return launch_job<true, false>(j, bits, mh, list.n * j.H, ncopy_max, list, PageMap{}, st);
}

hipError_t launch_quantize_kv_paged(const QuantJob& j, const SeqList& list, const PageMap& pm,
                                    int bits, int mh, int ncopy_max, hipStream_t st) {
  if (list.n == 0) return hipSuccess;
  return launch_job<true, true>(j, bits, mh, list.n * j.H, ncopy_max, list, pm, st);
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

hipError_t launch_quantize_v_tokens(const QuantJob& j, int bits, int mh, int B,
                                    const uint16_t* src, int src_stride, int src_row, int t0,
                                    int n, hipStream_t st, const uint16_t* k_new, int k_slot,
                                    const uint16_t* v_new, int v_slot) {
  if (n <= 0 && !k_new) return hipSuccess;
  const dim3 grid(B * j.H);
  dispatch(bits, mh, false, [&](auto Bt, auto M, auto) {
    quantize_v_tokens_kernel<Bt.value, M.value><<<grid, j.D, 0, st>>>(
        j, src, src_stride, src_row, t0, n, k_new, k_slot, v_new, v_slot);
  });
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

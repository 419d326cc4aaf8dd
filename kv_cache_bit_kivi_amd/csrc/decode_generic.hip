// Generic decode attention on the mixed cache (any supported shape), plus the
// split-combine kernel shared by every decode path.
//
// Method (study.space summary of "KIVI: A Tuning-Free Asymmetric 2bit
// Quantization for KV Cache"): scores are computed against the quantized
// grouped part and the full-precision residual part is combined with them.
// Here: o = softmax(scale * q.k) . v over the tq quantized tokens (keys and
// values dequantized in registers as code*scale + zero) and the tr residual
// fp16 tokens, binary32 accumulation.  With key outliers (KVQuant page,
// abstract: outliers isolated per vector), a key listed in its group's sparse
// row takes the kept fp16 value instead of the dense one.  With pre-RoPE keys
// (a.rope_theta > 0; same page: keys quantized before the rotary embedding)
// every key is rotated at its token index t before the dot product: pairs
// (i, i + D/2), angle t * rope_theta^(-2i/D) taken in binary64.  With the
// value window (a.vwin; scholarfeed "KIVI" quote page: a fixed-length buffer
// of recent full-precision tokens) the values of the R newest tokens come
// from v_res slot t % R and the older ones are dequantized.
//
// One block of 256 threads per (split, b*Hkv + h).  The block owns a
// contiguous token chunk and all r query heads of its KV head:
//   pass 1: one thread per token computes its r scores into LDS;
//   pass 2: block max / exp / sum per head;
//   pass 3: threads own (channel, token phase) and accumulate p * v.
// With one split the block writes fp16 output; otherwise it writes its
// (max, sum, unnormalised o) partial and the combine kernel merges them.
#include <math.h>

#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Code at position p of a packed row of n codes (a key row: D channels; a
// value row: one channel's 64 tokens of a tile) for b = 1..4 bits:
//   2, 4 bits: word p/E, bit b*(p%E), E = 32/b;  1 bit: word p/32, bit
//   beta(p%32);  3 bits: lo (word p/16, bits 2*(p%16)) + 4 * hi (word
//   n/16 + p/32, bit beta(p%32)),  beta(p) = 4*((p%16)/2) + 2*(p/16) + p%2.
__device__ __forceinline__ uint32_t code_at(const uint32_t* row, int n, int bits, int p) {
  auto beta = [](int q) { return 4 * ((q & 15) >> 1) + 2 * (q >> 4) + (q & 1); };
  if (bits == 3)
    return ((row[p >> 4] >> (2 * (p & 15))) & 3u) |
           (((row[(n >> 4) + (p >> 5)] >> beta(p & 31)) & 1u) << 2);
  if (bits == 1) return (row[p >> 5] >> beta(p & 31)) & 1u;
  const int E = 32 / bits;
  return (row[p / E] >> (bits * (p % E))) & ((1u << bits) - 1u);
}

// scale / zero element i of a metadata plane (binary32, or binary16 when mh)
__device__ __forceinline__ float meta_at(const void* p, size_t i, int mh) {
  return mh ? h2f(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

__device__ float block_reduce(float v, bool is_max, float* scratch) {
  for (int off = 32; off > 0; off >>= 1) {
    float o = __shfl_xor(v, off, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < kThreads / 64; i++) r = is_max ? fmaxf(r, scratch[i]) : r + scratch[i];
  return r;
}

// tokens scored per LDS round: the score buffer stays at 4-8 KB per head group
template <int RR>
constexpr int sub_tokens() { return RR <= 2 ? 1024 : 2048 / RR; }

template <int RR, bool RAG, bool PG>
__global__ void __launch_bounds__(kThreads)
decode_generic_kernel(DecodeArgs a, int chunk, LensT<RAG> lens) {
  constexpr int kSub = sub_tokens<RR>();
  extern __shared__ __align__(16) float sm[];
  const int r = a.r, D = a.D, G = a.G, bits = a.bits;
  float* sq = sm;                    // [r][D]   scale * q
  float* sp = sq + r * D;            // [r][kSub] scores, then weights
  float* so = sp + r * kSub;         // [kThreads/D][RR][D] pass-3 partials
  float* red = so + RR * kThreads;   // reduction scratch
  float* stat = red + 8;             // [RR] running max, [RR] running sum, [RR] rescale
  // pre-RoPE: pair frequencies, binary64 [D/2] (8-byte aligned after stat)
  double* th = reinterpret_cast<double*>(
      (reinterpret_cast<uintptr_t>(stat + 3 * RR) + 7) & ~static_cast<uintptr_t>(7));
  const bool rope = a.rope_theta > 0.f;

  const int split = blockIdx.x;
  const int u = seq_plane<RAG>(lens, blockIdx.y, a.H);   // b * H + h
  const int b = u / a.H, h = u % a.H;
  const int tq = seq_tq<RAG>(a, lens, b), tr = seq_tr<RAG>(a, lens, b);
  const int L = tq + tr;
  // quantized values: tq, or with the value window all but the R newest
  const int tv = a.vwin ? (L > a.R ? L - a.R : 0) : tq;
  if constexpr (RAG) chunk = (L + a.S - 1) / a.S;   // per sequence
  const int t0 = a.t_begin + split * chunk;
  const int t1 = min(L, t0 + chunk);
  const int W = D * bits / 32, WPC = 2 * bits, NG = D / G;   // words per key / value row

  const size_t kvp = (size_t)u;                   // plane index
  const int mh = a.mh;
  const size_t mb = mh ? 2 : 4;   // metadata element bytes
  // quantized token t: its slice plane (the contiguous plane, or the page
  // slice named by the block table) and its token inside that slice
  const size_t scap = PG ? (size_t)a.pages.page_tokens : (size_t)a.cap;
  auto slot = [&](int t, size_t& pl, int& lt) -> bool {
    if constexpr (PG) {
      return page_slot(a.pages, b, h, a.H, t, pl, lt);
    } else {
      pl = kvp;
      lt = t;
      return true;
    }
  };
  const uint16_t* kr = a.k_res + kvp * (size_t)a.R * D;
  const uint16_t* vr = a.v_res + kvp * (size_t)a.R * D;
  const size_t qrow0 = (size_t)b * a.H * r + (size_t)h * r;   // first query row

  for (int i = threadIdx.x; i < r * D; i += kThreads) sq[i] = a.scale * h2f(a.q[qrow0 * D + i]);
  if (threadIdx.x < RR) {
    stat[threadIdx.x] = -INFINITY;
    stat[RR + threadIdx.x] = 0.f;
  }
  if (rope)
    for (int i = threadIdx.x; i < D / 2; i += kThreads)
      th[i] = exp2(-(double)(2 * i) / (double)D * log2((double)a.rope_theta));
  __syncthreads();

  const int nsub = kThreads / D;
  const int d = threadIdx.x % D, sub = threadIdx.x / D;
  float o[RR];
#pragma unroll
  for (int i = 0; i < RR; i++) o[i] = 0.f;

  for (int c0 = t0; c0 < t1; c0 += kSub) {
    const int c1 = min(t1, c0 + kSub);
    const int nn = c1 - c0;
    // pass 1: scores of tokens [c0, c1)
    for (int t = c0 + threadIdx.x; t < c1; t += kThreads) {
      float acc[RR];
#pragma unroll
      for (int i = 0; i < RR; i++) acc[i] = 0.f;
      size_t pl;
      int lt;
      const bool quant = t < tq && slot(t, pl, lt);
      if (quant || t >= tq) {
        // key channel dd of token t: dequantized (outliers replaced by their
        // kept value), or the residual fp16 value
        const uint32_t* row = quant ? a.k_codes + (pl * scap + lt) * W : nullptr;
        const size_t m0 = quant ? (pl * (scap / G) + lt / G) * D : 0;
        const uint32_t* orow = a.k_out + m0 * a.n_out;   // [n_out][D] of this group
        const uint32_t my = quant ? (uint32_t)(lt % G) : 0u;
        const uint16_t* rrow = quant ? nullptr : kr + (size_t)(t - tq) * D;
        auto kval = [&](int dd) -> float {
          if (!quant) return h2f(rrow[dd]);
          float kh = (float)code_at(row, D, bits, dd) * meta_at(a.k_scale, m0 + dd, mh) +
                     meta_at(a.k_zero, m0 + dd, mh);
          for (int j = 0; j < a.n_out; j++) {
            const uint32_t w = orow[(size_t)j * D + dd];
            if ((w >> 16) == my) kh = h2f((uint16_t)(w & 0xFFFFu));
          }
          return kh;
        };
        if (rope) {
          const int hd = D / 2;
          for (int p = 0; p < hd; p++) {
            const float k0 = kval(p), k1 = kval(p + hd);
            double sn, cs;
            sincos(th[p] * (double)t, &sn, &cs);
            const float c = (float)cs, sf = (float)sn;
            const float kr0 = k0 * c - k1 * sf, kr1 = k0 * sf + k1 * c;
#pragma unroll
            for (int i = 0; i < RR; i++)
              if (i < r) acc[i] += sq[i * D + p] * kr0 + sq[i * D + p + hd] * kr1;
          }
        } else {
          for (int dd = 0; dd < D; dd++) {
            const float kh = kval(dd);
#pragma unroll
            for (int i = 0; i < RR; i++)
              if (i < r) acc[i] += sq[i * D + dd] * kh;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < RR; i++)
        if (i < r) sp[i * kSub + (t - c0)] = acc[i];
    }
    __syncthreads();

    // pass 2: online softmax statistics per head
    for (int i = 0; i < r; i++) {
      float m = -INFINITY;
      for (int j = threadIdx.x; j < nn; j += kThreads) m = fmaxf(m, sp[i * kSub + j]);
      m = block_reduce(m, true, red);
      const float m_old = stat[i];
      const float m_new = fmaxf(m_old, m);
      float l = 0.f;
      for (int j = threadIdx.x; j < nn; j += kThreads) {
        const float p = __expf(sp[i * kSub + j] - m_new);
        sp[i * kSub + j] = p;
        l += p;
      }
      l = block_reduce(l, false, red);
      if (threadIdx.x == 0) {
        const float alpha = __expf(m_old - m_new);   // 0 on the first sub-chunk
        stat[i] = m_new;
        stat[RR + i] = stat[RR + i] * alpha + l;
        stat[2 * RR + i] = alpha;
      }
      __syncthreads();
    }

    // pass 3: weighted values
    if (sub < nsub) {
#pragma unroll
      for (int i = 0; i < RR; i++)
        if (i < r) o[i] *= stat[2 * RR + i];
      for (int t = c0 + sub; t < c1; t += nsub) {
        float vh = 0.f;
        size_t pl;
        int lt;
        if (t < tv) {
          if (slot(t, pl, lt)) {
            const uint32_t* row =
                a.v_codes + pl * scap * D * bits / 32 + ((size_t)(lt / 64) * D + d) * WPC;
            const size_t mi = (pl * scap + lt) * NG + d / G;
            vh = (float)code_at(row, 64, bits, lt % 64) * meta_at(a.v_scale, mi, mh) +
                 meta_at(a.v_zero, mi, mh);
          }
        } else {
          vh = h2f(vr[(size_t)(a.vwin ? t % a.R : t - tq) * D + d]);
        }
#pragma unroll
        for (int i = 0; i < RR; i++)
          if (i < r) o[i] += sp[i * kSub + (t - c0)] * vh;
      }
    }
    __syncthreads();
  }

  // reduce the token phases: so[sub][i][d]
  for (int i = 0; i < RR; i++)
    if (i < r && sub < nsub) so[(sub * RR + i) * D + d] = o[i];
  __syncthreads();
  const bool empty = t1 <= t0;
  for (int idx = threadIdx.x; idx < r * D; idx += kThreads) {
    const int i = idx / D, dd = idx % D;
    float acc = 0.f;
    for (int s = 0; s < nsub; s++) acc += so[(s * RR + i) * D + dd];
    const size_t row = qrow0 + i;
    if (a.ws_stride == 1) {
      a.out[row * D + dd] = f2h(acc / stat[RR + i]);
    } else {
      const size_t rows = (size_t)a.B * a.H * r, WS = a.ws_stride;
      const size_t slot = (size_t)a.ws_slot0 + split;
      if (dd == 0) {
        a.ws[row * WS + slot] = empty ? -INFINITY : stat[i];
        a.ws[rows * WS + row * WS + slot] = empty ? 0.f : stat[RR + i];
      }
      a.ws[2 * rows * WS + (row * WS + slot) * D + dd] = empty ? 0.f : acc;
    }
  }
}

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ ws,
                                                      uint16_t* __restrict__ out, int rows,
                                                      int S, int D) {
  const int row = blockIdx.x;
  const float* m = ws + (size_t)row * S;
  const float* l = ws + (size_t)rows * S + (size_t)row * S;
  const float* o = ws + 2 * (size_t)rows * S + (size_t)row * S * D;
  float M = -INFINITY;
  for (int s = 0; s < S; s++) M = fmaxf(M, m[s]);
  float Ls = 0.f;
  for (int s = 0; s < S; s++) Ls += l[s] * __expf(m[s] - M);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < S; s++) acc += o[(size_t)s * D + d] * __expf(m[s] - M);
    out[(size_t)row * D + d] = f2h(acc / Ls);
  }
}

// ---- value window tail ---------------------------------------------------
// Tokens [a.t_begin, tq + tr) of one (b, h) plane for the matrix-core shape
// (D = 128, G = 32) without key outliers or pre-RoPE keys: keys from the
// codes (t < tq) or the key residual, values from the codes (t < L - R) or
// the window (slot t % R).  Each half wave takes its own token stream (every
// 2 NWV-th token; 16 waves, 8 for eight heads: the merge buffer stays at
// 32 KB), lane = 4 channels, scores by a butterfly sum over the half and an
// online softmax per head; the waves' states merge in LDS with the split-K
// partials [0, a.ws_slot0) that the matrix-core launch before it wrote
// (natural-log maxima), and the block writes the fp16 output.

// code at position p of a packed row of n codes, b = BITS (the layouts of
// code_at, with the width known at compile time)
template <int BITS>
__device__ __forceinline__ uint32_t code_at_t(const uint32_t* row, int n, int p) {
  if constexpr (BITS == 3) {
    const int q = p & 31;
    const int bt = 4 * ((q & 15) >> 1) + 2 * (q >> 4) + (q & 1);
    return ((row[p >> 4] >> (2 * (p & 15))) & 3u) | (((row[(n >> 4) + (p >> 5)] >> bt) & 1u) << 2);
  } else if constexpr (BITS == 1) {
    const int q = p & 31;
    const int bt = 4 * ((q & 15) >> 1) + 2 * (q >> 4) + (q & 1);
    return (row[p >> 5] >> bt) & 1u;
  } else {
    constexpr int E = 32 / BITS;
    return (row[p / E] >> (BITS * (p % E))) & ((1u << BITS) - 1u);
  }
}

// sum over the 32 lanes of a half wave (every lane of the half gets it)
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) v += __shfl_xor(v, off, 32);
  return v;
}

template <int RR>
constexpr int tail_waves() { return RR >= 8 ? 8 : 16; }

template <int BITS, bool MH, int RR, int NWV = tail_waves<RR>()>
__global__ void __launch_bounds__(NWV * 64) window_tail_kernel(DecodeArgs a) {
  constexpr int D = 128, G = 32, NG = D / G, W = D * BITS / 32, WPC = 2 * BITS;
  __shared__ float s_m[NWV][RR], s_l[NWV][RR];
  __shared__ float s_o[NWV][RR][D];
  const int u = blockIdx.x;                  // b * H + h
  const int b = u / a.H, h = u % a.H, r = a.r;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hf = lane >> 5, c0 = 4 * (lane & 31);   // half wave, its lane's 4 channels
  const int tq = a.tq, L = a.tq + a.tr, R = a.R;
  const int tv = L > R ? L - R : 0;
  const size_t qrow0 = (size_t)b * a.H * r + (size_t)h * r;
  float q[RR][4], m[RR], l[RR], o[RR][4];
#pragma unroll
  for (int i = 0; i < RR; i++) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      q[i][e] = i < r ? a.scale * h2f(a.q[(qrow0 + i) * D + c0 + e]) : 0.f;
      o[i][e] = 0.f;
    }
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  const size_t cap = a.cap;
  const uint32_t* kc = a.k_codes + (size_t)u * cap * W;
  const uint32_t* vc = a.v_codes + (size_t)u * cap * D * BITS / 32;
  const uint16_t* kr = a.k_res + (size_t)u * R * D;
  const uint16_t* vr = a.v_res + (size_t)u * R * D;
  // token stream 2 wv + hf: every 2 NWV-th token
#pragma unroll 2
  for (int t = a.t_begin + 2 * wv + hf; t < L; t += 2 * NWV) {
    float k[4], v[4];
    if (t < tq) {
      const uint32_t* row = kc + (size_t)t * W;
      const size_t mi = ((size_t)u * (cap / G) + t / G) * D + c0;
#pragma unroll
      for (int e = 0; e < 4; e++)
        k[e] = (float)code_at_t<BITS>(row, D, c0 + e) * meta_at(a.k_scale, mi + e, MH) +
               meta_at(a.k_zero, mi + e, MH);
    } else {
#pragma unroll
      for (int e = 0; e < 4; e++) k[e] = h2f(kr[(size_t)(t - tq) * D + c0 + e]);
    }
    if (t < tv) {
      const uint32_t* row0 = vc + ((size_t)(t / 64) * D + c0) * WPC;
      const size_t mi = ((size_t)u * cap + t) * NG + c0 / G;
      const float sc = meta_at(a.v_scale, mi, MH), z = meta_at(a.v_zero, mi, MH);
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = (float)code_at_t<BITS>(row0 + e * WPC, 64, t % 64) * sc + z;
    } else {
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = h2f(vr[(size_t)(t % R) * D + c0 + e]);
    }
#pragma unroll
    for (int i = 0; i < RR; i++) {
      if (i >= r) continue;
      const float sc = half_sum(q[i][0] * k[0] + q[i][1] * k[1] + q[i][2] * k[2] + q[i][3] * k[3]);
      const float mn = fmaxf(m[i], sc);
      const float alpha = __expf(m[i] - mn);   // (0 while m is -inf)
      const float p = __expf(sc - mn);
      l[i] = l[i] * alpha + p;
#pragma unroll
      for (int e = 0; e < 4; e++) o[i][e] = o[i][e] * alpha + p * v[e];
      m[i] = mn;
    }
  }
  // the two halves' streams -> one state per wave (lane and lane ^ 32 hold
  // the same channels)
#pragma unroll
  for (int i = 0; i < RR; i++) {
    const float m2 = __shfl_xor(m[i], 32, 64), l2 = __shfl_xor(l[i], 32, 64);
    const float mn = fmaxf(m[i], m2);
    const float f1 = mn == -INFINITY ? 0.f : __expf(m[i] - mn);
    const float f2 = mn == -INFINITY ? 0.f : __expf(m2 - mn);
    float oo[4];
#pragma unroll
    for (int e = 0; e < 4; e++) oo[e] = o[i][e] * f1 + __shfl_xor(o[i][e], 32, 64) * f2;
    if (lane == 0) {
      s_m[wv][i] = mn;
      s_l[wv][i] = l[i] * f1 + l2 * f2;
    }
    if (hf == 0) {
#pragma unroll
      for (int e = 0; e < 4; e++) s_o[wv][i][c0 + e] = oo[e];
    }
  }
  __syncthreads();
  const size_t rows = (size_t)a.B * a.H * r, WS = a.ws_stride;
  const int S0 = a.ws_slot0;   // the matrix-core partials
  for (int idx = threadIdx.x; idx < r * D; idx += NWV * 64) {
    const int i = idx / D, d = idx % D;
    const size_t row = qrow0 + i;
    const float* pm = a.ws + row * WS;
    const float* pl = a.ws + rows * WS + row * WS;
    const float* po = a.ws + 2 * rows * WS + row * WS * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; w++) M = fmaxf(M, s_m[w][i]);
    for (int sp = 0; sp < S0; sp++) M = fmaxf(M, pm[sp]);
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; w++) {
      const float f = __expf(s_m[w][i] - M);
      O += s_o[w][i][d] * f;
      Ls += s_l[w][i] * f;
    }
    for (int sp = 0; sp < S0; sp++) {
      const float f = __expf(pm[sp] - M);
      O += po[(size_t)sp * D + d] * f;
      Ls += pl[sp] * f;
    }
    a.out[row * D + d] = f2h(O / Ls);
  }
}

}  // namespace

bool window_tail_supported(int D, int G, int r, int outliers, bool rope) {
  return D == 128 && G == 32 && r >= 1 && r <= 8 && outliers == 0 && !rope;
}

hipError_t launch_window_tail(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.B * a.H);
  auto go = [&](auto B, auto M) {
    constexpr int BITS = decltype(B)::value;
    constexpr bool MH = decltype(M)::value;
    if (a.r == 1)
      window_tail_kernel<BITS, MH, 1><<<grid, tail_waves<1>() * 64, 0, st>>>(a);
    else if (a.r == 2)
      window_tail_kernel<BITS, MH, 2><<<grid, tail_waves<2>() * 64, 0, st>>>(a);
    else if (a.r <= 4)
      window_tail_kernel<BITS, MH, 4><<<grid, tail_waves<4>() * 64, 0, st>>>(a);
    else
      window_tail_kernel<BITS, MH, 8><<<grid, tail_waves<8>() * 64, 0, st>>>(a);
  };
  auto with_mh = [&](auto B) {
    if (a.mh) go(B, std::true_type{}); else go(B, std::false_type{});
  };
  switch (a.bits) {
    case 1: with_mh(std::integral_constant<int, 1>{}); break;
    case 2: with_mh(std::integral_constant<int, 2>{}); break;
    case 3: with_mh(std::integral_constant<int, 3>{}); break;
    default: with_mh(std::integral_constant<int, 4>{}); break;
  }
  return hipGetLastError();
}

size_t decode_generic_lds_bytes(int r, int D) {
  int rr = 1;
  while (rr < r) rr *= 2;
  const int sub = rr <= 2 ? 1024 : 2048 / rr;
  return sizeof(float) * ((size_t)r * D + (size_t)r * sub + (size_t)rr * kThreads + 8 + 3 * rr) +
         8 + sizeof(double) * (size_t)(D / 2);   // (+ the pre-RoPE frequencies)
}

template <bool RAG, bool PG>
static hipError_t launch_generic(const DecodeArgs& a, const LensT<RAG>& lens, hipStream_t st) {
  const int L = a.tq + a.tr - a.t_begin;   // tokens of the launch's range
  const int chunk = (L + a.S - 1) / a.S;   // (per sequence in the kernel when ragged)
  dim3 grid(a.S, a.B * a.H);
  const size_t lds = decode_generic_lds_bytes(a.r, a.D);
  if (a.r == 1)
    decode_generic_kernel<1, RAG, PG><<<grid, kThreads, lds, st>>>(a, chunk, lens);
  else if (a.r == 2)
    decode_generic_kernel<2, RAG, PG><<<grid, kThreads, lds, st>>>(a, chunk, lens);
  else if (a.r <= 4)
    decode_generic_kernel<4, RAG, PG><<<grid, kThreads, lds, st>>>(a, chunk, lens);
  else if (a.r <= 8)
    decode_generic_kernel<8, RAG, PG><<<grid, kThreads, lds, st>>>(a, chunk, lens);
  else
    decode_generic_kernel<16, RAG, PG><<<grid, kThreads, lds, st>>>(a, chunk, lens);
  return hipGetLastError();
}

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st) {
  return launch_generic<false, false>(a, NoLens{}, st);
}

hipError_t launch_decode_generic_ragged(const DecodeArgs& a, const SeqLens& lens, hipStream_t st) {
  return launch_generic<true, false>(a, lens, st);
}

hipError_t launch_decode_generic_paged(const DecodeArgs& a, const SeqLens& lens, hipStream_t st) {
  return launch_generic<true, true>(a, lens, st);
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t st) {
  const int rows = a.B * a.H * a.r;
  combine_kernel<<<rows, 128, 0, st>>>(a.ws, a.out, rows, a.ws_stride, a.D);
  return hipGetLastError();
}

}  // namespace kivi

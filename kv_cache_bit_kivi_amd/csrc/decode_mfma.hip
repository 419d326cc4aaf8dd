// Decode attention on the mixed cache with matrix-core (MFMA) contractions,
// for head_dim 128, group 32, 2- or 4-bit codes and GQA ratio r <= 8.
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
// Both contractions run on v_mfma_f32_16x16x32_f16 with the dense operand
// B = the codes, converted exactly to fp16 (2-bit nibbles via the e2m1
// convert with scale 2, 4-bit nibbles via the e4m3 convert with scale 2^9),
// and the operand A = the per-group factors q' (or p') split into fp16 hi +
// lo rows so the products keep ~22 significant bits:
//   keys:   A rows (head, hi|lo) x K=32 channels, B = 32 channels x 16 tokens
//   values: A rows (head, hi|lo) x K=32 tokens,   B = 32 tokens x 16 channels
// The K=32 slots a lane supplies map to code positions in the order the
// converts produce them (see k_pos / v_pos); A is written to LDS in that order.
//
// Work: one block of NW waves per (b*Hkv + h, split); every wave owns a
// contiguous run of 64-token value tiles plus a slice of the residual, walks
// it in chunks (scores of the chunk to LDS, chunk max, rescale, then P.V), and
// the block merges its waves in LDS.  One split writes fp16 output; more
// splits write (max, sum, o) partials for the combine kernel.
#include <math.h>

#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 32;
constexpr int kNG = kD / kG;   // value groups per token
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_read(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// all-lane reductions over the 64-lane wave (result uniform)
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0x128>(v);  // row_ror:8
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x122>(v);  // row_ror:2
  v += dpp<0x121>(v);  // row_ror:1
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0x128>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x122>(v));
  v = fmaxf(v, dpp<0x121>(v));
  return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 two-bit codes held one per nibble (upper two bits zero) -> 8 exact halves,
// slot s = nibble s
__device__ __forceinline__ half8 cvt_nib2(uint32_t x) {
  half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 0);
  half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 1);
  half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 2);
  half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 3);
  return half8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}
// one word of 8 four-bit codes -> 8 exact halves; slots 0..3 = even
// positions 0,2,4,6, slots 4..7 = odd positions 1,3,5,7
__device__ __forceinline__ half8 cvt_word4(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
  return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
__device__ __forceinline__ float4v mfma(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// slot of position q (0..7) inside a 4-bit word's half8
__device__ __forceinline__ int slot4(int q) { return (q & 1) ? 4 + (q >> 1) : (q >> 1); }

// Key side: channel c' (0..31 inside the lane group's 32 channels) -> (mfma m, slot s)
template <int BITS>
__device__ __forceinline__ void k_pos(int cp, int& m, int& s) {
  if (BITS == 2) {  // word (cp/16), even/odd nibble plane, nibble index
    m = 2 * (cp >> 4) + (cp & 1);
    s = (cp & 15) >> 1;
  } else {          // word cp/8
    m = cp >> 3;
    s = slot4(cp & 7);
  }
}
// Value side: token position p (0..15 inside the lane group's 16 tokens)
template <int BITS>
__device__ __forceinline__ void v_pos(int p, int& m, int& s) {
  if (BITS == 2) {
    m = p & 1;
    s = p >> 1;
  } else {
    m = p >> 3;
    s = slot4(p & 7);
  }
}

// value arr[2*g + hh] for lane group g without dynamic register indexing
template <int RR>
__device__ __forceinline__ float pick(const float (&arr)[RR], int g, int hh) {
  float v = arr[hh < RR ? hh : 0];
#pragma unroll
  for (int i = 1; i < (RR + 1) / 2; i++)
    if (g == i && 2 * i + hh < RR) v = arr[2 * i + hh];
  return v;
}

template <int RR>
struct Cfg {
  static constexpr int ROWS = 2 * RR;                       // A rows: (head, hi|lo)
  static constexpr int CH = RR <= 2 ? 512 : (RR == 4 ? 256 : 128);   // tokens / chunk
  static constexpr int CT = CH / 64;                        // tiles / chunk
  static constexpr int A_HALVES = kNG * 2 * ROWS * 32;      // value A (key A is smaller)
  static constexpr int LDS_A = A_HALVES / 2;                // floats
  static constexpr int LDS_SC = RR * CH;
  static constexpr int LDS_O = RR * kD + 2 * RR;
  static constexpr int LDS_WAVE = LDS_A + LDS_SC + LDS_O;   // floats per wave
};

template <int BITS, int RR, int NW>
__global__ void __launch_bounds__(NW * 64) decode_mfma_kernel(DecodeArgs a) {
  using C = Cfg<RR>;
  constexpr int ROWS = C::ROWS, CH = C::CH, CT = C::CT;
  constexpr int E = 32 / BITS;
  constexpr int W = kD / E;        // words per key row
  constexpr int WPC = 64 / E;      // words per channel per value tile
  __shared__ __align__(16) float smem[NW * C::LDS_WAVE];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n16 = lane & 15, kg = lane >> 4;
  const int S = a.S, H = a.H, r = a.r;
  const int u = blockIdx.x / S, split = blockIdx.x % S;
  const int b = u / H;
  const int tq = a.tq, tr = a.tr;

  float* my = smem + wv * C::LDS_WAVE;
  _Float16* lds_a = reinterpret_cast<_Float16*>(my);
  float* lds_sc = my + C::LDS_A;
  float* lds_o = lds_sc + C::LDS_SC;      // [RR][D], then m[RR], l[RR]

  const size_t plane = (size_t)u;
  const uint32_t* kc = a.k_codes + plane * (size_t)a.cap * W;
  const float* ksc = a.k_scale + plane * (size_t)(a.cap / kG) * kD;
  const float* kzr = a.k_zero + plane * (size_t)(a.cap / kG) * kD;
  const uint32_t* vc = a.v_codes + plane * (size_t)a.cap * (kD / E);
  const float* vsc = a.v_scale + plane * (size_t)a.cap * kNG;
  const float* vzr = a.v_zero + plane * (size_t)a.cap * kNG;
  const uint16_t* kr = a.k_res + plane * (size_t)a.R * kD;
  const uint16_t* vr = a.v_res + plane * (size_t)a.R * kD;
  const size_t qrow0 = (size_t)b * H * r + (size_t)(u % H) * r;

  // this wave's share: value tiles [t_begin, t_end) and residual [r_begin, r_end)
  const int NWT = S * NW, gw = split * NW + wv;
  const int nT = (tq + 63) / 64;
  const int t_begin = (int)((int64_t)gw * nT / NWT), t_end = (int)((int64_t)(gw + 1) * nT / NWT);
  const int r_begin = (int)((int64_t)gw * tr / NWT), r_end = (int)((int64_t)(gw + 1) * tr / NWT);

  // scaled query (log2 domain) for channels 2*lane, 2*lane+1
  const float qs = a.scale * kLog2e;
  float sq0[RR], sq1[RR];
#pragma unroll
  for (int h = 0; h < RR; h++) {
    sq0[h] = 0.f;
    sq1[h] = 0.f;
    if (h < r) {
      const uint32_t qq = *reinterpret_cast<const uint32_t*>(a.q + (qrow0 + h) * kD + 2 * lane);
      sq0[h] = qs * h2f((uint16_t)(qq & 0xFFFFu));
      sq1[h] = qs * h2f((uint16_t)(qq >> 16));
    }
  }

  float m_run[RR], l_acc[RR], l_res[RR], ores0[RR], ores1[RR];
  float gam[RR][kNG];
#pragma unroll
  for (int h = 0; h < RR; h++) {
    m_run[h] = -INFINITY;
    l_acc[h] = l_res[h] = ores0[h] = ores1[h] = 0.f;
#pragma unroll
    for (int j = 0; j < kNG; j++) gam[h][j] = 0.f;
  }
  float4v cv[8];
#pragma unroll
  for (int nb = 0; nb < 8; nb++) cv[nb] = float4v{0.f, 0.f, 0.f, 0.f};

  const bool a_row_ok = n16 < 2 * r;    // A rows beyond 2r stay zero

  // new chunk maximum -> rescale every running quantity
  auto rescale = [&](int ntok) {
    float alpha[RR];
    bool any = false;
#pragma unroll
    for (int h = 0; h < RR; h++) {
      alpha[h] = 1.f;
      if (h < r) {
        float mx = -INFINITY;
        for (int k = lane; k < ntok; k += 64) mx = fmaxf(mx, lds_sc[h * CH + k]);
        mx = wave_max(mx);
        const float m_new = fmaxf(m_run[h], mx);
        alpha[h] = fast_exp2(m_run[h] - m_new);
        any |= m_new != m_run[h];
        m_run[h] = m_new;
      }
    }
    if (any) {
#pragma unroll
      for (int h = 0; h < RR; h++) {
        l_acc[h] *= alpha[h];
        l_res[h] *= alpha[h];
        ores0[h] *= alpha[h];
        ores1[h] *= alpha[h];
#pragma unroll
        for (int j = 0; j < kNG; j++) gam[h][j] *= alpha[h];
      }
      const float a0 = pick<RR>(alpha, kg, 0), a1 = pick<RR>(alpha, kg, 1);
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        cv[nb][0] *= a0;
        cv[nb][1] *= a0;
        cv[nb][2] *= a1;
        cv[nb][3] *= a1;
      }
    }
  };

  // Everything one 64-token tile needs from memory, held in registers so the
  // next tile's loads are in flight while the current tile is computed.
  using KCode = typename std::conditional<BITS == 2, uint2, uint4>::type;
  using VCode = typename std::conditional<BITS == 2, uint32_t, uint2>::type;
  struct KTile {
    KCode c[4];        // codes of 4 x 16 tokens, 32 channels of this lane group
    float2 s[2], z[2]; // key scale / zero of channels 2*lane, 2*lane+1, 2 groups
  };
  struct VTile {
    VCode c[8];        // codes of 16 tokens of channel 16*nb + n16, nb = 0..7
    float4 s, z;       // value scale / zero of token lane, 4 groups
  };
  auto load_k = [&](int tile, KTile& kt) {
    const int tok0 = tile * 64;
    const bool half_tile = tok0 + 64 > tq;
#pragma unroll
    for (int mb = 0; mb < 4; mb++) {
      if (mb < 2 || !half_tile) {
        const size_t row = (size_t)tok0 + 16 * mb + n16;
        kt.c[mb] = *reinterpret_cast<const KCode*>(kc + row * W + (BITS == 2 ? 2 : 4) * kg);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (kb == 0 || !half_tile) {
        const size_t g = (size_t)(tok0 >> 5) + kb;
        kt.s[kb] = *reinterpret_cast<const float2*>(ksc + g * kD + 2 * lane);
        kt.z[kb] = *reinterpret_cast<const float2*>(kzr + g * kD + 2 * lane);
      }
    }
  };
  auto load_v = [&](int tile, VTile& vt) {
    const uint32_t* base = vc + (size_t)tile * kD * WPC;
#pragma unroll
    for (int nb = 0; nb < 8; nb++)
      vt.c[nb] = *reinterpret_cast<const VCode*>(base + (16 * nb + n16) * WPC +
                                                 (BITS == 2 ? 1 : 2) * kg);
    const size_t t = (size_t)tile * 64 + lane;
    vt.s = *reinterpret_cast<const float4*>(vsc + t * kNG);
    vt.z = *reinterpret_cast<const float4*>(vzr + t * kNG);
  };

  // scores of one tile -> lds_sc[h][i*64 + token]
  auto do_k = [&](int tile, int i, const KTile& kt) {
    const int tok0 = tile * 64;
    const bool half_tile = tok0 + 64 > tq;   // only the first 32 tokens exist
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (kb == 1 && half_tile) {
#pragma unroll
        for (int h = 0; h < RR; h++)
          if (h < r && lane < 32) lds_sc[h * CH + i * 64 + 32 + lane] = -INFINITY;
        continue;
      }
      const float2 s2 = kt.s[kb], z2 = kt.z[kb];
      float qa[RR], qb[RR], bpart[RR], beta[RR];
      float qmax = 0.f;
#pragma unroll
      for (int h = 0; h < RR; h++) {
        qa[h] = sq0[h] * s2.x;
        qb[h] = sq1[h] * s2.y;
        bpart[h] = sq0[h] * z2.x + sq1[h] * z2.y;
        qmax = fmaxf(qmax, fmaxf(fabsf(qa[h]), fabsf(qb[h])));
      }
      // power-of-two prescale keeps the fp16 hi part finite for any input
      qmax = wave_max(qmax);
      const int ex = max(0, (int)((__builtin_bit_cast(uint32_t, qmax) >> 23) & 0xFF) - 127 - 13);
      const float down = __builtin_bit_cast(float, (uint32_t)(127 - ex) << 23);
      const float up = __builtin_bit_cast(float, (uint32_t)(127 + ex) << 23);
      {
        int m0, s0, m1, s1;
        const int cp = (2 * lane) & 31;
        k_pos<BITS>(cp, m0, s0);
        k_pos<BITS>(cp + 1, m1, s1);
        const int kgc = (2 * lane) >> 5;
#pragma unroll
        for (int h = 0; h < RR; h++) {
          if (h < r) {
            const float x0 = qa[h] * down, x1 = qb[h] * down;
            const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
            const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
            lds_a[((m0 * ROWS + 2 * h) * 4 + kgc) * 8 + s0] = h0;
            lds_a[((m0 * ROWS + 2 * h + 1) * 4 + kgc) * 8 + s0] = l0;
            lds_a[((m1 * ROWS + 2 * h) * 4 + kgc) * 8 + s1] = h1;
            lds_a[((m1 * ROWS + 2 * h + 1) * 4 + kgc) * 8 + s1] = l1;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < RR; h++) beta[h] = h < r ? wave_sum(bpart[h]) : 0.f;
      __builtin_amdgcn_wave_barrier();
      half8 af[4];
#pragma unroll
      for (int m = 0; m < 4; m++) {
        af[m] = half8{0, 0, 0, 0, 0, 0, 0, 0};
        if (a_row_ok)
          af[m] = *reinterpret_cast<const half8*>(lds_a + ((m * ROWS + n16) * 4 + kg) * 8);
      }
      __builtin_amdgcn_wave_barrier();
      const float b0 = pick<RR>(beta, kg, 0), b1 = pick<RR>(beta, kg, 1);
#pragma unroll
      for (int mb2 = 0; mb2 < 2; mb2++) {
        const int mb = 2 * kb + mb2;
        float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
        if constexpr (BITS == 2) {
          const uint2 w = kt.c[mb];
#pragma unroll
          for (int wp = 0; wp < 2; wp++) {
            const uint32_t x = wp ? w.y : w.x;
            acc = mfma(af[2 * wp], cvt_nib2(x & 0x33333333u), acc);
            acc = mfma(af[2 * wp + 1], cvt_nib2((x >> 2) & 0x33333333u), acc);
          }
        } else {
          const uint4 w = kt.c[mb];
          acc = mfma(af[0], cvt_word4(w.x), acc);
          acc = mfma(af[1], cvt_word4(w.y), acc);
          acc = mfma(af[2], cvt_word4(w.z), acc);
          acc = mfma(af[3], cvt_word4(w.w), acc);
        }
        const int k = i * 64 + 16 * mb + n16;
        const int h0 = 2 * kg, h1 = 2 * kg + 1;
        if (h0 < r) lds_sc[h0 * CH + k] = (acc[0] + acc[1]) * up + b0;
        if (h1 < r) lds_sc[h1 * CH + k] = (acc[2] + acc[3]) * up + b1;
      }
    }
  };

  // P.V of one tile into the cv accumulators
  auto do_v = [&](int tile, int i, const VTile& vt) {
    const int t = tile * 64 + lane;              // this lane's token
    const bool valid = t < tq;
    const float sj[4] = {vt.s.x, vt.s.y, vt.s.z, vt.s.w};
    const float zj[4] = {valid ? vt.z.x : 0.f, valid ? vt.z.y : 0.f, valid ? vt.z.z : 0.f,
                         valid ? vt.z.w : 0.f};
    int mt, st;
    v_pos<BITS>(lane & 15, mt, st);
    const int kgt = lane >> 4;
#pragma unroll
    for (int h = 0; h < RR; h++) {
      if (h < r) {
        const float p = valid ? fast_exp2(lds_sc[h * CH + i * 64 + lane] - m_run[h]) : 0.f;
        l_acc[h] += p;
#pragma unroll
        for (int j = 0; j < kNG; j++) {
          gam[h][j] += p * zj[j];
          const float x = valid ? p * sj[j] : 0.f;
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)(x - (float)hi);
          lds_a[((((j * 2 + mt) * ROWS) + 2 * h) * 4 + kgt) * 8 + st] = hi;
          lds_a[((((j * 2 + mt) * ROWS) + 2 * h + 1) * 4 + kgt) * 8 + st] = lo;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kNG; j++) {
      half8 av0 = half8{0, 0, 0, 0, 0, 0, 0, 0}, av1 = av0;
      if (a_row_ok) {
        av0 = *reinterpret_cast<const half8*>(lds_a + (((j * 2 + 0) * ROWS + n16) * 4 + kg) * 8);
        av1 = *reinterpret_cast<const half8*>(lds_a + (((j * 2 + 1) * ROWS + n16) * 4 + kg) * 8);
      }
#pragma unroll
      for (int nbj = 0; nbj < 2; nbj++) {
        const int nb = 2 * j + nbj;
        if constexpr (BITS == 2) {
          const uint32_t x = vt.c[nb];
          cv[nb] = mfma(av0, cvt_nib2(x & 0x33333333u), cv[nb]);
          cv[nb] = mfma(av1, cvt_nib2((x >> 2) & 0x33333333u), cv[nb]);
        } else {
          const uint2 x = vt.c[nb];
          cv[nb] = mfma(av0, cvt_word4(x.x), cv[nb]);
          cv[nb] = mfma(av1, cvt_word4(x.y), cv[nb]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // software pipeline: the loads of step n+1 are issued before step n runs
  KTile kt;
  VTile vt;
  if (t_begin < t_end) load_k(t_begin, kt);
  for (int c0 = t_begin; c0 < t_end; c0 += CT) {
    const int nt = min(CT, t_end - c0);
    for (int i = 0; i < nt; i++) {
      const KTile cur = kt;
      if (i + 1 < nt)
        load_k(c0 + i + 1, kt);
      else
        load_v(c0, vt);
      do_k(c0 + i, i, cur);
    }
    __builtin_amdgcn_wave_barrier();
    rescale(nt * 64);
    for (int i = 0; i < nt; i++) {
      const VTile cur = vt;
      if (i + 1 < nt)
        load_v(c0 + i + 1, vt);
      else if (c0 + nt < t_end)
        load_k(c0 + nt, kt);
      do_v(c0 + i, i, cur);
    }
  }

  // ---------------- residual slice (full precision), VALU
  for (int c0 = r_begin; c0 < r_end; c0 += CH) {
    const int c1 = min(r_end, c0 + CH);
    for (int t = c0; t < c1; t++) {
      const uint32_t kk = *reinterpret_cast<const uint32_t*>(kr + (size_t)t * kD + 2 * lane);
      const float k0 = h2f((uint16_t)(kk & 0xFFFFu)), k1 = h2f((uint16_t)(kk >> 16));
#pragma unroll
      for (int h = 0; h < RR; h++) {
        if (h < r) {
          const float sc = wave_sum(sq0[h] * k0 + sq1[h] * k1);
          if (lane == 0) lds_sc[h * CH + (t - c0)] = sc;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    rescale(c1 - c0);
    for (int t = c0; t < c1; t++) {
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(vr + (size_t)t * kD + 2 * lane);
      const float v0 = h2f((uint16_t)(vv & 0xFFFFu)), v1 = h2f((uint16_t)(vv >> 16));
#pragma unroll
      for (int h = 0; h < RR; h++) {
        if (h < r) {
          const float p = fast_exp2(lds_sc[h * CH + (t - c0)] - m_run[h]);
          l_res[h] += p;
          ores0[h] += p * v0;
          ores1[h] += p * v1;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---------------- wave result -> LDS: o[h][d], m[h], l[h]
  {
    const int h0 = 2 * kg, h1 = 2 * kg + 1;
#pragma unroll
    for (int nb = 0; nb < 8; nb++) {
      if (h0 < r) lds_o[h0 * kD + 16 * nb + n16] = cv[nb][0] + cv[nb][1];
      if (h1 < r) lds_o[h1 * kD + 16 * nb + n16] = cv[nb][2] + cv[nb][3];
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < RR; h++) {
    if (h < r) {
      float gsum[kNG];
#pragma unroll
      for (int j = 0; j < kNG; j++) gsum[j] = wave_sum(gam[h][j]);
      const float lsum = wave_sum(l_acc[h]) + l_res[h];
      // channels 2*lane, 2*lane+1 lie in value group (2*lane)/32 = lane/16
      float gj = gsum[0];
#pragma unroll
      for (int j = 1; j < kNG; j++)
        if (kg == j) gj = gsum[j];
      lds_o[h * kD + 2 * lane] += gj + ores0[h];
      lds_o[h * kD + 2 * lane + 1] += gj + ores1[h];
      if (lane == 0) {
        lds_o[RR * kD + h] = m_run[h];
        lds_o[RR * kD + RR + h] = lsum;
      }
    }
  }
  __syncthreads();

  // ---------------- merge the block's waves
  for (int idx = threadIdx.x; idx < r * kD; idx += NW * 64) {
    const int h = idx / kD, d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) M = fmaxf(M, smem[w * C::LDS_WAVE + C::LDS_A + C::LDS_SC + RR * kD + h]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; w++) {
        const float* o = smem + w * C::LDS_WAVE + C::LDS_A + C::LDS_SC;
        const float f = fast_exp2(o[RR * kD + h] - M);
        O += o[h * kD + d] * f;
        L += o[RR * kD + RR + h] * f;
      }
    }
    const size_t row = qrow0 + h;
    if (S == 1) {
      a.out[row * kD + d] = f2h(O / L);
    } else {
      const size_t rows = (size_t)a.B * H * r;
      if (d == 0) {
        a.ws[row * S + split] = M * kLn2;          // natural-log units for the combine
        a.ws[rows * S + row * S + split] = L;
      }
      a.ws[2 * rows * S + (row * S + split) * kD + d] = O;
    }
  }
}

// blocks of 16 waves only where their LDS fits (r <= 2)
template <int BITS, int RR>
hipError_t launch_rr(const DecodeArgs& a, int nw, hipStream_t st) {
  const dim3 grid(a.B * a.H * a.S);
  if (nw == 16 && RR <= 2)
    decode_mfma_kernel<BITS, RR, (RR <= 2 ? 16 : 8)><<<grid, (RR <= 2 ? 16 : 8) * 64, 0, st>>>(a);
  else if (nw >= 8)
    decode_mfma_kernel<BITS, RR, 8><<<grid, 8 * 64, 0, st>>>(a);
  else
    decode_mfma_kernel<BITS, RR, 4><<<grid, 4 * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int decode_mfma_block_waves(int r, int nw) {
  if (nw == 16 && r <= 2) return 16;
  return nw >= 8 ? 8 : 4;
}

namespace {

template <int BITS>
hipError_t launch_bits(const DecodeArgs& a, int nw, hipStream_t st) {
  if (a.r == 1) return launch_rr<BITS, 1>(a, nw, st);
  if (a.r == 2) return launch_rr<BITS, 2>(a, nw, st);
  if (a.r <= 4) return launch_rr<BITS, 4>(a, nw, st);
  return launch_rr<BITS, 8>(a, nw, st);
}

}  // namespace

bool decode_mfma_supported(int D, int G, int r) { return D == kD && G == kG && r >= 1 && r <= 8; }

hipError_t launch_decode_mfma(const DecodeArgs& a, int nw, hipStream_t st) {
  return a.bits == 2 ? launch_bits<2>(a, nw, st) : launch_bits<4>(a, nw, st);
}

}  // namespace kivi

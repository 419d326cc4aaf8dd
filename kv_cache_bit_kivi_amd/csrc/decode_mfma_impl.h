// The matrix-core decode kernel template and its launch helpers, shared by
// the translation units that instantiate it: decode_mfma.hip (lengths
// uniform across the batch), decode_mfma_ragged.hip (per-sequence lengths),
// decode_mfma_paged.hip (paged store), and their key-outlier variants
// (decode_mfma_o1.hip, decode_mfma_o2.hip, decode_mfma_ragged_o.hip,
// decode_mfma_paged_o.hip).  The method and the kernel's design are
// described at the top of decode_mfma.hip.
#pragma once

#include <math.h>

#include <atomic>
#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __fp16 hrtz2 __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 32;
constexpr int kNG = kD / kG;   // value groups per token
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;   // log2 slack of the online-softmax reference

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

// 8 codes of at most two bits held one per nibble (upper bits zero) -> 8
// exact halves, slot s = nibble s.  The e2m1 value of nibble c is c/2, so
// scale 2 gives the codes and scale 8 four times them (the high plane of a
// three-bit code).
__device__ __forceinline__ half8 cvt_nib2(uint32_t x, float sc = 2.0f) {
  half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, sc, 0);
  half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, sc, 1);
  half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, sc, 2);
  half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, sc, 3);
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
// the same two code converts to bf16 (value side)
__device__ __forceinline__ bf16x8 cvt_nib2_bf(uint32_t x, float sc = 2.0f) {
  bf16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 0);
  bf16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 1);
  bf16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 2);
  bf16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 3);
  return bf16x8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}
__device__ __forceinline__ bf16x8 cvt_word4_bf(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);
  return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
__device__ __forceinline__ float4v mfma(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma_bf(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// (hi, lo) bf16 pairs of two binary32 values: hi = x truncated to bf16, lo =
// the remainder truncated; hi + lo = x within 2^-16 |x|, over the full
// binary32 exponent range.  Lane 0 of each pair holds x0, lane 1 x1.
__device__ __forceinline__ void split2_bf(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t u0 = __builtin_bit_cast(uint32_t, x0), u1 = __builtin_bit_cast(uint32_t, x1);
  const float r0 = x0 - __builtin_bit_cast(float, u0 & 0xFFFF0000u);
  const float r1 = x1 - __builtin_bit_cast(float, u1 & 0xFFFF0000u);
  hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // upper halves of u0, u1
  lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, r1), __builtin_bit_cast(uint32_t, r0),
                             0x07060302u);
}
// (hi, lo) fp16 pairs of two binary32 values: hi = x rounded toward zero,
// lo = the remainder rounded toward zero; hi + lo = x within 2^-20 |x|
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const hrtz2 h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
  const hrtz2 l = __builtin_amdgcn_cvt_pkrtz(x0 - (float)h.x, x1 - (float)h.y);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Raw buffer loads: a resource covers one plane; an offset at or past its end
// returns zeros and touches no memory.  Absent tiles and tokens are loaded at
// kOut instead of being branched around, so every wave issues one fixed load
// sequence and the in-order completion counter stays exact.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOut = 0x80000000u;   // past every plane (planes stay < 2^31 bytes)
// Cache policy of the streamed cache reads: non-temporal.  Every cache byte is
// read once per call, so keeping it out of the normal cache-allocation path
// costs nothing and measurably raises the achieved read bandwidth.
constexpr int kStream = 2;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream);
  return uint4{v.x, v.y, v.z, v.w};
}
// (bit-cast the whole vector: clang bit-casts an ext-vector element access
// from the vector's first element)
__device__ __forceinline__ float4 ld16f(rsrc_t r, uint32_t off) {
  const f32x4 v =
      __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream));
  return float4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ u32x4 ld16v(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream);
}
// one 16-byte slice of residual token t: from the residual plane (zeros past
// the slice), or from the new-token row when t is the freshly appended token.
// The two arms are exec-masked loads into one register: one load per lane.
__device__ __forceinline__ u32x4 ld_res(rsrc_t res, rsrc_t nw, int t, int t_end, int t_new,
                                        uint32_t row_bytes, uint32_t col) {
  u32x4 v;
  if (t != t_new)
    v = ld16v(res, t < t_end ? (uint32_t)t * row_bytes + col : kOut);
  else
    v = ld16v(nw, col);
  return v;
}
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ uint2 ld8(rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return uint2{v.x, v.y};
}
__device__ __forceinline__ uint2 ld8s(rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kStream);
  return uint2{v.x, v.y};
}
// four metadata values of a lane: binary32 as loaded, or four binary16 widened
__device__ __forceinline__ float4 meta4(float4 v) { return v; }
__device__ __forceinline__ float4 meta4(uint2 v) {
  return float4{h2f((uint16_t)(v.x & 0xFFFFu)), h2f((uint16_t)(v.x >> 16)),
                h2f((uint16_t)(v.y & 0xFFFFu)), h2f((uint16_t)(v.y >> 16))};
}

// slot of position q (0..7) inside a 4-bit word's half8
__device__ __forceinline__ int slot4(int q) { return (q & 1) ? 4 + (q >> 1) : (q >> 1); }

// Key side: channel c' (0..31 inside a lane group's 32 channels) -> (mfma m,
// slot s).  1 and 3 bits use the 2-bit mapping: the one-bit order puts code
// position p of a word in nibble plane m, nibble s of exactly this mapping.
template <int BITS>
__device__ __forceinline__ void k_pos(int cp, int& m, int& s) {
  if (BITS != 4) {  // word cp/16, even/odd nibble plane, nibble index
    m = 2 * (cp >> 4) + (cp & 1);
    s = (cp & 15) >> 1;
  } else {          // word cp/8
    m = cp >> 3;
    s = slot4(cp & 7);
  }
}
// Value side: token position p (0..15 inside a lane group's 16 tokens)
template <int BITS>
__device__ __forceinline__ void v_pos(int p, int& m, int& s) {
  if (BITS != 4) {
    m = p & 1;
    s = p >> 1;
  } else {
    m = p >> 3;
    s = slot4(p & 7);
  }
}

// Code of channel d (a compile-time constant after unrolling) from the W
// words of a token's key row, as a float (the documented row layouts: 2 and
// 4 bits little-endian; 1 bit at beta(d % 32) of word d / 32; 3 bits as the
// 2-bit plane, then the 1-bit plane of the high bits).
__device__ __forceinline__ constexpr int beta_pos(int p) {
  return 4 * ((p & 15) >> 1) + 2 * (p >> 4) + (p & 1);
}
template <int BITS>
__device__ __forceinline__ float key_code(const uint32_t* w, int d) {
  if constexpr (BITS == 2) {
    return (float)((w[d >> 4] >> (2 * (d & 15))) & 3u);
  } else if constexpr (BITS == 4) {
    return (float)((w[d >> 3] >> (4 * (d & 7))) & 15u);
  } else if constexpr (BITS == 1) {
    return (float)((w[d >> 5] >> beta_pos(d & 31)) & 1u);
  } else {
    return (float)(((w[d >> 4] >> (2 * (d & 15))) & 3u) |
                   (((w[kD / 16 + (d >> 5)] >> beta_pos(d & 31)) & 1u) << 2));
  }
}

// value arr[2*g + hh] for lane group g without dynamic register indexing
template <int R>
__device__ __forceinline__ float pick(const float (&arr)[R], int g, int hh) {
  float v = arr[hh < R ? hh : 0];
#pragma unroll
  for (int i = 1; i < (R + 1) / 2; i++)
    if (g == i && 2 * i + hh < R) v = arr[2 * i + hh];
  return v;
}

// floor(g * n / parts) for 0 <= g <= parts < 2^16 and n >= 0, exactly, in
// 32-bit arithmetic (g (n mod parts) < 2^32).  This keeps the wave-uniform
// prologue short: a 64-bit division expands to about a hundred scalar
// instructions, and the waves of a compute unit share one scalar unit.  (The
// C ABI caps the split count at 4096, so S * NW < 2^16.)
__device__ __forceinline__ int part_bound(int g, int n, int parts) {
  const uint32_t p = (uint32_t)parts, q = (uint32_t)n / p, r = (uint32_t)n - q * p;
  return (int)((uint32_t)g * q + ((uint32_t)g * r) / p);
}

// Block barrier that publishes LDS writes but, unlike __syncthreads, does
// not wait for the wave's outstanding global loads (lgkmcnt(0) only; the
// signal fences keep the compiler from moving memory accesses across it)
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int BITS, int R>
struct Cfg {
  static constexpr int ROWS = 2 * R;                    // A rows: (head, hi|lo)
  static constexpr int CH = 64;                         // score slots: one tile
  static constexpr int KC_BYTES = 64 * kD * BITS / 8;   // key codes of one tile
  static constexpr int VC_BYTES = 64 * kD * BITS / 8;   // value codes of one tile
  static constexpr int A_BYTES = kNG * 2 * ROWS * 64;   // value A (two key groups: same)
  static constexpr int RES_BYTES = 4 * ROWS * 64;       // residual key A
  static constexpr int SC_BYTES = R * CH * 4;
  static constexpr int O_BYTES = ((R * kD + 2 * R) * 4 + 15) / 16 * 16;  // keeps stg 16-aligned
  static constexpr int DUMMY_BYTES = 64;                // sink for writes of absent heads
  static constexpr int STG_BYTES = KC_BYTES + VC_BYTES; // staged codes of one tile
  static constexpr int WAVE_BYTES =
      A_BYTES + RES_BYTES + SC_BYTES + O_BYTES + DUMMY_BYTES + STG_BYTES;
  static constexpr int ZERO_BYTES = ROWS < 16 ? A_BYTES : 0;  // all-zero rows, per block
  static_assert(WAVE_BYTES % 16 == 0 && A_BYTES % 16 == 0, "b128 LDS accesses need 16-byte alignment");
};

// register budget of the occupancy target: one wave per SIMD for 8 heads and
// for pre-RoPE keys with several heads, two waves otherwise (blocks of 8 waves
// place two per SIMD).  Three waves per SIMD (12-wave blocks) fit the one-head
// 2-bit variant without spills (158 registers) but measured slower (28.1
// against 27.1 us on the batch-8 Llama layer).
template <int BITS, int R, bool ROPE = false, int KO = 0>
constexpr int waves_per_eu() {
  return (R >= 8 || (ROPE && R >= 2)) ? 1 : 2;
}

// tiles of loads in flight per wave: one (a second register set measured no
// faster at two waves per SIMD), two for 8 heads at one wave per SIMD
template <int BITS, int R>
constexpr int prefetch_depth() {
  return R >= 8 ? 2 : 1;
}

// Binary32 metadata: issue the next tile's scales and zeros before the
// current tile's compute, in a second register set (as binary16 metadata
// always does), or after it.  Measured on one box, same binary otherwise:
// before is faster with several heads per KV head (Mistral-shaped r = 4
// layer 57.8-58.1 against 59.9-61.4 us) and for ragged batches (51.9-52.3
// against 52.5-52.9 us), after is faster for one head with uniform lengths
// (batch-8 Llama layer 27.0-27.1 against 27.8-27.9 us) and for the paged
// store (27.7-28.0 against 28.9 us with 256-token pages).  Outlier and
// pre-RoPE variants keep the order they were tuned with.
template <int R, bool MH, bool RAG, bool PG, int KO, bool ROPE>
constexpr bool early_meta() {
  return MH || (KO == 0 && !ROPE && !PG && R <= 4 && (R >= 2 || RAG));
}

// KO: key outliers per (group, channel) (0, 1 or 2; a.n_out == KO).  Each
// lane loads the outlier words of its key group and channels cq..cq+3 with
// the tile's metadata.  The correction q_d * (kept value - zero) of every
// outlier (the dense code there is 0, so the dense score already holds
// q_d * zero) is one more matrix product per slot: the slot's positions
// become a plane of 0/1 codes in the 2-bit key-row layout (each lane owns
// the byte of its 4 channels in every token row, so plain byte stores build
// it), multiplied on the matrix cores by q * (value - zero) as hi/lo rows,
// into the same accumulators as the dense scores.
// ROPE: the cached keys are pre-RoPE (a.rope_theta > 0; KO == 0).  Key
// scores are computed lane-per-token on the VALU: the key is dequantized,
// rotated by the angle of its position inside the tile (a per-block table
// F[pair][lane]) and dotted with the query rotated back by the tile's first
// position (one binary64 sincos per pair and tile, so tiles can come in any
// order).
template <int BITS, int R, int NW, bool MH, bool RAG, bool PG, int KO, bool ROPE>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<BITS, R, ROPE, KO>(),
                                   waves_per_eu<BITS, R, ROPE, KO>())))
decode_mfma_kernel(DecodeArgs a, LensT<RAG> lens) {
  static_assert(!PG || RAG, "paged launches carry per-sequence lengths");
  using C = Cfg<BITS, R>;
  constexpr int ROWS = C::ROWS, CH = C::CH;
  constexpr int W = kD * BITS / 32;   // words per key row
  constexpr int WPC = 2 * BITS;       // words per channel per value tile
  static_assert(!(ROPE && KO > 0), "pre-RoPE keys take no outlier corrections here");
  // pre-RoPE: the block's table F[pair][lane] = (cos, sin)(theta_pair * lane);
  // per wave the tile's scale / zero pairs [group][pair][4] (2 KB: in the A
  // tile region, which the key product no longer uses, when it is that large,
  // else in a region of its own) and the rotated query [pair][head] (float2,
  // in the residual-A region: exactly its size)
  constexpr int RT_BYTES = ROPE ? 64 * 64 * 8 : 0;
  // (one head: 1 KB more for the per-pair constant terms of the folded form)
  constexpr int RW_BYTES = (ROPE && C::A_BYTES < 2048) ? (R == 1 ? 3072 : 2048) : 0;
  // outlier slot plane: 64 token rows x 32 bytes, in the staged key-code region
  // once the key product has read it, or in a region of its own (1-bit codes)
  constexpr int MK_BYTES = (KO > 0 && C::KC_BYTES < 2048) ? 2048 : 0;
  static_assert(!ROPE || C::RES_BYTES == 64 * R * 8, "rotated query fills the residual-A region");
  // several heads per KV head, stored keys: the zero term beta of every head
  // and key group is one more matrix product per tile (the scaled query rows
  // of the residual key product times the tile's key zeros), so the per-head
  // cross-lane sums leave the vector units; per wave the tile's key zeros as
  // binary16 [group][channel] (512 bytes)
  constexpr bool BMF = R >= 2 && !ROPE;
  constexpr int KZ_BYTES = BMF ? 2 * kD * 2 : 0;
  __shared__ __align__(16) char smem[C::ZERO_BYTES + NW * C::WAVE_BYTES + RT_BYTES +
                                     NW * (RW_BYTES + MK_BYTES + KZ_BYTES)];
  // tiles the block's waves have taken beyond their first two (shared tiles)
  __shared__ int tile_ctr;

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n16 = lane & 15, kg = lane >> 4;
  const int S = a.S, H = a.H;
  const int bs = (int)(blockIdx.x / (uint32_t)S);
  const int u = seq_plane<RAG>(lens, bs, H), split = (int)blockIdx.x - bs * S;
  const int b = (int)((uint32_t)u / (uint32_t)H), hh = u - b * H;
  const int tq = seq_tq<RAG>(a, lens, b), tr = seq_tr<RAG>(a, lens, b);

  char* zero = smem;
  char* my = smem + C::ZERO_BYTES + wv * C::WAVE_BYTES;
  char* lds_a = my;                                     // key / value A tiles
  char* lds_res = my + C::A_BYTES;                      // residual key A tile
  float* lds_sc = reinterpret_cast<float*>(lds_res + C::RES_BYTES);   // [R][CH]
  float* lds_o = reinterpret_cast<float*>(lds_res + C::RES_BYTES + C::SC_BYTES);
  float* lds_dummy = reinterpret_cast<float*>(reinterpret_cast<char*>(lds_o) + C::O_BYTES);
  char* stg = reinterpret_cast<char*>(lds_dummy) + C::DUMMY_BYTES;   // staged tile codes
  for (int i = threadIdx.x; i < C::ZERO_BYTES / 16; i += NW * 64)
    reinterpret_cast<uint4*>(zero)[i] = uint4{0, 0, 0, 0};
  if (threadIdx.x == 0) tile_ctr = 0;
  // (pre-RoPE launches publish these with the table, after the first loads)
  if constexpr (!ROPE) __syncthreads();
  float2* ftab = reinterpret_cast<float2*>(smem + C::ZERO_BYTES + NW * C::WAVE_BYTES);
  char* rope_wave = smem + C::ZERO_BYTES + NW * C::WAVE_BYTES + RT_BYTES + wv * RW_BYTES;
  char* mask_own = smem + C::ZERO_BYTES + NW * C::WAVE_BYTES + RT_BYTES + NW * RW_BYTES +
                   wv * MK_BYTES;
  char* kz_own = smem + C::ZERO_BYTES + NW * C::WAVE_BYTES + RT_BYTES +
                 NW * (RW_BYTES + MK_BYTES) + wv * KZ_BYTES;

  // per-(b, h) planes as buffer resources (uniform base, 32-bit lane offsets)
  const size_t plane = (size_t)u, cap = (size_t)a.cap;
  const rsrc_t r_kc = make_rsrc(a.k_codes + plane * cap * W, (uint32_t)(cap * W * 4));
  // metadata: MB bytes per value (binary16 or binary32)
  constexpr uint32_t MB = MH ? 2 : 4;
  using MetaT = std::conditional_t<MH, uint2, float4>;
  const size_t kmp = (cap / kG) * kD * MB, vmp = cap * kNG * MB;   // plane bytes
  const rsrc_t r_ks = make_rsrc(static_cast<const char*>(a.k_scale) + plane * kmp, (uint32_t)kmp);
  const rsrc_t r_kz = make_rsrc(static_cast<const char*>(a.k_zero) + plane * kmp, (uint32_t)kmp);
  const rsrc_t r_vc = make_rsrc(a.v_codes + plane * cap * (kD * BITS / 32), (uint32_t)(cap * (kD * BITS / 32) * 4));
  const rsrc_t r_vs = make_rsrc(static_cast<const char*>(a.v_scale) + plane * vmp, (uint32_t)vmp);
  const rsrc_t r_vz = make_rsrc(static_cast<const char*>(a.v_zero) + plane * vmp, (uint32_t)vmp);
  // key outliers: KO words per (group, channel), KO * 512 bytes per key group
  const size_t kop = (cap / kG) * KO * kD * 4;
  const rsrc_t r_ko = make_rsrc(a.k_out + plane * (kop / 4), (uint32_t)kop);
  const rsrc_t r_kr = make_rsrc(a.k_res + plane * (size_t)a.R * kD, (uint32_t)(a.R * kD * 2));
  const rsrc_t r_vr = make_rsrc(a.v_res + plane * (size_t)a.R * kD, (uint32_t)(a.R * kD * 2));
  // fused append: the new token (residual slot t_new) comes from its input row
  const bool fused = a.k_new != nullptr;
  const int t_new = fused ? tr - 1 : -1;
  const rsrc_t r_kn = make_rsrc(fused ? a.k_new + plane * kD : a.k_res, fused ? kD * 2 : 0);
  const rsrc_t r_vn = make_rsrc(fused ? a.v_new + plane * kD : a.v_res, fused ? kD * 2 : 0);
  const size_t qrow0 = (size_t)b * H * R + (size_t)hh * R;
  const rsrc_t r_q = make_rsrc(a.q + qrow0 * kD, (uint32_t)(R * kD * 2));

  // this wave's share: value tiles [t_begin, t_end) and residual [r_begin, r_end)
  const int NWT = S * NW, gw = split * NW + wv;
  const int nT = (tq + 63) / 64;
  const int t_begin = part_bound(gw, nT, NWT), t_end = part_bound(gw + 1, nT, NWT);
  const int r_begin = part_bound(gw, tr, NWT), r_end = part_bound(gw + 1, tr, NWT);
  // Shared tiles (a.share_tiles): the waves of the block take the split's
  // tiles [sb, se) as their loads return instead of keeping fixed runs, so a
  // wave whose loads come back late computes fewer tiles rather than holding
  // the block back.  Wave wv starts with sb + wv and sb + NW + wv; the k-th
  // tile taken from the block's counter is sb + 2 NW + k.  Tiles past t_lim
  // load as zeros and are never computed; a wave's tile indices increase, so
  // it computes every tile below t_lim that it takes.
  const bool share = a.share_tiles != 0;
  const int sb = part_bound(split, nT, S), se = part_bound(split + 1, nT, S);
  const int t_lim = share ? se : t_end;
  const int t_first = share ? sb + wv : t_begin;
  int t_given = share ? sb + NW + wv : t_begin + 1;   // last tile handed to this wave
  // taking a tile is split in two so that the LDS atomic's latency hides
  // behind a tile's compute: issue() reserves one (lane 0 holds the reply),
  // take() returns it
  auto issue = [&](int& pend) __attribute__((always_inline)) {
    if (share && lane == 0)
      pend = __hip_atomic_fetch_add(&tile_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto take = [&](const int& pend) __attribute__((always_inline)) -> int {
    return share ? sb + 2 * NW + __builtin_amdgcn_readfirstlane(pend) : ++t_given;
  };

  // Lane roles.  Every global load is 16 bytes per lane over 1 KB contiguous.
  //  key factors: lane -> key group kgrp = lane/32 of the tile and channels
  //    cq..cq+3 (cq = 4*(lane%32)), i.e. exactly its own 16-byte scale / zero
  //    load; channels cq, cq+2 (and cq+1, cq+3) sit in adjacent A slots, so
  //    hi/lo pairs are written as 32-bit words;
  //  value factors: lane -> token lane of the tile, its own 16-byte scale /
  //    zero load (4 value groups);
  //  codes: staged through LDS and re-read in the MFMA operand layout.
  //  One head per KV head (stored keys, no outliers): one key A operand
  //    serves both key groups (rows (group, hi|lo)) and one value A operand
  //    all four value groups (rows (group, hi|lo)), each output lane taking
  //    the rows of its own group, so each is read from LDS once per tile
  //    (otherwise the rows are (head, hi|lo) and each group has its own).
  constexpr bool SHA = R == 1 && KO == 0 && !ROPE;
  constexpr int KROWS = SHA ? 4 : ROWS;   // rows of the key A operand
  constexpr int VROWS = SHA ? 8 : ROWS;   // rows of the value A operand
  const int kgrp = lane >> 5, cq = 4 * (lane & 31);
  uint32_t kwr[2];      // A offsets of channel pairs (cq, cq+2), (cq+1, cq+3)
#pragma unroll
  for (int e = 0; e < 2; e++) {
    const int c = cq + e;
    int m, s;
    k_pos<BITS>(c & 31, m, s);
    kwr[e] = SHA ? (uint32_t)(((m * KROWS) * 4 + (c >> 5)) * 16 + 2 * s + (2 * kgrp) * 64)
                 : (uint32_t)(kgrp * (4 * ROWS * 64) + ((m * ROWS) * 4 + (c >> 5)) * 16 + 2 * s);
  }
  uint32_t kwr2[2];     // the same in the 2-bit operand order (outlier slot planes)
#pragma unroll
  for (int e = 0; e < 2; e++) {
    const int c = cq + e;
    int m, s;
    k_pos<2>(c & 31, m, s);
    kwr2[e] = (uint32_t)(kgrp * (4 * ROWS * 64) + ((m * ROWS) * 4 + (c >> 5)) * 16 + 2 * s);
  }
  int vm, vs0;
  v_pos<BITS>(lane & 15, vm, vs0);
  const uint32_t vwr = (uint32_t)(((vm * VROWS) * 4 + kg) * 16 + 2 * vs0);
  // A read bases: lanes of absent rows read the all-zero region instead
  const bool row_ok = n16 < ROWS;
  const char* a_rd = row_ok ? lds_a + (n16 * 4 + kg) * 16 : zero + kg * 16;
  const char* a_rdk = n16 < KROWS ? lds_a + (n16 * 4 + kg) * 16 : zero + kg * 16;
  const char* a_rdv = n16 < VROWS ? lds_a + (n16 * 4 + kg) * 16 : zero + kg * 16;
  const char* res_rd = row_ok ? lds_res + (n16 * 4 + kg) * 16 : zero + kg * 16;

  // Issue order matters: vector-memory loads complete in order, so the query
  // goes first, then the first residual batch, then the tile prefetch; waiting
  // for an earlier group never waits for a later one.
  uint2 q4r[R];
#pragma unroll
  for (int h = 0; h < R; h++) q4r[h] = ld8(r_q, (uint32_t)((h * kD + cq) * 2));
  __builtin_amdgcn_sched_barrier(0);

  // registers of a tile in flight: codes (2-bit uses x0..x3: key codes, then
  // value codes; 4-bit x0..x7), key scale / zero of key group kgrp, channels
  // cq..cq+3, value scale / zero of the token lane
  const uint32_t l16 = (uint32_t)lane * 16;
  // Paged store: the page slice of a tile (a scalar table lookup at a
  // wave-uniform index) and the tile's offset inside the slice.  Absent tiles
  // look up an entry that exists in the sequence's table row (tile t_first,
  // clamped to the sequence's last tile, or tile 0 when it has none) and
  // load nothing.
  const int P = a.pages.page_tokens;
  const int t_last = nT > 0 ? nT - 1 : 0;
  auto page_tile = [&](int tile, size_t& sp, uint32_t& lt64) __attribute__((always_inline)) {
    const int tu =
        __builtin_amdgcn_readfirstlane(tile < t_lim ? tile : (t_first < t_last ? t_first : t_last));
    int tok;
    const bool ok = page_slot(a.pages, b, hh, H, tu * 64, sp, tok);
    lt64 = (uint32_t)(tok / 64);
    return ok && tile < t_lim;
  };
  // codes / metadata of tile `tile` of this wave, or zeros (no memory access)
  // when it is past the wave's last tile.  Codes are reloaded as soon as they
  // are staged, metadata once the tile's compute has consumed them, so that
  // no register holds two generations at once (that would need copies, and a
  // copy waits for its load).
  auto load_codes = [&](int tile, uint4& x0, uint4& x1, uint4& x2, uint4& x3, uint4& x4,
                        uint4& x5, uint4& x6, uint4& x7) __attribute__((always_inline)) {
    uint32_t co = tile < t_lim ? (uint32_t)tile * C::KC_BYTES + l16 : kOut;  // KC == VC
    rsrc_t rkc = r_kc, rvc = r_vc;
    if constexpr (PG) {
      size_t sp;
      uint32_t lt;
      const bool ok = page_tile(tile, sp, lt);
      rkc = make_rsrc(a.k_codes + sp * P * W, (uint32_t)(P * W * 4));
      rvc = make_rsrc(a.v_codes + sp * P * (kD * BITS / 32), (uint32_t)(P * (kD * BITS / 32) * 4));
      co = ok ? lt * C::KC_BYTES + l16 : kOut;
    }
    if constexpr (BITS == 1) {
      x0 = ld16(rkc, co);
      x1 = ld16(rvc, co);
    } else if constexpr (BITS == 2) {
      x0 = ld16(rkc, co);
      x1 = ld16(rkc, co + 1024);
      x2 = ld16(rvc, co);
      x3 = ld16(rvc, co + 1024);
    } else if constexpr (BITS == 3) {
      x0 = ld16(rkc, co);
      x1 = ld16(rkc, co + 1024);
      x2 = ld16(rkc, co + 2048);
      x3 = ld16(rvc, co);
      x4 = ld16(rvc, co + 1024);
      x5 = ld16(rvc, co + 2048);
    } else {
      x0 = ld16(rkc, co);
      x1 = ld16(rkc, co + 1024);
      x2 = ld16(rkc, co + 2048);
      x3 = ld16(rkc, co + 3072);
      x4 = ld16(rvc, co);
      x5 = ld16(rvc, co + 1024);
      x6 = ld16(rvc, co + 2048);
      x7 = ld16(rvc, co + 3072);
    }
  };
  auto load_meta = [&](int tile, MetaT& ks, MetaT& kz, MetaT& vs, MetaT& vz, uint4& o0,
                       uint4& o1) __attribute__((always_inline)) {
    // 2 key groups x 128 channels, or 64 tokens x 4 value groups: 256 values
    // each, 4 per lane (converted to binary32 when the tile is computed)
    uint32_t mo = tile < t_lim ? (uint32_t)tile * (256 * MB) + lane * (4 * MB) : kOut;
    // outlier words j of key group 2*tile + kgrp, channels cq..cq+3
    uint32_t oo = tile < t_lim ? (uint32_t)((2 * tile + kgrp) * KO) * 512 + (lane & 31) * 16 : kOut;
    rsrc_t rks = r_ks, rkz = r_kz, rvs = r_vs, rvz = r_vz, rko = r_ko;
    if constexpr (PG) {
      size_t sp;
      uint32_t lt;
      const bool ok = page_tile(tile, sp, lt);
      const size_t kb = (size_t)(P / kG) * kD * MB, vb = (size_t)P * kNG * MB;  // slice bytes
      rks = make_rsrc(static_cast<const char*>(a.k_scale) + sp * kb, (uint32_t)kb);
      rkz = make_rsrc(static_cast<const char*>(a.k_zero) + sp * kb, (uint32_t)kb);
      rvs = make_rsrc(static_cast<const char*>(a.v_scale) + sp * vb, (uint32_t)vb);
      rvz = make_rsrc(static_cast<const char*>(a.v_zero) + sp * vb, (uint32_t)vb);
      mo = ok ? lt * (256 * MB) + lane * (4 * MB) : kOut;
      if constexpr (KO > 0) {
        const size_t ob = (size_t)(P / kG) * KO * kD * 4;
        rko = make_rsrc(a.k_out + sp * (ob / 4), (uint32_t)ob);
        oo = ok ? (uint32_t)((2 * lt + kgrp) * KO) * 512 + (lane & 31) * 16 : kOut;
      }
    }
    if constexpr (KO >= 1) o0 = ld16(rko, oo);
    if constexpr (KO >= 2) o1 = ld16(rko, oo == kOut ? kOut : oo + 512);
    if constexpr (MH) {
      ks = ld8s(rks, mo);
      kz = ld8s(rkz, mo);
      vs = ld8s(rvs, mo);
      vz = ld8s(rvz, mo);
    } else {
      ks = ld16f(rks, mo);
      kz = ld16f(rkz, mo);
      vs = ld16f(rvs, mo);
      vz = ld16f(rvz, mo);
    }
  };
  auto stage = [&](const uint4& x0, const uint4& x1, const uint4& x2, const uint4& x3,
                   const uint4& x4, const uint4& x5, const uint4& x6, const uint4& x7)
      __attribute__((always_inline)) {
    // 2*BITS loads of 1 KB: the tile's key codes, then its value codes
    uint4* d = reinterpret_cast<uint4*>(stg + l16);
    d[0] = x0;
    d[64] = x1;
    if constexpr (BITS >= 2) {
      d[128] = x2;
      d[192] = x3;
    }
    if constexpr (BITS >= 3) {
      d[256] = x4;
      d[320] = x5;
    }
    if constexpr (BITS == 4) {
      d[384] = x6;
      d[448] = x7;
    }
  };

  // residual slice, 16 tokens per batch.  Key lanes: token n16 of the batch,
  // channels 8*kg + 32*i .. +7 (MFMA B operand); value lanes: token group
  // tg = lane/16 (tokens tg, tg+4, tg+8, tg+12), channels 8*c8 .. 8*c8+7.
  // Tokens past the slice read zeros and weigh zero.  Under a fused append
  // every lane loads from both the residual and the new-token row, one of the
  // two offsets out of range, and ORs the results (no per-lane branch).
  const int tg = lane >> 4, c8 = lane & 15;
  u32x4 rk0, rk1, rk2, rk3;   // key rows (8 fp16 each, MFMA B operand)
  u32x4 rv0, rv1, rv2, rv3;   // value rows (8 fp16 each)
  auto load_res = [&](int t16) __attribute__((always_inline)) {
    const uint32_t rb = kD * 2;
    rk0 = ld_res(r_kr, r_kn, t16 + n16, r_end, t_new, rb, kg * 16);
    rk1 = ld_res(r_kr, r_kn, t16 + n16, r_end, t_new, rb, kg * 16 + 64);
    rk2 = ld_res(r_kr, r_kn, t16 + n16, r_end, t_new, rb, kg * 16 + 128);
    rk3 = ld_res(r_kr, r_kn, t16 + n16, r_end, t_new, rb, kg * 16 + 192);
    rv0 = ld_res(r_vr, r_vn, t16 + tg, r_end, t_new, rb, c8 * 16);
    rv1 = ld_res(r_vr, r_vn, t16 + tg + 4, r_end, t_new, rb, c8 * 16);
    rv2 = ld_res(r_vr, r_vn, t16 + tg + 8, r_end, t_new, rb, c8 * 16);
    rv3 = ld_res(r_vr, r_vn, t16 + tg + 12, r_end, t_new, rb, c8 * 16);
  };
  load_res(r_begin);
  __builtin_amdgcn_sched_barrier(0);

  // Loads run DEPTH tiles ahead of the compute, in DEPTH register sets used
  // round robin.  They are issued before the residual slice so that it
  // overlaps them.
  constexpr int DEPTH = prefetch_depth<BITS, R>();
  uint4 a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3, b4, b5, b6, b7;
  MetaT a_ks, a_kz, a_vs, a_vz, b_ks, b_kz, b_vs, b_vz;
  uint4 a_o0, a_o1, b_o0, b_o1;   // key-outlier words (KO > 0)
  // (the same issue order as the loop: codes A, meta A, codes B, meta B)
  load_codes(t_first, a0, a1, a2, a3, a4, a5, a6, a7);
  __builtin_amdgcn_sched_barrier(0);
  load_meta(t_first, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
  if constexpr (DEPTH == 2) {
    __builtin_amdgcn_sched_barrier(0);
    load_codes(t_given, b0, b1, b2, b3, b4, b5, b6, b7);
    __builtin_amdgcn_sched_barrier(0);
    load_meta(t_given, b_ks, b_kz, b_vs, b_vz, b_o0, b_o1);
  }
  __builtin_amdgcn_sched_barrier(0);

  // pre-RoPE: the block's table, built while the first loads are in flight
  // (the barrier after it waits for LDS only, not for those loads)
  // frequency of pair `lane`: rope_theta^(-2 lane / 128), binary64
  const double rp_lb = ROPE ? log2((double)a.rope_theta) : 0.0;
  const double rp_th = ROPE ? exp2(-(double)lane * (1.0 / 64.0) * rp_lb) : 0.0;
  if constexpr (ROPE) {
    // thread -> pair lane, lanes l0 .. l0 + 64/NW - 1 of the table: one
    // binary64 sincos, then exact-enough complex steps in binary64
    constexpr int LPT = 64 / NW;
    const int l0 = wv * LPT;
    double sn, c, ss, sc;
    sincos(rp_th * (double)l0, &sn, &c);
    sincos(rp_th, &ss, &sc);
#pragma unroll
    for (int k = 0; k < LPT; k++) {
      ftab[lane * 64 + l0 + k] = float2{(float)c, (float)sn};
      const double c2 = c * sc - sn * ss;
      sn = sn * sc + c * ss;
      c = c2;
    }
    lds_barrier();
  }

  // scaled query (log2 domain) of channels cq..cq+3, and its power-of-two
  // normalisation qn so that |q * qn| < 1 (then |q' * qn| < 65536 / 1.5)
  const float qs = a.scale * kLog2e;
  float sq[R][4];
  float qabs = 0.f;
#pragma unroll
  for (int h = 0; h < R; h++) {
    const uint2 q4 = q4r[h];
    sq[h][0] = qs * h2f((uint16_t)(q4.x & 0xFFFFu));
    sq[h][1] = qs * h2f((uint16_t)(q4.x >> 16));
    sq[h][2] = qs * h2f((uint16_t)(q4.y & 0xFFFFu));
    sq[h][3] = qs * h2f((uint16_t)(q4.y >> 16));
#pragma unroll
    for (int e = 0; e < 4; e++) qabs = fmaxf(qabs, fabsf(sq[h][e]));
  }
  qabs = wave_max(qabs);
  int qe = (int)((__builtin_bit_cast(uint32_t, qabs) >> 23) & 0xFF) - 126;  // qabs < 2^qe
  qe = qe < -100 ? -100 : (qe > 100 ? 100 : qe);
  const float qn = __builtin_bit_cast(float, (uint32_t)(127 - qe) << 23);
  const float qup = __builtin_bit_cast(float, (uint32_t)(127 + qe) << 23);
  float sqn[R][4];
#pragma unroll
  for (int h = 0; h < R; h++)
#pragma unroll
    for (int e = 0; e < 4; e++) sqn[h][e] = sq[h][e] * qn;

  // pre-RoPE: lane = pair (lane, lane + 64).  The query pair as a complex
  // number (scaled to the log2 domain); each tile rotates it back by its
  // first position T (one binary64 sincos per lane and tile, so the tiles
  // can come in any order).
  float qre[R], qim[R];
  if constexpr (ROPE) {
    const uint16_t* qp = a.q + qrow0 * kD;
#pragma unroll
    for (int h = 0; h < R; h++) {
      qre[h] = qs * h2f(qp[h * kD + lane]);
      qim[h] = qs * h2f(qp[h * kD + lane + 64]);
    }
  }
  float* rp_sz = reinterpret_cast<float*>(RW_BYTES ? rope_wave : lds_a);   // [g][pair][4]
  float2* rp_q = reinterpret_cast<float2*>(lds_res);                          // [pair][R]
  // writes the query rotated back by angle theta_pair * T (cos, sin given)
  auto rope_query = [&](float c, float sn) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < R; h++)
      rp_q[lane * R + h] = float2{qre[h] * c + qim[h] * sn, qim[h] * c - qre[h] * sn};
  };

  float m_run[R], l_acc[R], l_res[R];
  float gam[R][kNG];
  float ores[R][8];
#pragma unroll
  for (int h = 0; h < R; h++) {
    m_run[h] = -INFINITY;
    l_acc[h] = l_res[h] = 0.f;
#pragma unroll
    for (int j = 0; j < kNG; j++) gam[h][j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) ores[h][e] = 0.f;
  }
  // P.V partial outputs of the rows this lane holds (heads 2kg, 2kg+1): each
  // tile's products are summed (hi + lo rows) into these, so the product
  // accumulators are free between tiles (one head: 8 registers, not 32)
  constexpr int OH = R >= 2 ? 2 : 1;
  float oacc[8][OH];
#pragma unroll
  for (int nb = 0; nb < 8; nb++)
#pragma unroll
    for (int e = 0; e < OH; e++) oacc[nb][e] = 0.f;

  // score slot of head 2*kg + hh for token index k (absent heads go to a sink)
  auto sc_addr = [&](int hh, int k) __attribute__((always_inline)) -> float* {
    const int h = 2 * kg + hh;
    return h < R ? lds_sc + h * CH + k : lds_dummy + n16;
  };

  // new running maximum of each head -> rescale every running quantity (the
  // residual's value sums only while the residual is processed: afterwards
  // they wait in LDS and are rescaled once at the end)
  auto apply_max = [&](const float (&mxs)[R], bool in_res) __attribute__((always_inline)) {
    float alpha[R];
    bool any = false;
#pragma unroll
    for (int h = 0; h < R; h++) {
      // lazy reference: move it only when a score exceeds it by more than
      // 2^kLazy (p stays <= 2^kLazy; fine for the fp32 sums and the bf16 P.V
      // operand); a head without any finite score keeps -inf
      const bool grow = mxs[h] > m_run[h] + kLazy;
      const float m_new = grow ? mxs[h] : m_run[h];
      alpha[h] = grow ? fast_exp2(m_run[h] - m_new) : 1.f;
      any |= grow;
      m_run[h] = m_new;
    }
    if (any) {
#pragma unroll
      for (int h = 0; h < R; h++) {
        l_acc[h] *= alpha[h];
#pragma unroll
        for (int j = 0; j < kNG; j++) gam[h][j] *= alpha[h];
        if (in_res) {
          l_res[h] *= alpha[h];
#pragma unroll
          for (int e = 0; e < 8; e++) ores[h][e] *= alpha[h];
        }
      }
      const float a0 = pick<R>(alpha, kg, 0), a1 = pick<R>(alpha, kg, 1);
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        oacc[nb][0] *= a0;
        if constexpr (OH == 2) oacc[nb][OH - 1] *= a1;
      }
    }
  };
  // maximum over the ntok scores in LDS (residual batches)
  auto rescale = [&](int ntok) __attribute__((always_inline)) {
    float mxs[R];
#pragma unroll
    for (int h = 0; h < R; h++) mxs[h] = wave_max(lane < ntok ? lds_sc[h * CH + lane] : -INFINITY);
    apply_max(mxs, true);
  };

  // one tile (codes already staged in LDS): key scores -> LDS, online-softmax
  // rescale, P.V
  auto do_tile = [&](int tile, MetaT ksm, MetaT kzm, MetaT vsm, MetaT vzm, const uint4& o0,
                     const uint4& o1) __attribute__((always_inline)) {
    const float4 ks4 = meta4(ksm), kz4 = meta4(kzm), vs4 = meta4(vsm), vz4 = meta4(vzm);
    const bool half_tile = tile * 64 + 64 > tq;   // only the first 32 tokens exist
    // key factors (both groups at once: lanes 0-31 group 0, 32-63 group 1)
    const float ksv[4] = {ks4.x, ks4.y, ks4.z, ks4.w};
    const float kzv[4] = {kz4.x, kz4.y, kz4.z, kz4.w};
    if constexpr (!ROPE) {
    float beta0[R], beta1[R];
#pragma unroll
    for (int h = 0; h < R; h++) {
#pragma unroll
      for (int e = 0; e < 2; e++) {
        uint32_t hi, lo;
        split2(sqn[h][e] * ksv[e], sqn[h][e + 2] * ksv[e + 2], hi, lo);
        *reinterpret_cast<uint32_t*>(lds_a + kwr[e] + (2 * h) * 64) = hi;
        *reinterpret_cast<uint32_t*>(lds_a + kwr[e] + (2 * h + 1) * 64) = lo;
      }
      if constexpr (!BMF) {
        // (on the normalised query, scaled back by qup: a power of two)
        float bp = sqn[h][0] * kzv[0] + sqn[h][1] * kzv[1] + sqn[h][2] * kzv[2] + sqn[h][3] * kzv[3];
        bp += dpp<0x128>(bp);
        bp += dpp<0x124>(bp);
        bp += dpp<0x122>(bp);
        bp += dpp<0x121>(bp);
        beta0[h] = (lane_read(bp, 0) + lane_read(bp, 16)) * qup;
        beta1[h] = (lane_read(bp, 32) + lane_read(bp, 48)) * qup;
      }
    }
    if constexpr (BMF) {
      // this lane's four key zeros as binary16: exact, a zero is the minimum
      // of binary16 inputs (the group's, or of its dense rest)
      const hrtz2 z01 = __builtin_amdgcn_cvt_pkrtz(kzv[0], kzv[1]);
      const hrtz2 z23 = __builtin_amdgcn_cvt_pkrtz(kzv[2], kzv[3]);
      *reinterpret_cast<uint2*>(kz_own + (kgrp * kD + cq) * 2) =
          uint2{__builtin_bit_cast(uint32_t, z01), __builtin_bit_cast(uint32_t, z23)};
    }
    if (half_tile && lane < 32) {
#pragma unroll
      for (int h = 0; h < R; h++) lds_sc[h * CH + 32 + lane] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    const int ngr = half_tile ? 1 : 2;
    // per-lane maxima of the scores this lane produces (heads 2kg, 2kg+1)
    float mx0 = -INFINITY, mx1 = -INFINITY;
    // the key product of 16-token block mb (A tile af of its key group)
    auto key_block = [&](int mb, const half8 (&af)[4]) __attribute__((always_inline)) {
          float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
          const char* krow = stg + (16 * mb + n16) * W * 4;   // token 16mb + n16
          if constexpr (BITS == 1 || BITS == 3) {
            // one-bit plane: word kg, nibble bit-planes m = 0..3 (scale 2 for
            // 1-bit codes; for 3-bit codes the high bit, scale 8 = 4 * hi)
            const uint32_t x = *reinterpret_cast<const uint32_t*>(
                krow + (BITS == 3 ? 32 : 0) + kg * 4);
            const float sc = BITS == 3 ? 8.0f : 2.0f;
            acc = mfma(af[0], cvt_nib2(x & 0x11111111u, sc), acc);
            acc = mfma(af[1], cvt_nib2((x >> 1) & 0x11111111u, sc), acc);
            acc = mfma(af[2], cvt_nib2((x >> 2) & 0x11111111u, sc), acc);
            acc = mfma(af[3], cvt_nib2((x >> 3) & 0x11111111u, sc), acc);
          }
          if constexpr (BITS == 2 || BITS == 3) {
            // two-bit plane: words 2kg, 2kg + 1
            const uint2 x = *reinterpret_cast<const uint2*>(krow + kg * 8);
            acc = mfma(af[0], cvt_nib2(x.x & 0x33333333u), acc);
            acc = mfma(af[1], cvt_nib2((x.x >> 2) & 0x33333333u), acc);
            acc = mfma(af[2], cvt_nib2(x.y & 0x33333333u), acc);
            acc = mfma(af[3], cvt_nib2((x.y >> 2) & 0x33333333u), acc);
          }
          if constexpr (BITS == 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(stg + (16 * mb + n16) * W * 4 + kg * 16);
            acc = mfma(af[0], cvt_word4(x.x), acc);
            acc = mfma(af[1], cvt_word4(x.y), acc);
            acc = mfma(af[2], cvt_word4(x.z), acc);
            acc = mfma(af[3], cvt_word4(x.w), acc);
          }
          return acc;
    };
    // scores of block mb from its accumulators -> LDS, running lane maxima
    auto put_scores = [&](int mb, const float4v& acc, float b0, float b1)
        __attribute__((always_inline)) {
          const int k = 16 * mb + n16;
          const float s0 = (acc[0] + acc[1]) * qup + b0;
          const float s1 = (acc[2] + acc[3]) * qup + b1;
          *sc_addr(0, k) = s0;
          *sc_addr(1, k) = s1;
          mx0 = fmaxf(mx0, s0);
          mx1 = fmaxf(mx1, s1);
    };
    // the matrix-core sections run at raised wave priority: with two waves
    // per SIMD, the wave in its product keeps the matrix cores fed while the
    // other one's vector work fills the gaps (batch-8 Llama layer 27.55 ->
    // 27.32 us)
    __builtin_amdgcn_s_setprio(1);
    // zero terms of the heads in this lane's output rows (2kg, 2kg + 1) for
    // key group g: beta[g][hh]
    float bta[2][2];
    if constexpr (BMF) {
      // A = the scaled query rows (head, hi|lo) of the residual key product,
      // B = the key zeros, column n -> key group n & 1 (only columns 0 and 1
      // are used; a column's products depend on that column alone)
      float4v bacc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const half8 aq = *reinterpret_cast<const half8*>(res_rd + i * ROWS * 64);
        const half8 bz =
            *reinterpret_cast<const half8*>(kz_own + ((n16 & 1) * kD + 32 * i + 8 * kg) * 2);
        bacc = mfma(aq, bz, bacc);
      }
      // rows 2hh, 2hh + 1 of lane row kg are head 2kg + hh (hi, lo); the
      // columns of groups 0 and 1 are broadcast over the row (row_newbcast)
      const float s0 = (bacc[0] + bacc[1]) * qup, s1 = (bacc[2] + bacc[3]) * qup;
      bta[0][0] = dpp<0x150>(s0);
      bta[0][1] = dpp<0x150>(s1);
      bta[1][0] = dpp<0x151>(s0);
      bta[1][1] = dpp<0x151>(s1);
    } else {
#pragma unroll
      for (int g = 0; g < 2; g++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) bta[g][hh] = pick<R>(g ? beta1 : beta0, kg, hh);
    }
    if constexpr (SHA) {
      // rows (group g, hi|lo): block mb of group g takes rows 2g, 2g + 1
      half8 af[4];
#pragma unroll
      for (int m = 0; m < 4; m++)
        af[m] = *reinterpret_cast<const half8*>(a_rdk + m * KROWS * 64);
#pragma unroll
      for (int g = 0; g < 2; g++) {
        if (g < ngr) {
#pragma unroll
          for (int mb2 = 0; mb2 < 2; mb2++) {
            const int mb = 2 * g + mb2, k = 16 * mb + n16;
            const float4v acc = key_block(mb, af);
            const float s0 = (acc[2 * g] + acc[2 * g + 1]) * qup + (g ? beta1[0] : beta0[0]);
            *sc_addr(0, k) = s0;
            mx0 = fmaxf(mx0, s0);
          }
        }
      }
    } else if constexpr (KO == 0) {
#pragma unroll
      for (int g = 0; g < 2; g++) {
        if (g < ngr) {
          half8 af[4];
#pragma unroll
          for (int m = 0; m < 4; m++)
            af[m] = *reinterpret_cast<const half8*>(a_rd + g * (4 * ROWS * 64) + m * ROWS * 64);
#pragma unroll
          for (int mb2 = 0; mb2 < 2; mb2++)
            put_scores(2 * g + mb2, key_block(2 * g + mb2, af), bta[g][0], bta[g][1]);
        }
      }
    } else {
      // dense key products of all four blocks first, accumulators kept
      float4v accs[4];
#pragma unroll
      for (int g = 0; g < 2; g++) {
        if (g < ngr) {
          half8 af[4];
#pragma unroll
          for (int m = 0; m < 4; m++)
            af[m] = *reinterpret_cast<const half8*>(a_rd + g * (4 * ROWS * 64) + m * ROWS * 64);
#pragma unroll
          for (int mb2 = 0; mb2 < 2; mb2++) accs[2 * g + mb2] = key_block(2 * g + mb2, af);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // outlier slots: (a) A' = q * (kept value - zero) / 4 in the 2-bit
      // operand order, over the key-A region the dense product has read;
      // (b) the slot's positions as 0/1 codes in 2-bit key rows (a lane owns
      // byte cq/4 of each row: its 4 channels); (c) accs += A' x plane, the
      // plane converted with scale 8 so that a set code reads as 4
      char* mrow = MK_BYTES ? mask_own : stg;
      const uint32_t ow[2][4] = {{o0.x, o0.y, o0.z, o0.w}, {o1.x, o1.y, o1.z, o1.w}};
#pragma unroll
      for (int j = 0; j < KO; j++) {
        float dv[4];
        uint32_t pos[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          dv[e] = 0.25f * (h2f((uint16_t)(ow[j][e] & 0xFFFFu)) - kzv[e]);
          pos[e] = (ow[j][e] >> 16) & 31u;
        }
#pragma unroll
        for (int h = 0; h < R; h++)
#pragma unroll
          for (int e = 0; e < 2; e++) {
            uint32_t hi, lo;
            split2(sqn[h][e] * dv[e], sqn[h][e + 2] * dv[e + 2], hi, lo);
            *reinterpret_cast<uint32_t*>(lds_a + kwr2[e] + (2 * h) * 64) = hi;
            *reinterpret_cast<uint32_t*>(lds_a + kwr2[e] + (2 * h + 1) * 64) = lo;
          }
        reinterpret_cast<uint4*>(mrow + lane * 32)[0] = uint4{0, 0, 0, 0};
        reinterpret_cast<uint4*>(mrow + lane * 32)[1] = uint4{0, 0, 0, 0};
        __builtin_amdgcn_wave_barrier();
        if (!half_tile || kgrp == 0) {
#pragma unroll
          for (int e = 0; e < 4; e++) {
            uint32_t byte = 0;
#pragma unroll
            for (int e2 = 0; e2 < 4; e2++) byte |= (pos[e2] == pos[e] ? 1u : 0u) << (2 * e2);
            mrow[(32 * kgrp + pos[e]) * 32 + cq / 4] = (char)byte;
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int g = 0; g < 2; g++) {
          if (g < ngr) {
            half8 af[4];
#pragma unroll
            for (int m = 0; m < 4; m++)
              af[m] = *reinterpret_cast<const half8*>(a_rd + g * (4 * ROWS * 64) + m * ROWS * 64);
#pragma unroll
            for (int mb2 = 0; mb2 < 2; mb2++) {
              const int mb = 2 * g + mb2;
              const uint2 x = *reinterpret_cast<const uint2*>(mrow + (16 * mb + n16) * 32 + kg * 8);
              accs[mb] = mfma(af[0], cvt_nib2(x.x & 0x33333333u, 8.0f), accs[mb]);
              accs[mb] = mfma(af[1], cvt_nib2((x.x >> 2) & 0x33333333u, 8.0f), accs[mb]);
              accs[mb] = mfma(af[2], cvt_nib2(x.y & 0x33333333u, 8.0f), accs[mb]);
              accs[mb] = mfma(af[3], cvt_nib2((x.y >> 2) & 0x33333333u, 8.0f), accs[mb]);
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
#pragma unroll
      for (int g = 0; g < 2; g++) {
        if (g < ngr) {
#pragma unroll
          for (int mb2 = 0; mb2 < 2; mb2++) put_scores(2 * g + mb2, accs[2 * g + mb2], bta[g][0], bta[g][1]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_wave_barrier();
    // tile maximum per head straight from the MFMA output: reduce over the 16
    // token lanes of each row (heads 2kg, 2kg+1 live in lane row kg)
    {
      mx0 = fmaxf(mx0, dpp<0x128>(mx0));
      mx0 = fmaxf(mx0, dpp<0x124>(mx0));
      mx0 = fmaxf(mx0, dpp<0x122>(mx0));
      mx0 = fmaxf(mx0, dpp<0x121>(mx0));
      if constexpr (R >= 2) {
        mx1 = fmaxf(mx1, dpp<0x128>(mx1));
        mx1 = fmaxf(mx1, dpp<0x124>(mx1));
        mx1 = fmaxf(mx1, dpp<0x122>(mx1));
        mx1 = fmaxf(mx1, dpp<0x121>(mx1));
      }
      float mxs[R];
#pragma unroll
      for (int h = 0; h < R; h++) mxs[h] = lane_read((h & 1) ? mx1 : mx0, 16 * (h >> 1));
      apply_max(mxs, false);
    }
    } else {
      // pre-RoPE keys.  (1) this lane's 4 channels' scale / zero, stored per
      // pair as (s_lo, z_lo, s_hi, z_hi); (2) the query rotated back by the
      // tile's first position (lane = pair); (3) lane = token: dequantize,
      // rotate by the in-tile angle, dot with every head.
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int d = cq + e;
        *reinterpret_cast<float2*>(rp_sz + (kgrp * 64 + (d & 63)) * 4 + 2 * (d >> 6)) =
            float2{ksv[e], kzv[e]};
      }
      // one head: the query rotated back by the tile's position, P = (pr, pim),
      // stays in this lane (= pair); several heads share the rotated key
      float pr = 0.f, pim = 0.f;
      {
        double tsn, tc;
        sincos(rp_th * (64.0 * (double)tile), &tsn, &tc);
        const float c = (float)tc, sn = (float)tsn;
        if constexpr (R == 1) {
          pr = qre[0] * c + qim[0] * sn;
          pim = qim[0] * c - qre[0] * sn;
        } else {
          rope_query(c, sn);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // One head, folded form: with k0 = c0 s0 + z0, k1 = c1 s1 + z1 and the
      // in-tile angle (cos, sin), the pair adds cos * X + sin * Y where
      //   X = P_r k0 + P_i k1 = c0 (P_r s0) + c1 (P_i s1) + (P_r z0 + P_i z1)
      //   Y = P_i k0 - P_r k1 = c0 (P_i s0) - c1 (P_r s1) + (P_i z0 - P_r z1),
      // i.e. 6 FMAs per pair and token instead of 8.  Lane = pair computes the
      // six coefficients of both key groups; the four code factors replace its
      // (s, z) entries in place, the two constants go to their own 1 KB.
      float4* rp_co = reinterpret_cast<float4*>(rp_sz);                   // [g][pair]
      float2* rp_ce = reinterpret_cast<float2*>(rope_wave + 2048);        // [g][pair]
      if constexpr (R == 1) {
#pragma unroll
        for (int g = 0; g < 2; g++) {
          const float4 sz = rp_co[g * 64 + lane];   // (s0, z0, s1, z1) of pair `lane`
          rp_co[g * 64 + lane] = float4{pr * sz.x, pim * sz.z, pim * sz.x, -(pr * sz.z)};
          rp_ce[g * 64 + lane] = float2{pr * sz.y + pim * sz.w, pim * sz.y - pr * sz.w};
        }
        __builtin_amdgcn_wave_barrier();
      }
      uint32_t wd[W];
#pragma unroll
      for (int i = 0; i < W / 4; i++) {
        const uint4 x = *reinterpret_cast<const uint4*>(stg + lane * W * 4 + 16 * i);
        wd[4 * i] = x.x;
        wd[4 * i + 1] = x.y;
        wd[4 * i + 2] = x.z;
        wd[4 * i + 3] = x.w;
      }
      const float* szg = rp_sz + (lane >> 5) * 64 * 4;
      float acc[R];
#pragma unroll
      for (int h = 0; h < R; h++) acc[h] = 0.f;
      // pair i with the codes of channels i and i + 64
      auto pair = [&](int i, float c0, float c1) __attribute__((always_inline)) {
        if constexpr (R == 1) {
          const float4 co = rp_co[(lane >> 5) * 64 + i];
          const float2 ce = rp_ce[(lane >> 5) * 64 + i];
          const float X = fmaf(c0, co.x, fmaf(c1, co.y, ce.x));
          const float Y = fmaf(c0, co.z, fmaf(c1, co.w, ce.y));
          const float2 f = ftab[i * 64 + lane];
          acc[0] = fmaf(f.x, X, fmaf(f.y, Y, acc[0]));
          return;
        }
        const float4 sz = *reinterpret_cast<const float4*>(szg + 4 * i);
        const float k0 = fmaf(c0, sz.x, sz.y);
        const float k1 = fmaf(c1, sz.z, sz.w);
        const float2 f = ftab[i * 64 + lane];
        const float kr = f.x * k0 - f.y * k1, ki = f.y * k0 + f.x * k1;
#pragma unroll
        for (int h = 0; h < R; h++) {
          const float2 pq = rp_q[i * R + h];
          acc[h] = fmaf(pq.x, kr, fmaf(pq.y, ki, acc[h]));
        }
      };
      // one head, 2-bit codes: the coefficients and table entries of pair
      // i + 8 are read while pair i is computed (an 8-deep ring), so that
      // the compiler does not wait for each LDS read right before its use
      float4 pf_co[8];
      float2 pf_ce[8], pf_f[8];
      if constexpr (R == 1 && BITS == 2) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          pf_co[i] = rp_co[(lane >> 5) * 64 + i];
          pf_ce[i] = rp_ce[(lane >> 5) * 64 + i];
          pf_f[i] = ftab[i * 64 + lane];
        }
      }
      if constexpr (BITS == 2) {
        // a word holds 16 channels: its two nibble planes through the e2m1
        // convert (scale 2) give the codes as floats, two per instruction
        // (byte b of plane m -> positions 4b + m, 4b + 2 + m)
#pragma unroll
        for (int k = 0; k < 4; k++) {
          float lo[16], hi[16];
          const uint32_t wl[2] = {wd[k], wd[4 + k]};
#pragma unroll
          for (int x = 0; x < 2; x++) {
            float* o = x ? hi : lo;
#pragma unroll
            for (int m = 0; m < 2; m++) {
              const uint32_t pl = (wl[x] >> (2 * m)) & 0x33333333u;
              const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pl, 2.0f, 0);
              const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pl, 2.0f, 1);
              const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pl, 2.0f, 2);
              const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pl, 2.0f, 3);
              o[m] = v0[0];
              o[2 + m] = v0[1];
              o[4 + m] = v1[0];
              o[6 + m] = v1[1];
              o[8 + m] = v2[0];
              o[10 + m] = v2[1];
              o[12 + m] = v3[0];
              o[14 + m] = v3[1];
            }
          }
          if constexpr (R == 1) {
#pragma unroll
            for (int u = 0; u < 16; u++) {
              const int i = 16 * k + u;
              const float4 co = pf_co[i & 7];
              const float2 ce = pf_ce[i & 7];
              const float2 f = pf_f[i & 7];
              if (i + 8 < 64) {
                pf_co[i & 7] = rp_co[(lane >> 5) * 64 + i + 8];
                pf_ce[i & 7] = rp_ce[(lane >> 5) * 64 + i + 8];
                pf_f[i & 7] = ftab[(i + 8) * 64 + lane];
              }
              const float X = fmaf(lo[u], co.x, fmaf(hi[u], co.y, ce.x));
              const float Y = fmaf(lo[u], co.z, fmaf(hi[u], co.w, ce.y));
              acc[0] = fmaf(f.x, X, fmaf(f.y, Y, acc[0]));
            }
          } else {
#pragma unroll
          for (int u = 0; u < 16; u++) pair(16 * k + u, lo[u], hi[u]);
          }
        }
      } else if constexpr (BITS == 4) {
        // a word holds 8 channels: low and high nibbles as e4m3 bytes (scale
        // 2^9 gives the code) -> positions 0,2 | 4,6 and 1,3 | 5,7
#pragma unroll
        for (int k = 0; k < 8; k++) {
          float lo[8], hi[8];
          const uint32_t wl[2] = {wd[k], wd[8 + k]};
#pragma unroll
          for (int x = 0; x < 2; x++) {
            float* o = x ? hi : lo;
#pragma unroll
            for (int m = 0; m < 2; m++) {
              const uint32_t pl = (wl[x] >> (4 * m)) & 0x0F0F0F0Fu;
              const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pl, 512.0f, false);
              const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pl, 512.0f, true);
              o[m] = v0[0];
              o[2 + m] = v0[1];
              o[4 + m] = v1[0];
              o[6 + m] = v1[1];
            }
          }
#pragma unroll
          for (int u = 0; u < 8; u++) pair(8 * k + u, lo[u], hi[u]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 64; i++) pair(i, key_code<BITS>(wd, i), key_code<BITS>(wd, i + 64));
      }
      const bool tok_ok = tile * 64 + lane < tq;
      float mxs[R];
#pragma unroll
      for (int h = 0; h < R; h++) {
        const float sc = tok_ok ? acc[h] : -INFINITY;
        lds_sc[h * CH + lane] = sc;
        mxs[h] = wave_max(sc);
      }
      apply_max(mxs, false);
      __builtin_amdgcn_wave_barrier();
    }
    // P.V: value factors of token lane, 4 groups, hi/lo halves to LDS
    const bool valid = tile * 64 + lane < tq;
    // (absent tokens of a half tile: p = 0 and factors 0, so every product of
    // theirs is 0 whatever their unwritten scale / zero held; several heads
    // mask the factors once, one head each product, which compiles shorter)
    constexpr bool VM1 = R >= 2;
    const float vsv[4] = {VM1 && !valid ? 0.f : vs4.x, VM1 && !valid ? 0.f : vs4.y,
                          VM1 && !valid ? 0.f : vs4.z, VM1 && !valid ? 0.f : vs4.w};
    const float vzv[4] = {valid ? vz4.x : 0.f, valid ? vz4.y : 0.f, valid ? vz4.z : 0.f,
                          valid ? vz4.w : 0.f};
#pragma unroll
    for (int h = 0; h < R; h++) {
      const float p = valid ? fast_exp2(lds_sc[h * CH + lane] - m_run[h]) : 0.f;
      l_acc[h] += p;
#pragma unroll
      for (int j = 0; j < kNG; j++) gam[h][j] += p * vzv[j];
      // hi/lo halves of p * s for the group pairs (0,1), (2,3), two at a time
#pragma unroll
      for (int jj = 0; jj < kNG; jj += 2) {
        uint32_t hi, lo;
        split2_bf(VM1 || valid ? p * vsv[jj] : 0.f, VM1 || valid ? p * vsv[jj + 1] : 0.f, hi, lo);
        if constexpr (SHA) {
          // rows 2j (hi), 2j + 1 (lo) of group j
          char* d = lds_a + vwr + (uint32_t)(2 * jj * 64);
          *reinterpret_cast<uint16_t*>(d) = (uint16_t)hi;
          *reinterpret_cast<uint16_t*>(d + 64) = (uint16_t)lo;
          *reinterpret_cast<uint16_t*>(d + 128) = (uint16_t)(hi >> 16);
          *reinterpret_cast<uint16_t*>(d + 192) = (uint16_t)(lo >> 16);
          continue;
        }
        char* d0 = lds_a + vwr + (uint32_t)(jj * 2 * ROWS * 64);
        char* d1 = d0 + 2 * ROWS * 64;
        *reinterpret_cast<uint16_t*>(d0 + (2 * h) * 64) = (uint16_t)hi;
        *reinterpret_cast<uint16_t*>(d1 + (2 * h) * 64) = (uint16_t)(hi >> 16);
        *reinterpret_cast<uint16_t*>(d0 + (2 * h + 1) * 64) = (uint16_t)lo;
        *reinterpret_cast<uint16_t*>(d1 + (2 * h + 1) * 64) = (uint16_t)(lo >> 16);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const char* vstg = stg + C::KC_BYTES;
    bf16x8 sav0, sav1;   // the shared value A operand (both token halves)
    if constexpr (!ROPE) __builtin_amdgcn_s_setprio(1);
    if constexpr (SHA) {
      sav0 = *reinterpret_cast<const bf16x8*>(a_rdv);
      sav1 = *reinterpret_cast<const bf16x8*>(a_rdv + VROWS * 64);
    }
#pragma unroll
    for (int j = 0; j < kNG; j++) {
      const bf16x8 av0 =
          SHA ? sav0 : *reinterpret_cast<const bf16x8*>(a_rd + (j * 2 + 0) * ROWS * 64);
      const bf16x8 av1 =
          SHA ? sav1 : *reinterpret_cast<const bf16x8*>(a_rd + (j * 2 + 1) * ROWS * 64);
#pragma unroll
      for (int nbj = 0; nbj < 2; nbj++) {
        const int nb = 2 * j + nbj;
        float4v cvn = float4v{0.f, 0.f, 0.f, 0.f};   // this block's products
        const char* vrow = vstg + (16 * nb + n16) * WPC * 4;   // channel 16nb + n16
        if constexpr (BITS == 1 || BITS == 3) {
          // one-bit plane: word kg/2 holds this lane group's 16 tokens in
          // nibble bit-planes 2*(kg%2) (even tokens) and 2*(kg%2) + 1 (odd)
          const uint32_t x = *reinterpret_cast<const uint32_t*>(
              vrow + (BITS == 3 ? 16 : 0) + (kg >> 1) * 4);
          const float sc = BITS == 3 ? 8.0f : 2.0f;
          const uint32_t xs = x >> (2 * (kg & 1));
          cvn = mfma_bf(av0, cvt_nib2_bf(xs & 0x11111111u, sc), cvn);
          cvn = mfma_bf(av1, cvt_nib2_bf((xs >> 1) & 0x11111111u, sc), cvn);
        }
        if constexpr (BITS == 2 || BITS == 3) {
          // two-bit plane: word kg
          const uint32_t x = *reinterpret_cast<const uint32_t*>(vrow + kg * 4);
          cvn = mfma_bf(av0, cvt_nib2_bf(x & 0x33333333u), cvn);
          cvn = mfma_bf(av1, cvt_nib2_bf((x >> 2) & 0x33333333u), cvn);
        }
        if constexpr (BITS == 4) {
          const uint2 x = *reinterpret_cast<const uint2*>(vstg + (16 * nb + n16) * WPC * 4 + kg * 8);
          cvn = mfma_bf(av0, cvt_word4_bf(x.x), cvn);
          cvn = mfma_bf(av1, cvt_word4_bf(x.y), cvn);
        }
        if constexpr (SHA) {
          // group j's rows 2j, 2j + 1 sit in lane row j / 2
          oacc[nb][0] += cvn[2 * (j & 1)] + cvn[2 * (j & 1) + 1];
        } else {
          oacc[nb][0] += cvn[0] + cvn[1];
          if constexpr (OH == 2) oacc[nb][OH - 1] += cvn[2] + cvn[3];
        }
      }
    }
    if constexpr (!ROPE) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_wave_barrier();
  };

  // ---------------- residual slice (full precision), overlapping the tile loads
  // one batch of 16 tokens from rk*/rv*: scores by MFMA, values on the VALU
  half8 ar[4];
  auto res_batch = [&](int t16) __attribute__((always_inline)) {
    const int n = min(16, r_end - t16);
    if constexpr (ROPE) {
      // the query rotated back by the batch's first position tq + t16 (one
      // binary64 sincos per pair), then lane (token n16, quarter kg) takes
      // its 16 pairs (channels 32 m + 8 kg + s and + 64, m = 0, 1) from the
      // fp16 rows it holds, rotates them by the in-batch angle and reduces
      // over the four quarters
      {
        double sn, c;
        sincos(rp_th * (double)(tq + t16), &sn, &c);
        rope_query((float)c, (float)sn);
      }
      __builtin_amdgcn_wave_barrier();
      float part[R];
#pragma unroll
      for (int h = 0; h < R; h++) part[h] = 0.f;
      const u32x4 klo[2] = {rk0, rk1}, khi[2] = {rk2, rk3};
#pragma unroll
      for (int m = 0; m < 2; m++)
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const int i = 32 * m + 8 * kg + s;
          const uint32_t wl = klo[m][s >> 1], wh = khi[m][s >> 1];
          const float k0 = h2f((uint16_t)((s & 1) ? (wl >> 16) : (wl & 0xFFFFu)));
          const float k1 = h2f((uint16_t)((s & 1) ? (wh >> 16) : (wh & 0xFFFFu)));
          const float2 f = ftab[i * 64 + n16];
          const float kr = f.x * k0 - f.y * k1, ki = f.y * k0 + f.x * k1;
#pragma unroll
          for (int h = 0; h < R; h++) {
            const float2 pq = rp_q[i * R + h];
            part[h] = fmaf(pq.x, kr, fmaf(pq.y, ki, part[h]));
          }
        }
#pragma unroll
      for (int h = 0; h < R; h++) {
        part[h] += __shfl_xor(part[h], 16);
        part[h] += __shfl_xor(part[h], 32);
      }
      if (kg == 0 && n16 < n) {
#pragma unroll
        for (int h = 0; h < R; h++) lds_sc[h * CH + n16] = part[h];
      }
    } else {
    float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
    acc = mfma(ar[0], __builtin_bit_cast(half8, rk0), acc);
    acc = mfma(ar[1], __builtin_bit_cast(half8, rk1), acc);
    acc = mfma(ar[2], __builtin_bit_cast(half8, rk2), acc);
    acc = mfma(ar[3], __builtin_bit_cast(half8, rk3), acc);
    {
      const bool ok = n16 < n;
      float* p0 = ok ? sc_addr(0, n16) : lds_dummy + n16;
      float* p1 = ok ? sc_addr(1, n16) : lds_dummy + n16;
      *p0 = (acc[0] + acc[1]) * qup;
      *p1 = (acc[2] + acc[3]) * qup;
    }
    }
    __builtin_amdgcn_wave_barrier();
    rescale(n);
    const u32x4 vv[4] = {rv0, rv1, rv2, rv3};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int ti = tg + 4 * i;
      const bool ok = ti < n;
      const uint32_t w4[4] = {vv[i][0], vv[i][1], vv[i][2], vv[i][3]};
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        v[2 * e] = h2f((uint16_t)(w4[e] & 0xFFFFu));
        v[2 * e + 1] = h2f((uint16_t)(w4[e] >> 16));
      }
#pragma unroll
      for (int h = 0; h < R; h++) {
        const float p = ok ? fast_exp2(lds_sc[h * CH + (ok ? ti : 0)] - m_run[h]) : 0.f;
        if (c8 == 0) l_res[h] += p;     // each token counted once
#pragma unroll
        for (int e = 0; e < 8; e++) ores[h][e] += p * v[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // The first batch runs in every wave (an empty slice weighs zero), so that
  // its loads stay ahead of the tile loads instead of sinking into a branch.
  // Residual key A: row (h, hi|lo), MFMA i, lane group kgr, slot s <->
  // channel 32 i + 8 kgr + s.  Lanes 0-31 write channel pairs (cq, cq+1),
  // (cq+2, cq+3) from the scaled query already in registers.
  if (!ROPE && lane < 32) {
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int ch = cq + 2 * e;
      const uint32_t off =
          (uint32_t)((((ch >> 5) * ROWS) * 4 + ((ch & 31) >> 3)) * 16 + 2 * (ch & 7));
#pragma unroll
      for (int h = 0; h < R; h++) {
        uint32_t hi, lo;
        split2(sqn[h][2 * e], sqn[h][2 * e + 1], hi, lo);
        *reinterpret_cast<uint32_t*>(lds_res + off + (2 * h) * 64) = hi;
        *reinterpret_cast<uint32_t*>(lds_res + off + (2 * h + 1) * 64) = lo;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; i++) ar[i] = *reinterpret_cast<const half8*>(res_rd + i * ROWS * 64);
  // fused append: the lanes holding the new token store it into its residual
  // slot (one wave of one split per plane; no load in this launch reads the
  // slot, the token itself came from its input row)
  auto write_new = [&](int t16) __attribute__((always_inline)) {
    const int dn = t_new - t16;
    if (dn < 0 || dn >= 16) return;           // uniform: this batch lacks it
    const uint32_t row = (uint32_t)t_new * kD * 2;
    if (n16 == dn) {
      const uint32_t o = row + kg * 16;
      st16(r_kr, o, rk0);
      st16(r_kr, o + 64, rk1);
      st16(r_kr, o + 128, rk2);
      st16(r_kr, o + 192, rk3);
    }
    if (tg == (dn & 3)) {
      // i = dn / 4 is uniform: plain branches (a value select here would
      // become a pointer select over the captured registers)
      const uint32_t o = row + c8 * 16;
      const int i = dn >> 2;
      if (i == 0) st16(r_vr, o, rv0);
      else if (i == 1) st16(r_vr, o, rv1);
      else if (i == 2) st16(r_vr, o, rv2);
      else st16(r_vr, o, rv3);
    }
  };
  res_batch(r_begin);
  if (fused) write_new(r_begin);
  // slices longer than one batch (short contexts, few splits) load the rest here
  for (int t16 = r_begin + 16; t16 < r_end; t16 += 16) {
    load_res(t16);
    res_batch(t16);
    if (fused) write_new(t16);
  }
  // From here on the residual's sums only rescale: reduce them across lanes
  // now, while the first tile's loads are in flight, rather than after the
  // last tile (value partials: over the token groups in lanes c8, c8 + 16,
  // c8 + 32, c8 + 48; the probability sum over the whole wave)
#pragma unroll
  for (int h = 0; h < R; h++) {
    l_res[h] = wave_sum(l_res[h]);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      ores[h][e] += __shfl_xor(ores[h][e], 16);
      ores[h][e] += __shfl_xor(ores[h][e], 32);
    }
  }
  // ... and park them in this wave's output slot until the end, with the
  // running maximum they are referred to (the registers are free for the
  // tile loop): lane (tg, c8) keeps channels 8*c8 + 2*tg, 8*c8 + 2*tg + 1
  {
    const int tg = lane >> 4, c8 = lane & 15;
#pragma unroll
    for (int h = 0; h < R; h++) {
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        if (e == 2 * tg) rs0 = ores[h][e];
        if (e == 2 * tg + 1) rs1 = ores[h][e];
      }
      *reinterpret_cast<float2*>(lds_o + h * kD + 8 * c8 + 2 * tg) = float2{rs0, rs1};
      if (lane == 0) {
        lds_o[R * kD + h] = m_run[h];
        lds_o[R * kD + R + h] = l_res[h];
      }
    }
  }

  // ---------------- quantized tiles, DEPTH tiles of loads in flight
  // the scheduling barriers keep "stage the current tile, issue the loads of
  // the tile DEPTH later, compute the current tile" in that order, so no wait
  // for a later tile lands before the current compute.  Loads of tiles past
  // t_lim read zeros; the only branch in a loop (the second tile of an
  // iteration that has none) holds no load.
  // (cur: the tile in register set a; nxt: the tile loaded after it; the
  // pending replies pa, pb are each issued a tile's compute before they are
  // taken)
  int pa = 0, pb = 0;
  if constexpr (DEPTH == 2) {
    // set a holds cur, set b holds nxt; two replies in flight
    issue(pa);
    issue(pb);
    for (int cur = t_first, nxt = t_given; cur < t_lim;) {
      __builtin_amdgcn_sched_barrier(0);
      stage(a0, a1, a2, a3, a4, a5, a6, a7);
      const int c2 = take(pa);
      load_codes(c2, a0, a1, a2, a3, a4, a5, a6, a7);
      __builtin_amdgcn_sched_barrier(0);
      do_tile(cur, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
      __builtin_amdgcn_sched_barrier(0);
      load_meta(c2, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
      issue(pa);
      __builtin_amdgcn_sched_barrier(0);
      stage(b0, b1, b2, b3, b4, b5, b6, b7);
      const int c3 = take(pb);
      load_codes(c3, b0, b1, b2, b3, b4, b5, b6, b7);
      __builtin_amdgcn_sched_barrier(0);
      if (nxt < t_lim) do_tile(nxt, b_ks, b_kz, b_vs, b_vz, b_o0, b_o1);
      __builtin_amdgcn_sched_barrier(0);
      load_meta(c3, b_ks, b_kz, b_vs, b_vz, b_o0, b_o1);
      issue(pb);
      cur = c2;
      nxt = c3;
    }
  } else if constexpr (early_meta<R, MH, RAG, PG, KO, ROPE>()) {
    // the next tile's metadata is issued before the current tile's compute,
    // in a second register set, instead of after it (binary16 metadata: 26.2
    // -> 25.0 us on the batch-8 Llama layer; binary32: see early_meta)
    issue(pa);
    for (int cur = t_first, nxt = t_given; cur < t_lim;) {
      __builtin_amdgcn_sched_barrier(0);
      stage(a0, a1, a2, a3, a4, a5, a6, a7);
      load_codes(nxt, a0, a1, a2, a3, a4, a5, a6, a7);
      __builtin_amdgcn_sched_barrier(0);
      load_meta(nxt, b_ks, b_kz, b_vs, b_vz, b_o0, b_o1);
      __builtin_amdgcn_sched_barrier(0);
      do_tile(cur, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
      __builtin_amdgcn_sched_barrier(0);
      const int c2 = take(pa);
      issue(pa);
      stage(a0, a1, a2, a3, a4, a5, a6, a7);
      load_codes(c2, a0, a1, a2, a3, a4, a5, a6, a7);
      __builtin_amdgcn_sched_barrier(0);
      load_meta(c2, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
      __builtin_amdgcn_sched_barrier(0);
      if (nxt < t_lim) do_tile(nxt, b_ks, b_kz, b_vs, b_vz, b_o0, b_o1);
      __builtin_amdgcn_sched_barrier(0);
      cur = c2;
      nxt = take(pa);
      issue(pa);
    }
  } else {
    issue(pa);
    for (int cur = t_first, nxt = t_given; cur < t_lim;) {
      __builtin_amdgcn_sched_barrier(0);
      stage(a0, a1, a2, a3, a4, a5, a6, a7);
      load_codes(nxt, a0, a1, a2, a3, a4, a5, a6, a7);
      __builtin_amdgcn_sched_barrier(0);
      do_tile(cur, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
      __builtin_amdgcn_sched_barrier(0);
      load_meta(nxt, a_ks, a_kz, a_vs, a_vz, a_o0, a_o1);
      cur = nxt;
      nxt = take(pa);
      issue(pa);
    }
  }

  // ---------------- wave result -> LDS: o[h][d], m[h], l[h]
  // the residual's parked sums, read before the slot is overwritten, and the
  // factor 2^(m_res - m_run) that brings them to the final reference (the
  // product of the tile loop's rescale factors; 0 for an empty residual)
  float2 rpart[R];
  float rfac[R], lres[R];
  {
    const int tg = lane >> 4, c8 = lane & 15;
#pragma unroll
    for (int h = 0; h < R; h++) {
      rpart[h] = *reinterpret_cast<const float2*>(lds_o + h * kD + 8 * c8 + 2 * tg);
      const float mr = lds_o[R * kD + h];
      lres[h] = lds_o[R * kD + R + h];
      rfac[h] = mr == -INFINITY ? 0.f : fast_exp2(mr - m_run[h]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  {
    const int h0 = 2 * kg, h1 = 2 * kg + 1;
#pragma unroll
    for (int nb = 0; nb < 8; nb++) {
      // (shared value operand: channel 16 nb + n16 of the head is in lane row nb / 4)
      float* o0 = (SHA ? kg == (nb >> 2) : h0 < R) ? lds_o + (SHA ? 0 : h0 * kD) + 16 * nb + n16
                                                    : lds_dummy + n16;
      float* o1 = h1 < R ? lds_o + h1 * kD + 16 * nb + n16 : lds_dummy + n16;
      *o0 = oacc[nb][0];
      *o1 = OH == 2 ? oacc[nb][OH - 1] : 0.f;
    }
  }
  // residual P.V sums: lane (tg, c8) adds channels 8*c8+2*tg, 8*c8+2*tg+1
  // (value group c8/4) together with the Gamma term of that group
  __builtin_amdgcn_wave_barrier();
  {
    const int tg = lane >> 4, c8 = lane & 15, grp = c8 >> 2;
#pragma unroll
    for (int h = 0; h < R; h++) {
      float g[kNG];
#pragma unroll
      for (int j = 0; j < kNG; j++) g[j] = wave_sum(gam[h][j]);
      const float lsum = wave_sum(l_acc[h]) + lres[h] * rfac[h];
      float gj = g[0];
#pragma unroll
      for (int j = 1; j < kNG; j++)
        if (grp == j) gj = g[j];
      float2* op = reinterpret_cast<float2*>(lds_o + h * kD + 8 * c8 + 2 * tg);
      float2 o2 = *op;
      o2.x += gj + rpart[h].x * rfac[h];
      o2.y += gj + rpart[h].y * rfac[h];
      *op = o2;
      if (lane == 0) {
        lds_o[R * kD + h] = m_run[h];
        lds_o[R * kD + R + h] = lsum;
      }
    }
  }
  __syncthreads();

  // ---------------- merge the block's waves
  for (int idx = threadIdx.x; idx < R * kD; idx += NW * 64) {
    const int h = idx / kD, d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float* ow = reinterpret_cast<const float*>(smem + C::ZERO_BYTES + w * C::WAVE_BYTES +
                                                       C::A_BYTES + C::RES_BYTES + C::SC_BYTES);
      M = fmaxf(M, ow[R * kD + h]);
    }
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; w++) {
        const float* ow = reinterpret_cast<const float*>(
            smem + C::ZERO_BYTES + w * C::WAVE_BYTES + C::A_BYTES + C::RES_BYTES + C::SC_BYTES);
        const float f = fast_exp2(ow[R * kD + h] - M);
        O += ow[h * kD + d] * f;
        L += ow[R * kD + R + h] * f;
      }
    }
    const size_t row = qrow0 + h;
    if (a.ws_stride == 1) {
      a.out[row * kD + d] = f2h(O / L);
    } else {
      const size_t rows = (size_t)a.B * H * R, WS = a.ws_stride;
      const size_t slot = (size_t)a.ws_slot0 + split;
      if (d == 0) {
        a.ws[row * WS + slot] = M * kLn2;          // natural-log units for the combine
        a.ws[rows * WS + row * WS + slot] = L;
      }
      a.ws[2 * rows * WS + (row * WS + slot) * kD + d] = O;
    }
  }
}

template <int R>
constexpr int block_waves(int nw) {
  return (R >= 8 || nw < 8) ? 4 : 8;
}

template <int BITS, int R, bool MH, bool RAG, bool PG, int KO, bool ROPE>
hipError_t launch_m(const DecodeArgs& a, const LensT<RAG>& lens, int nw, hipStream_t st) {
  const dim3 grid(a.B * a.H * a.S);
  // (pre-RoPE keys with several heads per KV head run 4-wave blocks at the
  // one-wave register budget: at two waves per SIMD their rotated keys and
  // per-head sums spilled to scratch)
  constexpr bool kSmall = ROPE && R >= 2;
  if constexpr (kSmall) {
    decode_mfma_kernel<BITS, R, 4, MH, RAG, PG, KO, ROPE><<<grid, 4 * 64, 0, st>>>(a, lens);
  } else {
    if (block_waves<R>(nw) == 8)
      decode_mfma_kernel<BITS, R, (R < 8 ? 8 : 4), MH, RAG, PG, KO, ROPE>
          <<<grid, (R < 8 ? 8 : 4) * 64, 0, st>>>(a, lens);
    else
      decode_mfma_kernel<BITS, R, 4, MH, RAG, PG, KO, ROPE><<<grid, 4 * 64, 0, st>>>(a, lens);
  }
  return hipGetLastError();
}
template <int BITS, int R, bool RAG, bool PG, int KO, bool ROPE>
hipError_t launch_r(const DecodeArgs& a, const LensT<RAG>& lens, int nw, hipStream_t st) {
  return a.mh ? launch_m<BITS, R, true, RAG, PG, KO, ROPE>(a, lens, nw, st)
              : launch_m<BITS, R, false, RAG, PG, KO, ROPE>(a, lens, nw, st);
}

template <int BITS, bool RAG, bool PG, int KO, bool ROPE>
hipError_t launch_bits(const DecodeArgs& a, const LensT<RAG>& lens, int nw, hipStream_t st) {
  switch (a.r) {
    case 1: return launch_r<BITS, 1, RAG, PG, KO, ROPE>(a, lens, nw, st);
    case 2: return launch_r<BITS, 2, RAG, PG, KO, ROPE>(a, lens, nw, st);
    case 4: return launch_r<BITS, 4, RAG, PG, KO, ROPE>(a, lens, nw, st);
    default: return launch_r<BITS, 8, RAG, PG, KO, ROPE>(a, lens, nw, st);
  }
}

// every code width of one (lengths, store, outliers, pre-RoPE) family
template <bool RAG, bool PG, int KO, bool ROPE = false>
hipError_t launch_family(const DecodeArgs& a, const LensT<RAG>& lens, int nw, hipStream_t st) {
  switch (a.bits) {
    case 1: return launch_bits<1, RAG, PG, KO, ROPE>(a, lens, nw, st);
    case 2: return launch_bits<2, RAG, PG, KO, ROPE>(a, lens, nw, st);
    case 3: return launch_bits<3, RAG, PG, KO, ROPE>(a, lens, nw, st);
    default: return launch_bits<4, RAG, PG, KO, ROPE>(a, lens, nw, st);
  }
}

}  // namespace
}  // namespace kivi

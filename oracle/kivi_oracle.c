/*
 * kivi_oracle.c -- plain, slow, single-threaded CPU oracle for the KIVI
 * quantized KV cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library: it re-derives everything from the method's
 * description.
 *
 * Sources (web pages about the method):
 *   [KIVI-abs]  "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV
 *               Cache", mlsanity paper page, section "Abstract (arXiv)".
 *   [KIVI-sum]  study.space summary page of the same paper (one summary
 *               paragraph, no headings).
 *   [KIVI-quo]  scholarfeed.org "KIVI" quote page (one-line quotes from other
 *               papers about the method).
 *   [KVQ-abs]   "KVQuant: Towards 10 Million Context Length LLM Inference with
 *               KV Cache Quantization", codewithpapers.app paper page,
 *               abstract (per-vector dense-and-sparse quantization; keys
 *               quantized before the rotary positional embedding).
 *
 * What the pages fix, restated:
 *   - keys are quantized per channel: one group is one channel over a run
 *     of consecutive tokens; values are quantized per token: one group is a
 *     run of consecutive channels of one token [KIVI-abs]; the key groups
 *     span tokens, so tokens are grouped before keys are quantized [KIVI-sum];
 *   - the quantizer is asymmetric, low-bit (2-bit; 4-bit and 1-bit are also
 *     named) and tuning-free, i.e. uses no calibration [KIVI-abs title,
 *     KIVI-quo];
 *   - the cache is split into a quantized "grouped" part and a
 *     full-precision "residual" part of recent tokens; new tokens are
 *     appended along the token axis [KIVI-sum, KIVI-quo];
 *   - decode attention computes scores on the grouped part and combines the
 *     residual part with it [KIVI-sum].
 *
 * Readings where the pages are silent (the pages print no formula):
 *   - quantizer: z = min of the group, s = (max - min) / (2^b - 1),
 *     code = round-half-even((x - z) / s) clamped to [0, 2^b - 1];
 *     dequantized value = code * s + z.  Every codec step is one IEEE
 *     binary32 operation rounded to nearest-even, in the order written in
 *     quantize_group() below; divisions are true divisions.
 *   - a group whose max equals its min stores s = 0, z = that value and
 *     all-zero codes, so it dequantizes exactly;
 *   - attention: softmax(scale * q . k_t) over every cached token, no mask,
 *     in binary64 on the dequantized keys and values; a GQA query head hq
 *     reads KV head hq / r.
 *   - key outliers (optional, n_out > 0) [KVQ-abs: outliers are isolated per
 *     vector so that they do not stretch the quantization range]: the
 *     "vector" is one key group (one channel over G tokens, the range that
 *     an outlier would stretch); its n_out entries of largest magnitude
 *     (|x| of the binary16 input; equal magnitudes: the lower position
 *     first) form the sparse part and are kept exactly; the other G - n_out
 *     entries form the dense part, quantized as above with min and max taken
 *     over them alone; outlier positions get code 0 in the dense codes; a
 *     dequantized outlier position is its kept value.  No calibration: a
 *     fixed count per group, chosen from the group itself.
 *   - pre-RoPE keys (optional, rope_theta > 0) [KVQ-abs: keys are quantized
 *     before the rotary positional embedding]: the cache holds keys before
 *     the embedding (quantized and residual alike); attention applies it to
 *     each dequantized key at the key's position, its token index t in the
 *     sequence.  The embedding is the rotate-half form: channel pairs
 *     (i, i + D/2) for i < D/2, frequency f_i = rope_theta^(-2i/D), and
 *     (x, y) -> (x cos(f_i t) - y sin(f_i t), x sin(f_i t) + y cos(f_i t)).
 *     Queries arrive with the embedding already applied at their own
 *     position, as the model computes them.
 *
 *   - value sliding window (optional residual policy, v_window = 1)
 *     [KIVI-quo: a fixed-length buffer of recent full-precision tokens;
 *     KIVI-abs: values are quantized per token, so a single value token can
 *     be quantized on its own, while a key group needs G tokens]: the
 *     full-precision values are the R newest tokens.  When a token arrives
 *     and the cache holds L >= R tokens, the value of token L - R leaves the
 *     window and is quantized by itself (its per-token groups, as any
 *     value); keys keep the lazy flush of the whole key residual.  After any
 *     append, values [0, max(0, L - R)) are quantized and the rest are full
 *     precision; keys [0, tq) are quantized, tq >= L - R.  The window keeps
 *     value token t in slot t mod R of the value residual buffer.
 *
 * Packed layout (the library's documented storage contract, re-implemented
 * here independently from its description).  Codes are stored in "rows" of
 * n positions: a key row is one token's n = D channels, a value row is one
 * channel's n = 64 tokens of a 64-token tile.  A row of n codes of b bits
 * takes n*b/32 words; position p of a row sits at (word, bit):
 *   b = 2, 4 : word p/E, bit b*(p%E), E = 32/b (little-endian order);
 *   b = 1    : word p/32, bit beta(p%32),
 *              beta(p) = 4*((p%16)/2) + 2*(p/16) + p%2;
 *   b = 3    : code c = lo + 4*hi; lo at word p/16, bits 2*(p%16) (the
 *              2-bit order), hi at word n/16 + p/32, bit beta(p%32) (the
 *              1-bit order) -- the two-bit plane first, then the one-bit
 *              plane.
 *   K codes : [B][H][cap][D*b/32] words, one key row per token.
 *   V codes : [B][H][cap/64][D][2*b] words: tile t/64, channel d, position
 *             t%64 of that value row.
 *   K scale/zero : [B][H][cap/G][D] binary32.
 *   V scale/zero : [B][H][cap][D/G] binary32.
 *   residual K/V : [B][H][R][D] binary16.
 *   K outliers : [B][H][cap/G][n_out][D] words, a compressed sparse row
 *             store with rows of fixed length n_out (so the row offsets are
 *             implicit): row (group g, channel d) is words [g][0..n_out)[d],
 *             each (i << 16) | binary16 bits of the value at position i of
 *             the group, in increasing i.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC (x86-64 SSE
 * arithmetic, no excess precision).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define KIVIO_OK 0
#define KIVIO_EINVAL 1
#define KIVIO_ESHAPE 2
#define KIVIO_ECAPACITY 3

/* ---- binary16 -> binary32, exact (every half is a float) ---------------- */
float kivio_half_to_float(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) << 31;
  uint32_t exp = (h >> 10) & 0x1fu;
  uint32_t man = h & 0x3ffu;
  uint32_t bits;
  if (exp == 0) {
    if (man == 0) {
      bits = sign;
    } else {
      /* subnormal half: man * 2^-24, renormalise */
      int e = -1;
      do {
        man <<= 1;
        e++;
      } while ((man & 0x400u) == 0);
      man &= 0x3ffu;
      bits = sign | ((uint32_t)(127 - 15 - e) << 23) | (man << 13);
    }
  } else if (exp == 31) {
    bits = sign | 0x7f800000u | (man << 13);
  } else {
    bits = sign | ((exp - 15 + 127) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* ---- binary32 -> binary16, round to nearest even (IEEE 754) -------------- */
uint16_t kivio_float_to_half(float f) {
  uint32_t x;
  memcpy(&x, &f, sizeof x);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t exp = (x >> 23) & 0xffu;
  uint32_t man = x & 0x7fffffu;
  if (exp == 0xffu) /* inf / nan (nan keeps a payload bit) */
    return (uint16_t)(sign | 0x7c00u | (man ? 0x200u | (man >> 13) : 0u));
  const int e = (int)exp - 127; /* unbiased exponent of a normal float */
  if (exp == 0 || e < -25)      /* zero, float subnormal, or below half the
                                   smallest half subnormal: rounds to 0 */
    return (uint16_t)sign;
  man |= 0x800000u; /* 24-bit significand */
  if (e > 15) return (uint16_t)(sign | 0x7c00u); /* overflow -> inf */
  /* keep 11 significant bits for a normal half (e >= -14), fewer for a
     subnormal half; drop `shift` bits with round-half-even */
  const int shift = e >= -14 ? 13 : 13 + (-14 - e);
  uint32_t q = man >> shift;
  const uint32_t rem = man & ((1u << shift) - 1);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;
  /* q is the significand in half units: normal halves carry the implicit bit
     (value 0x400..0x800), subnormals do not; a carry into 0x800 bumps the
     exponent, which the addition below does by itself */
  uint32_t h;
  if (e >= -14)
    h = ((uint32_t)(e + 15) << 10) + (q - 0x400u);
  else
    h = q; /* subnormal (q may reach 0x400: the smallest normal) */
  if (h >= 0x7c00u) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | h);
}

static int words_per_row(int D, int bits) { return D * bits / 32; }

/* bit of position p (0..31) inside a one-bit word (the layout above) */
static int beta(int p) { return 4 * ((p % 16) / 2) + 2 * (p / 16) + p % 2; }

/* OR code c into position p of a row of n codes */
static void row_put(uint32_t* row, int n, int bits, int p, uint32_t c) {
  if (bits == 3) {
    row[p / 16] |= (c & 3u) << (2 * (p % 16));
    row[n / 16 + p / 32] |= (c >> 2) << beta(p % 32);
  } else if (bits == 1) {
    row[p / 32] |= c << beta(p % 32);
  } else {
    const int E = 32 / bits;
    row[p / E] |= c << (bits * (p % E));
  }
}

/* code at position p of a row of n codes */
static uint32_t row_get(const uint32_t* row, int n, int bits, int p) {
  if (bits == 3)
    return ((row[p / 16] >> (2 * (p % 16))) & 3u) |
           (((row[n / 16 + p / 32] >> beta(p % 32)) & 1u) << 2);
  if (bits == 1) return (row[p / 32] >> beta(p % 32)) & 1u;
  const int E = 32 / bits;
  return (row[p / E] >> (bits * (p % E))) & ((1u << bits) - 1u);
}

/* zero every word that position p of the row uses */
static void row_clear(uint32_t* row, int n, int bits, int p) {
  if (bits == 3) {
    row[p / 16] = 0;
    row[n / 16 + p / 32] = 0;
  } else {
    row[p / (32 / bits)] = 0;
  }
}

/* clear the bits of position p of the row (the other positions keep theirs) */
static void row_unset(uint32_t* row, int n, int bits, int p) {
  if (bits == 3) {
    row[p / 16] &= ~(3u << (2 * (p % 16)));
    row[n / 16 + p / 32] &= ~(1u << beta(p % 32));
  } else if (bits == 1) {
    row[p / 32] &= ~(1u << beta(p % 32));
  } else {
    const int E = 32 / bits;
    row[p / E] &= ~(((1u << bits) - 1u) << (bits * (p % E)));
  }
}

/* metadata element m of a scale / zero array: binary32, or binary16 when
 * meta_half (the variant with half-width scale and zero) */
static double meta_get(const void* a, size_t m, int meta_half) {
  if (meta_half) return (double)kivio_half_to_float(((const uint16_t*)a)[m]);
  return (double)((const float*)a)[m];
}
static void meta_put(void* a, size_t m, float v, int meta_half) {
  if (meta_half)
    ((uint16_t*)a)[m] = kivio_float_to_half(v);
  else
    ((float*)a)[m] = v;
}

/* Quantize one group of n binary32 values (already widened from binary16).
 * Writes n codes and the group's scale and zero.  The order of operations is
 * the reading stated in the file header.  skip (NULL = none) marks the
 * positions left out of the dense part (key outliers): min and max are taken
 * over the other positions only, and skipped positions get code 0. */
static void quantize_group(const float* xs, int n, int bits, const uint8_t* skip,
                           uint8_t* codes, float* scale_out, float* zero_out) {
  int first = 0;
  while (skip && skip[first]) first++;
  float mn = xs[first], mx = xs[first];
  for (int i = first + 1; i < n; i++) {
    if (skip && skip[i]) continue;
    if (xs[i] < mn) mn = xs[i];
    if (xs[i] > mx) mx = xs[i];
  }
  const float qmax = (float)((1 << bits) - 1);
  if (mx == mn) { /* constant group: exact */
    *scale_out = 0.0f;
    *zero_out = mn;
    for (int i = 0; i < n; i++) codes[i] = 0;
    return;
  }
  float range = mx - mn;      /* one binary32 rounding */
  float s = range / qmax;     /* one binary32 rounding */
  float z = mn;
  for (int i = 0; i < n; i++) {
    if (skip && skip[i]) {
      codes[i] = 0;
      continue;
    }
    float u = xs[i] - z;      /* one rounding, u >= 0 */
    float v = u / s;          /* one rounding */
    float c = rintf(v);       /* round half to even (default mode) */
    if (c > qmax) c = qmax;
    codes[i] = (uint8_t)c;
  }
  *scale_out = s;
  *zero_out = z;
}

/* The n_out positions of largest |x| in a group of n (equal magnitudes: the
 * lower position first), marked in skip[] and listed in pos[] in increasing
 * order [KVQ-abs; the selection rule is the reading in the file header]. */
static void select_outliers(const float* xs, int n, int n_out, uint8_t* skip, int* pos) {
  for (int i = 0; i < n; i++) skip[i] = 0;
  for (int j = 0; j < n_out; j++) {
    int best = -1;
    float best_mag = -1.0f;
    for (int i = 0; i < n; i++) {
      if (skip[i]) continue;
      float a = fabsf(xs[i]);
      if (a > best_mag) { /* strict: the first of equal magnitudes stays */
        best_mag = a;
        best = i;
      }
    }
    skip[best] = 1;
  }
  int m = 0;
  for (int i = 0; i < n; i++)
    if (skip[i]) pos[m++] = i;
}

static int check_common(int B, int H, int D, int bits, int G, int cap) {
  if (B < 1 || H < 1 || D < 1 || G < 1 || cap < 0) return KIVIO_EINVAL;
  if (bits < 1 || bits > 4) return KIVIO_EINVAL;
  if (D % G != 0) return KIVIO_ESHAPE;
  if ((D * bits) % 32 != 0) return KIVIO_ESHAPE;
  if (cap % 64 != 0 || cap % G != 0) return KIVIO_ESHAPE;
  return KIVIO_OK;
}

/* Key quantization, per channel over groups of G consecutive tokens
 * [KIVI-abs, KIVI-sum].  Source tokens [0, ntok) of k ([B][H][in_stride][D]
 * binary16) go to cache tokens [dst_off, dst_off + ntok).  With n_out > 0
 * each group also isolates its n_out outliers into `outl` (layout and rule
 * in the file header) [KVQ-abs]. */
int kivio_quantize_k(int B, int H, int D, int bits, int G, int cap, int meta_half,
                     const uint16_t* k, int in_stride, int ntok, int dst_off,
                     uint32_t* codes, void* scale, void* zero, int n_out, uint32_t* outl) {
  int rc = check_common(B, H, D, bits, G, cap);
  if (rc) return rc;
  if (n_out < 0 || n_out >= G || (n_out > 0 && !outl)) return KIVIO_EINVAL;
  if (ntok < 1 || ntok % G || dst_off < 0 || dst_off % G || in_stride < ntok)
    return KIVIO_ESHAPE;
  if (dst_off + ntok > cap) return KIVIO_ECAPACITY;
  const int W = words_per_row(D, bits);
  float xs[1024];
  uint8_t cs[1024], skip[1024];
  int pos[1024];
  if (G > 1024) return KIVIO_ESHAPE;
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++) {
      const uint16_t* src = k + ((size_t)b * H + h) * (size_t)in_stride * D;
      uint32_t* cw = codes + ((size_t)b * H + h) * (size_t)cap * W;
      const size_t mbase = ((size_t)b * H + h) * (size_t)(cap / G) * D;
      /* clear the destination rows, then OR codes in */
      for (int t = 0; t < ntok; t++)
        for (int w = 0; w < W; w++) cw[(size_t)(dst_off + t) * W + w] = 0;
      for (int g = 0; g < ntok / G; g++)
        for (int d = 0; d < D; d++) {
          for (int i = 0; i < G; i++)
            xs[i] = kivio_half_to_float(src[(size_t)(g * G + i) * D + d]);
          int gg = (dst_off / G) + g;
          if (n_out > 0) {
            select_outliers(xs, G, n_out, skip, pos);
            uint32_t* row = outl + (mbase + (size_t)gg * D) * n_out;  /* [gg][j][d] */
            for (int j = 0; j < n_out; j++)
              row[(size_t)j * D + d] =
                  ((uint32_t)pos[j] << 16) | src[(size_t)(g * G + pos[j]) * D + d];
          }
          float s, z;
          quantize_group(xs, G, bits, n_out > 0 ? skip : NULL, cs, &s, &z);
          meta_put(scale, mbase + (size_t)gg * D + d, s, meta_half);
          meta_put(zero, mbase + (size_t)gg * D + d, z, meta_half);
          for (int i = 0; i < G; i++) {
            int t = dst_off + g * G + i;
            row_put(cw + (size_t)t * W, D, bits, d, cs[i]);
          }
        }
    }
  return KIVIO_OK;
}

/* value row (within one (b, h) plane) holding token t of channel d */
static size_t v_row(int D, int bits, int t, int d) {
  const int WPC = 2 * bits; /* words per channel per 64-token tile */
  return ((size_t)(t / 64) * D + d) * WPC;
}

/* Value quantization, per token over groups of G consecutive channels
 * [KIVI-abs]; quantized tokens are appended along the token axis
 * [KIVI-sum]. */
int kivio_quantize_v(int B, int H, int D, int bits, int G, int cap, int meta_half,
                     const uint16_t* v, int in_stride, int ntok, int dst_off,
                     uint32_t* codes, void* scale, void* zero) {
  int rc = check_common(B, H, D, bits, G, cap);
  if (rc) return rc;
  if (ntok < 1 || ntok % G || dst_off < 0 || dst_off % G || in_stride < ntok)
    return KIVIO_ESHAPE;
  if (dst_off + ntok > cap) return KIVIO_ECAPACITY;
  const int NG = D / G;
  const size_t plane_words = (size_t)cap * D * bits / 32;
  float xs[1024];
  uint8_t cs[1024];
  if (G > 1024) return KIVIO_ESHAPE;
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++) {
      const uint16_t* src = v + ((size_t)b * H + h) * (size_t)in_stride * D;
      uint32_t* cw = codes + ((size_t)b * H + h) * plane_words;
      const size_t mbase = ((size_t)b * H + h) * (size_t)cap * NG;
      /* the token range is 32-aligned, so the words it uses hold no other tokens */
      for (int t = 0; t < ntok; t++)
        for (int d = 0; d < D; d++)
          row_clear(cw + v_row(D, bits, dst_off + t, d), 64, bits, (dst_off + t) % 64);
      for (int t = 0; t < ntok; t++)
        for (int j = 0; j < NG; j++) {
          for (int i = 0; i < G; i++)
            xs[i] = kivio_half_to_float(src[(size_t)t * D + j * G + i]);
          float s, z;
          quantize_group(xs, G, bits, NULL, cs, &s, &z);
          int tt = dst_off + t;
          meta_put(scale, mbase + (size_t)tt * NG + j, s, meta_half);
          meta_put(zero, mbase + (size_t)tt * NG + j, z, meta_half);
          for (int i = 0; i < G; i++) {
            int d = j * G + i;
            row_put(cw + v_row(D, bits, tt, d), 64, bits, tt % 64, cs[i]);
          }
        }
    }
  return KIVIO_OK;
}

/* Value quantization of one token per (b, h) [KIVI-abs: per token]: source
 * row `slot` of v ([B][H][in_stride][D]) becomes cache token t; the same
 * per-token groups as kivio_quantize_v, at any token position (the bits of
 * position t % 64 in the shared value rows are replaced, the other tokens'
 * bits are kept). */
int kivio_quantize_v_token(int B, int H, int D, int bits, int G, int cap, int meta_half,
                           const uint16_t* v, int in_stride, int slot, int t,
                           uint32_t* codes, void* scale, void* zero) {
  int rc = check_common(B, H, D, bits, G, cap);
  if (rc) return rc;
  if (slot < 0 || slot >= in_stride || t < 0) return KIVIO_ESHAPE;
  if (t >= cap) return KIVIO_ECAPACITY;
  const int NG = D / G;
  const size_t plane_words = (size_t)cap * D * bits / 32;
  float xs[1024];
  uint8_t cs[1024];
  if (G > 1024) return KIVIO_ESHAPE;
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++) {
      const uint16_t* src = v + (((size_t)b * H + h) * (size_t)in_stride + slot) * D;
      uint32_t* cw = codes + ((size_t)b * H + h) * plane_words;
      const size_t mbase = ((size_t)b * H + h) * (size_t)cap * NG;
      for (int j = 0; j < NG; j++) {
        for (int i = 0; i < G; i++) xs[i] = kivio_half_to_float(src[j * G + i]);
        float s, z;
        quantize_group(xs, G, bits, NULL, cs, &s, &z);
        meta_put(scale, mbase + (size_t)t * NG + j, s, meta_half);
        meta_put(zero, mbase + (size_t)t * NG + j, z, meta_half);
        for (int i = 0; i < G; i++) {
          uint32_t* row = cw + v_row(D, bits, t, j * G + i);
          row_unset(row, 64, bits, t % 64);
          row_put(row, 64, bits, t % 64, cs[i]);
        }
      }
    }
  return KIVIO_OK;
}

/* Streaming append of one decode token per (b, h) [KIVI-sum: the residual
 * part is kept in full precision and new tokens are appended; KIVI-quo: a
 * fixed-length residual of recent tokens].  Reading: when a token arrives
 * and the residual already holds R tokens, all R are quantized into the
 * grouped part first (keys and values alike), then the new token is stored
 * in the residual.  *tq, *tr are updated only on success.  A flush isolates
 * key outliers as kivio_quantize_k does (n_out, k_outl). */
int kivio_append(int B, int H, int D, int bits, int G, int R, int cap, int meta_half,
                 uint32_t* k_codes, void* ks, void* kz, uint32_t* v_codes,
                 void* vs, void* vz, uint16_t* k_res, uint16_t* v_res,
                 const uint16_t* k_new, const uint16_t* v_new, int* tq,
                 int* tr, int n_out, uint32_t* k_outl) {
  int rc = check_common(B, H, D, bits, G, cap);
  if (rc) return rc;
  if (R < G || R % G) return KIVIO_ESHAPE;
  if (n_out < 0 || n_out >= G || (n_out > 0 && !k_outl)) return KIVIO_EINVAL;
  int q = *tq, r = *tr;
  if (q < 0 || q % G || r < 0 || r > R) return KIVIO_ESHAPE;
  if (r == R) {
    if (q + R > cap) return KIVIO_ECAPACITY;
    rc = kivio_quantize_k(B, H, D, bits, G, cap, meta_half, k_res, R, R, q, k_codes, ks, kz,
                          n_out, k_outl);
    if (rc) return rc;
    rc = kivio_quantize_v(B, H, D, bits, G, cap, meta_half, v_res, R, R, q, v_codes, vs, vz);
    if (rc) return rc;
    q += R;
    r = 0;
  }
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++)
      for (int d = 0; d < D; d++) {
        size_t src = ((size_t)b * H + h) * D + d;
        size_t dst = (((size_t)b * H + h) * R + r) * D + d;
        k_res[dst] = k_new[src];
        v_res[dst] = v_new[src];
      }
  *tq = q;
  *tr = r + 1;
  return KIVIO_OK;
}

/* kivio_append under the value sliding window (the v_window reading in the
 * file header): the keys take exactly kivio_append's steps; v_res is the
 * window (value token t in slot t mod R).  With L = tq + tr tokens cached,
 * L >= R sends value token L - R (slot (L - R) mod R = L mod R) to the
 * value store first; the new value then takes slot L mod R.  *tq, *tr are
 * updated only on success, and nothing is written on an error. */
int kivio_append_vw(int B, int H, int D, int bits, int G, int R, int cap, int meta_half,
                    uint32_t* k_codes, void* ks, void* kz, uint32_t* v_codes,
                    void* vs, void* vz, uint16_t* k_res, uint16_t* v_res,
                    const uint16_t* k_new, const uint16_t* v_new, int* tq,
                    int* tr, int n_out, uint32_t* k_outl) {
  int rc = check_common(B, H, D, bits, G, cap);
  if (rc) return rc;
  if (R < G || R % G) return KIVIO_ESHAPE;
  if (n_out < 0 || n_out >= G || (n_out > 0 && !k_outl)) return KIVIO_EINVAL;
  int q = *tq, r = *tr;
  if (q < 0 || q % G || r < 0 || r > R) return KIVIO_ESHAPE;
  const int L = q + r;
  if (r == R && q + R > cap) return KIVIO_ECAPACITY;
  if (L >= R && L - R >= cap) return KIVIO_ECAPACITY;
  if (r == R) {
    rc = kivio_quantize_k(B, H, D, bits, G, cap, meta_half, k_res, R, R, q, k_codes, ks, kz,
                          n_out, k_outl);
    if (rc) return rc;
    q += R;
    r = 0;
  }
  if (L >= R) {
    rc = kivio_quantize_v_token(B, H, D, bits, G, cap, meta_half, v_res, R, L % R, L - R,
                                v_codes, vs, vz);
    if (rc) return rc;
  }
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++)
      for (int d = 0; d < D; d++) {
        size_t src = ((size_t)b * H + h) * D + d;
        k_res[(((size_t)b * H + h) * R + r) * D + d] = k_new[src];
        v_res[(((size_t)b * H + h) * R + L % R) * D + d] = v_new[src];
      }
  *tq = q;
  *tr = r + 1;
  return KIVIO_OK;
}

/* dequantized key / value of cache token t (< tq), channel d, in binary64 */
/* (sc, zr point at the plane's metadata; mb is the plane's element offset;
 * ow, n_out: the plane's key outliers, row (t/G, d), if any) */
static double dequant_k(const uint32_t* cw, const void* sc, const void* zr, size_t mb,
                        int meta_half, int D, int bits, int G, int t, int d,
                        const uint32_t* ow, int n_out) {
  for (int j = 0; j < n_out; j++) {
    uint32_t w = ow[((size_t)(t / G) * n_out + j) * D + d];
    if ((int)(w >> 16) == t % G) return (double)kivio_half_to_float((uint16_t)(w & 0xffffu));
  }
  const int W = words_per_row(D, bits);
  uint32_t c = row_get(cw + (size_t)t * W, D, bits, d);
  size_t m = mb + (size_t)(t / G) * D + d;
  return (double)c * meta_get(sc, m, meta_half) + meta_get(zr, m, meta_half);
}

static double dequant_v(const uint32_t* cw, const void* sc, const void* zr, size_t mb,
                        int meta_half, int D, int bits, int G, int t, int d) {
  uint32_t c = row_get(cw + v_row(D, bits, t, d), 64, bits, t % 64);
  size_t m = mb + (size_t)t * (D / G) + d / G;
  return (double)c * meta_get(sc, m, meta_half) + meta_get(zr, m, meta_half);
}

/* Rotary embedding of one key vector kv[D] at position t, in place (the
 * rotate-half form stated in the file header) [KVQ-abs]. */
static void rope_key(double* kv, int D, int t, double theta) {
  const int h = D / 2;
  for (int i = 0; i < h; i++) {
    const double f = pow(theta, -2.0 * (double)i / (double)D);
    const double a = f * (double)t;
    const double c = cos(a), s = sin(a);
    const double x = kv[i], y = kv[i + h];
    kv[i] = x * c - y * s;
    kv[i + h] = x * s + y * c;
  }
}

/* Decode attention over the mixed cache [KIVI-sum: scores on the grouped
 * part, then the residual part is combined with it], binary64 throughout.
 * q, out: [B][H*r][D].  Work space: 2*(tq+tr) doubles in `scratch`.  Keys
 * with isolated outliers (n_out > 0) dequantize through k_outl; with
 * rope_theta > 0 the cached keys are pre-RoPE and each is rotated at its
 * position before the dot product [KVQ-abs]. */
int kivio_decode_attn_vw(int B, int H, int r, int D, int bits, int G, int R,
                         int cap, int meta_half, const uint32_t* k_codes, const void* ks,
                         const void* kz, const uint32_t* v_codes,
                         const void* vs, const void* vz, const uint16_t* k_res,
                         const uint16_t* v_res, int tq, int tr, const uint16_t* q,
                         float softmax_scale, double* out, double* scratch,
                         int n_out, const uint32_t* k_outl, double rope_theta,
                         int v_window);

int kivio_decode_attn(int B, int H, int r, int D, int bits, int G, int R,
                      int cap, int meta_half, const uint32_t* k_codes, const void* ks,
                      const void* kz, const uint32_t* v_codes,
                      const void* vs, const void* vz, const uint16_t* k_res,
                      const uint16_t* v_res, int tq, int tr, const uint16_t* q,
                      float softmax_scale, double* out, double* scratch,
                      int n_out, const uint32_t* k_outl, double rope_theta) {
  return kivio_decode_attn_vw(B, H, r, D, bits, G, R, cap, meta_half, k_codes, ks, kz,
                              v_codes, vs, vz, k_res, v_res, tq, tr, q, softmax_scale, out,
                              scratch, n_out, k_outl, rope_theta, 0);
}

/* The same attention with the value residual read as the sliding window when
 * v_window = 1: values [0, max(0, L - R)) dequantized, value token t >= that
 * from slot t mod R of v_res. */
int kivio_decode_attn_vw(int B, int H, int r, int D, int bits, int G, int R,
                         int cap, int meta_half, const uint32_t* k_codes, const void* ks,
                         const void* kz, const uint32_t* v_codes,
                         const void* vs, const void* vz, const uint16_t* k_res,
                         const uint16_t* v_res, int tq, int tr, const uint16_t* q,
                         float softmax_scale, double* out, double* scratch,
                         int n_out, const uint32_t* k_outl, double rope_theta,
                         int v_window) {
  int rc = check_common(B, H, D, bits, G, cap);
  if (rc) return rc;
  if (r < 1) return KIVIO_EINVAL;
  if (n_out < 0 || n_out >= G || (n_out > 0 && !k_outl)) return KIVIO_EINVAL;
  if (!(rope_theta >= 0.0) || isinf(rope_theta) || D % 2 != 0 || D > 1024) return KIVIO_EINVAL;
  if (tq < 0 || tq % G || tq > cap || tr < 0 || tr > R || tq + tr < 1)
    return KIVIO_ESHAPE;
  if (v_window != 0 && v_window != 1) return KIVIO_EINVAL;
  const int Hq = H * r, W = words_per_row(D, bits);
  const int L = tq + tr;
  const int tv = v_window ? (L > R ? L - R : 0) : tq;   /* quantized value tokens */
  double* logit = scratch;
  double* p = scratch + L;
  for (int b = 0; b < B; b++)
    for (int hq = 0; hq < Hq; hq++) {
      const int h = hq / r;
      const size_t bh = (size_t)b * H + h;
      const uint32_t* kc = k_codes + bh * (size_t)cap * W;
      const size_t kmb = bh * (size_t)(cap / G) * D;
      const uint32_t* ko = n_out > 0 ? k_outl + kmb * n_out : NULL;
      const uint32_t* vc = v_codes + bh * (size_t)cap * D * bits / 32;
      const size_t vmb = bh * (size_t)cap * (D / G);
      const uint16_t* kr = k_res + bh * (size_t)R * D;
      const uint16_t* vr = v_res + bh * (size_t)R * D;
      const uint16_t* qv = q + ((size_t)b * Hq + hq) * D;
      for (int t = 0; t < L; t++) {
        double kvec[1024];
        for (int d = 0; d < D; d++)
          kvec[d] = (t < tq) ? dequant_k(kc, ks, kz, kmb, meta_half, D, bits, G, t, d, ko, n_out)
                             : (double)kivio_half_to_float(kr[(size_t)(t - tq) * D + d]);
        if (rope_theta > 0.0) rope_key(kvec, D, t, rope_theta);
        double dot = 0.0;
        for (int d = 0; d < D; d++) dot += (double)kivio_half_to_float(qv[d]) * kvec[d];
        logit[t] = (double)softmax_scale * dot;
      }
      double m = logit[0];
      for (int t = 1; t < L; t++)
        if (logit[t] > m) m = logit[t];
      double l = 0.0;
      for (int t = 0; t < L; t++) {
        p[t] = exp(logit[t] - m);
        l += p[t];
      }
      double* o = out + ((size_t)b * Hq + hq) * D;
      for (int d = 0; d < D; d++) {
        double acc = 0.0;
        for (int t = 0; t < L; t++) {
          const size_t slot = v_window ? (size_t)(t % R) : (size_t)(t - tq);
          double vv = (t < tv) ? dequant_v(vc, vs, vz, vmb, meta_half, D, bits, G, t, d)
                               : (double)kivio_half_to_float(vr[slot * D + d]);
          acc += p[t] * vv;
        }
        o[d] = acc / l;
      }
    }
  return KIVIO_OK;
}

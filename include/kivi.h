/*
 * kivi.h -- C ABI of the KIVI low-bit KV-cache library for AMD Instinct
 * MI355X (gfx950).
 *
 * The method ("KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV
 * Cache"; mlsanity paper page, Abstract; study.space summary page):
 *   - keys are quantized per channel, values per token, with asymmetric
 *     low-bit codes (2-bit; 4-bit also supported here);
 *   - the cache is a quantized "grouped" part plus a full-precision
 *     "residual" part of the most recent tokens; tokens are appended along
 *     the token axis, and key groups span G consecutive tokens;
 *   - decode attention scores the grouped part with a tiled product and
 *     combines the residual part with it.
 * The pages print no formula.  This library uses, for every group of G
 * values x: z = min(x), s = (max(x) - min(x)) / (2^b - 1),
 * code = round-half-even((x - z) / s) clamped to 2^b - 1, each step one IEEE
 * binary32 operation in that order (true division, no fused multiply-add);
 * a group with max == min stores s = 0, z = that value and zero codes.
 * Metadata width (kivi_shape.meta_half): s and z are stored as binary32, or,
 * with meta_half = 1, as binary16 rounded to nearest even from those binary32
 * values (the codes stay those of the binary32 computation; z, a binary16
 * input, is exact; s never overflows since it is at most 131008/3).
 * Dequantization always uses the stored values.
 *
 * Key outliers (kivi_shape.outliers = n > 0; "KVQuant: Towards 10 Million
 * Context Length LLM Inference with KV Cache Quantization", codewithpapers.app
 * paper page, abstract: outliers are isolated separately for each vector so
 * that they do not stretch the quantization range).  Here the vector is one
 * key group (one channel over G tokens).  Its n entries of largest magnitude
 * (equal magnitudes: the lower token first) are kept exactly in a sparse
 * store; the other G - n entries are quantized by the formula above with min
 * and max taken over them alone; outlier positions carry code 0 and
 * dequantize to their kept value.  Selection uses no calibration data.
 *
 * Pre-RoPE keys (kivi_shape.rope_theta > 0; the same KVQuant page: keys are
 * quantized before the rotary positional embedding): the cache stores the
 * keys it is given (quantized and residual) before the embedding, and the
 * decode applies the embedding to every dequantized key at its position, the
 * key's token index t in its sequence: channel pairs (i, i + D/2) for i <
 * D/2 are rotated by the angle t * rope_theta^(-2i/D) (the rotate-half form;
 * (x, y) -> (x cos - y sin, x sin + y cos)).  Queries are passed with the
 * embedding already applied at their own position, as a model computes them.
 *
 * Conventions for every function below:
 *   - All buffer pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), owned by the caller; the library never allocates, frees,
 *     reads back or synchronizes.  fp16 is IEEE binary16 bit patterns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream); all work
 *     is enqueued asynchronously on it, in order.
 *   - Return value: KIVI_OK or one of the error codes below.  Arguments are
 *     validated before any HIP call; on error nothing is enqueued and no
 *     output (including *cache) is modified.  Faults inside kernels surface
 *     at the caller's next synchronization, as for any HIP launch.
 *   - Every buffer pointer must be 16-byte aligned (KIVI_EALIGN otherwise).
 *   - Functions are reentrant; one kivi_cache must not be used from two host
 *     threads at once.
 *
 * Storage layout (E = 32 / bits codes per 32-bit word, little-endian bits):
 *   k_codes : uint32 [B][Hkv][cap][D/E]; channel d of token t is in word d/E
 *             at bits [bits*(d%E), +bits).
 *   k_scale, k_zero : meta [B][Hkv][cap/G][D]    (one pair per channel per
 *             group of G tokens); meta = float, or binary16 bits (uint16)
 *             when meta_half.  A key zero is the minimum of binary16 inputs
 *             and so a binary16 value; the decode relies on it (with several
 *             query heads per KV head it takes the zeros as binary16 matrix
 *             operands), so planes filled other than by this library's codec
 *             must keep that property.
 *   v_codes : uint32 [B][Hkv][cap/64][D][64/E]; 64-token tiles, channel-major
 *             inside a tile: token t, channel d is in tile t/64, word
 *             (t%64)/E of channel d, bits [bits*((t%64)%E), +bits).
 *   v_scale, v_zero : meta [B][Hkv][cap][D/G]    (one pair per token per
 *             group of G channels).
 *   k_res, v_res : fp16 [B][Hkv][R][D]; residual slot i holds cache token
 *             tq + i.
 *   queries / outputs : fp16 [B][Hkv*r][D]; query head h reads KV head h/r.
 *   k_outliers (outliers = n > 0): uint32 [B][Hkv][cap/G][n][D], a
 *             compressed-sparse-row store with rows of fixed length n (row
 *             offsets implicit): the row of (group g, channel d) is words
 *             [g][0..n)[d], each (i << 16) | fp16 bits of the key at token
 *             g*G + i, in increasing i.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kivi_status {
  KIVI_OK = 0,
  KIVI_EINVAL = 1,       /* null pointer, bits not in 1..4, a count < 1     */
  KIVI_ESHAPE = 2,       /* sizes inconsistent (see each function)          */
  KIVI_EALIGN = 3,       /* a buffer pointer not 16-byte aligned            */
  KIVI_ECAPACITY = 4,    /* the quantized store would overflow `capacity`   */
  KIVI_EWORKSPACE = 5,   /* decode workspace smaller than required          */
  KIVI_EUNSUPPORTED = 6, /* a (head_dim, group, bits) with no kernel here   */
  KIVI_EHIP = 7          /* a HIP launch or runtime call failed             */
};

/* Largest split count a decode call accepts (num_splits arguments). */
#define KIVI_MAX_SPLITS 4096

/* Static configuration of one cache (one attention layer).
 * Constraints (KIVI_ESHAPE unless noted):
 *   batch, num_kv_heads, gqa_ratio >= 1 (KIVI_EINVAL);
 *   bits in {1, 2, 3, 4} (KIVI_EINVAL);
 *   head_dim in {32, 64, 128, 256}, group in {32, 64, 128}, group divides
 *     head_dim (KIVI_EUNSUPPORTED for other head_dim/group values);
 *   residual >= group and a multiple of group;
 *   capacity >= 0, a multiple of 64 and of group;
 *   gqa_ratio <= 16;
 *   meta_half in {0, 1} (KIVI_EINVAL): 0 = binary32 scale / zero, 1 =
 *     binary16 (half the metadata bytes; a zero-initialised shape keeps
 *     binary32);
 *   outliers in 0..8 and < group (KIVI_EINVAL): key outliers isolated per
 *     key group (0, the zero-initialised value, = none; every cache then
 *     needs its k_outliers buffer);
 *   rope_theta finite and >= 0 (KIVI_EINVAL): 0 (the zero-initialised value)
 *     = keys used as stored; > 0 = pre-RoPE keys rotated at decode with this
 *     base (10000 for Llama-2);
 *   deterministic in {0, 1} (KIVI_EINVAL): 0 (the zero-initialised value) =
 *     the matrix-core decode lets the waves of a block take its 64-token
 *     tiles in the order their loads return, so the binary32 sums group
 *     differently from call to call and the output can differ in its last
 *     bits; 1 = every wave keeps a fixed run of tiles and repeated calls
 *     give identical bits (slower when some waves' loads return late).
 *     The generic kernel always uses fixed runs;
 *   v_window in {0, 1} (KIVI_EINVAL): the residual policy for values.  0 (the
 *     zero-initialised value) = values follow the keys: a token arriving at
 *     a full residual flushes all residual tokens, keys and values.  1 = a
 *     sliding window of values (scholarfeed "KIVI" quote page: a fixed-length
 *     buffer of recent full-precision tokens; "KIVI...", Abstract: values are
 *     quantized per token, so one value token can be quantized on its own):
 *     the R newest values stay fp16, value token t in slot t mod R of v_res,
 *     and a value leaving the window is quantized by itself; keys keep the
 *     lazy flush.  With L = tq + tr cached tokens, values [0, max(0, L - R))
 *     are quantized.  Uniform caches only (KIVI_EUNSUPPORTED for ragged and
 *     paged caches).  Decode: the whole 64-token tiles below L - R (keys
 *     and values quantized) on the matrix-core kernel where it takes the
 *     shape, in num_splits splits, and the other tokens as one more split-K
 *     partial (a dedicated kernel without key outliers or pre-RoPE keys,
 *     else the generic kernel); shapes the matrix-core kernel does not take
 *     run on the generic kernel alone. */
typedef struct {
  int32_t batch;
  int32_t num_kv_heads;
  int32_t gqa_ratio;
  int32_t head_dim;
  int32_t bits;
  int32_t group;
  int32_t residual;
  int32_t capacity;
  int32_t meta_half;
  int32_t outliers;
  float rope_theta;
  int32_t deterministic;
  int32_t v_window;
} kivi_shape;

/* One mixed-precision cache: device buffers (layouts above) plus the host-side
 * lengths: tq quantized tokens (a multiple of group, <= capacity) and tr
 * residual tokens (0 <= tr <= residual), equal for every sequence.  With
 * shape.v_window = 1, tq and tr count keys; the values are quantized up to
 * max(0, tq + tr - residual) and v_res holds the rest as the window. */
typedef struct {
  kivi_shape shape;
  uint32_t* k_codes;
  void* k_scale;     /* float, or uint16 binary16 bits when shape.meta_half */
  void* k_zero;
  uint32_t* v_codes;
  void* v_scale;
  void* v_zero;
  uint16_t* k_res;
  uint16_t* v_res;
  int32_t tq;
  int32_t tr;
  uint32_t* k_outliers;   /* shape.outliers > 0 only (NULL otherwise) */
} kivi_cache;

/* Bytes of each cache buffer for a shape (host arithmetic only, no HIP call).
 * Returns KIVI_OK and fills the six sizes, or a shape error. */
int kivi_cache_bytes(const kivi_shape* shape, size_t* k_codes, size_t* k_meta,
                     size_t* v_codes, size_t* v_meta, size_t* residual,
                     size_t* query);

/* Bytes of the key-outlier store of a shape: the contiguous layout above
 * when page_tokens == 0, else a page pool of num_pages pages of page_tokens
 * tokens ([num_pages][Hkv][page_tokens/G][n][D] words).  0 bytes when
 * shape.outliers == 0.  Host arithmetic only. */
int kivi_outlier_bytes(const kivi_shape* shape, int32_t page_tokens,
                       int32_t num_pages, size_t* bytes);

/* Per-channel key quantization ("KIVI...", Abstract: keys are grouped along
 * the channel dimension; study.space summary: the key groups span tokens).
 * Quantizes source tokens [0, ntok) of `k` (fp16 [B][Hkv][in_tok_stride][D])
 * into cache tokens [dst_tok_offset, dst_tok_offset + ntok) of `codes`,
 * `scale`, `zero` (layouts above; element type set by shape->meta_half).
 * Each (channel, group of G tokens) gets its own scale and zero; results are
 * bit-exact to the formula above.
 * ntok >= 1, ntok and dst_tok_offset multiples of group, in_tok_stride >=
 * ntok; dst_tok_offset + ntok > capacity gives KIVI_ECAPACITY. */
int kivi_quantize_k(const kivi_shape* shape, const uint16_t* k,
                    int32_t in_tok_stride, int32_t ntok,
                    int32_t dst_tok_offset, uint32_t* codes, void* scale,
                    void* zero, void* stream);

/* kivi_quantize_k with key outliers isolated (KVQuant page, abstract; the
 * rule at the top of this file): also writes the rows of the quantized
 * groups into `outliers` (layout of k_outliers above).  Requires
 * shape->outliers > 0 and outliers non-NULL (KIVI_EINVAL); kivi_quantize_k
 * requires shape->outliers == 0 (KIVI_EINVAL). */
int kivi_quantize_k_outliers(const kivi_shape* shape, const uint16_t* k,
                             int32_t in_tok_stride, int32_t ntok,
                             int32_t dst_tok_offset, uint32_t* codes,
                             void* scale, void* zero, uint32_t* outliers,
                             void* stream);

/* Per-token value quantization ("KIVI...", Abstract: values are quantized
 * per token).  Same arguments and rules as kivi_quantize_k; each (token,
 * group of G channels) gets its own scale and zero. */
int kivi_quantize_v(const kivi_shape* shape, const uint16_t* v,
                    int32_t in_tok_stride, int32_t ntok,
                    int32_t dst_tok_offset, uint32_t* codes, void* scale,
                    void* zero, void* stream);

/* Fill an empty cache from a prompt (study.space summary: the cache is split
 * into grouped and residual parts).  k, v: fp16 [B][Hkv][ntok][D].  Tokens
 * [0, tq) are quantized, tokens [tq, ntok) are copied into the residual.
 * Requires tq a multiple of group, 0 <= ntok - tq <= residual, tq <=
 * capacity.  On success sets cache->tq = tq, cache->tr = ntok - tq. */
int kivi_prefill(kivi_cache* cache, const uint16_t* k, const uint16_t* v,
                 int32_t ntok, int32_t tq, void* stream);

/* Append one decode token per (sequence, KV head) (study.space summary: new
 * tokens are appended along the token axis; scholarfeed "KIVI" quote page: a
 * fixed-length residual of recent full-precision key/value pairs).
 * k_new, v_new: fp16 [B][Hkv][D].  If the residual already holds `residual`
 * tokens, all of them are first quantized into tokens [tq, tq + residual) of
 * the grouped part (KIVI_ECAPACITY if that exceeds capacity), tq grows by
 * `residual` and tr becomes 0; then the token is stored in residual slot tr
 * and tr grows by 1.  cache->tq / tr change only on success. */
int kivi_append(kivi_cache* cache, const uint16_t* k_new,
                const uint16_t* v_new, void* stream);

/* Split count the decode call uses when num_splits == 0, for the current
 * cache lengths and the current device (queries the device's compute-unit
 * count once per device).  Returns >= 1, or a negative error code. */
int kivi_decode_auto_splits(const kivi_cache* cache);

/* Workspace bytes kivi_decode_attn needs for `num_splits` splits of the
 * context; num_splits == 0 returns a bound valid for the automatic split
 * count at every context length of this shape; 0 for an invalid shape or a
 * num_splits outside 0..KIVI_MAX_SPLITS.  With shape->v_window the bound
 * covers one more partial (the window's tail, below).  Host arithmetic
 * only. */
size_t kivi_decode_workspace_bytes(const kivi_shape* shape,
                                   int32_t num_splits);

/* Decode attention on the mixed cache (study.space summary: scores on the
 * grouped part by a tiled product, the residual part combined with it).
 * For every sequence b and query head h (KV head h/r):
 *   o = softmax_t(softmax_scale * q . k_t) . v_t over the tq dequantized and
 *   tr residual tokens (no mask), accumulated in binary32, written as fp16
 *   (round to nearest even).  q, out: fp16 [B][Hkv*r][D].
 * num_splits: number of context chunks per (b, KV head) reduced at the end
 *   (0 = automatic; at most KIVI_MAX_SPLITS and at most tq + tr, else
 *   KIVI_ESHAPE); workspace: device scratch of at least
 *   kivi_decode_workspace_bytes(shape, num_splits) bytes (may be NULL when
 *   that is 0).  Requires tq + tr >= 1 (KIVI_ESHAPE).  With
 *   shape.deterministic = 1 results are bit-identical between calls for a
 *   fixed split count (no floating-point atomics anywhere); with 0 they can
 *   differ in the last bits (tile order inside a block, above).
 * Key outliers (shape.outliers > 0): quantized keys are dequantized through
 *   cache->k_outliers (the kept value replaces the dense one); the
 *   matrix-core kernel handles outliers <= 2, larger counts use the generic
 *   kernel.
 * Pre-RoPE keys (shape.rope_theta > 0): every key is rotated at its token
 *   index before the dot product (rule at the top of this file); the
 *   matrix-core kernel scores keys on the vector units in that case and does
 *   not combine it with outliers (that combination uses the generic kernel). */
int kivi_decode_attn(const kivi_cache* cache, const uint16_t* q,
                     float softmax_scale, uint16_t* out, void* workspace,
                     size_t workspace_bytes, int32_t num_splits,
                     void* stream);

/* One decode step of a layer in one call: exactly kivi_append(cache, k_new,
 * v_new) followed by kivi_decode_attn(cache, q, ...) (study.space summary:
 * tokens are appended along the token axis, then attention reads the grouped
 * and residual parts), with the same results, bit for bit, and the same
 * errors, all checked before anything is enqueued (on error nothing is
 * enqueued and *cache is unchanged).  Where the matrix-core decode kernel
 * applies (head_dim 128, group 32, gqa_ratio 1, 2, 4 or 8) the append is
 * folded into that kernel: the new token is read from k_new / v_new directly
 * and written into its residual slot by the same launch, saving the separate
 * copy launch.  A full residual is still flushed first, as by kivi_append.
 * The workspace must cover the split count of the post-append lengths. */
int kivi_append_decode_attn(kivi_cache* cache, const uint16_t* k_new,
                            const uint16_t* v_new, const uint16_t* q,
                            float softmax_scale, uint16_t* out,
                            void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream);

/* Bytes of the library's own device scratch array used by
 * kivi_decode_attn_noalloc (one copy per GPU, held until the process ends). */
#define KIVI_SCRATCH_BYTES (8u << 20)

/* kivi_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same validation and results, bit for bit, as
 * kivi_decode_attn with the same split count, but the split-K partials live
 * in a device array of the library (KIVI_SCRATCH_BYTES per GPU) instead of a
 * caller workspace.  The call allocates nothing.  A split count whose
 * partials, kivi_decode_workspace_bytes(&cache->shape, num_splits), exceed
 * KIVI_SCRATCH_BYTES is refused with KIVI_EWORKSPACE before any HIP call
 * (num_splits == 0: the automatic count, checked after the compute-unit
 * query).  The first call on a device looks up that device's copy of the
 * array (a HIP symbol query; KIVI_EHIP if it fails).  Every call on one GPU
 * shares its array and leaves its last partials there; nothing in it needs
 * clearing (each call writes every partial it reads).  Calls that can
 * overlap on one GPU (other streams, other host threads) race on the array
 * and must be ordered by the caller. */
int kivi_decode_attn_noalloc(const kivi_cache* cache, const uint16_t* q,
                             float softmax_scale, uint16_t* out,
                             int32_t num_splits, void* stream);

/* ---- Ragged batches: a different length for every sequence ------------
 * In a serving batch every sequence has its own context length, so the
 * quantized and residual token counts differ per sequence (study.space
 * summary: tokens are appended along the token axis of each sequence's
 * grouped + residual cache; scholarfeed "KIVI" quote page: the residual is a
 * fixed-length buffer per sequence).  A kivi_ragged_cache has the same device
 * buffers and layouts as kivi_cache (every sequence owns `capacity` token
 * slots); its lengths are HOST arrays owned by the caller, tq[b] and tr[b]
 * for b < shape.batch, each obeying the kivi_cache rules (tq[b] a multiple of
 * group and <= capacity, 0 <= tr[b] <= residual).  Calls read them and, on
 * success, update them in place; on error nothing is enqueued and they are
 * unchanged.  Results for each sequence are bit-identical (codes, scales,
 * zeros, residual) to a one-sequence kivi_cache holding that sequence alone;
 * attention meets the same tolerance.  Per-sequence lengths travel with each
 * launch (batches above 128 sequences take several launches). */
typedef struct {
  kivi_shape shape;
  uint32_t* k_codes;
  void* k_scale;
  void* k_zero;
  uint32_t* v_codes;
  void* v_scale;
  void* v_zero;
  uint16_t* k_res;
  uint16_t* v_res;
  int32_t* tq;       /* host [batch] */
  int32_t* tr;       /* host [batch] */
  uint32_t* k_outliers;   /* shape.outliers > 0 only */
} kivi_ragged_cache;

/* Fill an empty ragged cache from padded prompts.  k, v: fp16
 * [B][Hkv][in_tok_stride][D]; sequence b has ntok[b] tokens (0 <= ntok[b] <=
 * in_tok_stride, host array); tokens [0, tq[b]) are quantized (tq[b] a
 * multiple of group, <= capacity: KIVI_ECAPACITY otherwise) and tokens
 * [tq[b], ntok[b]) copied into the residual (ntok[b] - tq[b] <= residual).
 * A sequence may be empty (ntok[b] = 0).  Sets cache->tq, cache->tr. */
int kivi_ragged_prefill(kivi_ragged_cache* cache, const uint16_t* k,
                        const uint16_t* v, int32_t in_tok_stride,
                        const int32_t* ntok, const int32_t* tq, void* stream);

/* Append one token to every sequence (k_new, v_new: fp16 [B][Hkv][D]).  Each
 * sequence whose residual is full is flushed first, as in kivi_append
 * (KIVI_ECAPACITY if any of them would overflow capacity). */
int kivi_ragged_append(kivi_ragged_cache* cache, const uint16_t* k_new,
                       const uint16_t* v_new, void* stream);

/* Split count kivi_ragged_decode_attn uses when num_splits == 0 (chosen for
 * the longest sequence).  Returns >= 1, or a negative error code. */
int kivi_ragged_decode_auto_splits(const kivi_ragged_cache* cache);

/* Decode attention for every sequence at its own lengths (the operation of
 * kivi_decode_attn).  Every sequence must hold at least one token
 * (KIVI_ESHAPE).  num_splits (0 = automatic, at most KIVI_MAX_SPLITS, else
 * KIVI_ESHAPE) applies to every sequence; a
 * split past a short sequence's end contributes nothing.  The workspace is
 * sized by kivi_decode_workspace_bytes(&cache->shape, num_splits). */
int kivi_ragged_decode_attn(const kivi_ragged_cache* cache, const uint16_t* q,
                            float softmax_scale, uint16_t* out,
                            void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream);

/* One decode step of a ragged batch: exactly kivi_ragged_append followed by
 * kivi_ragged_decode_attn (same validation, bit-identical results), with the
 * append folded into the decode launch where the matrix-core kernel
 * applies. */
int kivi_ragged_append_decode_attn(kivi_ragged_cache* cache,
                                   const uint16_t* k_new,
                                   const uint16_t* v_new, const uint16_t* q,
                                   float softmax_scale, uint16_t* out,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t num_splits, void* stream);

/* ---- Paged quantized store --------------------------------------------
 * A server keeps many sequences of unpredictable length, so the quantized
 * part of each sequence lives in fixed-size pages drawn from shared pools, as
 * in paged attention.  The scholarfeed "KIVI" quote page notes that a paged
 * pool of uniform-precision blocks does not fit a cache that mixes quantized
 * tokens with a fixed-length full-precision residual, and names separate
 * page tables as one way out: here the quantized tokens are paged (one block
 * table) and the residual keeps a fixed-length pool of its own per sequence,
 * so each pool holds one precision.  A page holds P = page_tokens consecutive tokens of
 * one sequence for every KV head; page p, head h is a "slice" with exactly the
 * layout of a kivi_cache plane of capacity P:
 *   k_codes : uint32 [num_pages][Hkv][P][D/E]
 *   k_scale, k_zero : meta [num_pages][Hkv][P/G][D]
 *   v_codes : uint32 [num_pages][Hkv][P/64][D][64/E]
 *   v_scale, v_zero : meta [num_pages][Hkv][P][D/G]
 *   k_outliers : uint32 [num_pages][Hkv][P/G][n][D] (outliers = n > 0)
 * Logical token t of sequence b is token t mod P of page
 * block_table[b * (capacity / P) + t / P].  The residual stays one
 * fixed-length pool per sequence: k_res, v_res fp16 [B][Hkv][R][D].
 * shape.capacity is the most tokens one sequence may quantize (a multiple of
 * P); P is a power of two, at least 64 and at least group (KIVI_ESHAPE
 * otherwise).  The block
 * table is a DEVICE int32 array [batch][capacity / P] (4-byte aligned) owned
 * and filled by the caller: every entry a call may touch must name a page
 * (the pages of tokens [0, tq[b]) for a decode, plus those of [tq[b],
 * tq[b] + residual) for a call that may flush, i.e. prefill and append), and
 * pages written by different sequences must be distinct.  Entries outside
 * [0, num_pages) are never written and read as zeros.  Lengths, validation,
 * updates and results are those of kivi_ragged_cache: each sequence is
 * bit-identical to the same sequence in a ragged (contiguous) cache. */
typedef struct {
  kivi_shape shape;
  int32_t page_tokens;
  int32_t num_pages;
  uint32_t* k_codes;
  void* k_scale;
  void* k_zero;
  uint32_t* v_codes;
  void* v_scale;
  void* v_zero;
  uint16_t* k_res;
  uint16_t* v_res;
  const int32_t* block_table;   /* device [batch][capacity / page_tokens] */
  int32_t* tq;                  /* host [batch] */
  int32_t* tr;                  /* host [batch] */
  uint32_t* k_outliers;         /* pool, shape.outliers > 0 only */
} kivi_paged_cache;

/* Bytes of each page pool for a shape, page size and page count (host
 * arithmetic only).  KIVI_OK, or a shape error. */
int kivi_paged_pool_bytes(const kivi_shape* shape, int32_t page_tokens,
                          int32_t num_pages, size_t* k_codes, size_t* k_meta,
                          size_t* v_codes, size_t* v_meta);

/* The kivi_ragged_* calls on a paged store (same arguments and rules). */
int kivi_paged_prefill(kivi_paged_cache* cache, const uint16_t* k,
                       const uint16_t* v, int32_t in_tok_stride,
                       const int32_t* ntok, const int32_t* tq, void* stream);
int kivi_paged_append(kivi_paged_cache* cache, const uint16_t* k_new,
                      const uint16_t* v_new, void* stream);
int kivi_paged_decode_auto_splits(const kivi_paged_cache* cache);
int kivi_paged_decode_attn(const kivi_paged_cache* cache, const uint16_t* q,
                           float softmax_scale, uint16_t* out, void* workspace,
                           size_t workspace_bytes, int32_t num_splits,
                           void* stream);
int kivi_paged_append_decode_attn(kivi_paged_cache* cache,
                                  const uint16_t* k_new, const uint16_t* v_new,
                                  const uint16_t* q, float softmax_scale,
                                  uint16_t* out, void* workspace,
                                  size_t workspace_bytes, int32_t num_splits,
                                  void* stream);

/* Short static description of a status code. */
const char* kivi_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */

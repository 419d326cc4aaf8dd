// C ABI entry points: argument validation (before any HIP call), launch
// configuration and the host-side cache lengths.  See include/kivi.h.
#include "kivi.h"

#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kivi_internal.h"

namespace {

using kivi::DecodeArgs;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// KIVI_EHIP for a failed HIP call; with the environment variable KIVI_DEBUG
// set, the HIP error's name goes to stderr first (the status code alone does
// not say which HIP error it was)
int hip_fail(hipError_t e, const char* where) {
  static const bool verbose = getenv("KIVI_DEBUG") != nullptr;
  if (verbose) fprintf(stderr, "kivi: %s: %s\n", where, hipGetErrorName(e));
  return KIVI_EHIP;
}

int check_shape(const kivi_shape* s) {
  if (!s) return KIVI_EINVAL;
  if (s->batch < 1 || s->num_kv_heads < 1 || s->gqa_ratio < 1) return KIVI_EINVAL;
  if (s->bits < 1 || s->bits > 4) return KIVI_EINVAL;
  if (s->meta_half != 0 && s->meta_half != 1) return KIVI_EINVAL;
  if (s->outliers < 0 || s->outliers > 8) return KIVI_EINVAL;   // (< every group size)
  if (!(s->rope_theta >= 0.f) || isinf(s->rope_theta)) return KIVI_EINVAL;
  if (s->deterministic != 0 && s->deterministic != 1) return KIVI_EINVAL;
  if (s->v_window != 0 && s->v_window != 1) return KIVI_EINVAL;
  const int D = s->head_dim, G = s->group;
  if (!(D == 32 || D == 64 || D == 128 || D == 256)) return KIVI_EUNSUPPORTED;
  if (!(G == 32 || G == 64 || G == 128)) return KIVI_EUNSUPPORTED;
  if (s->gqa_ratio > 16) return KIVI_EUNSUPPORTED;
  if (D % G != 0) return KIVI_ESHAPE;
  if (s->residual < G || s->residual % G != 0) return KIVI_ESHAPE;
  if (s->capacity < 0 || s->capacity % 64 != 0 || s->capacity % G != 0) return KIVI_ESHAPE;
  // 32-bit index arithmetic bound on one (b, h) plane of codes
  if ((int64_t)s->capacity * D > (int64_t)1 << 31) return KIVI_ESHAPE;
  return KIVI_OK;
}

int check_cache(const kivi_cache* c) {
  if (!c) return KIVI_EINVAL;
  int rc = check_shape(&c->shape);
  if (rc) return rc;
  const void* ptrs[] = {c->k_codes, c->k_scale, c->k_zero, c->v_codes,
                        c->v_scale, c->v_zero,  c->k_res,  c->v_res};
  for (const void* p : ptrs)
    if (!p) return KIVI_EINVAL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return KIVI_EALIGN;
  const kivi_shape& s = c->shape;
  if (s.outliers > 0 && !c->k_outliers) return KIVI_EINVAL;
  if (s.outliers > 0 && !aligned16(c->k_outliers)) return KIVI_EALIGN;
  if (c->tq < 0 || c->tq % s.group != 0 || c->tr < 0 || c->tr > s.residual)
    return KIVI_ESHAPE;
  if (c->tq > s.capacity) return KIVI_ECAPACITY;
  return KIVI_OK;
}

int check_quantize(const kivi_shape* s, const uint16_t* x, int32_t in_stride, int32_t ntok,
                   int32_t dst, const uint32_t* codes, const void* scale, const void* zero) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!x || !codes || !scale || !zero) return KIVI_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scale) || !aligned16(zero))
    return KIVI_EALIGN;
  if (ntok < 1 || ntok % s->group != 0 || dst < 0 || dst % s->group != 0 || in_stride < ntok)
    return KIVI_ESHAPE;
  if ((int64_t)dst + ntok > s->capacity) return KIVI_ECAPACITY;
  return KIVI_OK;
}

std::atomic<int> g_cu_count[64];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -KIVI_EHIP;
  if (dev < 64) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return -KIVI_EHIP;
  if (dev < 64) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Largest split count the automatic choice can return for a shape: a split
// count beyond 2048 (b, h) blocks buys nothing on a 256-CU device.
int max_auto_splits(const kivi_shape& s) {
  const int units = s.batch * s.num_kv_heads;
  return units >= 2048 ? 1 : (2048 + units - 1) / units;
}

// the matrix-core kernel takes the shape (its whole-tile part with the value
// window)
bool mfma_shape(const kivi_shape& s) {
  return kivi::decode_mfma_supported(s.head_dim, s.group, s.gqa_ratio, s.outliers,
                                     s.rope_theta > 0.f);
}
// the matrix-core kernel runs the whole decode (with the value window, the
// generic kernel takes the tokens whose values are in the window)
bool use_mfma(const kivi_shape& s) {
  return !s.v_window && kivi::decode_mfma_supported(s.head_dim, s.group, s.gqa_ratio, s.outliers,
                                     s.rope_theta > 0.f);
}

// waves per block of the matrix-core decode kernel
int mfma_waves() {
  static const int nw = [] {
    const char* e = getenv("KIVI_DECODE_WAVES");   // tuning override: 4 or 8
    int v = e ? atoi(e) : 8;
    return v >= 8 ? 8 : 4;
  }();
  return nw;
}

int auto_splits_for(const kivi_shape& s, int tq, int tr, int cus, bool mfma) {
  const int units = s.batch * s.num_kv_heads;
  const int L = tq + tr;
  int S;
  if (mfma) {
    // one round of blocks: as many splits as fill the resident block slots,
    // keeping at least two 64-token tiles per wave
    const int nw = kivi::decode_mfma_block_waves(s.gqa_ratio, mfma_waves());
    const int slots = cus * kivi::decode_mfma_blocks_per_cu(s.bits, s.gqa_ratio, mfma_waves());
    S = slots / units;
    const int by_work = ((tq + 63) / 64) / (2 * nw);
    if (S > by_work) S = by_work;
  } else {
    // about two blocks per compute unit, at least 256 tokens a split
    const int want = (2 * cus + units - 1) / units;
    const int by_len = (L + 255) / 256;
    S = want < by_len ? want : by_len;
  }
  if (S < 1) S = 1;
  const int cap = max_auto_splits(s);
  return S > cap ? cap : S;
}
int auto_splits(const kivi_shape& s, int tq, int tr, int cus) {
  return auto_splits_for(s, tq, tr, cus, use_mfma(s));
}

// The decode's plan at lengths (tq, tr): S_run splits of the main launch and
// S_ws partial slots per query row (1: the launch writes fp16 output).  With
// the value window, t_tiles whole 64-token tiles below max(0, L - R) (their
// keys and values quantized) go to the matrix-core kernel in S_run splits
// and the rest of the tokens (R to R + 63 of them) to the generic kernel as
// kMaxTailSplits more partials; t_tiles = 0 when the matrix-core kernel does
// not take the shape or no whole tile is there.  The device count is needed
// (KIVI_EHIP without one) only for an automatic split count.
// (One tail partial: its kernel takes the whole tail in one block per plane;
// on the generic kernel a step of the batch-8 Llama layer took 130 us with
// one and 169 us with up to eight splits of about 16 tokens each.)
constexpr int kMaxTailSplits = 1;
int tail_splits(int) { return kMaxTailSplits; }
int decode_plan(const kivi_shape& s, int tq, int tr, int num_splits, int* S_run, int* S_ws,
                int* t_tiles) {
  const int L = tq + tr, tv = L > s.residual ? L - s.residual : 0;
  *t_tiles = s.v_window && mfma_shape(s) ? tv / 64 * 64 : 0;
  int S = num_splits;
  if (S == 0) {
    const int cus = device_cu_count();
    if (cus < 0) return KIVI_EHIP;
    S = *t_tiles > 0 ? auto_splits_for(s, *t_tiles, 0, cus, true) : auto_splits(s, tq, tr, cus);
  }
  *S_run = S;
  *S_ws = *t_tiles > 0 ? S + tail_splits(L - *t_tiles) : S;
  return KIVI_OK;
}

size_t ws_bytes(const kivi_shape& s, int S) {
  if (S <= 1) return 0;
  const size_t rows = (size_t)s.batch * s.num_kv_heads * s.gqa_ratio;
  return rows * (size_t)S * (size_t)(s.head_dim + 2) * sizeof(float);
}

// A codec job writing into a cache's grouped store (sources, counts and the
// residual of a copy set by the caller).
kivi::QuantJob store_job(const kivi_shape& s, uint32_t* k_codes, void* k_scale, void* k_zero,
                         uint32_t* v_codes, void* v_scale, void* v_zero, uint32_t* k_out) {
  kivi::QuantJob j{};
  j.k_codes = k_codes;
  j.k_scale = k_scale;
  j.k_zero = k_zero;
  j.v_codes = v_codes;
  j.v_scale = v_scale;
  j.v_zero = v_zero;
  j.k_out = s.outliers > 0 ? k_out : nullptr;
  j.n_out = s.outliers;
  j.H = s.num_kv_heads;
  j.D = s.head_dim;
  j.G = s.group;
  j.cap = s.capacity;
  j.R = s.residual;
  return j;
}
kivi::QuantJob cache_job(const kivi_cache* c) {
  kivi::QuantJob j = store_job(c->shape, c->k_codes, c->k_scale, c->k_zero, c->v_codes,
                               c->v_scale, c->v_zero, c->k_outliers);
  j.k_res = c->k_res;
  j.v_res = c->v_res;
  return j;
}
// the flush of a full residual into tokens [tq, tq + R): keys and values in
// one launch
hipError_t launch_flush(const kivi_cache* c, int tq, hipStream_t st) {
  const kivi_shape& s = c->shape;
  kivi::QuantJob j = cache_job(c);
  j.k = c->k_res;
  j.v = c->v_res;
  j.in_stride = s.residual;
  j.do_k = j.do_v = 1;
  j.nq = s.residual;
  j.dst_off = tq;
  j.ncopy = 0;
  return kivi::launch_quantize_kv(j, s.bits, s.meta_half, s.batch, st);
}

// ---- value window (shape.v_window) ------------------------------------------
// Values keep the R newest tokens in v_res (token t in slot t % R); a value
// leaving the window is quantized by itself; keys follow the lazy flush.

// copies tokens [t0, t0 + n) of one tensor src ([B][H][stride][D]) into the
// window slots t % R of dst
hipError_t copy_window(const kivi_shape& s, const uint16_t* src, int stride, int t0, int n,
                       uint16_t* dst, hipStream_t st) {
  const int R = s.residual;
  while (n > 0) {
    const int slot = t0 % R, m = n < R - slot ? n : R - slot;
    hipError_t e = kivi::launch_copy_tokens(nullptr, src, stride, t0, nullptr, dst, R, slot, m,
                                            s.batch, s.num_kv_heads, s.head_dim, st);
    if (e != hipSuccess) return e;
    t0 += m;
    n -= m;
  }
  return hipSuccess;
}

// prefill: keys as without the window; values [0, ntok - R) quantized (whole
// 32-token chunks by the codec launch, the rest one token at a time), the
// newest min(ntok, R) values into the window
hipError_t prefill_window(const kivi_cache* c, const uint16_t* k, const uint16_t* v, int ntok,
                          int tq, hipStream_t st) {
  const kivi_shape& s = c->shape;
  const int tv = ntok > s.residual ? ntok - s.residual : 0, tv32 = tv / 32 * 32;
  hipError_t e = hipSuccess;
  if (tq > 0) {
    kivi::QuantJob j = cache_job(c);
    j.k = k;
    j.v = v;
    j.in_stride = ntok;
    j.do_k = 1;
    j.do_v = 0;
    j.nq = tq;
    j.dst_off = 0;
    j.ncopy = 0;
    if ((e = kivi::launch_quantize_kv(j, s.bits, s.meta_half, s.batch, st)) != hipSuccess)
      return e;
  }
  if (tv32 > 0) {
    kivi::QuantJob j = cache_job(c);
    j.k = k;
    j.v = v;
    j.in_stride = ntok;
    j.do_k = 0;
    j.do_v = 1;
    j.nq = tv32;
    j.dst_off = 0;
    j.ncopy = 0;
    if ((e = kivi::launch_quantize_kv(j, s.bits, s.meta_half, s.batch, st)) != hipSuccess)
      return e;
  }
  if ((e = kivi::launch_quantize_v_tokens(cache_job(c), s.bits, s.meta_half, s.batch, v, ntok,
                                          tv32, tv32, tv - tv32, st)) != hipSuccess)
    return e;
  if (ntok > tq &&
      (e = kivi::launch_copy_tokens(k, nullptr, ntok, tq, c->k_res, nullptr, s.residual, 0,
                                    ntok - tq, s.batch, s.num_kv_heads, s.head_dim, st)) !=
          hipSuccess)
    return e;
  return copy_window(s, v, ntok, tv, ntok - tv, c->v_res, st);
}

// lengths after a window append (the capacity checked), without any HIP call
int window_append_lengths(const kivi_cache* c, int* tq, int* tr) {
  const kivi_shape& s = c->shape;
  const int R = s.residual, L = c->tq + c->tr;
  const bool flush = c->tr == R;
  if (flush && (int64_t)c->tq + R > s.capacity) return KIVI_ECAPACITY;
  if (L >= R && L - R >= s.capacity) return KIVI_ECAPACITY;
  *tq = c->tq + (flush ? R : 0);
  *tr = (flush ? 0 : c->tr) + 1;
  return KIVI_OK;
}

// enqueues a window append (lengths already checked): the key flush when the
// key residual is full, the value leaving the window (token L - R, slot
// L % R) into the value store, then the new key and value
hipError_t append_window(const kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                         hipStream_t st) {
  const kivi_shape& s = c->shape;
  const int R = s.residual, L = c->tq + c->tr;
  const bool flush = c->tr == R;
  hipError_t e = hipSuccess;
  if (flush) {
    kivi::QuantJob j = cache_job(c);
    j.k = c->k_res;
    j.v = c->v_res;
    j.in_stride = R;
    j.do_k = 1;
    j.do_v = 0;
    j.nq = R;
    j.dst_off = c->tq;
    j.ncopy = 0;
    if ((e = kivi::launch_quantize_kv(j, s.bits, s.meta_half, s.batch, st)) != hipSuccess)
      return e;
  }
  // one launch: the leaving value (if any) quantized from its window slot,
  // then the new key and value written into their slots
  return kivi::launch_quantize_v_tokens(cache_job(c), s.bits, s.meta_half, s.batch, c->v_res,
                                        R, L % R, L - R, L >= R ? 1 : 0, st, k_new,
                                        flush ? 0 : c->tr, v_new, L % R);
}

// ---- ragged batches and the paged store -------------------------------------
// Both carry per-sequence host lengths; the paged store also a page map.  The
// calls below work on this common view.

struct Rg {
  const kivi_shape* s;
  uint32_t* k_codes;
  void* k_scale;
  void* k_zero;
  uint32_t* v_codes;
  void* v_scale;
  void* v_zero;
  uint16_t* k_res;
  uint16_t* v_res;
  int32_t* tq;
  int32_t* tr;
  bool paged;
  kivi::PageMap pm;   // paged: pools of pm.num_pages pages, device table [batch][max_pages]
  uint32_t* k_out;    // key outliers (shape.outliers > 0)
};

Rg view(const kivi_ragged_cache* c) {
  return Rg{&c->shape, c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero,
            c->k_res,  c->v_res,   c->tq,      c->tr,      false,      kivi::PageMap{nullptr, 0, 0, 0, 0},
            c->k_outliers};
}
Rg view(const kivi_paged_cache* c) {
  const int P = c->page_tokens > 0 ? c->page_tokens : 1;
  int shift = 0;
  while ((1 << shift) < P) shift++;
  return Rg{&c->shape, c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero,
            c->k_res,  c->v_res,   c->tq,      c->tr,      true,
            kivi::PageMap{c->block_table, c->page_tokens, c->shape.capacity / P, c->num_pages,
                          shift},
            c->k_outliers};
}

// buffers present and aligned, length arrays present (shape already checked)
int check_buffers(const Rg& g) {
  if (g.s->v_window) return KIVI_EUNSUPPORTED;   // (uniform caches only)
  const void* ptrs[] = {g.k_codes, g.k_scale, g.k_zero, g.v_codes,
                        g.v_scale, g.v_zero,  g.k_res,  g.v_res};
  for (const void* p : ptrs)
    if (!p) return KIVI_EINVAL;
  if (!g.tq || !g.tr) return KIVI_EINVAL;
  if (g.paged && !g.pm.table) return KIVI_EINVAL;
  if (g.s->outliers > 0 && !g.k_out) return KIVI_EINVAL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return KIVI_EALIGN;
  if (g.s->outliers > 0 && !aligned16(g.k_out)) return KIVI_EALIGN;
  if (g.paged && (reinterpret_cast<uintptr_t>(g.pm.table) & 3u)) return KIVI_EALIGN;
  return KIVI_OK;
}

int check_lengths(const Rg& g) {
  const kivi_shape& s = *g.s;
  for (int b = 0; b < s.batch; b++) {
    const int tq = g.tq[b], tr = g.tr[b];
    if (tq < 0 || tq % s.group != 0 || tr < 0 || tr > s.residual) return KIVI_ESHAPE;
    if (tq > s.capacity) return KIVI_ECAPACITY;
  }
  return KIVI_OK;
}

// page size and pool: P a power of two, at least 64 and the group, capacity
// a multiple of P, at least one page, page slices addressable with 32 bits
int check_pages(const kivi_paged_cache* c) {
  const kivi_shape& s = c->shape;
  const int P = c->page_tokens;
  if (P < 64 || (P & (P - 1)) != 0 || P % s.group != 0) return KIVI_ESHAPE;
  if (s.capacity % P != 0) return KIVI_ESHAPE;
  if (c->num_pages < 1) return KIVI_ESHAPE;
  if ((int64_t)P * s.head_dim > (int64_t)1 << 31) return KIVI_ESHAPE;
  return KIVI_OK;
}

int check_ragged(const kivi_ragged_cache* c) {
  if (!c) return KIVI_EINVAL;
  int rc = check_shape(&c->shape);
  if (rc) return rc;
  const Rg g = view(c);
  if ((rc = check_buffers(g))) return rc;
  return check_lengths(g);
}

int check_paged(const kivi_paged_cache* c) {
  if (!c) return KIVI_EINVAL;
  int rc = check_shape(&c->shape);
  if (rc) return rc;
  if ((rc = check_pages(c))) return rc;
  const Rg g = view(c);
  if ((rc = check_buffers(g))) return rc;
  return check_lengths(g);
}

// per-(b, h) plane extents of the contiguous cache buffers
struct PlaneSizes {
  size_t code_words, kmeta_bytes, vmeta_bytes, res_elems, kout_words;
};
PlaneSizes plane_sizes(const kivi_shape& s) {
  const size_t cap = s.capacity, D = s.head_dim, G = s.group, mb = s.meta_half ? 2 : 4;
  return {cap * D * s.bits / 32, (cap / G) * D * mb, cap * (D / G) * mb, (size_t)s.residual * D,
          (cap / G) * (size_t)s.outliers * D};
}

// Runs `launch(list)` over the items added with `add`, kMaxSeq at a time.
template <class F>
struct ListBatcher {
  kivi::SeqList list;
  F launch;
  int rc = KIVI_OK;
  explicit ListBatcher(F f) : launch(f) { list.n = 0; }
  void add(int seq, int a, int b, int c) {
    if (rc) return;
    list.seq[list.n] = seq;
    list.a[list.n] = a;
    list.b[list.n] = b;
    list.c[list.n] = c;
    if (++list.n == kivi::kMaxSeq) flush();
  }
  int flush() {
    if (!rc && list.n) rc = launch(list);
    list.n = 0;
    return rc;
  }
};
template <class F>
ListBatcher<F> batcher(F f) { return ListBatcher<F>(f); }

// One codec launch over list items of src ([batch][H][in_stride][D]) into the
// grouped store (contiguous planes, or the pages of the table): item i
// quantizes a[i] tokens of K and V of sequence seq[i] into its tokens
// [b[i], b[i] + a[i]) and copies the next c[i] tokens into its residual.
int enqueue_quantize_list(const Rg& g, const uint16_t* k_src, const uint16_t* v_src,
                          int in_stride, int ntok_max, int ncopy_max, const kivi::SeqList& L,
                          hipStream_t st) {
  const kivi_shape& s = *g.s;
  kivi::QuantJob j = store_job(s, g.k_codes, g.k_scale, g.k_zero, g.v_codes, g.v_scale,
                               g.v_zero, g.k_out);
  j.k = k_src;
  j.v = v_src;
  j.in_stride = in_stride;
  j.do_k = j.do_v = 1;
  j.nq = ntok_max;
  j.k_res = g.k_res;
  j.v_res = g.v_res;
  hipError_t e = g.paged ? kivi::launch_quantize_kv_paged(j, L, g.pm, s.bits, s.meta_half,
                                                          ncopy_max, st)
                         : kivi::launch_quantize_kv_list(j, L, s.bits, s.meta_half, ncopy_max,
                                                         st);
  return e == hipSuccess ? KIVI_OK : hip_fail(e, __func__);
}

// Quantizes the full residual of every sequence whose residual holds R tokens
// into its grouped store at tq[b] (the lazy flush).
int enqueue_ragged_flush(const Rg& g, hipStream_t st) {
  const kivi_shape& s = *g.s;
  const int R = s.residual;
  auto fl = batcher([&](const kivi::SeqList& L) {
    return enqueue_quantize_list(g, g.k_res, g.v_res, R, R, 0, L, st);
  });
  for (int b = 0; b < s.batch; b++)
    if (g.tr[b] == R) fl.add(b, R, g.tq[b], 0);
  return fl.flush();
}

// Writes token row b of k_new / v_new into residual slot slot[b].
int enqueue_ragged_token_copy(const Rg& g, const uint16_t* k_new, const uint16_t* v_new,
                              const std::vector<int>& slot, hipStream_t st) {
  const kivi_shape& s = *g.s;
  auto cp = batcher([&](const kivi::SeqList& L) {
    hipError_t e = kivi::launch_copy_tokens_list(k_new, v_new, 1, g.k_res, g.v_res, s.residual, L,
                                                 1, s.num_kv_heads, s.head_dim, st);
    return e == hipSuccess ? KIVI_OK : hip_fail(e, __func__);
  });
  for (int b = 0; b < s.batch; b++) cp.add(b, 0, slot[b], 1);
  return cp.flush();
}

// A validated ragged decode: split count and the lengths to decode at.
struct RaggedPlan {
  int S;
  std::vector<int> tq, tr;
};

int plan_ragged_decode(const Rg& g, std::vector<int> tq, std::vector<int> tr, const uint16_t* q,
                       uint16_t* out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                       RaggedPlan* plan) {
  if (!q || !out) return KIVI_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return KIVI_EALIGN;
  if (num_splits < 0) return KIVI_EINVAL;
  if (num_splits > KIVI_MAX_SPLITS) return KIVI_ESHAPE;
  const kivi_shape& s = *g.s;
  int max_tq = 0, max_tr = 0;
  for (int b = 0; b < s.batch; b++) {
    if (tq[b] + tr[b] < 1) return KIVI_ESHAPE;
    max_tq = std::max(max_tq, tq[b]);
    max_tr = std::max(max_tr, tr[b]);
  }
  int S = num_splits;
  if (S == 0) {
    const int cus = device_cu_count();
    if (cus < 0) return KIVI_EHIP;
    S = auto_splits(s, max_tq, max_tr, cus);
  }
  if (S > 1) {
    if (workspace_bytes < ws_bytes(s, S)) return KIVI_EWORKSPACE;
    if (!workspace) return KIVI_EINVAL;
    if (!aligned16(workspace)) return KIVI_EALIGN;
  }
  plan->S = S;
  plan->tq = std::move(tq);
  plan->tr = std::move(tr);
  return KIVI_OK;
}

// Decode launches over chunks of at most kMaxSeq sequences: query, output,
// residual and workspace pointers offset to the chunk, and either the
// contiguous cache planes or the block-table rows too; lengths by value.
int enqueue_ragged_decode(const Rg& g, const RaggedPlan& p, const uint16_t* q,
                          float softmax_scale, uint16_t* out, void* workspace,
                          const uint16_t* k_new, const uint16_t* v_new, hipStream_t st) {
  const kivi_shape& s = *g.s;
  const PlaneSizes ps = plane_sizes(s);
  const int H = s.num_kv_heads, r = s.gqa_ratio, D = s.head_dim, S = p.S;
  for (int c0 = 0; c0 < s.batch; c0 += kivi::kMaxSeq) {
    const int n = std::min(kivi::kMaxSeq, s.batch - c0);
    const size_t pl = (size_t)c0 * H;   // first plane of the chunk
    const size_t cp = g.paged ? 0 : pl; // first cache plane (pools are shared)
    DecodeArgs a;
    a.k_codes = g.k_codes + cp * ps.code_words;
    a.k_scale = static_cast<const char*>(g.k_scale) + cp * ps.kmeta_bytes;
    a.k_zero = static_cast<const char*>(g.k_zero) + cp * ps.kmeta_bytes;
    a.v_codes = g.v_codes + cp * ps.code_words;
    a.v_scale = static_cast<const char*>(g.v_scale) + cp * ps.vmeta_bytes;
    a.v_zero = static_cast<const char*>(g.v_zero) + cp * ps.vmeta_bytes;
    a.k_res = g.k_res + pl * ps.res_elems;
    a.v_res = g.v_res + pl * ps.res_elems;
    a.k_new = k_new ? k_new + pl * D : nullptr;
    a.v_new = v_new ? v_new + pl * D : nullptr;
    a.q = q + pl * r * D;
    a.out = out + pl * r * D;
    a.ws = S > 1 ? static_cast<float*>(workspace) + pl * r * (size_t)S * (D + 2) : nullptr;
    a.B = n;
    a.H = H;
    a.r = r;
    a.D = D;
    a.bits = s.bits;
    a.G = s.group;
    a.R = s.residual;
    a.cap = s.capacity;
    a.pages = g.pm;
    if (g.paged) a.pages.table = g.pm.table + (size_t)c0 * g.pm.max_pages;
    kivi::SeqLens lens;
    int mq = 0, mr = 0;
    for (int i = 0; i < n; i++) {
      lens.tq[i] = p.tq[c0 + i];
      lens.tr[i] = p.tr[c0 + i];
      mq = std::max(mq, lens.tq[i]);
      mr = std::max(mr, lens.tr[i]);
    }
    // longest sequences first (dispatch order; ties keep the batch order)
    for (int i = 0; i < n; i++) lens.order[i] = i;
    std::stable_sort(lens.order, lens.order + n, [&](int x, int y) {
      return lens.tq[x] + lens.tr[x] > lens.tq[y] + lens.tr[y];
    });
    a.tq = mq;   // (unused by the per-sequence kernels)
    a.tr = mr;
    a.S = S;
    a.mh = s.meta_half;
    a.scale = softmax_scale;
    a.k_out = s.outliers > 0 ? g.k_out + cp * ps.kout_words : nullptr;
    a.n_out = s.outliers;
    a.rope_theta = s.rope_theta;
    a.share_tiles = s.deterministic ? 0 : 1;
    a.vwin = 0;
    a.t_begin = 0;
    a.ws_stride = S;
    a.ws_slot0 = 0;
    hipError_t e;
    if (use_mfma(s))
      e = g.paged ? kivi::launch_decode_mfma_paged(a, lens, mfma_waves(), st)
                  : kivi::launch_decode_mfma_ragged(a, lens, mfma_waves(), st);
    else
      e = g.paged ? kivi::launch_decode_generic_paged(a, lens, st)
                  : kivi::launch_decode_generic_ragged(a, lens, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
    if (S > 1) {
      e = kivi::launch_combine(a, st);
      if (e != hipSuccess) return hip_fail(e, __func__);
    }
  }
  return KIVI_OK;
}

// lengths after appending one token to every sequence; false on overflow
bool ragged_after_append(const Rg& g, std::vector<int>& tq, std::vector<int>& tr,
                         std::vector<int>& slot) {
  const kivi_shape& s = *g.s;
  tq.resize(s.batch);
  tr.resize(s.batch);
  slot.resize(s.batch);
  for (int b = 0; b < s.batch; b++) {
    const bool flush = g.tr[b] == s.residual;
    if (flush && (int64_t)g.tq[b] + s.residual > s.capacity) return false;
    tq[b] = g.tq[b] + (flush ? s.residual : 0);
    slot[b] = flush ? 0 : g.tr[b];
    tr[b] = slot[b] + 1;
  }
  return true;
}

// The call bodies shared by the ragged and the paged entry points (arguments
// of the cache already validated).
int do_prefill(const Rg& g, const uint16_t* k, const uint16_t* v, int32_t in_tok_stride,
               const int32_t* ntok, const int32_t* tq, hipStream_t st) {
  if (!k || !v || !ntok || !tq) return KIVI_EINVAL;
  if (!aligned16(k) || !aligned16(v)) return KIVI_EALIGN;
  const kivi_shape& s = *g.s;
  if (in_tok_stride < 1) return KIVI_ESHAPE;
  for (int b = 0; b < s.batch; b++) {
    if (ntok[b] < 0 || ntok[b] > in_tok_stride || tq[b] < 0 || tq[b] % s.group != 0 ||
        ntok[b] < tq[b] || ntok[b] - tq[b] > s.residual)
      return KIVI_ESHAPE;
    if (tq[b] > s.capacity) return KIVI_ECAPACITY;
  }
  int max_tq = 0, max_n = 0;
  for (int b = 0; b < s.batch; b++) {
    max_tq = std::max(max_tq, (int)tq[b]);
    max_n = std::max(max_n, (int)(ntok[b] - tq[b]));
  }
  // one launch: each sequence's prefix quantized, its tail copied
  auto qz = batcher([&](const kivi::SeqList& L) {
    return enqueue_quantize_list(g, k, v, in_tok_stride, max_tq, max_n, L, st);
  });
  for (int b = 0; b < s.batch; b++)
    if (ntok[b] > 0) qz.add(b, tq[b], 0, ntok[b] - tq[b]);
  int rc = qz.flush();
  if (rc) return rc;
  for (int b = 0; b < s.batch; b++) {
    g.tq[b] = tq[b];
    g.tr[b] = ntok[b] - tq[b];
  }
  return KIVI_OK;
}

int do_append(const Rg& g, const uint16_t* k_new, const uint16_t* v_new, hipStream_t st) {
  if (!k_new || !v_new) return KIVI_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_EALIGN;
  std::vector<int> tq, tr, slot;
  if (!ragged_after_append(g, tq, tr, slot)) return KIVI_ECAPACITY;
  int rc = enqueue_ragged_flush(g, st);
  if (rc) return rc;
  if ((rc = enqueue_ragged_token_copy(g, k_new, v_new, slot, st))) return rc;
  for (int b = 0; b < g.s->batch; b++) {
    g.tq[b] = tq[b];
    g.tr[b] = tr[b];
  }
  return KIVI_OK;
}

int do_auto_splits(const Rg& g) {
  const int cus = device_cu_count();
  if (cus < 0) return cus;
  int max_tq = 0, max_tr = 0;
  for (int b = 0; b < g.s->batch; b++) {
    max_tq = std::max(max_tq, (int)g.tq[b]);
    max_tr = std::max(max_tr, (int)g.tr[b]);
  }
  return auto_splits(*g.s, max_tq, max_tr, cus);
}

int do_decode(const Rg& g, const uint16_t* q, float softmax_scale, uint16_t* out,
              void* workspace, size_t workspace_bytes, int32_t num_splits, hipStream_t st) {
  RaggedPlan p;
  const int B = g.s->batch;
  int rc = plan_ragged_decode(g, std::vector<int>(g.tq, g.tq + B), std::vector<int>(g.tr, g.tr + B),
                              q, out, workspace, workspace_bytes, num_splits, &p);
  if (rc) return rc;
  return enqueue_ragged_decode(g, p, q, softmax_scale, out, workspace, nullptr, nullptr, st);
}

int do_append_decode(const Rg& g, const uint16_t* k_new, const uint16_t* v_new,
                     const uint16_t* q, float softmax_scale, uint16_t* out, void* workspace,
                     size_t workspace_bytes, int32_t num_splits, hipStream_t st) {
  if (!k_new || !v_new) return KIVI_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_EALIGN;
  std::vector<int> tq, tr, slot;
  if (!ragged_after_append(g, tq, tr, slot)) return KIVI_ECAPACITY;
  RaggedPlan p;
  int rc = plan_ragged_decode(g, tq, tr, q, out, workspace, workspace_bytes, num_splits, &p);
  if (rc) return rc;
  if ((rc = enqueue_ragged_flush(g, st))) return rc;
  const bool fused = use_mfma(*g.s);
  if (!fused && (rc = enqueue_ragged_token_copy(g, k_new, v_new, slot, st))) return rc;
  rc = enqueue_ragged_decode(g, p, q, softmax_scale, out, workspace, fused ? k_new : nullptr,
                             fused ? v_new : nullptr, st);
  if (rc) return rc;
  for (int b = 0; b < g.s->batch; b++) {
    g.tq[b] = tq[b];
    g.tr[b] = tr[b];
  }
  return KIVI_OK;
}

}  // namespace

extern "C" {

const char* kivi_strerror(int status) {
  switch (status) {
    case KIVI_OK: return "ok";
    case KIVI_EINVAL: return "invalid argument (null pointer, bits, or count)";
    case KIVI_ESHAPE: return "inconsistent sizes";
    case KIVI_EALIGN: return "buffer not 16-byte aligned";
    case KIVI_ECAPACITY: return "quantized store capacity exceeded";
    case KIVI_EWORKSPACE: return "decode workspace too small";
    case KIVI_EUNSUPPORTED: return "unsupported head_dim / group / gqa_ratio";
    case KIVI_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int kivi_cache_bytes(const kivi_shape* s, size_t* k_codes, size_t* k_meta, size_t* v_codes,
                     size_t* v_meta, size_t* residual, size_t* query) {
  int rc = check_shape(s);
  if (rc) return rc;
  const size_t planes = (size_t)s->batch * s->num_kv_heads;
  const size_t cap = s->capacity, D = s->head_dim, G = s->group;
  const size_t codes = planes * cap * D * s->bits / 8;
  if (k_codes) *k_codes = codes;
  if (v_codes) *v_codes = codes;
  const size_t mb = s->meta_half ? 2 : sizeof(float);
  if (k_meta) *k_meta = planes * (cap / G) * D * mb;
  if (v_meta) *v_meta = planes * cap * (D / G) * mb;
  if (residual) *residual = planes * (size_t)s->residual * D * 2;
  if (query) *query = planes * (size_t)s->gqa_ratio * D * 2;
  return KIVI_OK;
}

int kivi_outlier_bytes(const kivi_shape* s, int32_t page_tokens, int32_t num_pages,
                       size_t* bytes) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!bytes) return KIVI_EINVAL;
  size_t slices = (size_t)s->batch * s->num_kv_heads, tokens = s->capacity;
  if (page_tokens != 0) {
    kivi_paged_cache c{};
    c.shape = *s;
    c.page_tokens = page_tokens;
    c.num_pages = num_pages;
    if ((rc = check_pages(&c))) return rc;
    slices = (size_t)num_pages * s->num_kv_heads;
    tokens = page_tokens;
  }
  *bytes = slices * (tokens / s->group) * (size_t)s->outliers * s->head_dim * 4;
  return KIVI_OK;
}

int kivi_quantize_k(const kivi_shape* s, const uint16_t* k, int32_t in_tok_stride, int32_t ntok,
                    int32_t dst, uint32_t* codes, void* scale, void* zero, void* stream) {
  int rc = check_quantize(s, k, in_tok_stride, ntok, dst, codes, scale, zero);
  if (rc) return rc;
  if (s->outliers != 0) return KIVI_EINVAL;   // kivi_quantize_k_outliers
  kivi::QuantJob j = store_job(*s, codes, scale, zero, nullptr, nullptr, nullptr, nullptr);
  j.k = k;
  j.in_stride = in_tok_stride;
  j.do_k = 1;
  j.nq = ntok;
  j.dst_off = dst;
  hipError_t e = kivi::launch_quantize_kv(j, s->bits, s->meta_half, s->batch,
                                          (hipStream_t)stream);
  return e == hipSuccess ? KIVI_OK : hip_fail(e, __func__);
}

int kivi_quantize_k_outliers(const kivi_shape* s, const uint16_t* k, int32_t in_tok_stride,
                             int32_t ntok, int32_t dst, uint32_t* codes, void* scale, void* zero,
                             uint32_t* outliers, void* stream) {
  int rc = check_quantize(s, k, in_tok_stride, ntok, dst, codes, scale, zero);
  if (rc) return rc;
  if (s->outliers < 1 || !outliers) return KIVI_EINVAL;
  if (!aligned16(outliers)) return KIVI_EALIGN;
  kivi::QuantJob j = store_job(*s, codes, scale, zero, nullptr, nullptr, nullptr, outliers);
  j.k = k;
  j.in_stride = in_tok_stride;
  j.do_k = 1;
  j.nq = ntok;
  j.dst_off = dst;
  hipError_t e = kivi::launch_quantize_kv(j, s->bits, s->meta_half, s->batch,
                                          (hipStream_t)stream);
  return e == hipSuccess ? KIVI_OK : hip_fail(e, __func__);
}

int kivi_quantize_v(const kivi_shape* s, const uint16_t* v, int32_t in_tok_stride, int32_t ntok,
                    int32_t dst, uint32_t* codes, void* scale, void* zero, void* stream) {
  int rc = check_quantize(s, v, in_tok_stride, ntok, dst, codes, scale, zero);
  if (rc) return rc;
  kivi::QuantJob j = store_job(*s, nullptr, nullptr, nullptr, codes, scale, zero, nullptr);
  j.v = v;
  j.in_stride = in_tok_stride;
  j.do_v = 1;
  j.nq = ntok;
  j.dst_off = dst;
  hipError_t e = kivi::launch_quantize_kv(j, s->bits, s->meta_half, s->batch,
                                          (hipStream_t)stream);
  return e == hipSuccess ? KIVI_OK : hip_fail(e, __func__);
}

int kivi_prefill(kivi_cache* c, const uint16_t* k, const uint16_t* v, int32_t ntok, int32_t tq,
                 void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!k || !v) return KIVI_EINVAL;
  if (!aligned16(k) || !aligned16(v)) return KIVI_EALIGN;
  const kivi_shape& s = c->shape;
  if (ntok < 1 || tq < 0 || tq % s.group != 0 || ntok - tq < 0 || ntok - tq > s.residual)
    return KIVI_ESHAPE;
  if (tq > s.capacity) return KIVI_ECAPACITY;
  if (s.v_window) {
    if (ntok > s.capacity + s.residual) return KIVI_ECAPACITY;
    hipError_t e = prefill_window(c, k, v, ntok, tq, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, __func__);
    c->tq = tq;
    c->tr = ntok - tq;
    return KIVI_OK;
  }
  // one launch: tokens [0, tq) quantized, [tq, ntok) copied into the residual
  kivi::QuantJob j = cache_job(c);
  j.k = k;
  j.v = v;
  j.in_stride = ntok;
  j.do_k = j.do_v = 1;
  j.nq = tq;
  j.dst_off = 0;
  j.ncopy = ntok - tq;
  hipError_t e = kivi::launch_quantize_kv(j, s.bits, s.meta_half, s.batch, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, __func__);
  c->tq = tq;
  c->tr = ntok - tq;
  return KIVI_OK;
}

int kivi_append(kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new, void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!k_new || !v_new) return KIVI_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_EALIGN;
  const kivi_shape& s = c->shape;
  hipStream_t st = (hipStream_t)stream;
  int tq = c->tq, tr = c->tr;
  if (s.v_window) {
    if ((rc = window_append_lengths(c, &tq, &tr))) return rc;
    hipError_t e = append_window(c, k_new, v_new, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
    c->tq = tq;
    c->tr = tr;
    return KIVI_OK;
  }
  if (tr == s.residual) {
    if ((int64_t)tq + s.residual > s.capacity) return KIVI_ECAPACITY;
    // flush: the full residual becomes the next quantized tokens; the copy
    // below is enqueued after, so slot 0 is read before it is overwritten
    hipError_t e = launch_flush(c, tq, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
    tq += s.residual;
    tr = 0;
  }
  hipError_t e = kivi::launch_copy_tokens(k_new, v_new, 1, 0, c->k_res, c->v_res, s.residual,
                                          tr, 1, s.batch, s.num_kv_heads, s.head_dim, st);
  if (e != hipSuccess) return hip_fail(e, __func__);
  c->tq = tq;
  c->tr = tr + 1;
  return KIVI_OK;
}

int kivi_decode_auto_splits(const kivi_cache* c) {
  int rc = check_cache(c);
  if (rc) return -rc;
  int S = 0, S_ws = 0, t_tiles = 0;
  if ((rc = decode_plan(c->shape, c->tq, c->tr, 0, &S, &S_ws, &t_tiles))) return -rc;
  return S;
}

size_t kivi_decode_workspace_bytes(const kivi_shape* s, int32_t num_splits) {
  if (check_shape(s) != KIVI_OK || num_splits < 0 || num_splits > KIVI_MAX_SPLITS) return 0;
  const int S = num_splits == 0 ? max_auto_splits(*s) : num_splits;
  // (the value window may need kMaxTailSplits more partial slots: its tail)
  return ws_bytes(*s, s->v_window ? S + kMaxTailSplits : S);
}

// Checks a decode at lengths (tq, tr) and fills the launch arguments; no HIP
// call except the (cached) compute-unit count.
static int prepare_decode(const kivi_cache* c, int tq, int tr, const uint16_t* q,
                          float softmax_scale, uint16_t* out, void* workspace,
                          size_t workspace_bytes, int32_t num_splits, DecodeArgs* a) {
  if (!q || !out) return KIVI_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return KIVI_EALIGN;
  if (num_splits < 0) return KIVI_EINVAL;
  const kivi_shape& s = c->shape;
  const int L = tq + tr;
  if (L < 1) return KIVI_ESHAPE;
  if (num_splits > 0 && (num_splits > L || num_splits > KIVI_MAX_SPLITS)) return KIVI_ESHAPE;
  int S = 0, S_ws = 0, t_tiles = 0;
  int rc = decode_plan(s, tq, tr, num_splits, &S, &S_ws, &t_tiles);
  if (rc) return rc;
  if (S_ws > 1) {
    if (workspace_bytes < ws_bytes(s, S_ws)) return KIVI_EWORKSPACE;
    if (!workspace) return KIVI_EINVAL;
    if (!aligned16(workspace)) return KIVI_EALIGN;
  }
  a->k_codes = c->k_codes;
  a->k_scale = c->k_scale;
  a->k_zero = c->k_zero;
  a->v_codes = c->v_codes;
  a->v_scale = c->v_scale;
  a->v_zero = c->v_zero;
  a->k_res = c->k_res;
  a->v_res = c->v_res;
  a->k_new = nullptr;
  a->v_new = nullptr;
  a->q = q;
  a->out = out;
  a->ws = static_cast<float*>(workspace);
  a->B = s.batch;
  a->H = s.num_kv_heads;
  a->r = s.gqa_ratio;
  a->D = s.head_dim;
  a->bits = s.bits;
  a->G = s.group;
  a->R = s.residual;
  a->cap = s.capacity;
  a->tq = tq;
  a->tr = tr;
  a->S = S;
  a->mh = s.meta_half;
  a->scale = softmax_scale;
  a->pages = kivi::PageMap{nullptr, 0, 0, 0, 0};
  a->k_out = s.outliers > 0 ? c->k_outliers : nullptr;
  a->n_out = s.outliers;
  a->rope_theta = s.rope_theta;
  a->share_tiles = s.deterministic ? 0 : 1;
  a->vwin = s.v_window;
  a->t_begin = t_tiles;      // (the value window's whole-tile part, when any)
  a->ws_stride = S_ws;
  a->ws_slot0 = 0;
  return KIVI_OK;
}

static int enqueue_decode(const kivi_shape& s, const DecodeArgs& a, hipStream_t st) {
  hipError_t e;
  if (s.v_window && a.t_begin > 0) {
    // value window: whole tiles [0, t_begin) on the matrix cores (keys and
    // values quantized, no residual) in slots [0, S), the tail [t_begin, L)
    // on the generic kernel in slots [S, ws_stride), then the combine over
    // all ws_stride slots
    DecodeArgs m = a;
    m.tq = a.t_begin;
    m.tr = 0;
    m.vwin = 0;
    m.t_begin = 0;
    if ((e = kivi::launch_decode_mfma(m, mfma_waves(), st)) != hipSuccess)
      return hip_fail(e, __func__);
    DecodeArgs g = a;
    g.S = a.ws_stride - a.S;
    g.ws_slot0 = a.S;
    if (kivi::window_tail_supported(s.head_dim, s.group, s.gqa_ratio, s.outliers,
                                    s.rope_theta > 0.f)) {
      // (the tail kernel merges every partial and writes the output itself)
      if ((e = kivi::launch_window_tail(g, st)) != hipSuccess) return hip_fail(e, __func__);
      return KIVI_OK;
    }
    if ((e = kivi::launch_decode_generic(g, st)) != hipSuccess) return hip_fail(e, __func__);
  } else {
    e = use_mfma(s) ? kivi::launch_decode_mfma(a, mfma_waves(), st)
                    : kivi::launch_decode_generic(a, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
  }
  if (a.ws_stride > 1) {
    e = kivi::launch_combine(a, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
  }
  return KIVI_OK;
}

int kivi_decode_attn(const kivi_cache* c, const uint16_t* q, float softmax_scale, uint16_t* out,
                     void* workspace, size_t workspace_bytes, int32_t num_splits,
                     void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  DecodeArgs a;
  rc = prepare_decode(c, c->tq, c->tr, q, softmax_scale, out, workspace, workspace_bytes,
                      num_splits, &a);
  if (rc) return rc;
  return enqueue_decode(c->shape, a, (hipStream_t)stream);
}

int kivi_append_decode_attn(kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                            const uint16_t* q, float softmax_scale, uint16_t* out,
                            void* workspace, size_t workspace_bytes, int32_t num_splits,
                            void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (!k_new || !v_new) return KIVI_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_EALIGN;
  const kivi_shape& s = c->shape;
  if (s.v_window) {
    // the window append's launches, then the decode at the new lengths
    int tq2 = 0, tr2 = 0;
    if ((rc = window_append_lengths(c, &tq2, &tr2))) return rc;
    DecodeArgs a;
    rc = prepare_decode(c, tq2, tr2, q, softmax_scale, out, workspace, workspace_bytes,
                        num_splits, &a);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = append_window(c, k_new, v_new, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
    if ((rc = enqueue_decode(s, a, st))) return rc;
    c->tq = tq2;
    c->tr = tr2;
    return KIVI_OK;
  }
  // lengths after the append (a full residual is flushed first)
  const bool flush = c->tr == s.residual;
  if (flush && (int64_t)c->tq + s.residual > s.capacity) return KIVI_ECAPACITY;
  const int tq = c->tq + (flush ? s.residual : 0);
  const int slot = flush ? 0 : c->tr;     // residual slot of the new token
  DecodeArgs a;
  rc = prepare_decode(c, tq, slot + 1, q, softmax_scale, out, workspace, workspace_bytes,
                      num_splits, &a);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (flush) {
    hipError_t e = launch_flush(c, c->tq, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
  }
  if (use_mfma(s)) {
    // the decode kernel reads the new token from its input rows and writes it
    // into the residual slot itself
    a.k_new = k_new;
    a.v_new = v_new;
  } else {
    hipError_t e = kivi::launch_copy_tokens(k_new, v_new, 1, 0, c->k_res, c->v_res,
                                            s.residual, slot, 1, s.batch, s.num_kv_heads,
                                            s.head_dim, st);
    if (e != hipSuccess) return hip_fail(e, __func__);
  }
  rc = enqueue_decode(s, a, st);
  if (rc) return rc;
  c->tq = tq;
  c->tr = slot + 1;
  return KIVI_OK;
}

// ---- decode without a caller workspace ----------------------------------------
// The split-K partials of kivi_decode_attn_noalloc live in this file-scope
// device array: every GPU the library runs on holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address is taken
// once per device with hipGetSymbolAddress and kept per device.
static __device__ __align__(256) float scratch[KIVI_SCRATCH_BYTES / sizeof(float)];

static std::atomic<void*> g_scratch_ptr[64];

// device address of this device's copy of `scratch`, or nullptr on a HIP error
static void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

int kivi_decode_attn_noalloc(const kivi_cache* c, const uint16_t* q, float softmax_scale,
                             uint16_t* out, int32_t num_splits, void* stream) {
  int rc = check_cache(c);
  if (rc) return rc;
  if (num_splits < 0) return KIVI_EINVAL;
  const int L = c->tq + c->tr;
  if (L < 1) return KIVI_ESHAPE;
  if (num_splits > 0 && (num_splits > L || num_splits > KIVI_MAX_SPLITS)) return KIVI_ESHAPE;
  // the split count's partials must fit the array (checked before any HIP
  // call when num_splits is given)
  int S = 0, S_ws = 0, t_tiles = 0;
  if ((rc = decode_plan(c->shape, c->tq, c->tr, num_splits, &S, &S_ws, &t_tiles))) return rc;
  if (ws_bytes(c->shape, S_ws) > (size_t)KIVI_SCRATCH_BYTES) return KIVI_EWORKSPACE;
  void* ws = S_ws > 1 ? scratch_address() : nullptr;
  if (S_ws > 1 && !ws) return KIVI_EHIP;
  DecodeArgs a;
  rc = prepare_decode(c, c->tq, c->tr, q, softmax_scale, out, ws,
                      S_ws > 1 ? KIVI_SCRATCH_BYTES : 0, S, &a);
  if (rc) return rc;
  return enqueue_decode(c->shape, a, (hipStream_t)stream);
}

// ---- ragged batches ---------------------------------------------------------

int kivi_ragged_prefill(kivi_ragged_cache* c, const uint16_t* k, const uint16_t* v,
                        int32_t in_tok_stride, const int32_t* ntok, const int32_t* tq,
                        void* stream) {
  if (!c) return KIVI_EINVAL;
  int rc = check_shape(&c->shape);
  if (rc) return rc;
  const Rg g = view(c);
  if ((rc = check_buffers(g))) return rc;
  return do_prefill(g, k, v, in_tok_stride, ntok, tq, (hipStream_t)stream);
}

int kivi_ragged_append(kivi_ragged_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                       void* stream) {
  int rc = check_ragged(c);
  if (rc) return rc;
  return do_append(view(c), k_new, v_new, (hipStream_t)stream);
}

int kivi_ragged_decode_auto_splits(const kivi_ragged_cache* c) {
  int rc = check_ragged(c);
  if (rc) return -rc;
  return do_auto_splits(view(c));
}

int kivi_ragged_decode_attn(const kivi_ragged_cache* c, const uint16_t* q, float softmax_scale,
                            uint16_t* out, void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream) {
  int rc = check_ragged(c);
  if (rc) return rc;
  return do_decode(view(c), q, softmax_scale, out, workspace, workspace_bytes, num_splits,
                   (hipStream_t)stream);
}

int kivi_ragged_append_decode_attn(kivi_ragged_cache* c, const uint16_t* k_new,
                                   const uint16_t* v_new, const uint16_t* q, float softmax_scale,
                                   uint16_t* out, void* workspace, size_t workspace_bytes,
                                   int32_t num_splits, void* stream) {
  int rc = check_ragged(c);
  if (rc) return rc;
  return do_append_decode(view(c), k_new, v_new, q, softmax_scale, out, workspace,
                          workspace_bytes, num_splits, (hipStream_t)stream);
}

// ---- paged store -------------------------------------------------------------

int kivi_paged_pool_bytes(const kivi_shape* s, int32_t page_tokens, int32_t num_pages,
                          size_t* k_codes, size_t* k_meta, size_t* v_codes, size_t* v_meta) {
  int rc = check_shape(s);
  if (rc) return rc;
  kivi_paged_cache c{};
  c.shape = *s;
  c.page_tokens = page_tokens;
  c.num_pages = num_pages;
  if ((rc = check_pages(&c))) return rc;
  const size_t slices = (size_t)num_pages * s->num_kv_heads;
  const size_t P = page_tokens, D = s->head_dim, G = s->group, mb = s->meta_half ? 2 : 4;
  if (k_codes) *k_codes = slices * P * D * s->bits / 8;
  if (v_codes) *v_codes = slices * P * D * s->bits / 8;
  if (k_meta) *k_meta = slices * (P / G) * D * mb;
  if (v_meta) *v_meta = slices * P * (D / G) * mb;
  return KIVI_OK;
}

int kivi_paged_prefill(kivi_paged_cache* c, const uint16_t* k, const uint16_t* v,
                       int32_t in_tok_stride, const int32_t* ntok, const int32_t* tq,
                       void* stream) {
  if (!c) return KIVI_EINVAL;
  int rc = check_shape(&c->shape);
  if (rc) return rc;
  if ((rc = check_pages(c))) return rc;
  const Rg g = view(c);
  if ((rc = check_buffers(g))) return rc;
  return do_prefill(g, k, v, in_tok_stride, ntok, tq, (hipStream_t)stream);
}

int kivi_paged_append(kivi_paged_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                      void* stream) {
  int rc = check_paged(c);
  if (rc) return rc;
  return do_append(view(c), k_new, v_new, (hipStream_t)stream);
}

int kivi_paged_decode_auto_splits(const kivi_paged_cache* c) {
  int rc = check_paged(c);
  if (rc) return -rc;
  return do_auto_splits(view(c));
}

int kivi_paged_decode_attn(const kivi_paged_cache* c, const uint16_t* q, float softmax_scale,
                           uint16_t* out, void* workspace, size_t workspace_bytes,
                           int32_t num_splits, void* stream) {
  int rc = check_paged(c);
  if (rc) return rc;
  return do_decode(view(c), q, softmax_scale, out, workspace, workspace_bytes, num_splits,
                   (hipStream_t)stream);
}

int kivi_paged_append_decode_attn(kivi_paged_cache* c, const uint16_t* k_new,
                                  const uint16_t* v_new, const uint16_t* q, float softmax_scale,
                                  uint16_t* out, void* workspace, size_t workspace_bytes,
                                  int32_t num_splits, void* stream) {
  int rc = check_paged(c);
  if (rc) return rc;
  return do_append_decode(view(c), k_new, v_new, q, softmax_scale, out, workspace,
                          workspace_bytes, num_splits, (hipStream_t)stream);
}

}  // extern "C"

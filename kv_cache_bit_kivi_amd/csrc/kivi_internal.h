// Internal declarations shared by the library's translation units.
// Not part of the public ABI (see include/kivi.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace kivi {

// Sequences handled by one launch over per-sequence lengths (larger batches
// are split into launches of at most this many sequences).
constexpr int kMaxSeq = 128;

// Per-sequence lengths of one ragged decode launch, passed by value: the
// sequences b = 0 .. B-1 of the launch (pointers already offset to them).
// order[] lists the sequences longest first: the blocks are dispatched in
// index order, so taking sequence order[i] for the i-th group of blocks
// starts the longest work first and lets the short work fill in behind it.
struct SeqLens {
  int tq[kMaxSeq];
  int tr[kMaxSeq];
  int order[kMaxSeq];
};

// A list of per-sequence work items, passed by value: item i works on
// sequence seq[i] of the launch's batch with three integer parameters whose
// meaning is the launcher's (documented there).
struct SeqList {
  int n;
  int seq[kMaxSeq];
  int a[kMaxSeq];
  int b[kMaxSeq];
  int c[kMaxSeq];
};

// Paged quantized store: the quantized tokens of sequence b, head h live in
// pages of `page_tokens` tokens drawn from a pool of `num_pages` pages; page
// p holds every head, and its (p, h) slice has the layout of a contiguous
// plane of capacity page_tokens.  Logical token t of sequence b is token
// t % page_tokens of page table[b * max_pages + t / page_tokens].  Entries
// outside [0, num_pages) read as zeros and are never written.
struct PageMap {
  const int* table;   // device [batch][max_pages]
  int page_tokens, max_pages, num_pages;
  int page_shift;     // log2(page_tokens): page sizes are powers of two
};

// (slice plane, token inside it) of logical token t of (sequence b, head h):
// the contiguous plane b*H + h itself, or the page slice holding t.  Returns
// false for a page outside the pool.  The table is read through the constant
// address space so that a wave-uniform lookup is a scalar load.
__device__ __forceinline__ bool page_slot(const PageMap& pm, int b, int h, int H, int t,
                                          size_t& plane, int& tok) {
  const __attribute__((address_space(4))) int* tbl =
      (const __attribute__((address_space(4))) int*)pm.table;
  const int pg = tbl[(size_t)b * pm.max_pages + (t >> pm.page_shift)];
  plane = (size_t)pg * H + h;
  tok = t & (pm.page_tokens - 1);
  return pg >= 0 && pg < pm.num_pages;
}

// Device pointers and lengths of one decode call.
struct DecodeArgs {
  const uint32_t* k_codes;
  const void* k_scale;   // float, or binary16 bits when mh
  const void* k_zero;
  const uint32_t* v_codes;
  const void* v_scale;
  const void* v_zero;
  const uint16_t* k_res;
  const uint16_t* v_res;
  // fused append: the token in residual slot tr - 1 is read from these rows
  // ([B][Hkv][D]) and written into the residual by the kernel; null otherwise
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* q;
  uint16_t* out;
  float* ws;          // split partials: m, l [rows][S], o [rows][S][D]
  int B, H, r, D, bits, G, R, cap, tq, tr, S;
  int mh;             // metadata stored as binary16 (1) or binary32 (0)
  float scale;
  PageMap pages;      // paged launches only (table null otherwise)
  // key outliers: n_out words per (key group, channel), [plane][cap/G][n_out][D]
  // (page slices [slice][P/G][n_out][D]); null when n_out == 0
  const uint32_t* k_out;
  int n_out;
  // > 0: the cached keys are pre-RoPE; decode rotates each key at its token
  // index (rotate-half pairs (i, i + D/2), frequency rope_theta^(-2i/D))
  float rope_theta;
  // 1: the waves of a block share its tiles in load-return order (matrix-core
  // kernel); 0: fixed per-wave runs (reproducible)
  int share_tiles;
  // 1: value sliding window (generic kernel): values [0, max(0, L - R))
  // quantized, value token t >= that in v_res slot t % R
  int vwin;
  // generic kernel: first token of the launch's range [t_begin, tq + tr)
  int t_begin;
  // split partials: ws_stride slots per query row, this launch's splits at
  // slots ws_slot0 .. ws_slot0 + S - 1 (ws_stride == 1: fp16 output instead)
  int ws_stride, ws_slot0;
};

// Kernel parameter of the decode kernels: nothing (uniform lengths, taken
// from DecodeArgs) or the launch's per-sequence lengths.
struct NoLens {};
template <bool RAG>
using LensT = std::conditional_t<RAG, SeqLens, NoLens>;
// lengths of sequence b of the launch
template <bool RAG>
__device__ __forceinline__ int seq_tq(const DecodeArgs& a, const LensT<RAG>& l, int b) {
  if constexpr (RAG) return l.tq[b]; else return a.tq;
}
template <bool RAG>
__device__ __forceinline__ int seq_tr(const DecodeArgs& a, const LensT<RAG>& l, int b) {
  if constexpr (RAG) return l.tr[b]; else return a.tr;
}
// (b, h) plane of the i-th group of blocks (i = sequence-major plane index)
template <bool RAG>
__device__ __forceinline__ int seq_plane(const LensT<RAG>& l, int i, int H) {
  if constexpr (RAG) return l.order[i / H] * H + i % H; else return i;
}

// Launchers: validate nothing (the C ABI layer did), return hipError_t of the
// launch.

// One launch of the codec (a prefill, a flush, or a quantize call): keys
// and/or values of `nq` source tokens ([*][H][in_stride][D], tokens
// [0, nq)) into destination tokens [dst_off, dst_off + nq) of the grouped
// store, and a copy of source tokens [nq, nq + ncopy) into residual slots
// [0, ncopy).  nq is a multiple of G (and of 32 for values).  Key outliers:
// n_out words per key group and channel into k_out (0: no isolation).
// List launches take nq, dst_off and ncopy per item (a[i], b[i], c[i]) and
// use the job's nq as the largest item's count.
struct QuantJob {
  const uint16_t* k;
  const uint16_t* v;
  int in_stride;
  int do_k, do_v;
  int nq, dst_off, ncopy;
  uint16_t* k_res;
  uint16_t* v_res;
  int R;
  uint32_t* k_codes;
  void* k_scale;      // float, or binary16 bits when metadata is half width
  void* k_zero;
  uint32_t* v_codes;
  void* v_scale;
  void* v_zero;
  uint32_t* k_out;
  int n_out;
  int H, D, G, cap;
};
hipError_t launch_quantize_kv(const QuantJob& j, int bits, int mh, int B, hipStream_t st);
// per-sequence items (the paged form writes quantized tokens into the page
// slices the table names; pm.page_tokens is the slice capacity, j.cap unused)
hipError_t launch_quantize_kv_list(const QuantJob& j, const SeqList& list, int bits, int mh,
                                   int ncopy_max, hipStream_t st);
hipError_t launch_quantize_kv_paged(const QuantJob& j, const SeqList& list, const PageMap& pm,
                                    int bits, int mh, int ncopy_max, hipStream_t st);
// Value window tail (decode tokens [a.t_begin, L) into split-K slot
// a.ws_slot0) for the shapes the dedicated kernel takes: D 128, G 32, no key
// outliers, no pre-RoPE keys, gqa ratio <= 8.
bool window_tail_supported(int D, int G, int r, int outliers, bool rope);
// (final: the kernel also merges split-K slots [0, a.ws_slot0), which the
// matrix-core launch before it wrote, with its own and writes the fp16
// output; no combine launch follows)
hipError_t launch_window_tail(const DecodeArgs& a, hipStream_t st);
// Value window: quantizes cache tokens [t0, t0 + n) of every (b, h) from
// source rows [src_row, src_row + n) of src ([B][H][src_stride][D]) into the
// value store of j (per-token groups; other tokens' code bits kept); with
// k_new (append: n <= 1), then writes the new token ([B][H][D] rows) into
// key-residual slot k_slot and window slot v_slot of j.k_res, j.v_res.
hipError_t launch_quantize_v_tokens(const QuantJob& j, int bits, int mh, int B,
                                    const uint16_t* src, int src_stride, int src_row, int t0,
                                    int n, hipStream_t st, const uint16_t* k_new = nullptr,
                                    int k_slot = 0, const uint16_t* v_new = nullptr,
                                    int v_slot = 0);
// Copies tokens [t0, t0 + n) of src ([B][H][src_stride][D]) into slots
// [slot0, slot0 + n) of dst ([B][H][dst_stride][D]), for K and V at once
// (a null source skips that tensor).
hipError_t launch_copy_tokens(const uint16_t* k_src, const uint16_t* v_src, int src_stride,
                              int t0, uint16_t* k_dst, uint16_t* v_dst, int dst_stride,
                              int slot0, int n, int B, int H, int D, hipStream_t st);
// Per-sequence copy: item i copies tokens [a[i], a[i] + c[i]) of sequence
// seq[i] of src into residual slots [b[i], b[i] + c[i]) (c[i] <= n_max).
hipError_t launch_copy_tokens_list(const uint16_t* k_src, const uint16_t* v_src, int src_stride,
                                   uint16_t* k_dst, uint16_t* v_dst, int dst_stride,
                                   const SeqList& list, int n_max, int H, int D, hipStream_t st);

// Generic decode kernel (any supported shape) + split combine.  The ragged
// variants take the launch's per-sequence lengths (a.tq / a.tr unused) and
// need every sequence to hold at least one token.
hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_generic_ragged(const DecodeArgs& a, const SeqLens& lens, hipStream_t st);
// paged store (a.pages; per-sequence lengths as in the ragged launch; the
// cache pointers are the pools, the sequence index b is the launch's
// sequence b0 + b with b0 = a.pages' row offset already applied to table)
hipError_t launch_decode_generic_paged(const DecodeArgs& a, const SeqLens& lens, hipStream_t st);
size_t decode_generic_lds_bytes(int r, int D);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t st);

// Matrix-core decode kernel: head_dim 128, group 32, gqa ratio 1, 2, 4 or 8,
// at most kMfmaMaxOutliers key outliers per group.
constexpr int kMfmaMaxOutliers = 2;
bool decode_mfma_supported(int D, int G, int r, int n_out, bool rope);
// nw: requested waves per block (4 or 8); the block size actually used
// for a gqa ratio r is decode_mfma_block_waves(r, nw)
hipError_t launch_decode_mfma(const DecodeArgs& a, int nw, hipStream_t st);
hipError_t launch_decode_mfma_ragged(const DecodeArgs& a, const SeqLens& lens, int nw,
                                     hipStream_t st);
hipError_t launch_decode_mfma_paged(const DecodeArgs& a, const SeqLens& lens, int nw,
                                    hipStream_t st);
int decode_mfma_block_waves(int r, int nw);
// The launches above for a.n_out = 1 or 2, one translation unit per
// variant family (called by the launchers above, not by the API layer).
hipError_t launch_decode_mfma_o1(const DecodeArgs& a, int nw, hipStream_t st);
hipError_t launch_decode_mfma_o2(const DecodeArgs& a, int nw, hipStream_t st);
hipError_t launch_decode_mfma_ragged_o(const DecodeArgs& a, const SeqLens& lens, int nw,
                                       hipStream_t st);
hipError_t launch_decode_mfma_paged_o(const DecodeArgs& a, const SeqLens& lens, int nw,
                                      hipStream_t st);
// ... and for pre-RoPE keys (a.rope_theta > 0, no outliers)
hipError_t launch_decode_mfma_rope(const DecodeArgs& a, int nw, hipStream_t st);
hipError_t launch_decode_mfma_ragged_rope(const DecodeArgs& a, const SeqLens& lens, int nw,
                                          hipStream_t st);
hipError_t launch_decode_mfma_paged_rope(const DecodeArgs& a, const SeqLens& lens, int nw,
                                         hipStream_t st);
// resident blocks per compute unit of that kernel variant (occupancy query)
int decode_mfma_blocks_per_cu(int bits, int r, int nw);

}  // namespace kivi

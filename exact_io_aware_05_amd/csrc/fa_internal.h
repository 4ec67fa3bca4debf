// Host-side launchers behind the C interface in fa.h.  Arguments are
// already validated; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct Shape {
  int B, Hq, Hkv, Nq, Nk, d;
  int causal;
  float scale;
  // sliding window around each query's place c = i + Nk - Nq on the key
  // axis: keys c - win_left .. c + win_right; -1 is no bound on that side
  int win_left = -1, win_right = -1;
};

// The mask of a Shape as the kernels take it: kind 0 none, 1 causal, 2 a
// band of keys c - wl .. c + wr around each row's place c = i + Nk - Nq.
// A bound that no row reaches past (wl >= Nk - 1, wr >= Nq - 1: every key
// lies on its visible side for every row) is no bound; the causal flag
// caps wr at 0; without a left bound the mask is causal (wr 0) or none.
// A band's bounds are returned capped at those values (Nk - 1, Nq - 1),
// which hides the same keys and keeps the key span of a row tile tight.
struct MaskBounds {
  int kind, wl, wr;
};
inline MaskBounds mask_bounds(const Shape& s) {
  const int big = s.Nq + s.Nk;
  int wl = s.win_left < 0 ? big : (s.win_left < big ? s.win_left : big);
  int wr = s.win_right < 0 ? big : (s.win_right < big ? s.win_right : big);
  if (s.causal) wr = 0;
  const bool left_free = wl >= s.Nk - 1;
  const bool right_free = wr >= s.Nq - 1;
  if (left_free && right_free) return {0, 0, 0};
  if (left_free && wr == 0) return {1, 0, 0};
  return {2, left_free ? s.Nk - 1 : wl, right_free ? s.Nq - 1 : wr};
}

// Blocks of `kb` keys that the band of one 32-row tile of the KV-split
// form can span, for sizing its chunks.  The tile's packed rows (G query
// heads per query) cover queries a / G .. (a + 31) / G, at most 31 / G + 2
// of them, so it sees at most 31 / G + 1 + wl + wr + 1 consecutive keys,
// which span at most span / kb + 2 blocks.
inline int band_tile_blocks(const Shape& s, const MaskBounds& m, int kb) {
  const int G = s.Hq / s.Hkv;
  const int nblk = (s.Nk + kb - 1) / kb;
  if (m.kind != 2) return nblk;
  const long long span = 31 / G + 2 + (long long)m.wl + m.wr;
  const long long blocks = (span < s.Nk ? span : s.Nk) / kb + 2;
  return blocks < nblk ? (int)blocks : nblk;
}

// Where the rows of one (sequence, head) live, in elements: batch, head and
// row strides of Q, K, V, O and of lse.  Fixed-length batches have cu_q =
// cu_k = nullptr.  Packed variable-length batches take sequence b's rows
// from cu_q[b] .. cu_q[b + 1] (and cu_k for K/V), the batch strides unused;
// Nq / Nk of the Shape are then the maximum lengths and total_q / total_k
// the row counts of the packed tensors.  Fixed-length batches may give each
// sequence its own key count, seqlen_k[b] (device, clamped to [0, Nk]; the
// rows past it are never read).  A paged cache (the paged instances of the
// prefill kernel) keeps key row r of sequence b in row r % page_size of
// page page_table[b][r / page_size], rows k_r elements apart across pages
// too, head h at h * k_h; k_b and v_b are then 0.
struct SeqLayout {
  long long q_b, q_h, q_r;
  long long k_b, k_h, k_r;
  long long l_b, l_h, l_r;
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int n_seq;  // sequences of a packed batch (cu_q, cu_k: n_seq + 1 entries)
  long long v_b, v_h, v_r;  // V (same as K unless given apart)
  long long o_b, o_h, o_r;  // O (same as Q unless given apart)
  const int* seqlen_k;      // per-sequence key counts, or nullptr
  const int* page_table;    // paged: [B, max_pages] page numbers
  int max_pages, page_shift, num_pages;  // page_size = 1 << page_shift
};

// V laid out like K and O like Q.
inline void same_vo(SeqLayout& l) {
  l.v_b = l.k_b;
  l.v_h = l.k_h;
  l.v_r = l.k_r;
  l.o_b = l.q_b;
  l.o_h = l.q_h;
  l.o_r = l.q_r;
}

// [B, H, N, d] contiguous tensors, lse [B, Hq, Nq].
inline SeqLayout dense_layout(const Shape& s) {
  SeqLayout l{};
  l.q_r = s.d;
  l.q_h = (long long)s.Nq * s.d;
  l.q_b = l.q_h * s.Hq;
  l.k_r = s.d;
  l.k_h = (long long)s.Nk * s.d;
  l.k_b = l.k_h * s.Hkv;
  l.l_r = 1;
  l.l_h = s.Nq;
  l.l_b = (long long)s.Hq * s.Nq;
  same_vo(l);
  return l;
}

// Rows of queries per prefill workgroup and keys per streamed K/V block.
constexpr int kPrefillRows = 256;
constexpr int kPrefillKeys = 64;
// Keys per block and query rows per wave in the KV-split kernel.
constexpr int kSplitKeys = 32;
constexpr int kSplitRows = 32;
constexpr int kMaxSplits = 4096;

// The tiled prefill kernel over the rows `lay` describes; a layout with a
// page table runs the paged instances (k and v are then the caches).
hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s,
                          const SeqLayout& lay, bool out_f32,
                          hipStream_t stream);

// Block-sparse mask of the prefill kernel: one byte per (block of
// kSparseRows query rows, block of kPrefillKeys keys), rows of nkb bytes;
// head h of batch b starts at mask + b * mb + h * mh (strides may be 0 to
// share a mask).  A zero byte skips the block.
constexpr int kSparseRows = 128;
constexpr int kSparseMaxKeyBlocks = 8191;  // the key-block list fills LDS
// Pages per sequence that the paged prefill form keeps in the same LDS
// list (one int per page); its pages hold whole 64-key blocks.
constexpr int kPagedPrefillMaxPages = 8192;
constexpr int kPagedPrefillMinPage = 64;
struct BlockMask {
  const uint8_t* mask;
  long long mb, mh;
  int nkb;
};

// Column-interval mask of the prefill kernel: key j of sequence b may be
// seen by the query rows bounds[2 (b mb + j)] .. bounds[2 (b mb + j) + 1]
// - 1 (int32 pairs, shared by the sequence's heads), on top of the causal
// flag.  A first kernel classifies each (sequence, 256-row query block, key
// block) once for all heads into `lists` (one int per key block, rows of
// lstride); each prefill workgroup then keeps the key blocks that any of
// its rows may see (at most kColMaxKeyBlocks) in an LDS list like a block
// mask's.  The LDS that the list gives up holds a ring of each listed
// block's bounds and per-wave visibility masks.
constexpr int kColMaxKeyBlocks = 6655;
struct ColMask {
  const int* bounds;
  long long mb;       // pairs between sequences
  int* lists;         // B * ceil(Nq / 256) rows of lstride ints (workspace)
  long long lstride;  // key blocks of 64 keys: ceil(Nk / 64)
};
// bytes of the classification rows of a column-mask call
size_t column_list_bytes(int B, int Nq, int Nk);

hipError_t launch_prefill_column(const void* q, const void* k, const void* v,
                                 void* o, float* lse, const Shape& s,
                                 const ColMask& cm, bool out_f32,
                                 hipStream_t stream);

hipError_t launch_prefill_sparse(const void* q, const void* k, const void* v,
                                 void* o, float* lse, const Shape& s,
                                 const BlockMask& bm, bool out_f32,
                                 hipStream_t stream);

// FP8 (E4M3) prefill, d = 128: q [B, Hq, Nq, d], k [B, Hkv, Nk, d], vt
// [B, Hkv, d, ldv] codes; descales per (batch, head) on the device.
hipError_t launch_prefill_fp8(const void* q, const void* k, const void* vt,
                              const float* q_descale, const float* k_descale,
                              const float* v_descale, void* o, float* lse,
                              const Shape& s, int ldv, bool out_f32,
                              hipStream_t stream);

hipError_t launch_splitkv(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s, bool out_f32,
                          int num_splits, void* workspace,
                          hipStream_t stream);

// A paged KV cache: k and v are [num_pages, page_size, Hkv, d]; sequence b
// owns pages table[b * max_pages + 0, 1, ...] in that order and its first
// seqlen[b] rows (clamped to max_pages * page_size); page numbers are
// clamped into [0, num_pages).  page_size is a power of two and a multiple
// of the 32-key block (a block never straddles two pages), and a chunk of
// the KV-split form spans fewer than 64 pages.  Shape::Nk is then
// max_pages * page_size.
struct PagedKv {
  const int* table;
  const int* seqlen;
  int max_pages, page_size, num_pages;
  int page_shift;  // log2(page_size)
};

// Most 32-key blocks per chunk for pages of `page_size` keys: a chunk of
// that many blocks holds the keys of 62 pages and, starting anywhere inside
// a page, touches at most 63 of them (the kernel keeps the chunk's page
// numbers one per lane of a wave).
inline int paged_max_blocks_per_chunk(int page_size) {
  return 62 * (page_size / kSplitKeys);
}

hipError_t launch_splitkv_paged(const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse,
                                const Shape& s, const PagedKv& pg,
                                bool out_f32, int num_splits, void* workspace,
                                hipStream_t stream);

// KV-split form over contiguous [B, Hkv, Nk, d] K/V of which sequence b
// uses its first seqlen[b] rows (clamped to [0, Nk]; Shape::Nk is the
// padded length).
hipError_t launch_splitkv_kvlen(const void* q, const void* k, const void* v,
                                void* o, float* lse, const Shape& s,
                                const int* seqlen, bool out_f32,
                                int num_splits, void* workspace,
                                hipStream_t stream);

size_t splitkv_workspace_bytes(long long rows, int d, int num_splits);

// Backward pass: D and lse * log2(e) per query row in `workspace`, then the
// dK/dV and dQ kernels.  `o` and `dout` are bf16.
hipError_t launch_backward(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, const Shape& s,
                           bool out_f32, void* workspace, hipStream_t stream);

size_t backward_workspace_bytes(long long rows);

}  // namespace fa

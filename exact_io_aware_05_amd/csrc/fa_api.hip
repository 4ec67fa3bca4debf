// C interface of the attention library (declared in include/fa.h):
// argument validation, choice between the prefill and KV-split forms,
// workspace handling and error reporting.  No HIP call happens before every
// argument check has passed.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = (int)e;
  return FA_ERR_HIP;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Head dimensions an entry point takes, as bit sets.  The prefill kernel
// runs d = 32 and 96 in its 64- and 128-column tiles (the columns past d
// masked) and d = 256 in a kernel of its own (dense layouts, optionally
// with per-sequence key counts); the KV-split kernel has instances for 32,
// 64, 128 and 256; fa_fwd and its variants take all five (d = 96 only in
// the prefill form); the backward kernels 64 and 128.
enum : unsigned { kD32 = 1, kD64 = 2, kD96 = 4, kD128 = 8, kD256 = 16 };
constexpr unsigned kDimsPrefill = kD32 | kD64 | kD96 | kD128;
constexpr unsigned kDimsAny = kDimsPrefill | kD256;
constexpr unsigned kDimsSplit = kD32 | kD64 | kD128 | kD256;
constexpr unsigned kDimsBwd = kD64 | kD128;

unsigned dim_bit(int d) {
  switch (d) {
    case 32: return kD32;
    case 64: return kD64;
    case 96: return kD96;
    case 128: return kD128;
    case 256: return kD256;
    default: return 0;
  }
}

// Checks shared by the entry points; pure host arithmetic.
int check_common(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                 int d, float scale, int out_dtype,
                 unsigned dims = kDimsPrefill) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1)
    return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (out_dtype != FA_OUT_BF16 && out_dtype != FA_OUT_F32)
    return FA_ERR_INVALID_ARG;
  if (!(dim_bit(d) & dims)) return FA_ERR_UNSUPPORTED;
  // element counts must stay well inside 64-bit offsets and 32-bit rows
  const long long rows_q = (long long)B * Hq * Nq;
  const long long rows_k = (long long)B * Hkv * Nk;
  if (rows_q > (1LL << 40) || rows_k > (1LL << 40)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Is the current device gfx950?  Cached per device id.
int check_device() {
  static int cache[64];  // 0 unknown, 1 supported, 2 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev >= 0 && dev < 64 && cache[dev]) return cache[dev] == 1 ? FA_OK : FA_ERR_UNSUPPORTED;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_status(e);
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cache[dev] = ok ? 1 : 2;
  return ok ? FA_OK : FA_ERR_UNSUPPORTED;
}

// Heuristic for the KV-split form: used when the packed query rows of one
// KV head (Nq * Hq / Hkv) are few (decode, short chunks); then enough chunks
// to give about 1024 waves (one per SIMD: the partial kernel holds its K/V
// prefetch ring in registers and runs one wave per SIMD), each with >= 4
// key blocks.
int default_splits(int B, int Hq, int Hkv, int Nq, int Nk) {
  const long long R = (long long)Nq * (Hq / Hkv);
  if (R > 64) return 0;
  const long long units = (long long)B * Hkv * ((R + fa::kSplitRows - 1) / fa::kSplitRows);
  const long long nblk = (Nk + fa::kSplitKeys - 1) / fa::kSplitKeys;
  long long s = (1024 + units - 1) / units;
  long long cap = nblk / 4;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > fa::kMaxSplits) s = fa::kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

// The chunk count of fa_fwd's choice for this shape (0: the prefill kernel;
// at d = 256 its own one-wave-per-SIMD kernel); d = 96 has only the prefill
// kernel.
int forward_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  int s = default_splits(B, Hq, Hkv, Nq, Nk);
  if (d == 96) s = 0;
  return s;
}

// Sizes the KV-split form cannot address (its wave count fits in an int).
bool splitkv_too_large(int B, int Hq, int Hkv, int Nq, int splits) {
  const long long rowtiles =
      ((long long)Nq * (Hq / Hkv) + fa::kSplitRows - 1) / fa::kSplitRows;
  return (long long)B * Hkv * rowtiles * splits > (1LL << 31) - 64;
}

constexpr int kMaxDevices = 64;

// ---- workspace of the KV-split form inside fa_fwd and fa_fwd_window, and
// of the column-mask classification inside fa_fwd_colmask
//
// One buffer per (device, stream), kept for the later calls on that stream:
// calls on one stream run in stream order, so each may reuse what the one
// before it used, and a call that needs more frees the old buffer and takes
// a larger one, both stream-ordered (hipFreeAsync / hipMallocAsync on the
// stream).  Taking and returning memory on every call cost about 50 us of
// host time per call on MI355X, more than the kernels of a short windowed
// decode.  (A stream handle is reused only once the destroyed stream's work
// has completed, so an entry never outlives the work that used it.)  Under
// graph capture, and past kMaxCachedStreams entries, a call takes its
// workspace with hipMallocAsync and returns it with hipFreeAsync, so that a
// captured graph owns its memory.
constexpr int kMaxCachedStreams = 32;
struct StreamWorkspace {
  int dev;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
std::mutex g_ws_mu;
StreamWorkspace g_ws[kMaxCachedStreams];
int g_ws_count = 0;

// Runs launch(ws) with a workspace of at least `bytes` bytes, taken as
// described above.
template <class F>
int with_workspace(hipStream_t stream, size_t bytes, F&& launch) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_status(e);
  if (cap == hipStreamCaptureStatusNone) {
    std::lock_guard<std::mutex> guard(g_ws_mu);
    int i = 0;
    while (i < g_ws_count && !(g_ws[i].dev == dev && g_ws[i].stream == stream))
      ++i;
    if (i < g_ws_count || g_ws_count < kMaxCachedStreams) {
      if (i == g_ws_count) g_ws[g_ws_count++] = {dev, stream, nullptr, 0};
      StreamWorkspace& w = g_ws[i];
      if (w.bytes < bytes) {
        if (w.ptr) {
          e = hipFreeAsync(w.ptr, stream);
          w.ptr = nullptr;
          w.bytes = 0;
          if (e != hipSuccess) return hip_status(e);
        }
        e = hipMallocAsync(&w.ptr, bytes, stream);
        if (e != hipSuccess) {
          w.ptr = nullptr;
          return hip_status(e);
        }
        w.bytes = bytes;
      }
      return hip_status(launch(w.ptr));
    }
  }
  void* ws = nullptr;
  e = hipMallocAsync(&ws, bytes, stream);
  if (e != hipSuccess) return hip_status(e);
  e = launch(ws);
  hipError_t e2 = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(e2);
}

// The KV-split form with its workspace as described above.
int run_splitkv(const void* q, const void* k, const void* v, void* o,
                float* lse, const fa::Shape& s, int splits, bool f32,
                hipStream_t stream) {
  const size_t bytes =
      fa::splitkv_workspace_bytes((long long)s.B * s.Hq * s.Nq, s.d, splits);
  return with_workspace(stream, bytes, [&](void* ws) {
    return fa::launch_splitkv(q, k, v, o, lse, s, f32, splits, ws, stream);
  });
}

// The prefill kernel (splits == 0) or the KV-split form.
int run_forward(const void* q, const void* k, const void* v, void* o,
                float* lse, const fa::Shape& s, int splits, bool f32,
                hipStream_t stream) {
  if (splits == 0)
    return hip_status(fa::launch_prefill(q, k, v, o, lse, s,
                                         fa::dense_layout(s), f32, stream));
  return run_splitkv(q, k, v, o, lse, s, splits, f32, stream);
}

// ---- scratch of the allocation-free entry point (fa_fwd_noalloc)
//
// The KV-split partials of one call live in this file-scope device array
// instead of memory taken per call.  Every GPU the library runs on holds its
// own copy until the process ends, at its own address: host code reaches it
// only through the pointer hipGetSymbolAddress returns with that device
// current (the array's name, used in host code, is a host-side stand-in and
// not a device address).  The partial kernel writes every (row, chunk) entry
// the merge kernel reads, so nothing needs clearing between calls; calls
// that overlap on one device (different streams) share the array and race.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch, looked up once per
// device.
int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported shape or device";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error (see fa_last_hip_error)";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: the call needs more scratch than the "
             "allocation-free entry point holds (fa_noalloc_scratch_bytes)";
    default: return "unknown fa status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

// The build passes the SHA-256 of its inputs; the marker lets a loader read
// it from the file without loading the library.
#ifndef FA_SOURCE_HASH
#define FA_SOURCE_HASH "unknown"
#endif
static const char kSourceHash[] = "FA_SOURCE_HASH=" FA_SOURCE_HASH;

const char* fa_source_hash(void) { return kSourceHash + 15; }

size_t fa_splitkv_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits) {
  if (B < 1 || Hq < 1 || Nq < 1 || d < 1 || num_splits < 1) return 0;
  return fa::splitkv_workspace_bytes((long long)B * Hq * Nq, d, num_splits);
}

int fa_default_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv) return 0;
  if (!dim_bit(d)) return 0;
  return forward_splits(B, Hq, Hkv, Nq, Nk, d);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int out_dtype, int num_splits,
                   void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype, kDimsSplit);
  if (st != FA_OK) return st;
  if (num_splits < 1 || num_splits > fa::kMaxSplits) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa::splitkv_workspace_bytes((long long)B * Hq * Nq, d,
                                                    num_splits))
    return FA_ERR_INVALID_ARG;
  // the partial kernel addresses one K or V head with 32-bit byte offsets
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  const long long rowtiles = ((long long)Nq * (Hq / Hkv) + fa::kSplitRows - 1) /
                             fa::kSplitRows;
  if ((long long)B * Hkv * rowtiles * num_splits > (1LL << 31) - 64)
    return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  return hip_status(fa::launch_splitkv(q, k, v, o, lse, s,
                                       out_dtype == FA_OUT_F32, num_splits,
                                       workspace, stream));
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
           float scale, int out_dtype, hipStream_t stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype, kDimsAny);
  if (st != FA_OK) return st;
  const int splits = forward_splits(B, Hq, Hkv, Nq, Nk, d);
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if (splits == 0 && (long long)B * Hq * qblk > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  if (splits > 0 && splitkv_too_large(B, Hq, Hkv, Nq, splits))
    return FA_ERR_UNSUPPORTED;
  // both kernels address one K/V head with 32-bit byte offsets
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  return run_forward(q, k, v, o, lse, s, splits, out_dtype == FA_OUT_F32,
                     stream);
}

size_t fa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int out_dtype, hipStream_t stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype, kDimsAny);
  if (st != FA_OK) return st;
  const int splits = forward_splits(B, Hq, Hkv, Nq, Nk, d);
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if (splits == 0 && (long long)B * Hq * qblk > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  if (splits > 0 && splitkv_too_large(B, Hq, Hkv, Nq, splits))
    return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  const size_t bytes =
      splits == 0 ? 0
                  : fa::splitkv_workspace_bytes((long long)B * Hq * Nq, d,
                                                splits);
  if (bytes > kNoAllocScratchBytes) return FA_ERR_TOO_LARGE;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  const bool f32 = out_dtype == FA_OUT_F32;
  if (splits == 0)
    return hip_status(fa::launch_prefill(q, k, v, o, lse, s,
                                         fa::dense_layout(s), f32, stream));
  void* ws = nullptr;
  st = scratch_on_device(&ws);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_splitkv(q, k, v, o, lse, s, f32, splits, ws,
                                       stream));
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o,
                  float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                  int causal, int window_left, int window_right, float scale,
                  int out_dtype, hipStream_t stream) {
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype, kDimsAny);
  if (st != FA_OK) return st;
  fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  s.win_left = window_left;
  s.win_right = window_right;
  // A bound that no query reaches past hides nothing (left >= Nk - 1,
  // right >= Nq - 1); what is left is no mask, the causal mask or a band.
  const fa::MaskBounds mb = fa::mask_bounds(s);
  if (mb.kind != 2)
    return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, mb.kind, scale,
                  out_dtype, stream);
  // the KV-split form when few query rows share a KV head, its chunks cut
  // from the keys a row tile's band can span
  const long long span =
      (long long)fa::band_tile_blocks(s, mb, fa::kSplitKeys) * fa::kSplitKeys;
  const int splits =
      forward_splits(B, Hq, Hkv, Nq, (int)(span < Nk ? span : Nk), d);
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if (splits == 0 && (long long)B * Hq * qblk > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  if (splits > 0 && splitkv_too_large(B, Hq, Hkv, Nq, splits))
    return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  return run_forward(q, k, v, o, lse, s, splits, out_dtype == FA_OUT_F32,
                     stream);
}

}  // extern "C" (reopened below)

namespace {

// Can a paged call run the prefill kernel?  Its 64-key blocks must lie
// inside one page (pages of at least 64 keys), a sequence's page numbers
// must fit the kernel's LDS list, and 64 rows of a page are addressed with
// 32-bit byte offsets.
bool paged_prefill_ok(int Hkv, int d, int page_size, int max_pages) {
  return (dim_bit(d) & kDimsPrefill) &&
         page_size >= fa::kPagedPrefillMinPage &&
         max_pages <= fa::kPagedPrefillMaxPages &&
         (long long)fa::kPrefillKeys * Hkv * d * 2 < (1LL << 31);
}

// The form a paged call with num_splits = 0 runs: 0 for the prefill kernel
// (many query rows per KV head, as fa_fwd decides, or d = 96), otherwise
// the KV-split form's chunk count (as fa_fwd would split a cache of the
// longest length, and enough chunks that none spans 64 pages); -1 when no
// form takes the shape.  Pure host arithmetic.
int paged_form(int B, int Hq, int Hkv, int Nq, int d, int page_size,
               int max_pages_per_seq) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Hq % Hkv) return -1;
  if (!(dim_bit(d) & kDimsAny)) return -1;
  if (page_size < fa::kSplitKeys || (page_size & (page_size - 1)) ||
      max_pages_per_seq < 1)
    return -1;
  const long long nk = (long long)page_size * max_pages_per_seq;
  if (nk > (1LL << 30)) return -1;
  const bool pre = paged_prefill_ok(Hkv, d, page_size, max_pages_per_seq);
  int s = default_splits(B, Hq, Hkv, Nq, (int)nk);
  if (d == 96) return pre ? 0 : -1;
  if (s == 0 && pre) return 0;
  if (s < 1) s = 1;
  const long long nblk = (nk + fa::kSplitKeys - 1) / fa::kSplitKeys;
  const long long per = fa::paged_max_blocks_per_chunk(page_size);
  const long long need = (nblk + per - 1) / per;
  if (s < need) s = (int)need;
  return s <= fa::kMaxSplits ? s : -1;
}

}  // namespace

extern "C" {

int fa_paged_num_splits(int B, int Hq, int Hkv, int Nq, int d, int page_size,
                        int max_pages_per_seq) {
  const int f = paged_form(B, Hq, Hkv, Nq, d, page_size, max_pages_per_seq);
  return f > 0 ? f : 0;
}

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                 void* o, float* lse, const int* page_table,
                 const int* seqlens_k, int B, int Hq, int Hkv, int Nq, int d,
                 int num_pages, int page_size, int max_pages_per_seq,
                 int causal, int window_left, int window_right, float scale,
                 int out_dtype, int num_splits, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  if (!page_table || !seqlens_k ||
      (reinterpret_cast<uintptr_t>(page_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return FA_ERR_INVALID_ARG;
  if (num_pages < 1 || max_pages_per_seq < 1 || page_size < fa::kSplitKeys ||
      (page_size & (page_size - 1)))
    return FA_ERR_INVALID_ARG;
  const long long nk = (long long)page_size * max_pages_per_seq;
  if (nk > (1LL << 30)) return FA_ERR_UNSUPPORTED;
  int st = check_common(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nq, (int)nk,
                        d, scale, out_dtype, kDimsAny);
  if (st != FA_OK) return st;
  if ((long long)num_pages * page_size * Hkv * d > (1LL << 46))
    return FA_ERR_UNSUPPORTED;
  if (num_splits < 0) return FA_ERR_INVALID_ARG;
  fa::Shape s{B, Hq, Hkv, Nq, (int)nk, d, causal, scale};
  s.win_left = window_left;
  s.win_right = window_right;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  int splits = num_splits;
  if (splits == 0) {
    splits = paged_form(B, Hq, Hkv, Nq, d, page_size, max_pages_per_seq);
    if (splits < 0) return FA_ERR_UNSUPPORTED;
    if (splits == 0) {
      // prefill form: the tiled kernel reads each 64-key block from its
      // page; no workspace
      st = check_device();
      if (st != FA_OK) return st;
      fa::SeqLayout lay{};
      lay.q_r = d;
      lay.q_h = (long long)Nq * d;
      lay.q_b = lay.q_h * Hq;
      lay.k_r = (long long)Hkv * d;
      lay.k_h = d;
      lay.k_b = 0;
      lay.l_r = 1;
      lay.l_h = Nq;
      lay.l_b = (long long)Hq * Nq;
      fa::same_vo(lay);
      lay.seqlen_k = seqlens_k;
      lay.page_table = page_table;
      lay.max_pages = max_pages_per_seq;
      lay.page_shift = shift;
      lay.num_pages = num_pages;
      return hip_status(fa::launch_prefill(q, k_cache, v_cache, o, lse, s,
                                           lay, out_dtype == FA_OUT_F32,
                                           stream));
    }
  }
  // KV-split form
  if (!(dim_bit(d) & kDimsSplit)) return FA_ERR_UNSUPPORTED;
  const long long nblk = (nk + fa::kSplitKeys - 1) / fa::kSplitKeys;
  if (splits > fa::kMaxSplits ||
      (nblk + splits - 1) / splits > fa::paged_max_blocks_per_chunk(page_size))
    return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes <
      fa::splitkv_workspace_bytes((long long)B * Hq * Nq, d, splits))
    return FA_ERR_INVALID_ARG;
  const long long rowtiles = ((long long)Nq * (Hq / Hkv) + fa::kSplitRows - 1) /
                             fa::kSplitRows;
  if ((long long)B * Hkv * rowtiles * splits > (1LL << 31) - 64)
    return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::PagedKv pg{page_table, seqlens_k, max_pages_per_seq, page_size,
                       num_pages, shift};
  return hip_status(fa::launch_splitkv_paged(q, k_cache, v_cache, o, lse, s,
                                             pg, out_dtype == FA_OUT_F32,
                                             splits, workspace, stream));
}

int fa_fwd_kvlen(const void* q, const void* k, const void* v, void* o,
                 float* lse, const int* seqlens_k, int B, int Hq, int Hkv,
                 int Nq, int Nk, int d, int causal, int window_left,
                 int window_right, float scale, int out_dtype, int num_splits,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  if (!seqlens_k || (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return FA_ERR_INVALID_ARG;
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype, kDimsAny);
  if (st != FA_OK) return st;
  // one K or V head is addressed with 32-bit byte offsets
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  if (num_splits < 0) return FA_ERR_INVALID_ARG;
  fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  s.win_left = window_left;
  s.win_right = window_right;
  const int splits = num_splits == 0 ? forward_splits(B, Hq, Hkv, Nq, Nk, d)
                                     : num_splits;
  if (splits == 0) {
    // prefill form (many query rows per KV head, or d = 96): the tiled
    // kernel with each sequence's key count; no workspace
    st = check_device();
    if (st != FA_OK) return st;
    fa::SeqLayout lay = fa::dense_layout(s);
    lay.seqlen_k = seqlens_k;
    return hip_status(fa::launch_prefill(q, k, v, o, lse, s, lay,
                                         out_dtype == FA_OUT_F32, stream));
  }
  if (!(dim_bit(d) & kDimsSplit)) return FA_ERR_UNSUPPORTED;
  if (splits > fa::kMaxSplits) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes <
      fa::splitkv_workspace_bytes((long long)B * Hq * Nq, d, splits))
    return FA_ERR_INVALID_ARG;
  const long long rowtiles = ((long long)Nq * (Hq / Hkv) + fa::kSplitRows - 1) /
                             fa::kSplitRows;
  if ((long long)B * Hkv * rowtiles * splits > (1LL << 31) - 64)
    return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  return hip_status(fa::launch_splitkv_kvlen(q, k, v, o, lse, s, seqlens_k,
                                             out_dtype == FA_OUT_F32, splits,
                                             workspace, stream));
}

int fa_fwd_fp8(const void* q, const void* k, const void* vt,
               const float* q_descale, const float* k_descale,
               const float* v_descale, void* o, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nk, int ldv, int d, int causal,
               float scale, int out_dtype, hipStream_t stream) {
  int st = check_common(q, k, vt, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype);
  if (st != FA_OK) return st;
  if (!q_descale || !k_descale || !v_descale ||
      (reinterpret_cast<uintptr_t>(q_descale) & 3u) ||
      (reinterpret_cast<uintptr_t>(k_descale) & 3u) ||
      (reinterpret_cast<uintptr_t>(v_descale) & 3u))
    return FA_ERR_INVALID_ARG;
  if (ldv < Nk || ldv % 64 != 0) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  // one head of K and of V^T is addressed with 32-bit byte offsets
  if ((long long)Nk * d > (1LL << 31) - 1 ||
      (long long)ldv * d > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if ((long long)B * Hq * qblk > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  return hip_status(fa::launch_prefill_fp8(q, k, vt, q_descale, k_descale,
                                           v_descale, o, lse, s, ldv,
                                           out_dtype == FA_OUT_F32, stream));
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   const long long* q_stride, const long long* k_stride,
                   const long long* v_stride, const long long* o_stride,
                   int causal, int window_left, int window_right, float scale,
                   int out_dtype, hipStream_t stream) {
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype);
  if (st != FA_OK) return st;
  if (!q_stride || !k_stride || !v_stride || !o_stride)
    return FA_ERR_INVALID_ARG;
  // every row starts on a 16-byte boundary: strides are multiples of 8
  // elements, and a row holds d elements
  const long long* all[4] = {q_stride, k_stride, v_stride, o_stride};
  for (const long long* t : all)
    for (int i = 0; i < 3; ++i)
      if (t[i] < 0 || t[i] % 8 != 0 || t[i] > (1LL << 40))
        return FA_ERR_INVALID_ARG;
  if (q_stride[2] < d || k_stride[2] < d || v_stride[2] < d ||
      o_stride[2] < d)
    return FA_ERR_INVALID_ARG;
  // one head of K and of V is addressed with 32-bit byte offsets
  if (((long long)Nk - 1) * k_stride[2] * 2 + 2LL * d > (1LL << 31) - 1 ||
      ((long long)Nk - 1) * v_stride[2] * 2 + 2LL * d > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if ((long long)B * Hq * qblk > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  s.win_left = window_left;
  s.win_right = window_right;
  fa::SeqLayout lay = fa::dense_layout(s);  // lse dense [B, Hq, Nq]
  lay.q_b = q_stride[0]; lay.q_h = q_stride[1]; lay.q_r = q_stride[2];
  lay.k_b = k_stride[0]; lay.k_h = k_stride[1]; lay.k_r = k_stride[2];
  lay.v_b = v_stride[0]; lay.v_h = v_stride[1]; lay.v_r = v_stride[2];
  lay.o_b = o_stride[0]; lay.o_h = o_stride[1]; lay.o_r = o_stride[2];
  return hip_status(fa::launch_prefill(q, k, v, o, lse, s, lay,
                                       out_dtype == FA_OUT_F32, stream));
}

int fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o,
                        float* lse, const unsigned char* block_mask,
                        long long mask_batch_stride, long long mask_head_stride,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        int causal, float scale, int out_dtype,
                        hipStream_t stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype);
  if (st != FA_OK) return st;
  if (!block_mask || mask_batch_stride < 0 || mask_head_stride < 0)
    return FA_ERR_INVALID_ARG;
  const int nkb = (Nk + fa::kPrefillKeys - 1) / fa::kPrefillKeys;
  if (nkb > fa::kSparseMaxKeyBlocks) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if ((long long)B * Hq * qblk > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  const fa::BlockMask bm{block_mask, mask_batch_stride, mask_head_stride, nkb};
  return hip_status(fa::launch_prefill_sparse(q, k, v, o, lse, s, bm,
                                              out_dtype == FA_OUT_F32,
                                              stream));
}

int fa_fwd_colmask(const void* q, const void* k, const void* v, void* o,
                   float* lse, const int* col_bounds, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, int causal, float scale,
                   int out_dtype, hipStream_t stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        out_dtype);
  if (st != FA_OK) return st;
  if (!col_bounds || (reinterpret_cast<uintptr_t>(col_bounds) & 7u))
    return FA_ERR_INVALID_ARG;
  const int nkb = (Nk + fa::kPrefillKeys - 1) / fa::kPrefillKeys;
  if (nkb > fa::kColMaxKeyBlocks) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d * 2 > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  const long long qblk = ((long long)Nq + fa::kPrefillRows - 1) / fa::kPrefillRows;
  if ((long long)B * Hq * qblk > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  return with_workspace(
      stream, fa::column_list_bytes(B, Nq, Nk), [&](void* ws) {
        const fa::ColMask cm{col_bounds, (long long)Nk,
                             static_cast<int*>(ws), (long long)nkb};
        return fa::launch_prefill_column(q, k, v, o, lse, s, cm,
                                         out_dtype == FA_OUT_F32, stream);
      });
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int Hq, int Hkv, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int d, int causal,
                  float scale, int out_dtype, hipStream_t stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q,
                        max_seqlen_k, d, scale, out_dtype);
  if (st != FA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_INVALID_ARG;
  if (total_q < 1 || total_k < 1) return FA_ERR_INVALID_ARG;
  // one sequence's K/V rows of one head are addressed with 32-bit byte
  // offsets; the grid covers every (sequence, head, 256-row block)
  if (((long long)max_seqlen_k - 1) * Hkv * d * 2 + 2LL * d > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  const long long qblk =
      ((long long)max_seqlen_q + fa::kPrefillRows - 1) / fa::kPrefillRows;
  // (the grid is rounded up to whole rounds of 8 units of Hq / Hkv heads)
  if (((long long)B * Hkv * qblk + 7) / 8 * 8 * (Hq / Hkv) > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  const fa::Shape s{B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, causal, scale};
  fa::SeqLayout lay{};
  lay.q_h = d;
  lay.q_r = (long long)Hq * d;
  lay.k_h = d;
  lay.k_r = (long long)Hkv * d;
  lay.l_h = total_q;
  lay.l_r = 1;
  lay.cu_q = cu_seqlens_q;
  lay.cu_k = cu_seqlens_k;
  lay.total_q = total_q;
  lay.total_k = total_k;
  lay.n_seq = B;
  fa::same_vo(lay);
  return hip_status(fa::launch_prefill(q, k, v, o, lse, s, lay,
                                       out_dtype == FA_OUT_F32, stream));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq) {
  if (B < 1 || Hq < 1 || Nq < 1) return 0;
  return fa::backward_workspace_bytes((long long)B * Hq * Nq);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
           float scale, int grad_dtype, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_window(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk,
                       d, causal, -1, -1, scale, grad_dtype, workspace,
                       workspace_bytes, stream);
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk,
                  void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                  int causal, int window_left, int window_right, float scale,
                  int grad_dtype, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        grad_dtype, kDimsBwd);
  if (st != FA_OK) return st;
  if (!dout || !dq || !dk || !dv || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
  const long long rows = (long long)B * Hq * Nq;
  if (workspace_bytes < fa::backward_workspace_bytes(rows))
    return FA_ERR_INVALID_ARG;
  // the kernels address one head of Q / dO (and of K / V) with 32-bit byte
  // offsets, up to one 128-row step past its end
  if (((long long)Nq + 128) * d * 2 > (1LL << 31) - 1 ||
      ((long long)Nk + 128) * d * 2 > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  // grids: one workgroup per 128 keys of a KV head, per 128 rows of a
  // query head, and per 256 threads of the row preprocessing
  if ((long long)B * Hkv * ((Nk + 127) / 128) > (1LL << 31) - 1 ||
      (long long)B * Hq * ((Nq + 127) / 128) > (1LL << 31) - 1 ||
      rows * (d / 8) / 256 > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != FA_OK) return st;
  fa::Shape s{B, Hq, Hkv, Nq, Nk, d, causal, scale};
  s.win_left = window_left;
  s.win_right = window_right;
  return hip_status(fa::launch_backward(q, k, v, o, lse, dout, dq, dk, dv, s,
                                        grad_dtype == FA_OUT_F32, workspace,
                                        stream));
}

}  // extern "C"

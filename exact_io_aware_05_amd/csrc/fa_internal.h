// Host-side launchers behind the C interface in fa.h.  Arguments are
// already validated; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct Shape {
  int B, Hq, Hkv, Nq, Nk, d;
  int causal;
  float scale;
  // sliding window around each query's place c = i + Nk - Nq on the key
  // axis: keys c - win_left .. c + win_right; -1 is no bound on that side
  int win_left = -1, win_right = -1;
};

// Where the rows of one (sequence, head) live, in elements: batch, head and
// row strides of Q and O (same shape), of K and V, and of lse.  Fixed-length
// batches have cu_q = cu_k = nullptr.  Packed variable-length batches take
// sequence b's rows from cu_q[b] .. cu_q[b + 1] (and cu_k for K/V), the
// batch stride unused; Nq / Nk of the Shape are then the maximum lengths and
// total_q / total_k the row counts of the packed tensors.
struct SeqLayout {
  long long q_b, q_h, q_r;
  long long k_b, k_h, k_r;
  long long l_b, l_h, l_r;
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int n_seq;  // sequences of a packed batch (cu_q, cu_k: n_seq + 1 entries)
};

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
  return l;
}

// Rows of queries per prefill workgroup and keys per streamed K/V block.
constexpr int kPrefillRows = 256;
constexpr int kPrefillKeys = 64;
// Keys per block and query rows per wave in the KV-split kernel.
constexpr int kSplitKeys = 32;
constexpr int kSplitRows = 32;
constexpr int kMaxSplits = 4096;

hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s,
                          const SeqLayout& lay, bool out_f32,
                          hipStream_t stream);

hipError_t launch_splitkv(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s, bool out_f32,
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

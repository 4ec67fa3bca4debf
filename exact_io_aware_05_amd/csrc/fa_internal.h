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
};

// Rows of queries per prefill workgroup and keys per streamed K/V block.
constexpr int kPrefillRows = 256;
constexpr int kPrefillKeys = 64;
// Keys per block and query rows per wave in the KV-split kernel.
constexpr int kSplitKeys = 32;
constexpr int kSplitRows = 32;
constexpr int kMaxSplits = 4096;

hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s, bool out_f32,
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

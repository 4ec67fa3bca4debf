// Tiled attention forward (prefill): one workgroup per (batch, query head,
// block of 128 query rows), 4 waves of 32 query rows each.
//
// Method ("FlashAttention Analysis", ryotta.opik.net, section 3 "Tiling +
// Online Softmax"): the Q block stays resident (in registers, as matrix-core
// operands) while K/V blocks of 64 keys stream from HBM through LDS; per
// query row a running max m and running sum l are kept, the accumulated
// output is rescaled by 2^(m_old - m_new) whenever the max grows, and O is
// divided by l once at the end.  Scale and mask are applied inside the same
// pass (same page, section 2).  One fp32 logsumexp per row is written
// (FlashAttention version/GPU/training-cost guide, tool.smithlab.co.kr,
// attention-memory section).  Work is split over (batch, head, Q block), so
// one head spreads over many compute units ("FlashAttention-2 (KO)",
// systems-analysis.info, "Improved parallelism").
//
// gfx950 mapping:
// * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16):
//   a lane owns one query row and 16 of the keys of each 32-key half, so the
//   row max needs 16 in-lane steps and one v_permlane32_swap, and the row
//   sum needs no exchange until the epilogue (each lane keeps a partial l).
// * Keys are stored in LDS in an order (bits 2 and 3 of the key index
//   swapped) that makes the score registers r = 0..7 of a lane hold 8
//   consecutive keys, which is exactly the B operand layout of the P V
//   product: P needs no shuffle between the two products.
// * O is accumulated transposed too, O^T = V^T P^T, so the per-row rescale
//   factor is one scalar per lane.  V^T operands come from row-major V in
//   LDS through the transposing LDS read ds_read_b64_tr_b16.
// * K and V tiles are XOR-swizzled in LDS so that the matrix-operand reads
//   of a wave hit distinct banks.
// * Double-buffered LDS with register prefetch of the next block: one
//   barrier per block.
// * Causal: K/V blocks past the diagonal are never loaded; waves whose rows
//   are entirely before a block skip its math; masking is evaluated only on
//   blocks that cross the diagonal or the key tail.  Heavy Q blocks (near
//   the end of the sequence) are scheduled first, and the query heads of one
//   KV-head group run next to each other on the same XCD so that they share
//   K/V in its L2.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BR = kPrefillRows;
constexpr int BC = kPrefillKeys;
constexpr int NT = 256;  // 4 waves

// LDS row position of key j (within a 64-key tile): bits 2 and 3 swapped.
__device__ __forceinline__ int key_slot(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// 16-byte chunk swizzles (chunk index XOR a function of the LDS row).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Register staging of one BC x D bf16 tile, 16 bytes per thread per step.
template <int D>
struct Stage {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int N = BC * CPR / NT;       // chunks per thread
  u32x4 r[N];

  __device__ __forceinline__ void load(const uint16_t* rows, int row0,
                                       int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * NT + tid;
      const int row = c / CPR, w = c % CPR;
      const int grow = row0 + row;
      if (grow < nrows)
        r[i] = ldg16(rows + (int64_t)grow * D + w * 8);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store_k(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * NT + tid;
      const int row = key_slot(c / CPR), w = c % CPR;
      *reinterpret_cast<u32x4*>(lds + row * (2 * D) +
                                ((w ^ swz_k<D>(row)) * 16)) = r[i];
    }
  }
  __device__ __forceinline__ void store_v(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * NT + tid;
      const int row = c / CPR, w = c % CPR;
      *reinterpret_cast<u32x4*>(lds + row * (2 * D) +
                                ((w ^ swz_v<D>(row)) * 16)) = r[i];
    }
  }
};

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int Nq, int Nk, float c2,
    int n_qblk, int n_items) {
  constexpr int ROWB = 2 * D;            // bytes per LDS row
  constexpr int TILE = BC * ROWB;        // bytes per K or V tile
  constexpr int NTILE = D / 32;          // O^T accumulator tiles
  constexpr int NSTEP = D / 16;          // k-steps of the score product
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;

  // ---- work item: (b, kv head, Q block, head in group); heavy blocks first
  const int item = xcd_contiguous(blockIdx.x, n_items);
  const int G = Hq / Hkv;
  const int g = item % G;
  const int t1 = item / G;
  const int jq = t1 % n_qblk;
  const int bh = t1 / n_qblk;  // b * Hkv + hkv
  const int qblk = CAUSAL ? (n_qblk - 1 - jq) : jq;
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int hq = hkv * G + g;
  const int q0 = qblk * BR;
  const int off = Nk - Nq;

  const int64_t qhead = (int64_t)(b * Hq + hq) * Nq;
  const uint16_t* kh = k + (int64_t)bh * Nk * D;
  const uint16_t* vh = v + (int64_t)bh * Nk * D;

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, q0 + BR + off);
  const int nblk = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // ---- Q^T operand fragments: lane holds q[row][16t + 8h .. +7]
  const int qrow = q0 + wave * 32 + col;
  bf16x8 qf[NSTEP];
  {
    const bool ok = qrow < Nq;
    const uint16_t* qp = q + (qhead + (ok ? qrow : 0)) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      u32x4 x = ok ? ldg16(qp + 16 * t) : u32x4{0u, 0u, 0u, 0u};
      qf[t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 acc[NTILE];
#pragma unroll
  for (int i = 0; i < NTILE; ++i) acc[i] = f32x16{};
  float m = -INFINITY;  // running max, log2 units (score * scale * log2 e)
  float l = 0.f;        // running sum over this lane's keys

  Stage<D> ks, vs;
  if (nblk > 0) {
    ks.load(kh, 0, Nk, tid);
    vs.load(vh, 0, Nk, tid);
    ks.store_k(smem, tid);
    vs.store_v(smem + TILE, tid);
  }
  __syncthreads();

  const int wrow0 = q0 + wave * 32;  // first query row of this wave
  const int lg = lane >> 4, lp = lane & 15;

  for (int j = 0; j < nblk; ++j) {
    const int kb = j * BC;
    const bool has_next = j + 1 < nblk;
    if (has_next) {
      ks.load(kh, kb + BC, Nk, tid);
      vs.load(vh, kb + BC, Nk, tid);
    }
    const char* Ks = smem + (j & 1) * 2 * TILE;
    const char* Vs = Ks + TILE;

    // waves whose every row precedes this block's first key skip the math
    const bool active = !CAUSAL || kb <= wrow0 + 31 + off;
    if (active) {
      // ---- S^T = K Q^T for the two 32-key halves
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int t = 0; t < NSTEP; ++t) {
        const int w = 2 * t + h;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            Ks + col * ROWB + ((w ^ swz_k<D>(col)) * 16));
        const bf16x8 kc = *reinterpret_cast<const bf16x8*>(
            Ks + (32 + col) * ROWB + ((w ^ swz_k<D>(32 + col)) * 16));
        s0 = mfma32x32x16(ka, qf[t], s0);
        s1 = mfma32x32x16(kc, qf[t], s1);
      }

      // ---- mask (only on blocks crossing the key tail or the diagonal)
      const bool need_mask =
          (kb + BC > Nk) || (CAUSAL && kb + BC - 1 > wrow0 + off);
      uint32_t vis = 0xffffffffu;  // bit r: s0[r]; bit 16 + r: s1[r]
      if (need_mask) {
        vis = 0;
        const int lim = CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key <= lim) vis |= 1u << r;
          if (key + 32 <= lim) vis |= 1u << (16 + r);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!(vis & (1u << r))) s0[r] = -INFINITY;
          if (!(vis & (1u << (16 + r)))) s1[r] = -INFINITY;
        }
      }

      // ---- online softmax (log2 domain)
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = pair_max(mx);
      const float m_new = fmaxf(m, mx * c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      m = m_new;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p0 = exp2_fast(fmaf(s0[r], c2, -m_use));
        float p1 = exp2_fast(fmaf(s1[r], c2, -m_use));
        if (need_mask) {
          if (!(vis & (1u << r))) p0 = 0.f;
          if (!(vis & (1u << (16 + r)))) p1 = 0.f;
        }
        s0[r] = p0;
        s1[r] = p1;
        rs += p0 + p1;
      }
      l = alpha * l + rs;
#pragma unroll
      for (int i = 0; i < NTILE; ++i) acc[i] *= alpha;

      bf16x8 pb[4];
      pb[0] = to_bf16x8(s0, 0);
      pb[1] = to_bf16x8(s0, 8);
      pb[2] = to_bf16x8(s1, 0);
      pb[3] = to_bf16x8(s1, 8);

      // ---- O^T += V^T P^T
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int vrow = 16 * s + 8 * (lg >> 1) + (lp >> 2);
#pragma unroll
        for (int tt = 0; tt < NTILE; ++tt) {
          const int u = 8 * tt + 4 * (lg & 1) + (lp & 3);
          const int sw = 2 * swz_v<D>(vrow);  // 8-byte chunk units
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const lds_i16x4* p0 = (const lds_i16x4*)(
              (__attribute__((address_space(3))) char*)(
                  Vs + vrow * ROWB + ((u ^ sw) * 8)));
          const lds_i16x4* p1 = (const lds_i16x4*)(
              (__attribute__((address_space(3))) char*)(
                  Vs + (vrow + 4) * ROWB + ((u ^ sw) * 8)));
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              const_cast<lds_i16x4*>(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              const_cast<lds_i16x4*>(p1));
          u32x4 va;
          va[0] = __builtin_bit_cast(u32x2, lo)[0];
          va[1] = __builtin_bit_cast(u32x2, lo)[1];
          va[2] = __builtin_bit_cast(u32x2, hi)[0];
          va[3] = __builtin_bit_cast(u32x2, hi)[1];
          acc[tt] = mfma32x32x16(__builtin_bit_cast(bf16x8, va), pb[s],
                                 acc[tt]);
        }
      }
    }

    if (has_next) {
      char* nb = smem + ((j + 1) & 1) * 2 * TILE;
      ks.store_k(nb, tid);
      vs.store_v(nb + TILE, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O / l, lse = (m + log2 l) ln 2
  const float lt = pair_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v =
      lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  if (qrow < Nq) {
    const int64_t orow = (qhead + qrow) * D;
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int c = 32 * tt + 8 * gg + 4 * h;
        const float x0 = acc[tt][4 * gg + 0] * inv;
        const float x1 = acc[tt][4 * gg + 1] * inv;
        const float x2 = acc[tt][4 * gg + 2] * inv;
        const float x3 = acc[tt][4 * gg + 3] * inv;
        if (OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow + c) =
              f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + orow + c) =
              u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      }
    }
    if (h == 0) lse[qhead + qrow] = lse_v;
  }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch(const void* q, const void* k, const void* v, void* o,
                  float* lse, const Shape& s, hipStream_t stream) {
  const int n_qblk = (s.Nq + BR - 1) / BR;
  const long long n_items = (long long)s.B * s.Hq * n_qblk;
  const float c2 = s.scale * kLog2e;
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, OUT_F32>),
                     dim3((unsigned)n_items), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), o, lse, s.Hq, s.Hkv,
                     s.Nq, s.Nk, c2, n_qblk, (int)n_items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s, bool out_f32,
                          hipStream_t stream) {
  const bool c = s.causal != 0;
#define FA_DISPATCH(D_)                                                    \
  if (s.d == D_) {                                                         \
    if (c)                                                                 \
      return out_f32 ? launch<D_, true, true>(q, k, v, o, lse, s, stream)  \
                     : launch<D_, true, false>(q, k, v, o, lse, s, stream); \
    return out_f32 ? launch<D_, false, true>(q, k, v, o, lse, s, stream)   \
                   : launch<D_, false, false>(q, k, v, o, lse, s, stream); \
  }
  FA_DISPATCH(128)
  FA_DISPATCH(64)
#undef FA_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace fa

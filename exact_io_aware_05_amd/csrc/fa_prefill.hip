// Tiled attention forward (prefill): one workgroup per (batch, query head,
// block of 128 query rows), 4 waves of 32 query rows each.
//
// Method ("FlashAttention Analysis", ryotta.opik.net, section 3 "Tiling +
// Online Softmax"): the Q block stays resident (in registers, as matrix-core
// operands) while K/V blocks of 64 keys stream from HBM through LDS; per
// query row a running max m and running sum l are kept, the accumulated
// output is rescaled by 2^(m_old - m_new) when the max grows, and O is
// divided by l once at the end.  Scale and mask are applied inside the same
// pass (same page, section 2).  One fp32 logsumexp per row is written
// (FlashAttention version/GPU/training-cost guide, tool.smithlab.co.kr,
// attention-memory section).  Work is split over (batch, head, Q block), so
// one head spreads over many compute units ("FlashAttention-2 (KO)",
// systems-analysis.info, "Improved parallelism"), and the row statistics
// stay inside one wave ("Optimised work split inside a block").
//
// gfx950 mapping:
// * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16):
//   a lane owns one query row and 16 of the keys of each 32-key half, so the
//   row max needs in-lane steps and one v_permlane32_swap, and the row sum
//   needs no exchange until the epilogue (each lane keeps a partial l).
// * Keys are stored in LDS in an order (bits 2 and 3 of the key index
//   swapped) that makes score registers r = 0..7 of a lane hold 8
//   consecutive keys, which is exactly the B-operand layout of the P V
//   product: P needs no shuffle between the two products.
// * O is accumulated transposed too, O^T = V^T P^T, so the per-row rescale
//   factor is one scalar per lane.  V^T operands come from row-major V in
//   LDS through the transposing read ds_read_b64_tr_b16.
// * K/V tiles move HBM -> LDS with buffer_load ... lds (no staging
//   registers, no VALU); a buffer resource per head makes reads past the
//   last key return zeros, so tails need no branches.  LDS rows are padded
//   (K: 16 bytes, V: 64 bytes) so that the operand reads of a wave hit
//   distinct banks and every read address is a per-lane base plus an
//   immediate offset.  Double-buffered: one barrier per 64-key block.
// * The output rescale is lazy: the reference max used for the
//   exponentials only moves when some row's max grew by more than 2^8, so
//   almost every block skips the 64 multiplies per lane.  The result is the
//   same real-arithmetic quantity (the factor cancels in O = acc / l).
// * Causal: K/V blocks past the diagonal are never loaded; waves whose rows
//   all precede a block skip its math; masking runs only on blocks that
//   cross the diagonal or the key tail.  Heavy Q blocks (late rows) are
//   scheduled first, and the query heads of one KV-head group run next to
//   each other on the same XCD so that they share K/V in its L2.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BR = kPrefillRows;
constexpr int BC = kPrefillKeys;
constexpr int NT = 256;  // 4 waves
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) void lds_void;

// LDS row position of key j (within a 64-key tile): bits 2 and 3 swapped.
__device__ __forceinline__ int key_slot(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

template <int D>
struct Layout {
  static constexpr int ROWB = 2 * D;             // bytes of one K/V row
  static constexpr int KCH = D / 8 + 1;          // 16-byte chunks per K row
  static constexpr int VCH = D / 8 + 4;          // ... per V row (padded)
  static constexpr int KSTRIDE = 16 * KCH;       // 272 (D=128) / 144
  static constexpr int VSTRIDE = 16 * VCH;       // 320 (D=128) / 192
  static constexpr int KBYTES = BC * KSTRIDE;
  static constexpr int VBYTES = BC * VSTRIDE;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KINS = KCH;               // 1 KiB DMA instructions
  static constexpr int VINS = VCH;
  static constexpr int KPW = (KINS + 3) / 4;     // per wave (max)
  static constexpr int VPW = (VINS + 3) / 4;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base,
                                                       uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

// Starts the HBM -> LDS copy of K/V block `blk` into LDS stage `stage`:
// each wave issues its share of 1 KiB buffer_load ... lds instructions.
// Reads past key Nk return zeros (buffer range check).
template <int D>
__device__ __forceinline__ void issue_dma(char* smem, const char* kh,
                                          const char* vh, int Nk, int blk,
                                          int stage, int wave,
                                          const uint32_t* koff,
                                          const uint32_t* voff) {
  using L = Layout<D>;
  const int kb = blk * BC;
  const uint32_t rem = (uint32_t)(Nk - kb) * L::ROWB;
  const __amdgpu_buffer_rsrc_t rk = rsrc(kh + (int64_t)kb * L::ROWB, rem);
  const __amdgpu_buffer_rsrc_t rv = rsrc(vh + (int64_t)kb * L::ROWB, rem);
  char* base = smem + stage * L::STAGE;
#pragma unroll
  for (int n = 0; n < L::KPW; ++n) {
    const int i = wave + 4 * n;
    if (i < L::KINS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (lds_void*)(base + 1024 * i), 16, koff[n], 0, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < L::VPW; ++n) {
    const int i = wave + 4 * n;
    if (i < L::VINS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_void*)(base + L::KBYTES + 1024 * i), 16, voff[n], 0, 0, 0);
  }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int Nq, int Nk, float c2,
    int n_qblk, int n_items) {
  using L = Layout<D>;
  constexpr int NTILE = D / 32;  // O^T accumulator tiles
  constexpr int NSTEP = D / 16;  // k-steps of the score product
  __shared__ __attribute__((aligned(1024))) char smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const char* kh = reinterpret_cast<const char*>(k + (int64_t)bh * Nk * D);
  const char* vh = reinterpret_cast<const char*>(v + (int64_t)bh * Nk * D);

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, q0 + BR + off);
  const int nblk = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // ---- per-lane DMA source offsets (bytes within a block of 64 rows)
  uint32_t koff[L::KPW], voff[L::VPW];
#pragma unroll
  for (int n = 0; n < L::KPW; ++n) {
    const int gch = 64 * (wave + 4 * n) + lane;
    const int row = gch / L::KCH, c = gch % L::KCH;
    koff[n] = key_slot(row & 63) * L::ROWB + (c < D / 8 ? c : 0) * 16;
  }
#pragma unroll
  for (int n = 0; n < L::VPW; ++n) {
    const int gch = 64 * (wave + 4 * n) + lane;
    const int row = gch / L::VCH, c = gch % L::VCH;
    voff[n] = (row & 63) * L::ROWB + (c < D / 8 ? c : 0) * 16;
  }
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
  float m = -INFINITY;  // reference max in use, log2 units
  float l = 0.f;        // running sum over this lane's keys (fp32 weights)
  float lb = 0.f;       // same over the bf16-rounded weights

  // per-lane LDS read bases (bytes from the stage start)
  const int k_rd = col * L::KSTRIDE + 16 * h;
  const int lg = lane >> 4, lp = lane & 15;
  const int v_rd = L::KBYTES + (8 * (lg >> 1) + (lp >> 2)) * L::VSTRIDE +
                   (4 * (lg & 1) + (lp & 3)) * 8;

  if (nblk > 0)
    issue_dma<D>(smem, kh, vh, Nk, 0, 0, wave, koff, voff);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  const int wrow0 = q0 + wave * 32;  // first query row of this wave

  // One 64-key block.  MASK selects the variant that hides keys past the
  // causal limit or past Nk; it is only used for the trailing blocks.
  auto block = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kb = j * BC;
    if (j + 1 < nblk)
      issue_dma<D>(smem, kh, vh, Nk, j + 1, (j + 1) & 1, wave, koff, voff);
    const char* st = smem + (j & 1) * L::STAGE;

    // waves whose every row precedes this block's first key skip the math
    const bool active = !CAUSAL || kb <= wrow0 + 31 + off;
    if (active) {
      // ---- S^T = K Q^T for the two 32-key halves
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      const char* kp = st + k_rd;
#pragma unroll
      for (int t = 0; t < NSTEP; ++t) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp + 32 * t);
        const bf16x8 kc = *reinterpret_cast<const bf16x8*>(
            kp + 32 * L::KSTRIDE + 32 * t);
        s0 = mfma32x32x16(ka, qf[t], s0);
        s1 = mfma32x32x16(kc, qf[t], s1);
      }

      if (MASK) {
        // key index of register r (half 0): kb + 16(r/8) + 8h + r%8
        const int lim =
            (CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1) - kb - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 16 * (r >> 3) + (r & 7);
          if (kr > lim) s0[r] = -INFINITY;
          if (kr + 32 > lim) s1[r] = -INFINITY;
        }
      }

      // ---- online softmax, log2 domain, lazy reference max
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
      mx = pair_max(mx) * c2;
      if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleThreshold) != 0) {
        const float m_new = fmaxf(m, mx);
        // unchanged rows (including rows with nothing visible yet) keep
        // factor 1; a first visible key gives 2^-inf = 0
        const float alpha = (m_new == m) ? 1.f : exp2_fast(m - m_new);
        m = m_new;
        l *= alpha;
        lb *= alpha;
#pragma unroll
        for (int i = 0; i < NTILE; ++i) acc[i] *= alpha;
      }
      // P is rounded to bf16 once.  The rounded weights feed the P V
      // product and their own row sum lb, so O = acc / lb is an exact
      // convex combination of V rows up to fp32 summation; the fp32 sum l
      // of the unrounded weights gives lse.
      const float msub = (m == -INFINITY) ? 0.f : m;
      u32x4 pk[4];
      float rs = 0.f, rb0 = 0.f, rb1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = exp2_fast(fmaf(s0[r], c2, -msub));
        const float e1 = exp2_fast(fmaf(s0[r + 1], c2, -msub));
        const float e2 = exp2_fast(fmaf(s1[r], c2, -msub));
        const float e3 = exp2_fast(fmaf(s1[r + 1], c2, -msub));
        rs += e0;
        rs += e1;
        rs += e2;
        rs += e3;
        const uint32_t a = pack_bf16x2(e0, e1);
        const uint32_t c = pack_bf16x2(e2, e3);
        pk[r >> 3][(r >> 1) & 3] = a;
        pk[2 + (r >> 3)][(r >> 1) & 3] = c;
        rb0 = add_bf16x2(a, rb0);
        rb1 = add_bf16x2(c, rb1);
      }
      l += rs;
      lb += rb0 + rb1;
      bf16x8 pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = __builtin_bit_cast(bf16x8, pk[i]);

      // ---- O^T += V^T P^T
      const char* vp = st + v_rd;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int tt = 0; tt < NTILE; ++tt) {
          const char* a0 = vp + s * 16 * L::VSTRIDE + tt * 64;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(
                  (__attribute__((address_space(3))) char*)a0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(
                  (__attribute__((address_space(3))) char*)(
                      a0 + 4 * L::VSTRIDE)));
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

    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's DMA for block j+1
    __syncthreads();
  };

  // Block j needs no mask when (j + 1) * BC <= Nk and, if causal, when its
  // last key is visible to the workgroup's first row: (j + 1) * BC <=
  // q0 + off + 1.  Both conditions hold for a prefix of the blocks.
  int j_mask = Nk / BC;
  if (CAUSAL) j_mask = min(j_mask, max(0, q0 + off + 1) / BC);
  j_mask = min(j_mask, nblk);
  int j = 0;
  for (; j < j_mask; ++j) block(j, std::false_type{});
  for (; j < nblk; ++j) block(j, std::true_type{});

  // ---- epilogue: O = O / l, lse = (m + log2 l) ln 2
  const float lt = pair_sum(l);
  const float lbt = pair_sum(lb);
  const float inv = lbt > 0.f ? 1.f / lbt : 0.f;
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
  // scale 0 is run as the smallest normal scale: every exponent is then
  // below 2^-24 in magnitude, so each weight is exactly 1, and -inf scores
  // stay -inf (no 0 * inf)
  const float c2 = fmaxf(s.scale * kLog2e, 1.17549435e-38f);
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

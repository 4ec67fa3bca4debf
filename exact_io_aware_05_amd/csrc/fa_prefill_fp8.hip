// Tiled attention forward on FP8 (OCP E4M3) inputs, head dimension 128:
// one workgroup per (batch, query head, block of 256 query rows), 8 waves of
// 32 query rows each, K/V blocks of 64 keys streamed through LDS.
//
// Method: the tiled online softmax of the bf16 prefill kernel ("FlashAttention
// Analysis", ryotta.opik.net, section 3 "Tiling + Online Softmax"); the 8-bit
// path of FlashAttention-3 ("FlashAttention-2 (KO)", systems-analysis.info,
// comparison with later versions: 8-bit floating point for extra speed; the
// training-cost guide, tool.smithlab.co.kr, FAQ: the FP8 forward is a
// low-precision computation).  Both products run on the 8-bit matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, 64-deep contractions, twice the bf16 rate):
//   S^T = K Q^T   with Q, K in E4M3 (real values code * per-head descale),
//   O^T += V^T P^T with P rounded to E4M3 and V stored transposed
//                  ([B, Hkv, d, Nk]: the key axis is the contraction axis,
//                  and an 8-bit operand lane holds 32 consecutive keys).
// The descales fold into the exponent scale (Q, K) and the epilogue (V).
//
// gfx950 mapping (as in the bf16 kernel where not said otherwise):
// * A and B operands of the 8-bit product hold the same 32 k-slots per lane
//   half, so any byte order works as long as both operands use it: K rows
//   and Q rows are read with the same head-dimension order, V^T rows and P
//   with the same key order.
// * Keys sit in LDS in an order that makes a lane's 16 score registers of
//   one 32-key half 16 consecutive keys (16 h .. 16 h + 15): C register r
//   of lane half h is tile row 8 (r / 4) + 4 h + r % 4, and tile row s holds
//   key 16 (s/4 % 2) + 4 (s/8) + s % 4.  P then packs into the B operand in
//   register order, and the V^T operand is two contiguous 16-byte reads.
// * Weights are kept at most 448 (the largest E4M3 magnitude; the convert
//   turns 464 and above into NaN): the lazy reference max moves when a
//   lane's block sum would pass 448, and a moved reference sits 4 (in log2
//   units) below the row max, so weights reach down to 2^-13 of the row max
//   before they flush to zero.  O is normalised by the fp32 sum of the
//   unrounded weights (the sum of the E4M3-rounded weights would cost three
//   more vector instructions per pair of scores).
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int D = 128;
constexpr int BR = kPrefillRows;   // 256 query rows per workgroup
constexpr int BC = kPrefillKeys;   // 64 keys per K/V block
constexpr int NW = BR / 32;        // 8 waves
constexpr int NT = 64 * NW;
constexpr int NS = 4;              // ring stages of K and of V^T
constexpr int TBYTES = BC * D;     // one K or V^T tile: 8 KiB
constexpr int VBASE = NS * TBYTES;
constexpr int LDS_BYTES = 2 * NS * TBYTES;
constexpr float kMaxLaneSum = 448.f;  // largest E4M3 magnitude
constexpr float kBias = 4.f;          // a moved reference sits 4 below max

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// V^T tile: row d holds the block's 64 keys (64 bytes); its 16-byte chunk
// c sits at chunk c ^ vswz8(d): the 16 lanes of one read (16 consecutive d,
// the same c) then hit 16 different bank groups.
__device__ __forceinline__ int vswz8(int d) { return (d >> 2) & 3; }

// C += A B on the 8-bit matrix cores, E4M3 operands, no block scales (a
// zero scale operand is the unit scale)
__device__ __forceinline__ void mfma8(i32x8 a, i32x8 b, f32x16& c) {
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0,
                                                      0);
}

// Workgroup barrier that neither waits for the copies in flight nor lets
// the compiler move memory accesses across it (the loop's explicit vmcnt
// waits order the ring; __syncthreads would wait for every copy).
__device__ __forceinline__ void barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt with vmcnt = N (expcnt, lgkmcnt left free); gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// HBM -> LDS copies of key block `blk` of one head, one 1 KiB buffer_load
// ... lds instruction per wave for each tile.  K: wave w copies chunk w of
// the head dimension (16 bytes) of all 64 rows; rows at or past Nk read as
// zeros (the resource ends at row Nk - 1).  V^T: wave w copies rows
// 16 w .. 16 w + 15, keys kb .. kb + 63 (ldv, a multiple of 64, keeps
// them inside the row); keys Nk .. ldv - 1 are padding with zero weight,
// and a block past Nk is a copy of zeros.
__device__ __forceinline__ void copy_k(char* dst, const uint8_t* kh, int Nk,
                                       int blk, int wave, uint32_t k_off) {
  const int kb = blk * BC;
  const int rows = Nk - kb;
  const uint32_t range = rows > 0 ? (uint32_t)((rows - 1) * D + 16) : 0u;
  const __amdgpu_buffer_rsrc_t r =
      buffer_rsrc(kh + (int64_t)min(kb, Nk) * D + 16 * wave, range);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (lds_void*)(dst + 1024 * wave), 16, k_off, 0, 0, 0);
}
__device__ __forceinline__ void copy_vt(char* dst, const uint8_t* vth, int Nk,
                                        int ldv, int blk, int wave,
                                        uint32_t v_off) {
  const int kb = blk * BC;
  const uint32_t range = kb < Nk ? (uint32_t)(15 * ldv + 64) : 0u;
  const __amdgpu_buffer_rsrc_t r =
      buffer_rsrc(vth + (int64_t)(16 * wave) * ldv + min(kb, Nk), range);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (lds_void*)(dst + 1024 * wave), 16, v_off, 0, 0, 0);
}

struct RowState {
  float m;  // reference max in use, log2 units (weights use m - kBias)
  float l;  // sum of the fp32 weights
};

// Matrix phase of one wave for block j: O^T += V_{j-1}^T P_{j-1}^T (if PV),
// then S_j^T = K_j Q^T (if QK), 32-key halves into s0 / s1.  Operand reads
// run DEPTH products ahead.
template <bool PV, bool QK>
__device__ __forceinline__ void matrix_phase(const char* kp,
                                             const char* const* vp,
                                             const i32x8* qf,
                                             const i32x8& pk, f32x16* acc,
                                             f32x16& s0, f32x16& s1) {
  constexpr int NPV = PV ? 4 : 0;  // P V products (output tile)
  constexpr int NQK = QK ? 4 : 0;  // score products (t, half)
  constexpr int NOP = NPV + NQK;
  constexpr int DEPTH = 4;
  i32x8 op[NOP > 0 ? NOP : 1];
  // product i < NPV: P V tile i; otherwise score product q = i - NPV with
  // t = q >> 1 (head-dimension 64-slice), half = q & 1
  auto order = [&](int slot) {
    if (NPV == 0 || NQK == 0) return slot;
    return (slot & 1) ? NPV + (slot >> 1) : (slot >> 1);
  };
  auto read = [&](int i) {
    u32x4 lo, hi;
    if (i < NPV) {
      // V^T rows d = 32 i + col: keys 16 h .. +15 and 32 + 16 h .. +15
      lo = *reinterpret_cast<const u32x4*>(vp[0] + 2048 * i);
      hi = *reinterpret_cast<const u32x4*>(vp[1] + 2048 * i);
    } else {
      const int q = i - NPV, t = q >> 1, half = q & 1;
      // K tile row 32 half + col: head-dimension chunks 4 t + 2 h, + 1
      const char* a = kp + 4096 * t + 512 * half;
      lo = *reinterpret_cast<const u32x4*>(a);
      hi = *reinterpret_cast<const u32x4*>(a + 1024);
    }
    i32x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    op[i] = v;
  };
  if (QK) {
    s0 = f32x16{};
    s1 = f32x16{};
  }
#pragma unroll
  for (int i = 0; i < DEPTH && i < NOP; ++i) read(order(i));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int slot = 0; slot < NOP; ++slot) {
    if (slot + DEPTH < NOP) read(order(slot + DEPTH));
    const int i = order(slot);
    if (i < NPV) {
      mfma8(op[i], pk, acc[i]);
    } else {
      const int q = i - NPV, t = q >> 1;
      if (q & 1)
        mfma8(op[i], qf[t], s1);
      else
        mfma8(op[i], qf[t], s0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Softmax phase of one wave for block j: optional mask (`lim`: last
// visible key relative to this lane's first key of each half; register r
// holds relative key r, half 1 adds 32), weights p = 2^(s c2 - (m - 4))
// rounded to E4M3 once into pk, and the row sum.  When a lane's block sum
// would pass 448 (or a row has no reference yet) the block is redone with
// the reference moved to the row max; then the state is rescaled and true
// is returned with the factor in `alpha`.
template <bool MASK>
__device__ __forceinline__ bool softmax_phase(const f32x16& s0,
                                              const f32x16& s1, int lim,
                                              float c2, RowState& st,
                                              float& alpha, i32x8& pk) {
  auto hide0 = [&](int r) { return MASK && r > lim; };
  auto hide1 = [&](int r) { return MASK && r + 32 > lim; };
  auto weights = [&](float msub, float* rs) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float e0 = exp2_fast(fmaf(s0[r], c2, -msub));
      float e1 = exp2_fast(fmaf(s0[r + 1], c2, -msub));
      float e2 = exp2_fast(fmaf(s1[r], c2, -msub));
      float e3 = exp2_fast(fmaf(s1[r + 1], c2, -msub));
      if (hide0(r)) e0 = 0.f;
      if (hide0(r + 1)) e1 = 0.f;
      if (hide1(r)) e2 = 0.f;
      if (hide1(r + 1)) e3 = 0.f;
      rs[(r >> 1) & 1] += e0 + e1;
      rs[2 + ((r >> 1) & 1)] += e2 + e3;
      // bytes r, r + 1 of the half's 16 (dword r / 4, word (r / 2) % 2)
      const int w = r >> 2;
      if (r & 2) {
        pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, pk[w], true);
        pk[4 + w] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, pk[4 + w], true);
      } else {
        pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
        pk[4 + w] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, 0, false);
      }
    }
  };
  float rs[4];
  weights(st.m - kBias, rs);
  const float lsum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
  const bool redo = __builtin_amdgcn_ballot_w64(!(lsum <= kMaxLaneSum) ||
                                                st.m == -INFINITY) != 0;
  if (!redo) {
    st.l += lsum;
    return false;
  }
  float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int r = 0; r < 16; ++r)
    mq[r & 3] = fmaxf(fmaxf(mq[r & 3], hide0(r) ? -INFINITY : s0[r]),
                      hide1(r) ? -INFINITY : s1[r]);
  float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
  mx = pair_max(mx) * c2;
  const float m_new = fmaxf(st.m, mx);
  alpha = (m_new == st.m) ? 1.f : exp2_fast(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
  weights((st.m == -INFINITY) ? 0.f : st.m - kBias, rs);
  st.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  return true;
}

template <bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NT, 1) void prefill_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ vt, const float* __restrict__ q_descale,
    const float* __restrict__ k_descale, const float* __restrict__ v_descale,
    void* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int Nq,
    int Nk, int ldv, float c2base, int n_qblk, int n_items) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_a = wave < NW / 2;
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
  // kept a normal number, like the scale itself, so that the row max times
  // c2 never meets -inf * 0
  const float c2 =
      fmaxf(c2base * q_descale[b * Hq + hq] * k_descale[bh], 1.17549435e-38f);
  const float vscale = v_descale[bh];
  const uint8_t* kh = k + (int64_t)bh * Nk * D;
  const uint8_t* vth = vt + (int64_t)bh * D * ldv;

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, q0 + BR + off);
  const int nblk = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const int wrow0 = q0 + wave * 32;
  int w_mask = Nk / BC;
  if (CAUSAL) w_mask = min(w_mask, max(0, wrow0 + off + 1) / BC);

  // ---- per-lane DMA source offsets.  K: lane = tile row, holding key
  // j = key of tile row lane (chunk `wave` of the head dimension).  V^T:
  // lane -> row 16 wave + lane / 4 (the wave part is in the resource), its
  // physical chunk lane % 4 holds source chunk (lane % 4) ^ vswz8(row).
  int kj;
  {
    const int s = lane & 31;  // tile row within the half
    kj = (lane & 32) | (((s >> 2) & 1) << 4) | (((s >> 3) & 3) << 2) | (s & 3);
  }
  const uint32_t k_off = (uint32_t)(kj * D);
  const uint32_t v_off =
      (uint32_t)((lane >> 2) * ldv + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));

  // ---- Q^T operands: lane holds q[row][64 t + 32 h .. +31], t = 0, 1
  const int qrow = wrow0 + col;
  i32x8 qf[2];
  {
    const bool ok = qrow < Nq;
    const uint8_t* qp = q + ((int64_t)(b * Hq + hq) * Nq + (ok ? qrow : 0)) * D +
                        32 * h;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // every lane loads (its address is kept inside the tensor), then
      // zeros: a load under a branch leaves the compiler unsure at the main
      // loop whether it has landed, and it then waits for every copy in
      // flight in every iteration
      u32x4 a = ldg16(qp + 64 * t), c = ldg16(qp + 64 * t + 16);
      if (!ok) a = c = u32x4{0u, 0u, 0u, 0u};
      i32x8 v;
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = c[0]; v[5] = c[1]; v[6] = c[2]; v[7] = c[3];
      qf[t] = v;
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  RowState st{-INFINITY, 0.f};

  // per-lane LDS read bases.  K: tile row col of half 0 in chunk 2 h; the
  // matrix phase adds 4096 t (chunks 4 t), 512 half (rows 32 half) and
  // 1024 (the next chunk).  V^T: rows 32 tt + col, chunks h and 2 + h.
  const int k_rd = 2048 * h + 16 * col;
  int v_rd[2];
  {
    const int d0 = col;  // + 32 tt, which keeps vswz8 (32 tt is 0 mod 16)
    v_rd[0] = VBASE + 64 * d0 + 16 * ((h) ^ vswz8(d0));
    v_rd[1] = VBASE + 64 * d0 + 16 * ((2 + h) ^ vswz8(d0));
  }
  // this lane's last visible key relative to its first key of each half
  const int lim0 = (CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1) - 16 * h;

  f32x16 s0, s1;
  i32x8 pk;

  bool rescale = false;
  float alpha = 1.f;
  auto mphase = [&](int j, auto qk_tag) {
    if (rescale) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    }
    const int vs = ((j + NS - 1) % NS) * TBYTES;
    const char* vp[2] = {smem + vs + v_rd[0], smem + vs + v_rd[1]};
    __builtin_amdgcn_s_setprio(1);
    matrix_phase<true, decltype(qk_tag)::value>(
        smem + (j % NS) * TBYTES + k_rd, vp, qf, pk, acc, s0, s1);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- K/V ring as in the bf16 kernel: K_{j+3} and V_{j+2} are issued at
  // the start of the softmax phase of iteration j; group A waits for its
  // copies of iteration j at the end of iteration j+2, group B at the end
  // of iteration j+1.
  constexpr int OPS = 2;  // copy instructions per wave per block
  const int kv_rows = max(kv_end, 0);
  auto copies = [&](int j) {
    copy_k(smem + ((j + 3) % NS) * TBYTES, kh, kv_rows, j + 3, wave, k_off);
    copy_vt(smem + VBASE + ((j + 2) % NS) * TBYTES, vth, kv_rows, ldv, j + 2,
            wave, v_off);
  };
  // prologue: K_0, K_1, K_2, V_0, V_1, fully waited; the V^T stage before
  // block 0 is zeroed (block 0's matrix phase multiplies it by the all-zero
  // "previous" P, and 0 times stale NaN bits would not be 0)
#pragma unroll
  for (int b0 = 0; b0 < 3; ++b0)
    copy_k(smem + b0 * TBYTES, kh, kv_rows, b0, wave, k_off);
#pragma unroll
  for (int b0 = 0; b0 < 2; ++b0)
    copy_vt(smem + VBASE + b0 * TBYTES, vth, kv_rows, ldv, b0, wave, v_off);
#pragma unroll
  for (int i = tid; i < TBYTES / 16; i += NT)
    reinterpret_cast<u32x4*>(smem + VBASE + 3 * TBYTES)[i] =
        u32x4{0u, 0u, 0u, 0u};
  wait_vmcnt<0>();
  __syncthreads();

#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = 0;
  if (!group_a) __syncthreads();
  for (int j = 0; j < nblk; ++j) {
    mphase(j, std::true_type{});
    barrier();
    copies(j);
    if (j >= w_mask)
      rescale = softmax_phase<true>(s0, s1, lim0 - j * BC, c2, st, alpha, pk);
    else
      rescale = softmax_phase<false>(s0, s1, lim0 - j * BC, c2, st, alpha, pk);
    if (group_a)
      wait_vmcnt<2 * OPS>();
    else
      wait_vmcnt<OPS>();
    barrier();
  }
  if (nblk > 0) mphase(nblk, std::false_type{});
  wait_vmcnt<0>();  // no copy may be in flight when the wave ends
  __syncthreads();
  if (group_a) __syncthreads();

  // ---- epilogue: O = vscale acc / l, lse = (m - 4 + log2 l) ln 2
  const float lt = pair_sum(st.l);
  const float inv = lt > 0.f ? vscale / lt : 0.f;
  const float lse_v =
      lt > 0.f ? (st.m - kBias + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  if (qrow < Nq) {
    const int64_t orow = ((int64_t)(b * Hq + hq) * Nq + qrow) * D;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
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
    if (h == 0) lse[(int64_t)(b * Hq + hq) * Nq + qrow] = lse_v;
  }
}

template <bool CAUSAL, bool OUT_F32>
hipError_t launch(const void* q, const void* k, const void* vt,
                  const float* qd, const float* kd, const float* vd, void* o,
                  float* lse, const Shape& s, int ldv, hipStream_t stream) {
  const int n_qblk = (s.Nq + BR - 1) / BR;
  const long long n_items = (long long)s.B * s.Hq * n_qblk;
  const float c2 = fmaxf(s.scale * kLog2e, 1.17549435e-38f);
  hipLaunchKernelGGL((prefill_fp8_kernel<CAUSAL, OUT_F32>),
                     dim3((unsigned)n_items), dim3(NT), 0, stream,
                     static_cast<const uint8_t*>(q),
                     static_cast<const uint8_t*>(k),
                     static_cast<const uint8_t*>(vt), qd, kd, vd, o, lse, s.Hq,
                     s.Hkv, s.Nq, s.Nk, ldv, c2, n_qblk, (int)n_items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp8(const void* q, const void* k, const void* vt,
                              const float* q_descale, const float* k_descale,
                              const float* v_descale, void* o, float* lse,
                              const Shape& s, int ldv, bool out_f32,
                              hipStream_t stream) {
  if (s.d != D) return hipErrorInvalidValue;
  if (s.causal)
    return out_f32 ? launch<true, true>(q, k, vt, q_descale, k_descale,
                                        v_descale, o, lse, s, ldv, stream)
                   : launch<true, false>(q, k, vt, q_descale, k_descale,
                                         v_descale, o, lse, s, ldv, stream);
  return out_f32 ? launch<false, true>(q, k, vt, q_descale, k_descale,
                                       v_descale, o, lse, s, ldv, stream)
                 : launch<false, false>(q, k, vt, q_descale, k_descale,
                                        v_descale, o, lse, s, ldv, stream);
}

}  // namespace fa

// Tiled attention forward (prefill): one workgroup per (batch, query head,
// block of 256 query rows), 8 waves of 32 query rows each.
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
//   last key return zeros, so tails need no branches.  K is stored
//   column-major in 16-byte chunks (chunk c of all 64 rows is one
//   contiguous KiB), V row-major with 8-byte chunks XOR-swizzled by row:
//   each DMA instruction then reads from a per-lane base plus a scalar
//   offset, the operand reads of a wave hit distinct banks, and every read
//   address is a per-lane base plus an immediate.
// * Matrix cores and vector ALUs are kept busy together by running the two
//   halves of the workgroup half a block apart ("ping-pong"): waves 0-3 and
//   waves 4-7 share the SIMDs pairwise, and between two workgroup barriers
//   one group issues its matrix products (P_{j-1} V_{j-1}, then
//   S_j = Q K_j^T) while the other group does its softmax, then they swap.
//   A wave raises its issue priority during its matrix phase.
// * The rescale is lazy: the reference max m used for the exponentials
//   moves only when a block's weights against it would exceed 2^64 (or a
//   row has no reference yet), so almost every block skips both the row
//   max and the 64 multiplies per lane of the output rescale.  The result
//   is the same real-arithmetic quantity: m cancels in O = acc / l and in
//   lse = m + log l, and weights up to 2^64 keep every sum far inside the
//   fp32 range.
// * Causal: K/V blocks past the diagonal are never loaded; a wave whose rows
//   all precede a block skips its math for that block; masking runs only on
//   blocks that cross the wave's diagonal or the key tail.  Heavy Q blocks
//   (late rows) are scheduled first, and the query heads of one KV-head
//   group run next to each other on the same XCD so that they share K/V in
//   its L2.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BR = kPrefillRows;   // 256 query rows per workgroup
constexpr int BC = kPrefillKeys;   // 64 keys per K/V block
constexpr int NW = BR / 32;        // 8 waves
constexpr int NT = 64 * NW;
constexpr float kMaxLaneSum = 1.8446744e19f;  // 2^64

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

// LDS row position of key j (within a 64-key tile): bits 2 and 3 swapped.
__device__ __forceinline__ int key_slot(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

template <int D>
struct Layout {
  static constexpr int ROWB = 2 * D;          // bytes of one K/V row
  static constexpr int KBYTES = BC * ROWB;    // one K buffer (16 KiB at 128)
  static constexpr int VBYTES = BC * ROWB;    // one V buffer
  static constexpr int NS = 4;                // ring stages of K and of V
  static constexpr int VBASE = NS * KBYTES;   // [K0..K3 | V0..V3]
  static constexpr int TOTAL = NS * (KBYTES + VBYTES);
  static constexpr int NINS = KBYTES / 1024;  // 1 KiB DMA instructions
  static constexpr int NTILE = D / 32;        // O^T accumulator tiles
  static constexpr int NSTEP = D / 16;        // k-steps of the score product
};

// V swizzle: 8-byte chunk u of row r is stored at u ^ vswz(r).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 8 * (r & 3) : 8 * ((r >> 1) & 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base,
                                                       uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

// Starts the HBM -> LDS copy of block `blk` (64 rows) of one K or V head
// (`head`: its row 0; rows `rsb` bytes apart) into the LDS buffer at `dst`,
// shared by the NW waves: wave w issues 1 KiB buffer_load ... lds
// instructions i = w, w + NW, ...; instruction i reads from lane offset
// `lane_off` plus `step * i` bytes.  Rows at or past Nk read as zeros
// (buffer range check on the per-instruction resource, which ends at the
// end of row Nk - 1); a block wholly past Nk is a copy of zeros, which
// keeps the number of copies per loop iteration fixed.
template <int D>
__device__ __forceinline__ void copy_block(char* dst, const char* head,
                                           int Nk, int blk, int wave,
                                           uint32_t lane_off, int step,
                                           int rsb) {
  // (Nk here: number of rows that may be read; later rows read as zeros.
  // A head spans less than 2^31 bytes, so 32-bit offsets suffice.)
  using L = Layout<D>;
  const int kb = min(blk * BC, Nk);
  const char* base = head + (int64_t)kb * rsb;
  const int rem = kb < Nk ? (Nk - kb - 1) * rsb + L::ROWB : 0;
#pragma unroll
  for (int n = 0; n < L::NINS / NW; ++n) {
    const int i = wave + NW * n;
    const int left = rem - step * i;
    const __amdgpu_buffer_rsrc_t r =
        rsrc(base + step * i, (uint32_t)(left > 0 ? left : 0));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)(dst + 1024 * i), 16, lane_off, 0, 0, 0);
  }
}

// s_waitcnt with vmcnt = N (expcnt, lgkmcnt left free); gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Running softmax state of one lane (one query row, half of its keys).
struct RowState {
  float m;   // reference max in use, log2 units
  float l;   // sum of the fp32 weights (gives lse)
  float lb;  // sum of the bf16-rounded weights (normalises O)
};

// Matrix phase of one wave for block j: O^T += V_{j-1}^T P_{j-1}^T (if
// PV), then S_j^T = K_j Q^T (if QK), 32-key halves into s0 / s1.
//   kp: lane K read address in buffer j;  vp: lane V read addresses (per
//   output tile) in buffer j - 1.
// The operand reads run DEPTH matrix products ahead of their use (the
// order is pinned with sched_barrier): in this phase only one wave per SIMD
// issues matrix products, so an exposed LDS round trip would idle the
// matrix core.
template <int D, bool PV, bool QK>
__device__ __forceinline__ void matrix_phase(const char* kp,
                                             const char* const* vp,
                                             const bf16x8* qf,
                                             const u32x4* pk, f32x16* acc,
                                             f32x16& s0, f32x16& s1) {
  using L = Layout<D>;
  constexpr int NPV = PV ? 4 * L::NTILE : 0;  // P V products (s, tile)
  constexpr int NQK = QK ? 2 * L::NSTEP : 0;  // score products (t, half)
  constexpr int NOP = NPV + NQK;
  constexpr int DEPTH = 4;
  i16x4 vlo[NPV > 0 ? NPV : 1], vhi[NPV > 0 ? NPV : 1];
  bf16x8 kop[NQK > 0 ? NQK : 1];
  // Issue order: P V and score products alternate (when both are present)
  // so that two products on the same accumulator are several slots apart.
  // Product index i < NPV: P V product i; otherwise score product i - NPV.
  auto order = [&](int slot) {
    if (NPV == 0 || NQK == 0) return slot;
    const int k = slot >> 1;
    if (NPV == NQK) return (slot & 1) ? NPV + k : k;
    return slot < 2 * (NPV < NQK ? NPV : NQK) ? ((slot & 1) ? NPV + k : k)
                                              : slot;  // not reached
  };
  // operand read of product i
  auto read = [&](int i) {
    if (i < NPV) {
      const int s = i / L::NTILE, tt = i % L::NTILE;
      const char* a0 = vp[tt] + s * 16 * L::ROWB;
      vlo[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)((lds_char*)a0));
      vhi[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)((lds_char*)(a0 + 4 * L::ROWB)));
    } else {
      const int q = i - NPV, t = q >> 1, half = q & 1;
      // chunk 2t + h of LDS rows col (+ 32 for the second half)
      kop[q] = *reinterpret_cast<const bf16x8*>(kp + 2048 * t + 512 * half);
    }
  };
  if (QK) {
    s0 = f32x16{};
    s1 = f32x16{};
  }
  static_assert(NPV == 0 || NQK == 0 || NPV == NQK, "product counts");
#pragma unroll
  for (int i = 0; i < DEPTH && i < NOP; ++i) read(order(i));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int slot = 0; slot < NOP; ++slot) {
    if (slot + DEPTH < NOP) read(order(slot + DEPTH));
    const int i = order(slot);
    if (i < NPV) {
      const int s = i / L::NTILE, tt = i % L::NTILE;
      u32x4 va;
      va[0] = __builtin_bit_cast(u32x2, vlo[i])[0];
      va[1] = __builtin_bit_cast(u32x2, vlo[i])[1];
      va[2] = __builtin_bit_cast(u32x2, vhi[i])[0];
      va[3] = __builtin_bit_cast(u32x2, vhi[i])[1];
      acc[tt] = mfma32x32x16(__builtin_bit_cast(bf16x8, va),
                             __builtin_bit_cast(bf16x8, pk[s]), acc[tt]);
    } else {
      const int q = i - NPV, t = q >> 1;
      if (q & 1)
        s1 = mfma32x32x16(kop[q], qf[t], s1);
      else
        s0 = mfma32x32x16(kop[q], qf[t], s0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Softmax phase of one wave for block j: optional mask (`lim`: last
// visible key relative to this lane's first key of the block; register r of
// half 0 holds relative key 16(r/8) + r%8, half 1 adds 32; with a band,
// also `lo`: the first visible key, same reference), weights
// p = 2^(s c2 - m) against the reference max m, rounded to bf16 once into
// pk, and the row sums.  When the weights would grow past 2^64 (or a row
// has no reference yet) the block is redone with m moved to the row max;
// then the state is rescaled and true is returned, with the factor in
// `alpha`, because the accumulators must be scaled before the next P V.
// The rounded weights feed P V and their own row sum lb, so O = acc / lb
// is an exact convex combination of V rows up to fp32 summation; the fp32
// sum l of the unrounded weights gives lse.
// With COL, a column-interval mask as well: bit i of `cbits` hides this
// lane's key of score register i (i < 16: s0, else s1 register i - 16).
template <bool MASK, bool LOWER = false, bool COL = false>
__device__ __forceinline__ bool softmax_phase(const f32x16& s0,
                                              const f32x16& s1, int lim,
                                              int lo, float c2, RowState& st,
                                              float& alpha, u32x4* pk,
                                              uint32_t cbits = 0) {
  // The mask never overwrites the score registers (that would make the
  // masked and unmasked variants rejoin with copies): hidden keys are left
  // out of the max and get weight 0 after the exponential.
  auto hidden = [&](int key) {
    return MASK && (key > lim || (LOWER && key < lo));
  };
  auto hide0 = [&](int r) {
    return hidden(16 * (r >> 3) + (r & 7)) | (COL && ((cbits >> r) & 1u));
  };
  auto hide1 = [&](int r) {
    return hidden(16 * (r >> 3) + (r & 7) + 32) |
           (COL && ((cbits >> (16 + r)) & 1u));
  };
  // weights p = 2^(s c2 - msub) (0 for hidden keys), rounded to bf16 once
  // into pk; partial sums of the fp32 and of the rounded weights
  auto weights = [&](float msub, float* rs, float* rb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rs[i] = 0.f;
      rb[i] = 0.f;
    }
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
      rs[0] += e0;
      rs[1] += e1;
      rs[2] += e2;
      rs[3] += e3;
      const uint32_t a = pack_bf16x2(e0, e1);
      const uint32_t c = pack_bf16x2(e2, e3);
      pk[r >> 3][(r >> 1) & 3] = a;
      pk[2 + (r >> 3)][(r >> 1) & 3] = c;
      if (r & 2) {
        rb[2] = add_bf16x2(a, rb[2]);
        rb[3] = add_bf16x2(c, rb[3]);
      } else {
        rb[0] = add_bf16x2(a, rb[0]);
        rb[1] = add_bf16x2(c, rb[1]);
      }
    }
  };
  float rs[4], rb[4];
  // Fast path: the weights against the reference max m in use, without
  // looking for the block's max.  They are kept when every lane's sum stays
  // at most 2^64 (so every weight is <= 2^64, and the running sums and
  // accumulators stay far inside fp32 range); otherwise, and while a row
  // has no reference max yet, the block is redone below.
  weights(st.m, rs, rb);
  const float lsum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
  const bool redo = __builtin_amdgcn_ballot_w64(!(lsum <= kMaxLaneSum) ||
                                                st.m == -INFINITY) != 0;
  if (!redo) {
    st.l += lsum;
    st.lb += (rb[0] + rb[1]) + (rb[2] + rb[3]);
    return false;
  }
  // Slow path: the row max of the block (four independent max3 chains,
  // then combined); the reference moves to it where it grew, the state is
  // rescaled, and the weights are recomputed.
  float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int r = 0; r < 16; ++r)
    mq[r & 3] = fmaxf(fmaxf(mq[r & 3], hide0(r) ? -INFINITY : s0[r]),
                      hide1(r) ? -INFINITY : s1[r]);
  float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
  mx = pair_max(mx) * c2;
  const float m_new = fmaxf(st.m, mx);
  // unchanged rows (including rows with nothing visible yet) keep factor
  // 1; a first visible key gives 2^-inf = 0
  alpha = (m_new == st.m) ? 1.f : exp2_fast(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
  st.lb *= alpha;
  weights((st.m == -INFINITY) ? 0.f : st.m, rs, rb);
  st.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  st.lb += (rb[0] + rb[1]) + (rb[2] + rb[3]);
  return true;
}

// Mask modes: kNone, kCausal (key j visible to row i iff j <= i + Nk - Nq),
// kBand (iff i + Nk - Nq - wl <= j <= i + Nk - Nq + wr, wl and wr >= 0).
constexpr int kNone = 0, kCausal = 1, kBand = 2;

template <int D, int MODE, bool OUT_F32, bool SPARSE = false,
          bool COLUMN = false>
__global__ __launch_bounds__(NT, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int Nq_max, int Nk_max,
    float c2, int n_qblk, int n_items, SeqLayout lay, int wl, int wr,
    BlockMask bmask, ColMask cmask) {
  constexpr bool CAUSAL = MODE == kCausal;
  constexpr bool BAND = MODE == kBand;
  static_assert(!(SPARSE && BAND), "block masks go with no mask or causal");
  static_assert(!(COLUMN && (SPARSE || BAND)),
                "column masks go with no mask or causal");
  // a list of key blocks in LDS drives the loop (block or column mask)
  constexpr bool LISTED = SPARSE || COLUMN;
  constexpr int BLKBITS = COLUMN ? 0xFFFF : 0xFFFFFF;
  using L = Layout<D>;
  // block-sparse: the key blocks this workgroup computes, in order (bits
  // 0..23 the block, bit 24 / 25 set when the rows of group A / B use it),
  // then their count
  __shared__ int blist[LISTED ? kSparseMaxKeyBlocks + 1 : 1];
  constexpr int NTILE = L::NTILE;
  constexpr int NSTEP = L::NSTEP;
  __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_a = wave < NW / 2;
  const int h = lane >> 5, col = lane & 31;

  // ---- work item: (b, kv head, Q block, head in group); heavy blocks first
  const int G = Hq / Hkv;
  int g, jq, bh;  // bh = b * Hkv + hkv
  if (lay.cu_q) {
    // packed batch of unequal sequences: unit u = (Q block rank jq, bh),
    // jq outermost, so the blocks of every sequence are ordered by their
    // index from the top (the heaviest first under the causal mask).  Unit
    // u runs on XCD u % 8 and its G query heads one after another there
    // (they read the same K/V), so every XCD takes every 8th unit of the
    // ordered list.  The grid is the unit count times G, rounded up to a
    // multiple of 8 G; the surplus workgroups exit here.
    const int s8 = blockIdx.x >> 3;
    g = s8 % G;
    const int u = 8 * (s8 / G) + (blockIdx.x & 7);
    const int n_bh = lay.n_seq * Hkv;
    if (u >= n_bh * n_qblk) return;
    jq = u / n_bh;
    bh = u % n_bh;
  } else {
    // equal sequences: each XCD takes one contiguous range of items
    // (b, kv head, Q block, head in group), so a KV head's Q blocks share
    // that XCD's L2
    const int item = xcd_contiguous(blockIdx.x, n_items);
    g = item % G;
    const int t1 = item / G;
    jq = t1 % n_qblk;
    bh = t1 / n_qblk;
  }
  const int qblk = MODE != kNone ? (n_qblk - 1 - jq) : jq;
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int hq = hkv * G + g;
  const int q0 = qblk * BR;

  // this sequence's rows: element offsets of its row 0 in this head
  int Nq = Nq_max, Nk = Nk_max;
  int64_t qbase, kbase, vbase, obase, lbase;
  if (lay.cu_q) {
    // packed variable-length batch; lengths clamped into the packed
    // tensors whatever the offsets hold
    const int qs = min(max(lay.cu_q[b], 0), lay.total_q);
    const int ks = min(max(lay.cu_k[b], 0), lay.total_k);
    Nq = min(min(max(lay.cu_q[b + 1] - qs, 0), lay.total_q - qs), Nq_max);
    Nk = min(min(max(lay.cu_k[b + 1] - ks, 0), lay.total_k - ks), Nk_max);
    qbase = qs * lay.q_r + hq * lay.q_h;
    kbase = ks * lay.k_r + hkv * lay.k_h;
    vbase = ks * lay.v_r + hkv * lay.v_h;
    obase = qs * lay.o_r + hq * lay.o_h;
    lbase = qs * lay.l_r + hq * lay.l_h;
  } else {
    qbase = b * lay.q_b + hq * lay.q_h;
    kbase = b * lay.k_b + hkv * lay.k_h;
    vbase = b * lay.v_b + hkv * lay.v_h;
    obase = b * lay.o_b + hq * lay.o_h;
    lbase = b * lay.l_b + hq * lay.l_h;
  }
  // a Q block past this sequence's rows has nothing to do (the test is
  // uniform over the workgroup, so no wave is left at a barrier)
  if (q0 >= Nq) return;
  const int off = Nk - Nq;
  const int rsb = (int)(2 * lay.k_r);   // bytes between K rows
  const int rsbv = (int)(2 * lay.v_r);  // bytes between V rows
  const char* kh = reinterpret_cast<const char*>(k + kbase);
  const char* vh = reinterpret_cast<const char*>(v + vbase);

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, q0 + BR + off);
  // band: keys from the first row's lower bound to the last row's upper one
  int j0 = 0;
  if (BAND) {
    kv_end = min(Nk, min(q0 + BR, Nq) + off + wr);
    j0 = max(0, q0 + off - wl) / BC;
  }
  const int nblk = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // ---- block-sparse: wave 0 lists the key blocks below nblk that either
  // 128-row half of this workgroup keeps (mask rows 2 qblk and 2 qblk + 1)
  int n_act = nblk;
  if (SPARSE) {
    if (wave == 0) {
      const uint8_t* ma = bmask.mask + b * bmask.mb + hq * bmask.mh +
                          (int64_t)(2 * qblk) * bmask.nkb;
      const bool has_b = q0 + BR / 2 < Nq;
      int cnt = 0;
      for (int base = 0; base < nblk; base += 64) {
        const int i = base + lane;
        const bool ua = i < nblk && ma[i] != 0;
        const bool ub = i < nblk && has_b && ma[bmask.nkb + i] != 0;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(ua || ub);
        const int pos =
            cnt + (int)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (ua || ub) blist[pos] = i | (ua ? 1 << 24 : 0) | (ub ? 1 << 25 : 0);
        cnt += (int)__builtin_popcountll(bal);
      }
      if (lane == 0) blist[kSparseMaxKeyBlocks] = cnt;
    }
    __syncthreads();
    n_act = __builtin_amdgcn_readfirstlane(blist[kSparseMaxKeyBlocks]);
  }
  // ---- column mask: every wave classifies the key blocks wave, wave + NW,
  // ... below nblk (lane = key of the block) into blist[block]: bits 0..15
  // the block, bit 16 + w set when some key of the block is hidden from
  // some row of wave w (that wave then tests every key), bits 24 / 25 when
  // some row of half A / B may see some key.  Wave 0 then drops the blocks
  // neither half sees, in place and in order.
  if (COLUMN) {
    const int* cb = cmask.bounds + 2 * ((int64_t)b * cmask.mb);
    constexpr int UNR = 4;
    for (int kb0 = wave; kb0 < nblk; kb0 += UNR * NW) {
      int blo[UNR], bhi[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int key = (kb0 + NW * u) * BC + lane;
        blo[u] = 0;
        bhi[u] = 0;
        if (kb0 + NW * u < nblk && key < kv_end) {
          const int2 x = *reinterpret_cast<const int2*>(cb + 2 * key);
          blo[u] = x.x;
          bhi[u] = x.y;
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int kb = kb0 + NW * u;
        if (kb >= nblk) break;
        const int key = kb * BC + lane;
        const bool valid = key < kv_end;
        // rows that may see this key: its interval, and (causal) from its
        // place on
        const int vlo = CAUSAL ? max(blo[u], key - off) : blo[u];
        const int vhi = bhi[u];
        uint32_t bits = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int r0 = q0 + 32 * w, r1 = min(r0 + 32, Nq);
          const bool all_vis =
              r0 >= r1 || !valid || (blo[u] <= r0 && bhi[u] >= r1);
          if (__builtin_amdgcn_ballot_w64(all_vis) != ~0ull)
            bits |= 1u << (16 + w);
        }
        const int ha1 = min(q0 + BR / 2, Nq), hb1 = min(q0 + BR, Nq);
        if (__builtin_amdgcn_ballot_w64(valid && vlo < ha1 && vhi > q0 &&
                                        vlo < vhi) != 0)
          bits |= 1u << 24;
        if (__builtin_amdgcn_ballot_w64(valid && vlo < hb1 &&
                                        vhi > q0 + BR / 2 && vlo < vhi) != 0)
          bits |= 1u << 25;
        if (lane == 0) blist[kb] = kb | (int)bits;
      }
    }
    __syncthreads();
    if (wave == 0) {
      int cnt = 0;
      for (int base = 0; base < nblk; base += 64) {
        const int i = base + lane;
        const int e = i < nblk ? blist[i] : 0;
        const bool kept = ((e >> 24) & 3) != 0;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(kept);
        const int pos =
            cnt + (int)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
        // (every lane has read its entry before any lane writes, and an
        // entry moves only down, never past an unread one)
        if (kept) blist[pos] = e;
        cnt += (int)__builtin_popcountll(bal);
      }
      if (lane == 0) blist[kSparseMaxKeyBlocks] = cnt;
    }
    __syncthreads();
    n_act = __builtin_amdgcn_readfirstlane(blist[kSparseMaxKeyBlocks]);
  }
  // key block at ring position p: p itself, or the p-th listed block (past
  // the list: a block past Nk, whose copies are zeros)
  auto blk_at = [&](int p) {
    if (!LISTED) return p;
    return p < n_act ? __builtin_amdgcn_readfirstlane(blist[p] & BLKBITS)
                     : nblk + 1;
  };

  // this wave's rows: blocks from w_mask on may hide keys from one of them
  // (past the causal limit of its first row, or past Nk)
  const int wrow0 = q0 + wave * 32;
  int w_mask = Nk / BC;
  if (CAUSAL) w_mask = min(w_mask, max(0, wrow0 + off + 1) / BC);
  // band: also blocks before w_lo may hide keys (below the lower bound of
  // the wave's last row)
  int w_lo = 0;
  if (BAND) {
    w_mask = min(w_mask, max(0, wrow0 + off + wr + 1) / BC);
    w_lo = (max(0, wrow0 + 31 + off - wl) + BC - 1) / BC;
  }

  // ---- per-lane DMA source offsets.  K: instruction i copies 16-byte
  // chunk i of all 64 rows (lane = LDS row, holding key key_slot(lane)).
  // V: instruction i copies the rows of its KiB, lane -> (row, chunk) with
  // the 16-byte chunk index XOR-swizzled by the row.
  const uint32_t k_off = (uint32_t)(key_slot(lane) * rsb);
  uint32_t v_off;
  {
    const int row = lane / (L::ROWB / 16);   // row within the KiB
    const int p = lane % (L::ROWB / 16);     // physical 16-byte chunk
    v_off = (uint32_t)(row * rsbv) + ((p ^ (vswz<D>(row) >> 1)) * 16);
  }
  const int v_step = (1024 / L::ROWB) * rsbv;  // rows of one KiB

  // ---- Q^T operand fragments: lane holds q[row][16t + 8h .. +7]
  const int qrow = wrow0 + col;
  bf16x8 qf[NSTEP];
  {
    const bool ok = qrow < Nq;
    const uint16_t* qp = q + qbase + (ok ? qrow : 0) * lay.q_r + 8 * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      u32x4 x = ok ? ldg16(qp + 16 * t) : u32x4{0u, 0u, 0u, 0u};
      qf[t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 acc[NTILE];
#pragma unroll
  for (int i = 0; i < NTILE; ++i) acc[i] = f32x16{};
  RowState st{-INFINITY, 0.f, 0.f};

  // per-lane LDS read bases.  K: chunk 2t + h of LDS row col sits at
  // (2t + h) KiB + 16 col.  V (transposing read): 16-lane group lg, lane lp
  // reads row 8(lg/2) + lp/4 (+16 s, +4), 8-byte chunk 8 tt + 4(lg%2) +
  // lp%4, swizzled by the row.
  const int k_rd = 1024 * h + 16 * col;
  const int lg = lane >> 4, lp = lane & 15;
  int v_rd[NTILE];
  {
    const int vrow = 8 * (lg >> 1) + (lp >> 2);
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
      const int u = 8 * tt + 4 * (lg & 1) + (lp & 3);
      v_rd[tt] = L::VBASE + vrow * L::ROWB + ((u ^ vswz<D>(vrow)) * 8);
    }
  }
  // this lane's row limit relative to its first key of block 0
  const int lim0 = (CAUSAL ? min(Nk - 1, qrow + off)
                    : BAND ? min(Nk - 1, qrow + off + wr)
                           : Nk - 1) - 8 * h;
  const int lo0 = BAND ? qrow + off - wl - 8 * h : 0;

  f32x16 s0, s1;    // scores of the block in flight
  u32x4 pk[4];      // bf16 weights of the previous block

  // matrix phase for block j: P_{j-1} V_{j-1} (P is zero before block 0),
  // then the scores of block j when QK
  bool rescale = false;  // scale acc by alpha before the next P V
  float alpha = 1.f;
  // (block-sparse: `pv` / `qk` false skip the products of a block this
  // wave's half does not keep)
  auto mphase = [&](int j, auto qk_tag, bool pv = true, bool qk = true) {
    if (rescale) {
#pragma unroll
      for (int i = 0; i < NTILE; ++i) acc[i] *= alpha;
    }
    const char* vp[NTILE];
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt)
      vp[tt] = smem + ((j + L::NS - 1) % L::NS) * L::VBYTES + v_rd[tt];
    const char* kp = smem + (j % L::NS) * L::KBYTES + k_rd;
    constexpr bool QK = decltype(qk_tag)::value;
    __builtin_amdgcn_s_setprio(1);
    if (!LISTED || (pv && qk)) {
      matrix_phase<D, true, QK>(kp, vp, qf, pk, acc, s0, s1);
    } else if (pv) {
      matrix_phase<D, true, false>(kp, vp, qf, pk, acc, s0, s1);
    } else if (QK && qk) {
      matrix_phase<D, false, QK>(kp, vp, qf, pk, acc, s0, s1);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- K/V ring: NS = 4 stages each; block b's K and V live in stage
  // b % 4.  In iteration j every wave issues its share of the copies of
  // K_{j+3} and V_{j+2} at the start of its softmax phase (vector memory
  // issue then overlaps vector ALU work).  A stage is refilled only after
  // both groups' last reads of it.  The copies are complete at the
  // iteration's closing barrier: its release fence waits for every
  // outstanding direct-to-LDS copy (they write LDS), so the explicit waits
  // below only state the weakest order the ring needs (the first reader of
  // K_{j+3} / V_{j+2} is group A's matrix phase of iteration j+3).
  constexpr int OPS = 2 * (L::NINS / NW);  // copy instructions per wave
  const int kv_rows = max(kv_end, 0);      // rows past this are not needed
  auto copies = [&](int j) {
    copy_block<D>(smem + ((j + 3) % L::NS) * L::KBYTES, kh, kv_rows,
                  blk_at(j + 3), wave, k_off, 16, rsb);
    copy_block<D>(smem + L::VBASE + ((j + 2) % L::NS) * L::VBYTES, vh,
                  kv_rows, blk_at(j + 2), wave, v_off, v_step, rsbv);
  };
  // prologue: K_j0, K_j0+1, K_j0+2, V_j0, V_j0+1 (all waves), fully
  // waited (j0 = 0 unless a band starts later).  The V stage before j0 is
  // zeroed: block j0's matrix phase multiplies it by the all-zero
  // "previous" P, and 0 * (stale NaN/Inf bits) would not be 0.
#pragma unroll
  for (int b0 = 0; b0 < 3; ++b0)
    copy_block<D>(smem + ((j0 + b0) % L::NS) * L::KBYTES, kh, kv_rows,
                  blk_at(j0 + b0), wave, k_off, 16, rsb);
#pragma unroll
  for (int b0 = 0; b0 < 2; ++b0)
    copy_block<D>(smem + L::VBASE + ((j0 + b0) % L::NS) * L::VBYTES, vh,
                  kv_rows, blk_at(j0 + b0), wave, v_off, v_step, rsbv);
#pragma unroll
  for (int i = tid; i < L::VBYTES / 16; i += NT)
    reinterpret_cast<u32x4*>(smem + L::VBASE +
                             ((j0 + L::NS - 1) % L::NS) * L::VBYTES)[i] =
        u32x4{0u, 0u, 0u, 0u};
  wait_vmcnt<0>();
  __syncthreads();

  // ---- main loop.  Every wave runs the same code, one barrier after each
  // phase; group B enters one barrier late (an extra barrier before the
  // loop) and group A leaves one late (an extra barrier at the end).
  // Barrier n of one group then meets barrier n+1 of the other, so while
  // group A runs the matrix phase of block j, group B runs the softmax of
  // block j-1, and while A runs the softmax of j, B runs the matrix phase
  // of j.  A block past all of a wave's rows (causal) goes through the
  // masked softmax and contributes zero weights.
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = u32x4{0u, 0u, 0u, 0u};
  if (!group_a) __syncthreads();
  // (ring position j holds key block jb: j itself, or the j-th listed
  // block of a block-sparse mask; a listed block that this wave's half does
  // not keep goes through the masked softmax with every key hidden)
  bool keep_prev = false;  // block-sparse: this half kept position j - 1
  for (int j = j0; j < n_act; ++j) {
    int jb = j;
    bool keep = true;
    bool colm = false;  // column mask: this wave tests every key
    if (LISTED) {
      const int e = __builtin_amdgcn_readfirstlane(blist[j]);
      jb = e & BLKBITS;
      keep = (e >> (group_a ? 24 : 25)) & 1;
      if (COLUMN) colm = keep && ((e >> (16 + wave)) & 1);
    }
    // the row bounds of the block's keys, one per lane, loaded before the
    // matrix phase (keys past Nk are hidden by the limit anyway)
    int clo = 0, chi = 0;
    if (COLUMN && colm) {
      const int key = jb * BC + lane;
      if (key < Nk) {
        const int2 x = *reinterpret_cast<const int2*>(
            cmask.bounds + 2 * ((int64_t)b * cmask.mb + key));
        clo = x.x;
        chi = x.y;
      }
    }
    mphase(j, std::true_type{}, keep_prev, keep);
    __syncthreads();
    copies(j);
    if (LISTED && !keep)
      rescale = false;  // nothing of this block enters this half's rows
    else if (COLUMN && colm) {
      // this lane's 32 keys against its row: key 16 (i / 8 % 2) + i % 8
      // + 8 h (+ 32 for i >= 16) of the block, its bounds fetched from the
      // lane that loaded them
      uint32_t cbits = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int r = i & 15;
        const int key = 16 * (r >> 3) + (r & 7) + 8 * h + 32 * (i >> 4);
        const int klo = __builtin_amdgcn_ds_bpermute(4 * key, clo);
        const int khi = __builtin_amdgcn_ds_bpermute(4 * key, chi);
        cbits |= (uint32_t)((qrow < klo) | (qrow >= khi)) << i;
      }
      rescale = softmax_phase<true, false, true>(s0, s1, lim0 - jb * BC, 0,
                                                 c2, st, alpha, pk, cbits);
    }
    else if (jb >= w_mask || (BAND && jb < w_lo))
      rescale = softmax_phase<true, BAND>(s0, s1, lim0 - jb * BC,
                                          lo0 - jb * BC, c2, st, alpha, pk);
    else
      rescale = softmax_phase<false>(s0, s1, lim0 - jb * BC, 0, c2, st,
                                     alpha, pk);
    keep_prev = keep;
    if (group_a)
      wait_vmcnt<2 * OPS>();  // own copies of iteration j-2 have landed
    else
      wait_vmcnt<OPS>();      // own copies of iteration j-1 have landed
    __syncthreads();
  }
  if (n_act > j0)  // P V of the last block
    mphase(n_act, std::false_type{}, LISTED ? keep_prev : true);
  __syncthreads();
  if (group_a) __syncthreads();

  // ---- epilogue: O = O / lb, lse = (m + log2 l) ln 2
  const float lt = pair_sum(st.l);
  const float lbt = pair_sum(st.lb);
  const float inv = lbt > 0.f ? 1.f / lbt : 0.f;
  const float lse_v =
      lt > 0.f ? (st.m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  if (qrow < Nq) {
    const int64_t orow = obase + qrow * lay.o_r;
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
    if (h == 0) lse[lbase + qrow * lay.l_r] = lse_v;
  }
}

template <int D, int MODE, bool OUT_F32, bool SPARSE = false,
          bool COLUMN = false>
hipError_t launch(const void* q, const void* k, const void* v, void* o,
                  float* lse, const Shape& s, const SeqLayout& lay, int wl,
                  int wr, hipStream_t stream, const BlockMask& bm = {},
                  const ColMask& cm = {}) {
  const int n_qblk = (s.Nq + BR - 1) / BR;
  long long n_items = (long long)s.B * s.Hq * n_qblk;
  // packed batch: whole rounds of 8 units of G heads (the tail's surplus
  // workgroups exit at once)
  if (lay.cu_q) {
    const long long per = 8LL * (s.Hq / s.Hkv);
    const long long units = (long long)s.B * s.Hkv * n_qblk;
    n_items = (units + 7) / 8 * per;
  }
  // scale 0 is run as the smallest normal scale: every exponent is then
  // below 2^-24 in magnitude, so each weight is exactly 1, and -inf scores
  // stay -inf (no 0 * inf)
  const float c2 = fmaxf(s.scale * kLog2e, 1.17549435e-38f);
  hipLaunchKernelGGL((prefill_kernel<D, MODE, OUT_F32, SPARSE, COLUMN>),
                     dim3((unsigned)n_items), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), o, lse, s.Hq, s.Hkv,
                     s.Nq, s.Nk, c2, n_qblk, (int)n_items, lay, wl, wr, bm,
                     cm);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_mode(const void* q, const void* k, const void* v, void* o,
                       float* lse, const Shape& s, const SeqLayout& lay,
                       int wl, int wr, bool out_f32, hipStream_t stream) {
  return out_f32 ? launch<D, MODE, true>(q, k, v, o, lse, s, lay, wl, wr,
                                         stream)
                 : launch<D, MODE, false>(q, k, v, o, lse, s, lay, wl, wr,
                                          stream);
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o,
                    float* lse, const Shape& s, const SeqLayout& lay,
                    bool out_f32, hipStream_t stream) {
  const MaskBounds m = mask_bounds(s);
  if (m.kind == 0)
    return launch_mode<D, kNone>(q, k, v, o, lse, s, lay, 0, 0, out_f32,
                                 stream);
  if (m.kind == 1)
    return launch_mode<D, kCausal>(q, k, v, o, lse, s, lay, 0, 0, out_f32,
                                   stream);
  return launch_mode<D, kBand>(q, k, v, o, lse, s, lay, m.wl, m.wr, out_f32,
                               stream);
}

}  // namespace

template <int D>
hipError_t launch_sparse_d(const void* q, const void* k, const void* v,
                           void* o, float* lse, const Shape& s,
                           const BlockMask& bm, bool out_f32,
                           hipStream_t stream) {
  const SeqLayout lay = dense_layout(s);
  if (s.causal)
    return out_f32 ? launch<D, kCausal, true, true>(q, k, v, o, lse, s, lay,
                                                    0, 0, stream, bm)
                   : launch<D, kCausal, false, true>(q, k, v, o, lse, s, lay,
                                                     0, 0, stream, bm);
  return out_f32 ? launch<D, kNone, true, true>(q, k, v, o, lse, s, lay, 0, 0,
                                                stream, bm)
                 : launch<D, kNone, false, true>(q, k, v, o, lse, s, lay, 0,
                                                 0, stream, bm);
}

template <int D>
hipError_t launch_column_d(const void* q, const void* k, const void* v,
                           void* o, float* lse, const Shape& s,
                           const ColMask& cm, bool out_f32,
                           hipStream_t stream) {
  const SeqLayout lay = dense_layout(s);
  if (s.causal)
    return out_f32 ? launch<D, kCausal, true, false, true>(
                         q, k, v, o, lse, s, lay, 0, 0, stream, {}, cm)
                   : launch<D, kCausal, false, false, true>(
                         q, k, v, o, lse, s, lay, 0, 0, stream, {}, cm);
  return out_f32 ? launch<D, kNone, true, false, true>(q, k, v, o, lse, s, lay,
                                                       0, 0, stream, {}, cm)
                 : launch<D, kNone, false, false, true>(
                       q, k, v, o, lse, s, lay, 0, 0, stream, {}, cm);
}

hipError_t launch_prefill_column(const void* q, const void* k, const void* v,
                                 void* o, float* lse, const Shape& s,
                                 const ColMask& cm, bool out_f32,
                                 hipStream_t stream) {
  if (s.d == 128)
    return launch_column_d<128>(q, k, v, o, lse, s, cm, out_f32, stream);
  if (s.d == 64)
    return launch_column_d<64>(q, k, v, o, lse, s, cm, out_f32, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_sparse(const void* q, const void* k, const void* v,
                                 void* o, float* lse, const Shape& s,
                                 const BlockMask& bm, bool out_f32,
                                 hipStream_t stream) {
  if (s.d == 128)
    return launch_sparse_d<128>(q, k, v, o, lse, s, bm, out_f32, stream);
  if (s.d == 64)
    return launch_sparse_d<64>(q, k, v, o, lse, s, bm, out_f32, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s,
                          const SeqLayout& lay, bool out_f32,
                          hipStream_t stream) {
  if (s.d == 128)
    return launch_d<128>(q, k, v, o, lse, s, lay, out_f32, stream);
  if (s.d == 64) return launch_d<64>(q, k, v, o, lse, s, lay, out_f32, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

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
//   last key return zeros, so tails need no branches.  The copies stay in
//   flight across the loop's barriers (which carry no memory fence), up to
//   three blocks ahead at d = 128 and seven at d = 64 (a ring of 4 or 8
//   stages); explicit vmcnt waits order them.  K is stored
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

template <int D, int NS_ = 4>
struct Layout {
  static constexpr int ROWB = 2 * D;          // bytes of one K/V row
  static constexpr int KBYTES = BC * ROWB;    // one K buffer (16 KiB at 128)
  static constexpr int VBYTES = BC * ROWB;    // one V buffer
  static constexpr int NS = NS_;              // ring stages of K and of V
  static constexpr int VBASE = NS * KBYTES;   // [K stages | V stages]
  static constexpr int TOTAL = NS * (KBYTES + VBYTES);
  static constexpr int NINS = KBYTES / 1024;  // 1 KiB DMA instructions
  static constexpr int NTILE = D / 32;        // O^T accumulator tiles
  static constexpr int NSTEP = D / 16;        // k-steps of the score product
};

// V swizzle: 8-byte chunk u of row r is stored at u ^ vswz(r).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D >= 128 ? 8 * (r & 3) : 8 * ((r >> 1) & 1);
}

// One 1 KiB HBM -> LDS copy instruction (buffer_load_dwordx4 ... lds):
// lane l reads 16 bytes at byte offset voff of the buffer [base, base +
// bytes) (zeros past its end) and writes them to LDS at dst + 16 l.  It is
// written in assembly so that the compiler does not track it: its own
// tracking of such copies cannot tell ring stages apart and would wait for
// every copy in flight before each LDS read.  The explicit vmcnt waits of
// the caller order the copies.  (The copy reads its LDS address from M0, one
// wait state after M0 is written.)
__device__ __forceinline__ void dma16(char* dst, const char* base,
                                      uint32_t bytes, uint32_t voff) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const u32x4 r = {
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) &
          0xFFFFu,
      (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((lds_char*)dst));
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "{m0}"(m));
}

// Workgroup barrier that neither waits for outstanding copies nor lets the
// compiler move memory accesses across it (the explicit vmcnt waits before
// it give the order the ring needs).
__device__ __forceinline__ void barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// This lane's index, computed where it is used: the compiler can neither
// hoist nor merge it, so a loop does not keep it (or values derived from
// it) in a register across its busiest part, where a kept value would be
// spilled.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile(
      "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
      "v_mbcnt_hi_u32_b32 %0, -1, %0"
      : "=v"(l));
  return l;
}

// Starts the HBM -> LDS copy of block `blk` (64 rows) of one K or V head
// (`head`: its row 0; rows `rsb` bytes apart) into the LDS buffer at `dst`,
// shared by the NW waves: wave w issues 1 KiB buffer_load ... lds
// instructions i = w, w + NW, ...; instruction i reads from lane offset
// `lane_off` plus `step * i` bytes.  Rows at or past Nk read as zeros
// (buffer range check on the per-instruction resource, which ends at the
// end of row Nk - 1); a block wholly past Nk is a copy of zeros, which
// keeps the number of copies per loop iteration fixed.  `rowb`: bytes of a
// row in memory (2 d, less than the tile's row when the head dimension d is
// narrower than the tile); instructions i >= `zero_from` copy zeros (the K
// chunks of columns past d).
// The copy instructions of one block whose row 0 is at `base`, of which
// the first `rem` bytes may be read (0: a copy of zeros).
template <int D, int NWAVES = NW>
__device__ __forceinline__ void copy_rows(char* dst, const char* base,
                                          int rem, int wave,
                                          uint32_t lane_off, int step,
                                          int zero_from) {
  using L = Layout<D>;
#pragma unroll
  for (int n = 0; n < L::NINS / NWAVES; ++n) {
    const int i = wave + NWAVES * n;
    const int left = i < zero_from ? rem - step * i : 0;
    dma16(dst + 1024 * i, base + step * i, (uint32_t)(left > 0 ? left : 0),
          lane_off);
  }
}

template <int D, int NWAVES = NW>
__device__ __forceinline__ void copy_block(char* dst, const char* head,
                                           int Nk, int blk, int wave,
                                           uint32_t lane_off, int step,
                                           int rsb, int rowb,
                                           int zero_from = 1 << 30) {
  // (Nk here: number of rows that may be read; later rows read as zeros.
  // A head spans less than 2^31 bytes, so 32-bit offsets suffice.)
  // (a block before the first, blk < 0, is a copy of zeros too)
  const int kb = min(max(blk, 0) * BC, Nk);
  const char* base = head + (int64_t)kb * rsb;
  const int rem = (blk >= 0 && kb < Nk) ? (Nk - kb - 1) * rsb + rowb : 0;
  copy_rows<D, NWAVES>(dst, base, rem, wave, lane_off, step, zero_from);
}

// The same for a block of a paged cache: `roff` is the byte offset of the
// block's row 0 from `head` (its page's row), or negative for a block that
// is not read (a copy of zeros); rows from `rows` on read as zeros.  The
// block lies inside one page, so 32-bit lane offsets suffice.
template <int D>
__device__ __forceinline__ void copy_block_paged(char* dst, const char* head,
                                                 int64_t roff, int rows,
                                                 int wave, uint32_t lane_off,
                                                 int step, int rsb, int rowb,
                                                 int zero_from = 1 << 30) {
  const int rem = roff >= 0 ? (min(rows, BC) - 1) * rsb + rowb : 0;
  copy_rows<D>(dst, head + (roff >= 0 ? roff : 0), rem, wave, lane_off, step,
               zero_from);
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
// With COL, a column-interval mask as well: `cm` (LDS) holds one word per
// key of the block from this lane's first key on (key 8h of the block),
// whose bit `crow` (this lane's row within its wave) says whether the row
// may see the key.
template <bool MASK, bool LOWER = false, bool COL = false>
__device__ __forceinline__ bool softmax_phase(const f32x16& s0,
                                              const f32x16& s1, int lim,
                                              int lo, float c2, RowState& st,
                                              float& alpha, u32x4* pk,
                                              const uint32_t* cm = nullptr,
                                              int crow = 0) {
  // The mask never overwrites the score registers (that would make the
  // masked and unmasked variants rejoin with copies): hidden keys are left
  // out of the max and get weight 0 after the exponential.
  auto hidden = [&](int key) {
    return MASK && (key > lim || (LOWER && key < lo));
  };
  auto hide0 = [&](int r) { return hidden(16 * (r >> 3) + (r & 7)); };
  auto hide1 = [&](int r) { return hidden(16 * (r >> 3) + (r & 7) + 32); };
  // column mask words of the keys of score registers r of s0 (keys 0..7
  // and 16..23 from cm) and of s1 (32 further on), and the lane's bit of
  // one of them as 0 or all ones
  uint32_t cw0[16], cw1[16];
  if (COL) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kq = 16 * (q >> 1) + 4 * (q & 1);
      const u32x4 a = *reinterpret_cast<const u32x4*>(cm + kq);
      const u32x4 b = *reinterpret_cast<const u32x4*>(cm + 32 + kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cw0[4 * q + e] = a[e];
        cw1[4 * q + e] = b[e];
      }
    }
  }
  auto vis = [&](uint32_t w) {
    return (uint32_t)__builtin_amdgcn_sbfe((int)w, (unsigned)crow, 1u);
  };
  auto keep = [&](float e, uint32_t w) {
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, e) & vis(w));
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
      if (COL) {
        e0 = keep(e0, cw0[r]);
        e1 = keep(e1, cw0[r + 1]);
        e2 = keep(e2, cw1[r]);
        e3 = keep(e3, cw1[r + 1]);
      }
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
  for (int r = 0; r < 16; ++r) {
    const bool h0 = hide0(r) || (COL && vis(cw0[r]) == 0u);
    const bool h1 = hide1(r) || (COL && vis(cw1[r]) == 0u);
    mq[r & 3] = fmaxf(fmaxf(mq[r & 3], h0 ? -INFINITY : s0[r]),
                      h1 ? -INFINITY : s1[r]);
  }
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

// Column mask, once per call for all heads: one wave per (sequence, query
// block of BR rows, key block of BC keys below the block's causal limit),
// lane = key, writes the block's entry for the prefill kernel's list: bits
// 0..15 the block, bit 16 + w set when the interval of some key hides it
// from some row of wave w (rows BR-block + 32 w ..) that would otherwise see
// it (that wave then tests every key), bit 24 + w when some row of wave w
// may see some key.  Entries past a query block's causal limit are not
// written (the prefill kernel reads only those below it).
template <bool CAUSAL>
__global__ __launch_bounds__(256) void column_list_kernel(
    ColMask cm, int Nq, int Nk, int n_qblk, long long n_waves) {
  const int lane = threadIdx.x & 63;
  const long long wv =
      (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= n_waves) return;
  const int kb = (int)(wv % cm.lstride);
  const long long t = wv / cm.lstride;
  const int qblk = (int)(t % n_qblk);
  const int b = (int)(t / n_qblk);
  const int q0 = qblk * BR;
  const int off = Nk - Nq;
  const int kv_end = CAUSAL ? min(Nk, q0 + BR + off) : Nk;
  if (kb * BC >= kv_end) return;  // whole wave: past the block's keys
  const int key = kb * BC + lane;
  const bool valid = key < kv_end;
  int lo = 0, hi = 0;
  if (valid) {
    const int2 x = *reinterpret_cast<const int2*>(
        cm.bounds + 2 * ((int64_t)b * cm.mb + key));
    lo = x.x;
    hi = x.y;
  }
  // rows that may see this key: its interval, and (causal) from its place on
  const int vlo = CAUSAL ? max(lo, key - off) : lo;
  uint32_t bits = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int w0 = q0 + 32 * w, r1 = min(w0 + 32, Nq);
    // the rows of wave w whose view of the key the interval decides: all of
    // them, or under the causal mask those from the first row that sees the
    // key (the causal limit hides it from the others)
    const int r0 = CAUSAL ? max(w0, key - off) : w0;
    const bool all_vis = r0 >= r1 || !valid || (lo <= r0 && hi >= r1);
    if (__builtin_amdgcn_ballot_w64(all_vis) != ~0ull) bits |= 1u << (16 + w);
    // some row of the wave may see the key
    if (__builtin_amdgcn_ballot_w64(valid && max(vlo, w0) < min(hi, r1)) != 0)
      bits |= 1u << (24 + w);
  }
  if (lane == 0) cm.lists[t * cm.lstride + kb] = kb | (int)bits;
}

template <int D, int MODE, bool OUT_F32, bool SPARSE = false,
          bool COLUMN = false, bool PAGED = false>
__global__ __launch_bounds__(NT, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int Nq_max, int Nk_max,
    float c2, int n_qblk, int n_items, SeqLayout lay, int wl, int wr,
    BlockMask bmask, ColMask cmask, int dq) {
  constexpr bool CAUSAL = MODE == kCausal;
  constexpr bool BAND = MODE == kBand;
  static_assert(!(SPARSE && BAND), "block masks go with no mask or causal");
  static_assert(!(COLUMN && (SPARSE || BAND)),
                "column masks go with no mask or causal");
  // a list of key blocks in LDS drives the loop (block or column mask)
  constexpr bool LISTED = SPARSE || COLUMN;
  static_assert(!(PAGED && LISTED), "paged caches go with the band masks");
  constexpr int BLKBITS = COLUMN ? 0xFFFF : 0xFFFFFF;
  // K/V ring depth: 8 stages of 8 KiB blocks at d = 64, 4 of 16 KiB at
  // d = 128 (128 KiB of LDS either way, leaving 32 KiB for the block list
  // of the listed variants; a fifth stage at d = 128 measured slower)
  constexpr int NSTG = D == 64 ? 8 : 4;
  using L = Layout<D, NSTG>;
  // block-sparse: each half has a ring of its own, half of the stages (its
  // waves copy and read only its blocks); NSR stages per ring, ring base
  // stage gofs, CW waves share a ring's copies
  constexpr int NSR = SPARSE ? NSTG / 2 : NSTG;
  constexpr int CW = SPARSE ? NW / 2 : NW;
  // block-sparse: the key blocks this workgroup computes, in order (bits
  // 0..23 the block, bit 24 / 25 set when the rows of group A / B use it),
  // then their count
  // paged cache: the page numbers of the pages this workgroup reads
  // column mask: the same list (bits 0..15 the block, bit 16 + w set when
  // wave w must test its rows key by key, bit 24 + w when some row of wave
  // w may see some key), a ring stage per K stage holding the listed
  // block's 64 bound pairs, and one visibility word per key and wave
  constexpr int LMAX = COLUMN ? kColMaxKeyBlocks : kSparseMaxKeyBlocks;
  __shared__ int blist[LISTED  ? LMAX + 1
                       : PAGED ? kPagedPrefillMaxPages
                               : 1];
  __shared__ __attribute__((aligned(16))) int cbnd[COLUMN ? NSTG * 2 * BC : 1];
  __shared__ __attribute__((aligned(16))) uint32_t cmk[COLUMN ? NW * BC : 1];
  constexpr int NTILE = L::NTILE;
  constexpr int NSTEP = L::NSTEP;
  __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_a = wave < NW / 2;
  const int h = lane >> 5, col = lane & 31;
  const int gofs = SPARSE && !group_a ? NSR : 0;
  const int cwave = SPARSE ? (wave & (CW - 1)) : wave;

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
    const int n_bh = lay.n_seq * Hkv;
    if ((Hkv & 7) == 0) {
      // KV heads a multiple of 8: XCD x takes the KV heads x, x + 8, ... of
      // every sequence (the same work on every XCD) and runs them one
      // (sequence, KV head) after another, Q-block ranks heavy first, so
      // that its concurrent workgroups share that head's K/V in its L2
      const int p = s8 / G;
      jq = p % n_qblk;
      bh = 8 * (p / n_qblk) + (blockIdx.x & 7);
    } else {
      const int u = 8 * (s8 / G) + (blockIdx.x & 7);
      if (u >= n_bh * n_qblk) return;
      jq = u / n_bh;
      bh = u % n_bh;
    }
  } else if (((n_items / (n_qblk * G)) & 7) == 0) {
    // equal sequences, KV heads a multiple of 8: each XCD (which receives
    // every 8th workgroup in launch order) takes whole KV heads, so a KV
    // head's Q blocks share that XCD's L2, and runs their items Q-block
    // rank first: the heaviest blocks of all its heads go first, which
    // keeps the in-order dispatch balanced under the causal mask
    const int per = (n_items / (n_qblk * G)) >> 3;  // KV heads per XCD
    const int x = blockIdx.x & 7, sx = blockIdx.x >> 3;
    g = sx % G;
    const int t1 = sx / G;
    bh = x * per + t1 % per;
    jq = t1 / per;
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
    // (a sequence's own key count, clamped into the cache)
    if (lay.seqlen_k) Nk = min(max(lay.seqlen_k[b], 0), Nk_max);
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

  // ---- paged cache: the page numbers of the pages that hold blocks j0 ..
  // nblk - 1, clamped into the pool, go to LDS (the host keeps a sequence's
  // pages within the list, and its length within its pages: the last page
  // read is at most max_pages - 1)
  int p0 = 0;
  if (PAGED) {
    p0 = (j0 * BC) >> lay.page_shift;
    const int np =
        nblk > j0 ? ((nblk * BC - 1) >> lay.page_shift) - p0 + 1 : 0;
    const int* tb = lay.page_table + (int64_t)b * lay.max_pages + p0;
    for (int i = tid; i < np; i += NT)
      blist[i] = min(max(tb[i], 0), lay.num_pages - 1);
    __syncthreads();
  }

  // ---- block-sparse: each 128-row half lists the key blocks below nblk
  // that its own mask row keeps (wave 0: row 2 qblk, for rows q0 ..; wave
  // NW/2: row 2 qblk + 1), entry p of half X in 16-bit slot 2p + X, its
  // count in slot 2 LMAX + X.  The halves then walk their lists side by
  // side, each with its own copy ring, so that both have a block to work on
  // in every iteration until the shorter list ends.
  int n_act = nblk;
  int n_mine = 0;  // block-sparse: entries of this wave's half
  if (SPARSE) {
    uint16_t* bl16 = reinterpret_cast<uint16_t*>(blist);
    if (wave == 0 || wave == NW / 2) {
      const int X = wave == 0 ? 0 : 1;
      const bool has = q0 + X * (BR / 2) < Nq;
      const uint8_t* ma = bmask.mask + b * bmask.mb + hq * bmask.mh +
                          (int64_t)(2 * qblk + X) * bmask.nkb;
      int cnt = 0;
      for (int base = 0; base < nblk; base += 64) {
        const int i = base + lane;
        const bool u = has && i < nblk && ma[i] != 0;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(u);
        const int pos =
            cnt + (int)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (u) bl16[2 * pos + X] = (uint16_t)i;
        cnt += (int)__builtin_popcountll(bal);
      }
      if (lane == 0) bl16[2 * LMAX + X] = (uint16_t)cnt;
    }
    __syncthreads();
    const int cnts = __builtin_amdgcn_readfirstlane(blist[LMAX]);
    const int na = cnts & 0xFFFF, nb = (cnts >> 16) & 0xFFFF;
    n_act = max(na, nb);
    n_mine = group_a ? na : nb;
  }
  // ---- column mask: the classification of this query block's key blocks
  // below nblk (one int each: bits 0..15 the block, bit 16 + w when wave w
  // must test its rows key by key, bit 24 + w when some row of wave w may
  // see some key), made once for all heads by column_list_kernel; the
  // waves keep the blocks some wave sees, in order, wave w compacting the
  // entries w * 64 .. w * 64 + 63 of each round of NW * 64 (the per-wave
  // counts of a round in the first NW words of the mask area, unused
  // before the main loop)
  if (COLUMN) {
    const int* ge = cmask.lists + (int64_t)(b * n_qblk + qblk) * cmask.lstride;
    uint32_t* ccnt = cmk;
    int total = 0;
    for (int base = 0; base < nblk; base += 64 * NW) {
      const int i = base + 64 * wave + lane;
      const int e = i < nblk ? ge[i] : 0;
      const bool kept = ((e >> 24) & 0xFF) != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(kept);
      if (lane == 0) ccnt[wave] = (uint32_t)__builtin_popcountll(bal);
      __syncthreads();
      int pre = total, all = total;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = (int)ccnt[w];
        pre += w < wave ? c : 0;
        all += c;
      }
      if (kept)
        blist[pre + (int)__builtin_popcountll(bal & ((1ull << lane) - 1ull))] =
            e;
      total = all;
      __syncthreads();  // (ccnt is reused by the next round)
    }
    n_act = __builtin_amdgcn_readfirstlane(total);
  }
  // list entry of ring position p (past the list: block nblk + 1, past
  // Nk, whose copies are zeros, and no keep bits).  The entries of the
  // positions whose copies are in flight stay in scalar registers, ent[i]
  // for position j + i at the start of iteration j, so that each iteration
  // reads one entry from LDS.
  // block-sparse: a half's own entries, bit 24 set (its rows keep the
  // block)
  auto entry = [&](int p) {
    if constexpr (SPARSE) {
      const uint16_t* bl16 = reinterpret_cast<const uint16_t*>(blist);
      return p < n_mine ? __builtin_amdgcn_readfirstlane(
                              bl16[2 * p + (group_a ? 0 : 1)]) |
                              (1 << 24)
                        : nblk + 1;
    }
    return p < n_act ? __builtin_amdgcn_readfirstlane(blist[p]) : nblk + 1;
  };
  int ent[LISTED ? NSR - 1 : 1];

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

  // ---- Q^T operand fragments: lane holds q[row][16t + 8h .. +7]; zeros
  // past the head dimension dq (a narrower head in this tile: with the K
  // columns past dq copied as zeros too, the scores are those of dq)
  const int qrow = wrow0 + col;
  bf16x8 qf[NSTEP];
  {
    const bool ok = qrow < Nq;
    const uint16_t* qp = q + qbase + (ok ? qrow : 0) * lay.q_r + 8 * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      u32x4 x = (ok && 16 * t + 8 * h < dq) ? ldg16(qp + 16 * t)
                                            : u32x4{0u, 0u, 0u, 0u};
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
      vp[tt] = smem + (gofs + (j + NSR - 1) % NSR) * L::VBYTES + v_rd[tt];
    const char* kp = smem + (gofs + j % NSR) * L::KBYTES + k_rd;
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

  // ---- K/V ring: NS stages each; block b's K and V live in stage b % NS.
  // Group g of copies is K_g and V_{g-1}; iteration j issues group
  // j + NS - 1 at the start of its softmax phase (vector memory issue then
  // overlaps vector ALU work).  A stage is refilled only after both groups'
  // last reads of it (those of block j - 1, before this iteration's first
  // barrier).  The loop's barriers carry no memory fence, so copies stay
  // in flight across them: at the end of iteration j group A waits for its
  // own copies of iteration j - (NS - 2) and group B (one barrier behind)
  // for those of iteration j - (NS - 3); the first reader of K_{j+NS-1} /
  // V_{j+NS-2}, group A's matrix phase of iteration j + NS - 1, comes after
  // both waits and a barrier.
  // copy instructions per wave and block (column mask: one more, for the
  // block's bounds)
  constexpr int OPS = 2 * (L::NINS / CW) + (COLUMN ? 1 : 0);
  const int kv_rows = max(kv_end, 0);      // rows past this are not needed
  // (V_{j0-1}, before the first block, is a copy of zeros: block j0's
  // matrix phase multiplies it by the all-zero "previous" P, and 0 *
  // (stale NaN/Inf bits) would not be 0)
  // paged cache: byte offset of block blk's row 0 from the head's base
  // (its page's row, K and V alike), negative for a block past the keys;
  // groups are issued in order, so V_{g-1} reuses K_{g-1}'s offset
  int64_t prev_ro = -1;
  auto page_off = [&](int blk) -> int64_t {
    const int kb = blk * BC;
    if (kb >= kv_rows) return -1;
    const int pg = __builtin_amdgcn_readfirstlane(
        blist[(kb >> lay.page_shift) - p0]);
    return (((int64_t)pg << lay.page_shift) |
            (kb & ((1 << lay.page_shift) - 1))) * rsb;
  };
  // group g: K of key block kblk, V of key block vblk (the block of
  // position g - 1; negative: a copy of zeros)
  auto group = [&](int g, int kblk, int vblk) {
    if constexpr (PAGED) {
      const int64_t ro = page_off(g);
      copy_block_paged<D>(smem + (g % L::NS) * L::KBYTES, kh, ro,
                          kv_rows - g * BC, wave, k_off, 16, rsb, 2 * dq,
                          dq / 8);
      copy_block_paged<D>(
          smem + L::VBASE + ((g + L::NS - 1) % L::NS) * L::VBYTES, vh,
          g > j0 ? prev_ro : -1, kv_rows - (g - 1) * BC, wave, v_off, v_step,
          rsbv, 2 * dq);
      prev_ro = ro;
    } else {
      if constexpr (COLUMN) {
        // bounds of the keys of the block at position g into stage g % NS:
        // wave w copies keys 8w .. 8w + 7 (64 bytes, four lanes); keys past
        // Nk read as zeros (an empty interval)
        const int kk = min(kblk * BC + 8 * wave, Nk);
        const char* src = reinterpret_cast<const char*>(
            cmask.bounds + 2 * ((int64_t)b * cmask.mb + kk));
        const int ln = lane_now();
        if (ln < 4)
          dma16(reinterpret_cast<char*>(cbnd) + (g % NSR) * 8 * BC +
                    64 * wave,
                src, (uint32_t)min(Nk - kk, 8) * 8u, 16 * ln);
      }
      copy_block<D, CW>(smem + (gofs + g % NSR) * L::KBYTES, kh, kv_rows,
                        kblk, cwave, k_off, 16, rsb, 2 * dq, dq / 8);
      copy_block<D, CW>(
          smem + L::VBASE + (gofs + (g + NSR - 1) % NSR) * L::VBYTES, vh,
          kv_rows, vblk, cwave, v_off, v_step, rsbv, 2 * dq);
    }
  };
  auto copies = [&](int j) {
    const int g = j + NSR - 1;
    if constexpr (LISTED) {
      const int en = entry(g);
      group(g, en & BLKBITS, ent[NSR - 2] & BLKBITS);
#pragma unroll
      for (int i = 0; i + 1 < NSR - 1; ++i) ent[i] = ent[i + 1];
      ent[NSR - 2] = en;
    } else {
      group(g, g, g - 1);
    }
  };
  // prologue: groups j0 .. j0 + NS - 2.  The first two must have landed for
  // every wave before the loop: group B's first wait in the loop comes one
  // barrier too late for group j0 + 1.
#pragma unroll
  for (int i = 0; i < NSR - 1; ++i) {
    const int g = j0 + i;
    if constexpr (LISTED) {
      ent[i] = entry(g);
      group(g, ent[i] & BLKBITS, i > 0 ? ent[i - 1] & BLKBITS : -1);
    } else {
      group(g, g, i > 0 ? g - 1 : -1);
    }
  }
  // (block-sparse: each half reads only its own ring, so its first block
  // is all it needs)
  if constexpr (SPARSE)
    wait_vmcnt<(NSR - 2) * OPS>();
  else
    wait_vmcnt<(L::NS - 3) * OPS>();
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
    if constexpr (LISTED) {
      const int e = ent[0];
      jb = e & BLKBITS;
      keep = (e >> 24) & 1;  // block mask: this half has a block here
      if (COLUMN) {
        keep = (e >> (24 + wave)) & 1;
        colm = keep && ((e >> (16 + wave)) & 1);
      }
    }
    mphase(j, std::true_type{}, keep_prev, keep);
    barrier();
    copies(j);
    if (LISTED && !keep)
      rescale = false;  // nothing of this block enters this wave's rows
    else if (COLUMN && colm) {
      // each key's visibility to the 32 rows of this wave as a bit mask
      // (lane = key of the block), from its interval clamped to the rows;
      // rows from which the limit hides the key anyway (causal, or a key
      // past Nk) count as seeing it
      const int ln = lane_now();
      const int2 x = *reinterpret_cast<const int2*>(
          cbnd + (j % NSR) * 2 * BC + 2 * ln);
      const int ra = min(max(x.x, wrow0), wrow0 + 32) - wrow0;
      const int rb = min(max(x.y, wrow0), wrow0 + 32) - wrow0;
      uint32_t m = rb <= ra        ? 0u
                   : rb - ra >= 32 ? ~0u
                                   : ((1u << (rb - ra)) - 1u) << ra;
      const int key = jb * BC + ln;
      if (CAUSAL) {
        const int cd = min(max(key - off - wrow0, 0), 32);
        m |= cd >= 32 ? ~0u : (1u << cd) - 1u;
      }
      if (key >= Nk) m = ~0u;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(m);
      if (__builtin_amdgcn_ballot_w64(m != m0) == 0) {
        // every key of the block has the same rows: a row either sees all
        // of them the limit lets through or none
        rescale = softmax_phase<true>(s0, s1,
                                      ((m0 >> col) & 1u) ? lim0 - jb * BC
                                                         : -1,
                                      0, c2, st, alpha, pk);
      } else {
        cmk[wave * BC + ln] = m;
        rescale = softmax_phase<true, false, true>(
            s0, s1, lim0 - jb * BC, 0, c2, st, alpha, pk,
            cmk + wave * BC + 8 * h, col);
      }
    }
    else if (jb >= w_mask || (BAND && jb < w_lo))
      rescale = softmax_phase<true, BAND>(s0, s1, lim0 - jb * BC,
                                          lo0 - jb * BC, c2, st, alpha, pk);
    else
      rescale = softmax_phase<false>(s0, s1, lim0 - jb * BC, 0, c2, st,
                                     alpha, pk);
    keep_prev = keep;
    if constexpr (SPARSE)
      wait_vmcnt<(NSR - 2) * OPS>();  // own ring: the next block, landed
    else if (group_a)
      wait_vmcnt<(L::NS - 2) * OPS>();
    else
      wait_vmcnt<(L::NS - 3) * OPS>();
    barrier();
  }
  if (n_act > j0)  // P V of the last block
    mphase(n_act, std::false_type{}, LISTED ? keep_prev : true);
  wait_vmcnt<0>();  // no copy may be in flight when the wave ends
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
      if (32 * tt >= dq) break;  // (columns past the head dimension)
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


// ---- d = 256: one wave per SIMD
//
// At d = 256 a wave's Q^T fragments (64 registers) and O^T accumulators
// (128) leave no room for two waves per SIMD, so the ping-pong schedule
// above does not fit.  This kernel runs one wave per SIMD (its 512 VGPRs
// and AGPRs): a workgroup of 4 waves takes 128 query rows, 32 per wave,
// with the same products, layouts, lazy reference max and epilogue.  Each
// wave issues its matrix phase (P_{j-1} V_{j-1}, then S_j) and then the
// softmax of block j.  The K/V ring has two stages of 64-key blocks (32 KiB
// each for K and for V, 128 KiB of LDS): group j + 1 (K_{j+1}, V_j) is
// issued at the top of iteration j into the stages that blocks j - 1 and
// j - 2 used, which every wave finished reading before the barrier that
// ended iteration j - 1, and it is waited for at the end of iteration j,
// so one whole iteration hides its latency.
constexpr int BR256 = 128;              // query rows per workgroup
constexpr int NW256 = BR256 / 32;       // 4 waves

template <int MODE, bool OUT_F32>
__global__ __launch_bounds__(64 * NW256, 1) void prefill256_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int Nq, int Nk_max, float c2,
    int n_qblk, int n_items, SeqLayout lay, int wl, int wr) {
  constexpr int D = 256;
  constexpr bool CAUSAL = MODE == kCausal;
  constexpr bool BAND = MODE == kBand;
  using L = Layout<D, 2>;
  constexpr int NTILE = L::NTILE;
  constexpr int NSTEP = L::NSTEP;
  __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  // ---- work item: (b, kv head, Q block, head in group); heavy blocks
  // first, and the XCD mapping of prefill_kernel
  const int G = Hq / Hkv;
  int g, jq, bh;
  if (((n_items / (n_qblk * G)) & 7) == 0) {
    const int per = (n_items / (n_qblk * G)) >> 3;
    const int x = blockIdx.x & 7, sx = blockIdx.x >> 3;
    g = sx % G;
    const int t1 = sx / G;
    bh = x * per + t1 % per;
    jq = t1 / per;
  } else {
    const int item = xcd_contiguous(blockIdx.x, n_items);
    g = item % G;
    const int t1 = item / G;
    jq = t1 % n_qblk;
    bh = t1 / n_qblk;
  }
  const int qblk = MODE != kNone ? (n_qblk - 1 - jq) : jq;
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int hq = hkv * G + g;
  const int q0 = qblk * BR256;
  if (q0 >= Nq) return;
  // (a sequence's own key count, clamped into the cache)
  const int Nk = lay.seqlen_k ? min(max(lay.seqlen_k[b], 0), Nk_max) : Nk_max;
  const int64_t qbase = b * lay.q_b + hq * lay.q_h;
  const int64_t obase = b * lay.o_b + hq * lay.o_h;
  const int64_t lbase = b * lay.l_b + hq * lay.l_h;
  const int off = Nk - Nq;
  const int rsb = (int)(2 * lay.k_r);
  const int rsbv = (int)(2 * lay.v_r);
  const char* kh = reinterpret_cast<const char*>(k + b * lay.k_b + hkv * lay.k_h);
  const char* vh = reinterpret_cast<const char*>(v + b * lay.v_b + hkv * lay.v_h);

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, q0 + BR256 + off);
  int j0 = 0;
  if (BAND) {
    kv_end = min(Nk, min(q0 + BR256, Nq) + off + wr);
    j0 = max(0, q0 + off - wl) / BC;
  }
  const int nblk = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const int kv_rows = max(kv_end, 0);

  const int wrow0 = q0 + wave * 32;
  int w_mask = Nk / BC;
  if (CAUSAL) w_mask = min(w_mask, max(0, wrow0 + off + 1) / BC);
  int w_lo = 0;
  if (BAND) {
    w_mask = min(w_mask, max(0, wrow0 + off + wr + 1) / BC);
    w_lo = (max(0, wrow0 + 31 + off - wl) + BC - 1) / BC;
  }

  // ---- per-lane DMA source offsets (K: chunk i of all 64 rows per
  // instruction; V: two 512-byte rows per instruction, 16-byte chunks
  // XOR-swizzled by the tile row; wave w issues instructions w, w + 4, ...,
  // so bit 1 of the tile rows of its V instructions is bit 0 of w)
  const uint32_t k_off = (uint32_t)(key_slot(lane) * rsb);
  uint32_t v_off;
  {
    const int row = lane >> 5;                  // row within the KiB
    const int p = lane & 31;                    // physical 16-byte chunk
    const int trow = 2 * (wave & 1) + row;      // tile row modulo 4
    v_off = (uint32_t)(row * rsbv) + ((p ^ (vswz<D>(trow) >> 1)) * 16);
  }
  const int v_step = 2 * rsbv;

  const int qrow = wrow0 + col;
  bf16x8 qf[NSTEP];
  {
    const bool ok = qrow < Nq;
    const uint16_t* qp = q + qbase + (ok ? qrow : 0) * lay.q_r + 8 * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, ok ? ldg16(qp + 16 * t)
                                            : u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 acc[NTILE];
#pragma unroll
  for (int i = 0; i < NTILE; ++i) acc[i] = f32x16{};
  RowState st{-INFINITY, 0.f, 0.f};

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
  const int lim0 = (CAUSAL ? min(Nk - 1, qrow + off)
                    : BAND ? min(Nk - 1, qrow + off + wr)
                           : Nk - 1) - 8 * h;
  const int lo0 = BAND ? qrow + off - wl - 8 * h : 0;

  f32x16 s0, s1;
  u32x4 pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = u32x4{0u, 0u, 0u, 0u};
  bool rescale = false;
  float alpha = 1.f;

  // group g: K_g into K stage g % 2, V_{g-1} into V stage (g + 1) % 2
  // (V_{j0-1} is a copy of zeros: the all-zero "previous" P multiplies it)
  auto group = [&](int gi) {
    copy_block<D, NW256>(smem + (gi & 1) * L::KBYTES, kh, kv_rows, gi, wave,
                         k_off, 16, rsb, 2 * D);
    copy_block<D, NW256>(smem + L::VBASE + ((gi + 1) & 1) * L::VBYTES, vh,
                         kv_rows, gi > j0 ? gi - 1 : -1, wave, v_off, v_step,
                         rsbv, 2 * D);
  };
  group(j0);
  wait_vmcnt<0>();
  __syncthreads();

  for (int j = j0; j < nblk; ++j) {
    group(j + 1);
    if (rescale) {
#pragma unroll
      for (int i = 0; i < NTILE; ++i) acc[i] *= alpha;
    }
    {
      const char* vp[NTILE];
#pragma unroll
      for (int tt = 0; tt < NTILE; ++tt)
        vp[tt] = smem + ((j + 1) & 1) * L::VBYTES + v_rd[tt];
      const char* kp = smem + (j & 1) * L::KBYTES + k_rd;
      matrix_phase<D, true, true>(kp, vp, qf, pk, acc, s0, s1);
    }
    if (j >= w_mask || (BAND && j < w_lo))
      rescale = softmax_phase<true, BAND>(s0, s1, lim0 - j * BC,
                                          lo0 - j * BC, c2, st, alpha, pk);
    else
      rescale = softmax_phase<false>(s0, s1, lim0 - j * BC, 0, c2, st, alpha,
                                     pk);
    wait_vmcnt<0>();
    barrier();
  }
  if (nblk > j0) {  // P V of the last block
    if (rescale) {
#pragma unroll
      for (int i = 0; i < NTILE; ++i) acc[i] *= alpha;
    }
    const char* vp[NTILE];
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt)
      vp[tt] = smem + ((nblk + 1) & 1) * L::VBYTES + v_rd[tt];
    matrix_phase<D, true, false>(smem, vp, qf, pk, acc, s0, s1);
  }

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
          bool COLUMN = false, bool PAGED = false>
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
  hipLaunchKernelGGL((prefill_kernel<D, MODE, OUT_F32, SPARSE, COLUMN, PAGED>),
                     dim3((unsigned)n_items), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), o, lse, s.Hq, s.Hkv,
                     s.Nq, s.Nk, c2, n_qblk, (int)n_items, lay, wl, wr, bm,
                     cm, s.d);
  return hipGetLastError();
}

template <int MODE, bool OUT_F32>
hipError_t launch256(const void* q, const void* k, const void* v, void* o,
                     float* lse, const Shape& s, const SeqLayout& lay, int wl,
                     int wr, hipStream_t stream) {
  const int n_qblk = (s.Nq + BR256 - 1) / BR256;
  const long long n_items = (long long)s.B * s.Hq * n_qblk;
  const float c2 = fmaxf(s.scale * kLog2e, 1.17549435e-38f);
  hipLaunchKernelGGL((prefill256_kernel<MODE, OUT_F32>), dim3((unsigned)n_items),
                     dim3(64 * NW256), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), o, lse, s.Hq, s.Hkv,
                     s.Nq, s.Nk, c2, n_qblk, (int)n_items, lay, wl, wr);
  return hipGetLastError();
}

// d = 256 (dense layout, optionally per-sequence key counts)
hipError_t launch_prefill256(const void* q, const void* k, const void* v,
                             void* o, float* lse, const Shape& s,
                             const SeqLayout& lay, bool out_f32,
                             hipStream_t stream) {
  if (lay.cu_q || lay.page_table) return hipErrorInvalidValue;
  const MaskBounds m = mask_bounds(s);
  if (m.kind == 0)
    return out_f32 ? launch256<kNone, true>(q, k, v, o, lse, s, lay, 0, 0, stream)
                   : launch256<kNone, false>(q, k, v, o, lse, s, lay, 0, 0, stream);
  if (m.kind == 1)
    return out_f32 ? launch256<kCausal, true>(q, k, v, o, lse, s, lay, 0, 0, stream)
                   : launch256<kCausal, false>(q, k, v, o, lse, s, lay, 0, 0, stream);
  return out_f32 ? launch256<kBand, true>(q, k, v, o, lse, s, lay, m.wl, m.wr, stream)
                 : launch256<kBand, false>(q, k, v, o, lse, s, lay, m.wl, m.wr, stream);
}

template <int D, int MODE, bool PAGED>
hipError_t launch_mode(const void* q, const void* k, const void* v, void* o,
                       float* lse, const Shape& s, const SeqLayout& lay,
                       int wl, int wr, bool out_f32, hipStream_t stream) {
  return out_f32 ? launch<D, MODE, true, false, false, PAGED>(
                       q, k, v, o, lse, s, lay, wl, wr, stream)
                 : launch<D, MODE, false, false, false, PAGED>(
                       q, k, v, o, lse, s, lay, wl, wr, stream);
}

template <int D, bool PAGED>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o,
                    float* lse, const Shape& s, const SeqLayout& lay,
                    bool out_f32, hipStream_t stream) {
  const MaskBounds m = mask_bounds(s);
  if (m.kind == 0)
    return launch_mode<D, kNone, PAGED>(q, k, v, o, lse, s, lay, 0, 0,
                                        out_f32, stream);
  if (m.kind == 1)
    return launch_mode<D, kCausal, PAGED>(q, k, v, o, lse, s, lay, 0, 0,
                                          out_f32, stream);
  return launch_mode<D, kBand, PAGED>(q, k, v, o, lse, s, lay, m.wl, m.wr,
                                      out_f32, stream);
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
  {
    const int n_qblk = (s.Nq + BR - 1) / BR;
    const long long n_waves = (long long)s.B * n_qblk * cm.lstride;
    if (s.causal)
      hipLaunchKernelGGL(column_list_kernel<true>,
                         dim3((unsigned)((n_waves + 3) / 4)), dim3(256), 0,
                         stream, cm, s.Nq, s.Nk, n_qblk, n_waves);
    else
      hipLaunchKernelGGL(column_list_kernel<false>,
                         dim3((unsigned)((n_waves + 3) / 4)), dim3(256), 0,
                         stream, cm, s.Nq, s.Nk, n_qblk, n_waves);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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

size_t column_list_bytes(int B, int Nq, int Nk) {
  const long long n_qblk = ((long long)Nq + BR - 1) / BR;
  const long long nkb = ((long long)Nk + BC - 1) / BC;
  return (size_t)(B * n_qblk * nkb) * sizeof(int);
}

hipError_t launch_prefill_column(const void* q, const void* k, const void* v,
                                 void* o, float* lse, const Shape& s,
                                 const ColMask& cm, bool out_f32,
                                 hipStream_t stream) {
  if (s.d == 128 || s.d == 96)
    return launch_column_d<128>(q, k, v, o, lse, s, cm, out_f32, stream);
  if (s.d == 64 || s.d == 32)
    return launch_column_d<64>(q, k, v, o, lse, s, cm, out_f32, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_sparse(const void* q, const void* k, const void* v,
                                 void* o, float* lse, const Shape& s,
                                 const BlockMask& bm, bool out_f32,
                                 hipStream_t stream) {
  if (s.d == 128 || s.d == 96)
    return launch_sparse_d<128>(q, k, v, o, lse, s, bm, out_f32, stream);
  if (s.d == 64 || s.d == 32)
    return launch_sparse_d<64>(q, k, v, o, lse, s, bm, out_f32, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s,
                          const SeqLayout& lay, bool out_f32,
                          hipStream_t stream) {
  // head dimension 96 runs in the 128-column tile and 32 in the 64-column
  // one, the columns past d masked (Q and K read as zeros, O not stored);
  // 256 in its own kernel
  if (s.d == 256)
    return launch_prefill256(q, k, v, o, lse, s, lay, out_f32, stream);
  const bool paged = lay.page_table != nullptr;
  if (s.d == 128 || s.d == 96)
    return paged ? launch_d<128, true>(q, k, v, o, lse, s, lay, out_f32, stream)
                 : launch_d<128, false>(q, k, v, o, lse, s, lay, out_f32,
                                        stream);
  if (s.d == 64 || s.d == 32)
    return paged ? launch_d<64, true>(q, k, v, o, lse, s, lay, out_f32, stream)
                 : launch_d<64, false>(q, k, v, o, lse, s, lay, out_f32,
                                       stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

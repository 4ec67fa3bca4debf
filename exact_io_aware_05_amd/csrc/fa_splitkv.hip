// KV-split attention forward (the Flash-Decoding form: "FlashAttention
// Analysis", ryotta.opik.net, "Flash-Decoding" paragraph).  With one query
// and thousands of cached keys there are too few query rows to fill the GPU,
// so the key axis is cut into chunks that are processed in parallel, each
// producing an unnormalised partial result (m, l, O~); a second kernel
// combines the chunks with the log-sum-exp rule.
//
// Partial kernel: one wave per (batch, KV head, block of 32 packed query
// rows, chunk).  The packed rows are the (query, head-in-group) pairs of
// one KV head, so the Hq/Hkv query heads that share a KV head read each
// K/V byte once.  The step is HBM-bound; the waves of a workgroup are
// independent (no barrier), each streaming its 32-key blocks through a
// ring of 4 (the loads of the next 3 blocks in flight while one is
// computed; at d = 256 a ring of 2, so that the four waves' K slots fit in
// LDS), with non-temporal loads:
// * K moves HBM -> LDS with buffer_load ... lds, each instruction reading
//   four whole rows (coalesced), into a per-wave LDS slot in a swizzled
//   row-major layout; S^T = K Q^T on v_mfma_f32_32x32x16_bf16 then reads
//   its A operands from LDS without bank conflicts.  The contraction index
//   (head dimension) is permuted so that a lane's operands are one
//   contiguous half row of K; Q uses the same permutation.  Score register
//   r of a lane holds key 16(r/8) + 8h + r%8 (the A-operand row order is
//   chosen for that), which is the B-operand layout of P for the P V step.
// * O^T = V^T P^T: a lane loads 8 consecutive V rows at head-dimension
//   columns 4 col .. 4 col + 3 into registers (whole rows per
//   instruction) and v_perm_b32 repacks them into the A operands of 4
//   output tiles, where tile t, operand row a is head-dimension column
//   4a + t.
// * Every load is issued unconditionally through buffer resources that end
//   at the chunk's last key, so the number of loads in flight is the same
//   on every path and the compiler waits for exactly the block it needs.
// Merge kernel: one wave per output row, chunks visited in order.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int KB = kSplitKeys;  // 32 keys per block
constexpr int NT = 256;         // 4 independent waves per workgroup
// Cache policy of the K/V loads: non-temporal (each cached byte is read
// once per KV head, so keeping it in the caches only evicts other data).
constexpr int kStreamAux = 2;

typedef __attribute__((address_space(3))) void lds_void;

// K of one 32-key block sits in a per-wave LDS slot, row-major with 16-byte
// chunk c of row r stored at chunk c ^ kswz(r): the 16 lanes that read one
// operand chunk of 16 different rows then hit 16 different bank groups.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D >= 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : ((r >> 1) & 3);
}

// Per-wave state of one 32-key block: K copied HBM -> LDS by buffer_load
// ... lds (each instruction reads whole rows, so the loads are coalesced),
// V loaded into registers.
template <int D>
struct KvRegs {
  static constexpr int NSTEP = D / 16;  // score k-steps
  static constexpr int CPL = D / 32;    // V columns per lane (= O^T tiles)
  static constexpr int KBYTES = KB * 2 * D;   // one K slot
  static constexpr int NI = KBYTES / 1024;    // copy instructions per block
  static constexpr int RPK = 1024 / (2 * D);  // K rows per instruction
  static constexpr int OPS = NI + 16;         // loads per block
  // V: [k-step s][row e] -> CPL bf16 values (CPL/2 dwords)
  uint32_t vr[2][8][CPL >= 2 ? CPL / 2 : 1];

  // source offset of this lane within copy instruction i: row RPK i +
  // lane / CPR of the block, the chunk that the swizzle puts at lane % CPR
  static __device__ __forceinline__ uint32_t k_lane_off(int i) {
    constexpr int CPR = 2 * D / 16;
    const int lane = threadIdx.x & 63;
    const int r = lane / CPR, p = lane % CPR;
    return (uint32_t)(r * 2 * D + 16 * (p ^ kswz<D>(RPK * i + r)));
  }

  // Loads block rows kb .. kb + 31: V into registers, then K into the LDS
  // slot (the K copies are the last OPS_K loads of a block, which the
  // explicit wait before the K reads counts on).
  // Every load is issued unconditionally through buffer resources that end
  // at row `end` (the chunk's last key + 1), so rows past it arrive as
  // zeros without touching memory, and the number of loads in flight is
  // the same on every path (which lets the compiler wait for just the
  // block it needs).
  __device__ __forceinline__ void load(char* kslot, const uint32_t* koff,
                                       const uint16_t* kh,
                                       __amdgpu_buffer_rsrc_t vrs, int kb,
                                       int end, int h, int col) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int vrow = kb + 16 * s + 8 * h + e;
        const int off = vrow * (2 * D) + 2 * CPL * col;
        if (CPL == 8) {
          const u32x4 x = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kStreamAux));
#pragma unroll
          for (int c = 0; c < CPL / 2; ++c) vr[s][e][c] = x[c];
        } else if (CPL == 4) {
          const u32x2 x = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, kStreamAux));
          vr[s][e][0] = x[0];
          vr[s][e][CPL / 2 - 1] = x[1];
        } else if (CPL == 2) {
          vr[s][e][0] =
              __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, kStreamAux);
        } else {
          vr[s][e][0] =
              __builtin_amdgcn_raw_buffer_load_b16(vrs, off, 0, kStreamAux);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r0 = kb + RPK * i;
      const uint32_t rem = r0 < end ? (uint32_t)(end - r0) * (2 * D) : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          buffer_rsrc(kh + (int64_t)r0 * D, rem),
          (lds_void*)(kslot + 1024 * i), 16, koff[i % (16 / RPK)], 0, 0,
          kStreamAux);
    }
  }

  // The same loads for a block whose rows are `rs` bytes apart starting at
  // `kbase` / `vbase` (a page of a paged cache), of which the first
  // `rows` exist; `koff` holds the lane offsets for that row pitch.
  __device__ __forceinline__ void load_rows(char* kslot, const uint32_t* koff,
                                            const uint16_t* kbase,
                                            const uint16_t* vbase, int rows,
                                            int rs, int h, int col) {
    const uint32_t vrange = rows > 0 ? (uint32_t)((rows - 1) * rs + 2 * D) : 0u;
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vbase, vrange);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int off = (16 * s + 8 * h + e) * rs + 2 * CPL * col;
        if (CPL == 8) {
          const u32x4 x = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kStreamAux));
#pragma unroll
          for (int c = 0; c < CPL / 2; ++c) vr[s][e][c] = x[c];
        } else if (CPL == 4) {
          const u32x2 x = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, kStreamAux));
          vr[s][e][0] = x[0];
          vr[s][e][CPL / 2 - 1] = x[1];
        } else if (CPL == 2) {
          vr[s][e][0] =
              __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, kStreamAux);
        } else {
          vr[s][e][0] =
              __builtin_amdgcn_raw_buffer_load_b16(vrs, off, 0, kStreamAux);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int left = rows - RPK * i;
      const uint32_t rem = left > 0 ? (uint32_t)((left - 1) * rs + 2 * D) : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          buffer_rsrc(reinterpret_cast<const char*>(kbase) +
                          (int64_t)RPK * i * rs,
                      rem),
          (lds_void*)(kslot + 1024 * i), 16, koff[i % (16 / RPK)], 0, 0,
          kStreamAux);
    }
  }

  // lane offsets of load_rows for rows `rs` bytes apart
  static __device__ __forceinline__ uint32_t k_lane_off_rows(int i, int rs) {
    constexpr int CPR = 2 * D / 16;
    const int lane = threadIdx.x & 63;
    const int r = lane / CPR, p = lane % CPR;
    return (uint32_t)(r * rs + 16 * (p ^ kswz<D>(RPK * i + r)));
  }

  // K operand of k-step t for lane (col, h): row kr of the block (the
  // A-operand row order realised by the bit swap), head-dimension chunk
  // (D/16) h + t (each lane half covers one contiguous half row)
  static __device__ __forceinline__ bf16x8 kop(const char* kslot, int kr,
                                               int h, int t) {
    const int c = (D / 16) * h + t;
    return *reinterpret_cast<const bf16x8*>(kslot + kr * (2 * D) +
                                            16 * (c ^ kswz<D>(kr)));
  }

  // A operand (V^T) of output tile tt for k-step s: 8 keys of column
  // CPL * col + tt, keys in the order e = 0..7.
  __device__ __forceinline__ bf16x8 vop(int s, int tt) const {
    const int dw = tt >> 1;
    const uint32_t sel = (tt & 1) ? 0x07060302u : 0x05040100u;
    u32x4 a;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = __builtin_amdgcn_perm(vr[s][2 * j + 1][dw], vr[s][2 * j][dw], sel);
    return __builtin_bit_cast(bf16x8, a);
  }
};

// Mask kinds: none, causal (key j visible to query i iff j <= i + Nk - Nq),
// band (iff i + Nk - Nq - wl <= j <= i + Nk - Nq + wr).  With a band the
// chunks of a row tile cut the blocks from its first row's lower bound on,
// not from key 0.
constexpr int kNone = 0, kCausal = 1, kBand = 2;

template <int D, int MODE, bool PAGED = false>
__global__ __launch_bounds__(NT, 1) void splitkv_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ ws_o,
    f32x4* __restrict__ ws_ml, int Hq, int Hkv, int Nq, int Nk_arg, float c2,
    int n_rowtiles, int num_splits, int blocks_per_split, int n_items, int wl,
    int wr, PagedKv pg) {
  constexpr bool CAUSAL = MODE == kCausal;
  constexpr bool BAND = MODE == kBand;
  constexpr int NSTEP = D / 16;
  constexpr int CPL = D / 32;
  const int lane = threadIdx.x & 63;
  // wave index, uniform (so buffer resources and LDS bases of copies stay
  // in scalar registers instead of going through per-lane loops)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * (NT / 64) + wave;
  if (item >= n_items) return;  // whole wave leaves; no barrier below
  const int h = lane >> 5, col = lane & 31;

  const int sp = item % num_splits;
  const int t1 = item / num_splits;
  const int rt = t1 % n_rowtiles;
  const int bh = t1 / n_rowtiles;  // b * Hkv + hkv
  const int b = bh / Hkv, hkv = bh % Hkv;
  // keys of this sequence: all of them, or its own cache length (paged, or
  // a padded contiguous cache with lengths), clamped into the cache
  const int Nk =
      PAGED ? min(max(pg.seqlen[b], 0), pg.max_pages * pg.page_size)
      : pg.seqlen ? min(max(pg.seqlen[b], 0), Nk_arg)
                  : Nk_arg;
  const int G = Hq / Hkv;
  const int R = Nq * G;
  const int prow = rt * 32 + col;  // packed (query, head-in-group) row
  const bool row_ok = prow < R;
  const int iq = row_ok ? prow / G : 0;
  const int hq = hkv * G + (row_ok ? prow % G : 0);
  const int off = Nk - Nq;
  const int64_t qrow_id = (int64_t)(b * Hq + hq) * Nq + iq;

  // Q^T operand with the permuted head dimension: step t, lane half h
  // covers columns (D/2) h + 8t .. +7.
  bf16x8 qf[NSTEP];
  {
    const uint16_t* qp = q + qrow_id * D + (D / 2) * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
      qf[t] = __builtin_bit_cast(
          bf16x8, row_ok ? ldg16(qp + 8 * t) : u32x4{0u, 0u, 0u, 0u});
  }

  // (contiguous heads are Nk_arg rows apart, padded or not)
  const uint16_t* kh = k + (int64_t)bh * Nk_arg * D;
  const uint16_t* vh = v + (int64_t)bh * Nk_arg * D;
  // paged: bytes between the rows of one page and head, the chunk's first
  // page, and its page numbers, one per lane (clamped into the cache)
  const int rs = PAGED ? Hkv * D * 2 : 2 * D;
  int first_page = 0, page_of_lane = 0;
  const int nblk_all = (Nk + KB - 1) / KB;
  // queries of the first and last packed rows of this tile
  const int first_q = (rt * 32) / G;
  const int last_q = min(R - 1, rt * 32 + 31) / G;
  const int blk_base = BAND ? max(0, first_q + off - wl) / KB : 0;
  const int blk0 = blk_base + sp * blocks_per_split;
  int blk1 = min(blk0 + blocks_per_split, nblk_all);
  if (PAGED) {
    first_page = (blk0 * KB) >> pg.page_shift;
    const int pi = first_page + lane;
    const int pv = pi < pg.max_pages ? pg.table[(int64_t)b * pg.max_pages + pi]
                                     : 0;
    page_of_lane = min(max(pv, 0), pg.num_pages - 1);
  }
  if (CAUSAL || BAND) {
    // last key visible to the last packed row of this tile
    const int kv_end = min(Nk, last_q + off + (BAND ? wr : 0) + 1);
    blk1 = min(blk1, kv_end > 0 ? (kv_end + KB - 1) / KB : 0);
  }
  const int lim = CAUSAL ? min(Nk - 1, iq + off)
                  : BAND ? min(Nk - 1, iq + off + wr)
                         : Nk - 1;
  // smallest per-row limit in this row tile (its first packed row)
  const int lim_first = CAUSAL ? min(Nk - 1, first_q + off)
                        : BAND ? min(Nk - 1, first_q + off + wr)
                               : Nk - 1;
  // band: this row's first visible key, and the largest such bound in the
  // tile (its last packed row)
  const int lo = BAND ? iq + off - wl : 0;
  const int lo_last = BAND ? last_q + off - wl : 0;

  f32x16 acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = f32x16{};
  float m = -INFINITY, l = 0.f, lb = 0.f;
  const int krow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);

  // K/V blocks stream through a ring of PF register buffers: the loads of
  // the next PF - 1 blocks are in flight while a block is computed (the
  // step is HBM-bound, and one wave per SIMD needs that many bytes in
  // flight to cover the memory latency).  The loop is unrolled by PF so
  // that every buffer index is a compile-time constant.
  // (d = 256: two buffers, so that the four waves' K slots fit in LDS)
  constexpr int PF = D == 256 ? 2 : 4;
  using KV = KvRegs<D>;
  __shared__ __attribute__((aligned(1024))) char kring[NT / 64][PF][KV::KBYTES];
  char (*slots)[KV::KBYTES] = kring[wave];
  uint32_t koff[16 / KV::RPK];
#pragma unroll
  for (int i = 0; i < 16 / KV::RPK; ++i)
    koff[i] = PAGED ? KV::k_lane_off_rows(i, rs) : KV::k_lane_off(i);
  // rows this chunk reads: up to its last block (or the causal limit)
  const int end = min(Nk, max(blk1, blk0) * KB);
  const __amdgpu_buffer_rsrc_t vrs =
      buffer_rsrc(vh, (uint32_t)max(end, 0) * (2 * D));
  // starts the loads of block `blk` into a ring buffer and its K slot
  auto issue = [&](KV& bf, char* slot, int blk) {
    if (PAGED) {
      // the block's page (the chunk spans fewer than 64 pages), then its
      // rows inside that page
      const int kb = blk * KB;
      const int pslot = min(max((kb >> pg.page_shift) - first_page, 0), 63);
      const int page = __builtin_amdgcn_readlane(page_of_lane, pslot);
      const int64_t row0 =
          (((int64_t)page << pg.page_shift) + (kb & (pg.page_size - 1))) *
              Hkv * D +
          (int64_t)hkv * D;
      bf.load_rows(slot, koff, k + row0, v + row0, min(end - kb, KB), rs, h,
                   col);
    } else {
      bf.load(slot, koff, kh, vrs, blk * KB, end, h, col);
    }
  };
  KV buf[PF];
#pragma unroll
  for (int u = 0; u < PF - 1; ++u) issue(buf[u], slots[u], blk0 + u);
  auto compute = [&](const KV& cur, const char* kslot, int blk) {
    const int kb = blk * KB;
    // The compiler does not order these LDS reads after the copies that
    // filled the slot PF - 1 blocks ago, so wait for them here: the loads of
    // the PF - 1 later blocks are issued after this block's K copies (more
    // than the counter holds means those copies have completed).
    constexpr int kAfter = (PF - 1) * KV::OPS;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((kAfter > 62 ? 62 : kAfter) & 15 |
                               (((kAfter > 62 ? 62 : kAfter) >> 4) << 14) |
                               0x0F70);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
      s = mfma32x32x16(KV::kop(kslot, krow, h, t), qf[t], s);

    const bool need_mask = kb + KB - 1 > lim_first || (BAND && kb < lo_last);
    uint32_t vis = 0xffffu;
    if (need_mask) {
      vis = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 16 * (r >> 3) + 8 * h + (r & 7);
        if (key <= lim && (!BAND || key >= lo)) vis |= 1u << r;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!(vis & (1u << r))) s[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m, mx * c2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    // weights rounded to bf16 once: the rounded weights feed the P V
    // product and their own sum lb (normalises O); the fp32 sum l gives lse
    u32x4 pk[2];
    float rs = 0.f, rb = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float pa = exp2_fast(fmaf(s[r], c2, -m_use));
      float pc = exp2_fast(fmaf(s[r + 1], c2, -m_use));
      if (need_mask && !(vis & (1u << r))) pa = 0.f;
      if (need_mask && !(vis & (1u << (r + 1)))) pc = 0.f;
      rs += pa;
      rs += pc;
      const uint32_t w = pack_bf16x2(pa, pc);
      pk[r >> 3][(r >> 1) & 3] = w;
      rb = add_bf16x2(w, rb);
    }
    l = alpha * l + rs;
    lb = alpha * lb + rb;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] *= alpha;
    const bf16x8 p0 = __builtin_bit_cast(bf16x8, pk[0]);
    const bf16x8 p1 = __builtin_bit_cast(bf16x8, pk[1]);
#pragma unroll
    for (int tt = 0; tt < CPL; ++tt) {
      acc[tt] = mfma32x32x16(cur.vop(0, tt), p0, acc[tt]);
      acc[tt] = mfma32x32x16(cur.vop(1, tt), p1, acc[tt]);
    }
  };

  for (int blk = blk0; blk < blk1; blk += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      // refill the buffer the previous step consumed (past the chunk's end
      // the loads read zeros and are never used)
      issue(buf[(u + PF - 1) % PF], slots[(u + PF - 1) % PF],
            blk + u + PF - 1);
      if (blk + u < blk1) compute(buf[u], slots[u], blk + u);
    }
  }
  // no copy into LDS may still be in flight when the wave ends
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- partial result of this chunk (unnormalised O, max m, sum l)
  const float lt = pair_sum(l);
  const float lbt = pair_sum(lb);
  if (row_ok) {
    float* op = ws_o + (qrow_id * num_splits + sp) * D;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 8 * gg + 4 * h + e;  // operand row -> columns CPL*a + tt
        if (CPL >= 4) {
#pragma unroll
          for (int c = 0; c < CPL; c += 4)
            *reinterpret_cast<f32x4*>(op + CPL * a + c) =
                f32x4{acc[c][4 * gg + e], acc[c + 1][4 * gg + e],
                      acc[c + 2][4 * gg + e], acc[c + 3][4 * gg + e]};
        } else if (CPL == 2) {
          *reinterpret_cast<float2*>(op + CPL * a) =
              float2{acc[0][4 * gg + e], acc[CPL - 1][4 * gg + e]};
        } else {
          op[a] = acc[0][4 * gg + e];
        }
      }
    }
    if (h == 0) ws_ml[qrow_id * num_splits + sp] = f32x4{m, lt, lbt, 0.f};
  }
}

// One wave per output row; each lane owns D/64 columns (d = 32: lanes
// 0..31 one column each, the others idle).
template <int D, bool OUT_F32>
__global__ __launch_bounds__(NT) void splitkv_merge_kernel(
    const float* __restrict__ ws_o, const f32x4* __restrict__ ws_ml,
    void* __restrict__ o, float* __restrict__ lse, long long n_rows,
    int num_splits) {
  constexpr int CPL = D >= 64 ? D / 64 : 1;
  const int lane = threadIdx.x & 63;
  const bool has_col = CPL * lane < D;
  const long long row = (long long)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const f32x4* ml = ws_ml + row * num_splits;
  float M = -INFINITY;
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, ml[s][0]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, LB = 0.f;
  float a[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) a[i] = 0.f;
  const float* op = ws_o + row * num_splits * D + CPL * lane;
  for (int s = 0; s < num_splits; ++s) {
    const f32x4 x = ml[s];
    const float w = exp2_fast(x[0] - Mu);  // empty chunk: m = -inf -> 0
    L += w * x[1];
    LB += w * x[2];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (has_col) a[i] += w * op[(int64_t)s * D + i];
  }
  const float inv = LB > 0.f ? 1.f / LB : 0.f;
  if (!has_col) {
    // no column of this row for this lane
  } else if (OUT_F32) {
    float* dst = static_cast<float*>(o) + row * D + CPL * lane;
#pragma unroll
    for (int i = 0; i < CPL; ++i) dst[i] = a[i] * inv;
  } else {
    uint16_t* dst = static_cast<uint16_t*>(o) + row * D + CPL * lane;
    if (CPL == 4) {
      *reinterpret_cast<u32x2*>(dst) =
          u32x2{pack_bf16x2(a[0] * inv, a[1] * inv),
                pack_bf16x2(a[2] * inv, a[CPL - 1] * inv)};
    } else if (CPL == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(a[0] * inv, a[CPL - 1] * inv);
    } else {
      const uint32_t pk = pack_bf16x2(a[0] * inv, 0.f);
      dst[0] = (uint16_t)(pk & 0xffffu);
    }
  }
  if (lane == 0)
    lse[row] = L > 0.f ? (Mu + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

template <int D, int MODE, bool OUT_F32, bool PAGED>
hipError_t launch(const void* q, const void* k, const void* v, void* o,
                  float* lse, const Shape& s, int num_splits, void* ws,
                  const MaskBounds& mb, const PagedKv& pg,
                  hipStream_t stream) {
  const int G = s.Hq / s.Hkv;
  const long long R = (long long)s.Nq * G;
  const int n_rowtiles = (int)((R + kSplitRows - 1) / kSplitRows);
  // blocks a tile's chunks cover: all of the keys, or the blocks the band
  // of a tile can span
  const int nblk = band_tile_blocks(s, mb, KB);
  const int bps = (nblk + num_splits - 1) / num_splits;
  const long long n_items = (long long)s.B * s.Hkv * n_rowtiles * num_splits;
  const long long n_rows = (long long)s.B * s.Hq * s.Nq;
  float* ws_o = static_cast<float*>(ws);
  f32x4* ws_ml = reinterpret_cast<f32x4*>(ws_o + n_rows * num_splits * D);
  const float c2 = s.scale * kLog2e;
  const unsigned wpb = NT / 64;
  hipLaunchKernelGGL((splitkv_partial_kernel<D, MODE, PAGED>),
                     dim3((unsigned)((n_items + wpb - 1) / wpb)), dim3(NT), 0,
                     stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), ws_o, ws_ml, s.Hq, s.Hkv,
                     s.Nq, s.Nk, c2, n_rowtiles, num_splits, bps,
                     (int)n_items, mb.wl, mb.wr, pg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((splitkv_merge_kernel<D, OUT_F32>),
                     dim3((unsigned)((n_rows + wpb - 1) / wpb)), dim3(NT), 0,
                     stream, ws_o, ws_ml, o, lse, n_rows, num_splits);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o,
                    float* lse, const Shape& s, bool out_f32, int num_splits,
                    void* ws, const PagedKv& pg, hipStream_t stream) {
  const MaskBounds mb = mask_bounds(s);
#define FA_MODE(M_)                                                          \
  return out_f32 ? launch<D, M_, true, PAGED>(q, k, v, o, lse, s, num_splits, \
                                              ws, mb, pg, stream)            \
                 : launch<D, M_, false, PAGED>(q, k, v, o, lse, s,           \
                                               num_splits, ws, mb, pg, stream);
  if (mb.kind == 0) { FA_MODE(kNone) }
  if (mb.kind == 1) { FA_MODE(kCausal) }
  FA_MODE(kBand)
#undef FA_MODE
}

}  // namespace

size_t splitkv_workspace_bytes(long long rows, int d, int num_splits) {
  // per (row, chunk): d fp32 partial outputs + (m, l, lb, unused)
  return (size_t)rows * (size_t)num_splits * ((size_t)d * 4 + 16);
}

hipError_t launch_splitkv(const void* q, const void* k, const void* v,
                          void* o, float* lse, const Shape& s, bool out_f32,
                          int num_splits, void* workspace,
                          hipStream_t stream) {
  const PagedKv none{};
  if (s.d == 256)
    return launch_d<256, false>(q, k, v, o, lse, s, out_f32, num_splits,
                                workspace, none, stream);
  if (s.d == 128)
    return launch_d<128, false>(q, k, v, o, lse, s, out_f32, num_splits,
                                workspace, none, stream);
  if (s.d == 64)
    return launch_d<64, false>(q, k, v, o, lse, s, out_f32, num_splits,
                               workspace, none, stream);
  if (s.d == 32)
    return launch_d<32, false>(q, k, v, o, lse, s, out_f32, num_splits,
                               workspace, none, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_splitkv_kvlen(const void* q, const void* k, const void* v,
                                void* o, float* lse, const Shape& s,
                                const int* seqlen, bool out_f32,
                                int num_splits, void* workspace,
                                hipStream_t stream) {
  PagedKv lens{};
  lens.seqlen = seqlen;
  if (s.d == 256)
    return launch_d<256, false>(q, k, v, o, lse, s, out_f32, num_splits,
                                workspace, lens, stream);
  if (s.d == 128)
    return launch_d<128, false>(q, k, v, o, lse, s, out_f32, num_splits,
                                workspace, lens, stream);
  if (s.d == 64)
    return launch_d<64, false>(q, k, v, o, lse, s, out_f32, num_splits,
                               workspace, lens, stream);
  if (s.d == 32)
    return launch_d<32, false>(q, k, v, o, lse, s, out_f32, num_splits,
                               workspace, lens, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_splitkv_paged(const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse,
                                const Shape& s, const PagedKv& pg,
                                bool out_f32, int num_splits, void* workspace,
                                hipStream_t stream) {
  if (s.d == 256)
    return launch_d<256, true>(q, k_cache, v_cache, o, lse, s, out_f32,
                               num_splits, workspace, pg, stream);
  if (s.d == 128)
    return launch_d<128, true>(q, k_cache, v_cache, o, lse, s, out_f32,
                               num_splits, workspace, pg, stream);
  if (s.d == 64)
    return launch_d<64, true>(q, k_cache, v_cache, o, lse, s, out_f32,
                              num_splits, workspace, pg, stream);
  if (s.d == 32)
    return launch_d<32, true>(q, k_cache, v_cache, o, lse, s, out_f32,
                              num_splits, workspace, pg, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

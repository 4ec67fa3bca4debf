// Attention backward pass by recomputation ("FlashAttention Analysis",
// ryotta.opik.net, section 4 "Recomputation"): the probabilities are not
// stored; every kernel recomputes the scores of its tiles from Q and K and
// rebuilds P = exp(S - lse) from the one logsumexp per row the forward pass
// kept (FlashAttention version/GPU/training-cost guide, tool.smithlab.co.kr,
// attention-memory section).  With D_i = dO_i . O_i,
//     dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q,
// each KV head collecting the gradients of all query heads that read it.
//
// Three kernels, no atomics (every output element has one owner):
// * bwd_pre_kernel: D and lse in log2 units per query row, into the
//   workspace.
// * bwd_dkdv_kernel: one workgroup of 8 waves per (batch, KV head, 128
//   keys), in two roles over four groups of 32 keys: waves 0-3 hold K as
//   matrix-core operands, form S = Q K^T and P = exp2(S c - lse2), and
//   accumulate dV^T += dO^T P; waves 4-7 hold V, form dP = dO V^T, take P
//   from the first group through LDS, form dS = P (dP - D) and accumulate
//   dK^T += Q^T dS.  The two waves of a key group share a SIMD, so one
//   wave's vector work runs under the other's matrix products.  Tiles of 64
//   query rows of every query head of the group stream through LDS
//   (double-buffered), row steps from the last one down (without a band
//   the group's query heads inside a step).  Scores use v_mfma_f32_32x32x16_bf16 with lane = one
//   key and 16 query rows; the query rows are read in an order (bits 2 and
//   3 of the row index swapped) that makes a lane's score registers 8
//   consecutive rows, so P and dS serve as B operands as they are, and dO^T
//   and Q^T come from the row-major tiles through the transposing LDS read
//   ds_read_b64_tr_b16.
// * bwd_dq_kernel: one workgroup of 4 waves per (batch, query head, 128
//   query rows), 32 rows per wave with Q and dO in registers; K / V tiles
//   of 64 keys stream through LDS (double-buffered).  Per half tile:
//   S^T = K Q^T and dP^T = V dO^T (lane = one query row, 16 keys, key order
//   swapped the same way), dS^T in registers, then dQ += dS K with dS as
//   the A operand as it is and K read transposed.
// Tiles move HBM -> LDS with buffer_load ... lds, issued at the start of the
// step before the one that reads them; a buffer resource per copy ends at
// the head's last row, so tails arrive as zeros and are masked.  LDS tiles
// are row-major with a 16-byte-chunk XOR swizzle (no bank conflicts in
// either read direction), and operand reads run four products ahead of
// their matrix products.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int NT = 256;  // 4 waves

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

// Row of a 32-row tile that feeds operand row r: bits 2 and 3 swapped, so
// C-fragment register i of a lane holds tile row 16(i/8) + 8h + i%8.
__device__ __forceinline__ int row_slot(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int D>
struct Tiles {
  static constexpr int ROWP = 2 * D;   // LDS row (bytes)
  static constexpr int NSTEP = D / 16;  // k-steps over the head dim
  static constexpr int NTILE = D / 32;  // 32-column tiles of the head dim
};

// LDS tile swizzle: 16-byte chunk c of tile row r is stored at chunk
// c ^ swz(r).  Tiles are read both along rows (16-byte reads, 16 lanes on
// 16 different rows) and down columns (transposing 8-byte reads, 32 lanes
// on 4 rows x 64 bytes); with 64 banks of 4 bytes, swz spreads the 16 rows
// of the first over all 16 chunk positions of a 256-byte bank line and the
// 4 rows of the second over the four 64-byte quarters of it, so neither
// read nor the row-wise tile store has a bank conflict.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                  : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// A / B operand (8 bf16) of lane (row or column `lr` = lane % 32, half h)
// for k-step t of a tile row: head dims 16t + 8h .. +7 of LDS row `row`.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char* tile, int row,
                                              int h, int t) {
  using T = Tiles<D>;
  return *reinterpret_cast<const bf16x8*>(
      tile + row * T::ROWP + 16 * ((2 * t + h) ^ swz<D>(row)));
}

// Transposing operand read: lane (lr, h) gets the 8 values of column
// 32 ct + lr at tile rows 16 ks + 8h .. +7 (two ds_read_b64_tr_b16; within
// a 16-lane group, lane j addresses row base + j/4, columns 4(j%4) .. +3).
template <int D>
__device__ __forceinline__ bf16x8 col_operand(const char* tile, int ct,
                                              int ks) {
  using T = Tiles<D>;
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4, lp = lane & 15;
  const int row = 16 * ks + 8 * (lg >> 1) + (lp >> 2);
  // 16-byte chunk of columns 32 ct + 16 (lg % 2) + 4 (lp % 4) .. +3, and
  // the 8-byte half of it
  const int chunk = 4 * ct + 2 * (lg & 1) + ((lp & 3) >> 1);
  const int part = 8 * (lp & 1);
  const char* a0 = tile + row * T::ROWP + 16 * (chunk ^ swz<D>(row)) + part;
  const char* a1 =
      tile + (row + 4) * T::ROWP + 16 * (chunk ^ swz<D>(row + 4)) + part;
  const i16x4 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_char*)a0));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_char*)a1));
  u32x4 va;
  va[0] = __builtin_bit_cast(u32x2, lo)[0];
  va[1] = __builtin_bit_cast(u32x2, lo)[1];
  va[2] = __builtin_bit_cast(u32x2, hi)[0];
  va[3] = __builtin_bit_cast(u32x2, hi)[1];
  return __builtin_bit_cast(bf16x8, va);
}

// bf16 operand of k-step ks (0, 1) from a C fragment: registers 8 ks ..
// 8 ks + 7.
__device__ __forceinline__ bf16x8 pack_operand(const f32x16& c, int ks) {
  return to_bf16x8(c, 8 * ks);
}

// Runs N matrix products in program order; product i gets one operand from
// LDS through read(i), issued DEPTH products before its use so that LDS
// latency hides under the products in between.
template <int N, int DEPTH, class Read, class Mfma>
__device__ __forceinline__ void lds_pipeline(Read read, Mfma mfma) {
  bf16x8 ring[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH && i < N; ++i) ring[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = ring[i % DEPTH];
    if (i + DEPTH < N) ring[i % DEPTH] = read(i + DEPTH);
    mfma(i, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i and lse_i in log2 units, per query row.  One 16-byte
// chunk (8 values) per lane; D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(NT) void bwd_pre_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ dvec,
    float* __restrict__ lse2, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long t = (long long)blockIdx.x * NT + threadIdx.x;
  const long long row = t / LPR;
  const int c = (int)(t % LPR);
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = ldg16(o + row * D + 8 * c);
    const u32x4 b = ldg16(dout + row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the element out first: a bit cast of a vector element itself
      // reads the vector's first element
      const uint32_t ai = a[i], bi = b[i];
      const bf16x2 x = __builtin_bit_cast(bf16x2, ai);
      const bf16x2 y = __builtin_bit_cast(bf16x2, bi);
      s = fmaf((float)x[0], (float)y[0], s);
      s = fmaf((float)x[1], (float)y[1], s);
    }
  }
  // sum over the LPR lanes of the row (fixed butterfly order)
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
  if (row < rows && c == 0) {
    dvec[row] = s;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(0) alone (expcnt, lgkmcnt left free); gfx9 encoding.
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// HBM -> LDS copies of 64-row tiles with buffer_load ... lds (no staging
// registers).  Instruction n of a tile fills LDS bytes [1 KiB n, 1 KiB
// (n + 1)) = tile rows RPK n .. RPK n + RPK - 1; lane j writes the 16 bytes
// at 16 j, so it reads the logical chunk that the swizzle puts there.  The
// buffer resource of each instruction starts at its first row and ends at
// the head's last row, so rows past the end arrive as zeros.
template <int D>
struct TileDma {
  static constexpr int RPK = 1024 / (2 * D);  // rows per instruction
  static constexpr int NI = 64 / RPK;         // instructions per tile
  static constexpr int CPR = 2 * D / 16;      // 16-byte chunks per row
  // source offset of this lane within instruction n (depends on n only
  // through n % (16 / RPK))
  static __device__ __forceinline__ uint32_t lane_off(int n) {
    const int lane = threadIdx.x & 63;
    const int r = lane / CPR, p = lane % CPR;
    return (uint32_t)(r * (2 * D) + 16 * (p ^ swz<D>(RPK * n + r)));
  }
  // instruction n of the tile of rows r0 .. r0 + 63 of `head` (`rows` rows
  // of 2D bytes) into the LDS tile `dst`
  static __device__ __forceinline__ void issue(char* dst, const char* head,
                                               int rows, int r0, int n,
                                               uint32_t loff) {
    const int64_t start = (int64_t)(r0 + RPK * n) * (2 * D);
    const int64_t total = (int64_t)rows * (2 * D);
    const uint32_t rem = start < total ? (uint32_t)(total - start) : 0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        buffer_rsrc(head + start, rem), (lds_void*)(dst + 1024 * n), 16, loff,
        0, 0, 0);
  }
  // 64 fp32 values v[r0 .. r0 + 63] (zeros past `rows`) into `dst`; one
  // wave's instruction
  static __device__ __forceinline__ void issue_vec(float* dst, const float* v,
                                                   int rows, int r0) {
    const uint32_t rem = r0 < rows ? (uint32_t)(rows - r0) * 4u : 0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        buffer_rsrc(v + r0, rem), (lds_void*)dst, 4,
        (uint32_t)(threadIdx.x & 63) * 4u, 0, 0, 0);
  }
};

// lse2 / D of the 16 score registers of one 32-row half (register i holds
// tile row 16(i/8) + 8h + i%8 of the half)
__device__ __forceinline__ void row_stats(const float* v, int h, float* out) {
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(v + 16 * (i >> 3) + 8 * h +
                                                    (i & 7));
#pragma unroll
    for (int e = 0; e < 4; ++e) out[i + e] = a[e];
  }
}

// dK/dV kernel: 8 waves in two roles over the same 4 groups of 32 keys.
// Waves 0-3 hold K and accumulate dV (they form P); waves 4-7 hold V and
// accumulate dK (they form dP and dS).  A P wave and the dS wave of the same
// keys share a SIMD, so one wave's vector work runs under the other's
// matrix products.
constexpr int NT2 = 512;

// Mask kinds: none, causal (key j visible to query i iff j <= i + Nk - Nq),
// band (iff i + Nk - Nq - wl <= j <= i + Nk - Nq + wr).
constexpr int kNone = 0, kCausal = 1, kBand = 2;

template <int D, int MODE, bool OUT_F32>
__global__ __launch_bounds__(NT2, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ dvec, const float* __restrict__ lse2,
    void* __restrict__ dk, void* __restrict__ dv, int Hq, int Hkv, int Nq,
    int Nk, float c2, float scale, int n_kblk, int wl, int wr) {
  constexpr bool CAUSAL = MODE == kCausal;
  constexpr bool BAND = MODE == kBand;
  using T = Tiles<D>;
  constexpr int NSTEP = T::NSTEP, NTILE = T::NTILE;
  constexpr int QR = 64;  // query rows per step
  using Dma = TileDma<D>;
  // one stage: [Q tile | dO tile | lse2[64] | D[64]]
  constexpr int STAGE = 2 * QR * T::ROWP + 2 * QR * 4;
  // P handed from the P waves to the dS waves, fp32: per key group 2 halves
  // x 4 chunks x 64 lanes x 4 values, chunk-major (conflict-free)
  constexpr int XFLOATS = 2 * 4 * 64 * 4;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE +
                                                      4 * XFLOATS * 4];

  const int lane = threadIdx.x & 63;
  // wave index, uniform (so buffer resources and LDS bases of copies stay
  // in scalar registers instead of going through per-lane loops)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, col = lane & 31;
  const bool pw = wave < 4;  // P wave (K, dV) or dS wave (V, dK)
  const int kw = wave & 3;   // key group
  float* xw = reinterpret_cast<float*>(smem + 2 * STAGE) + kw * XFLOATS;

  // work item: (b, kv head, key block of 128); causal: early keys (more
  // query rows to visit) first
  const int item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int kblk = item % n_kblk;
  const int bh = item / n_kblk;  // b * Hkv + hkv
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int G = Hq / Hkv;
  const int off = Nk - Nq;
  const int kfirst = kblk * 128;
  const int key = kfirst + kw * 32 + col;  // this lane's key

  // K (P waves) or V (dS waves) of the group's keys as B operands: lane
  // (col, h) holds [key][16t + 8h .. +7]
  bf16x8 kv[NSTEP];
  {
    const uint16_t* src = (pw ? k : v) + ((int64_t)bh * Nk + key) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
      kv[t] = __builtin_bit_cast(bf16x8, key < Nk ? ldg16(src + 16 * t)
                                                  : u32x4{0u, 0u, 0u, 0u});
  }
  f32x16 acc[NTILE];  // dV^T (P waves) or dK^T / scale (dS waves)
#pragma unroll
  for (int i = 0; i < NTILE; ++i) acc[i] = f32x16{};

  // query rows that can see a key of this workgroup (causal: rows i with
  // i + off >= its first key; band: also i + off - wl <= its last key), in
  // steps of QR rows, for each of the G query heads of the group
  const int t_begin = CAUSAL ? max(0, kfirst - off) / QR
                      : BAND ? max(0, kfirst - off - wr) / QR
                             : 0;
  const int t_end =
      BAND ? (max(0, min(Nq, kfirst + 128 - off + wl)) + QR - 1) / QR
           : (Nq + QR - 1) / QR;
  const int n_it = G * max(0, t_end - t_begin);
  const bool keys_in = kfirst + 128 <= Nk;
  const int arow = row_slot(col);  // tile row read for operand row col

  // copies of one step: 2 * NI tile instructions spread over the 8 waves
  // (instruction i = wave + 8 m: tile i / NI, part i % NI, the same part
  // modulo the swizzle period for every m), lse2 by wave 0, D by wave 1
  static_assert((2 * Dma::NI) % 8 == 0, "copy split");
  const uint32_t loff = Dma::lane_off(wave);
  // Row steps run from the last one down, so that the workgroups of one KV
  // head sweep the same Q / dO tiles at about the same time and share them
  // in L2.  Without a band they all start at the last row and stop at
  // different rows (causal), so the G query heads of a step come next to
  // each other and the sweeps stay in step across heads.  With a band each
  // workgroup's rows are a window that starts 128 rows after the previous
  // key block's, so the workgroups run staggered by design; there the
  // heads come one after another, which keeps the rows read at one time to
  // one head's (heads inside a step multiply them by G and overflow L2).
  constexpr bool HEADS_INNER = !BAND;
  int pg = 0, pt = t_end - 1;  // query head and row step of the next copy
  auto copy_step = [&](char* dst) {
    const int64_t qh = (int64_t)(b * Hq + hkv * G + pg) * Nq;
    const int r0 = pt * QR;
#pragma unroll
    for (int m = 0; m < 2 * Dma::NI / 8; ++m) {
      const int i = wave + 8 * m;
      const bool second = i >= Dma::NI;
      Dma::issue(dst + (second ? QR * T::ROWP : 0),
                 reinterpret_cast<const char*>((second ? dout : q) + qh * D),
                 Nq, r0, i % Dma::NI, loff);
    }
    float* st = reinterpret_cast<float*>(dst + 2 * QR * T::ROWP);
    if (wave == 0) Dma::issue_vec(st, lse2 + qh, Nq, r0);
    if (wave == 1) Dma::issue_vec(st + QR, dvec + qh, Nq, r0);
    if (HEADS_INNER) {
      if (++pg == G) {
        pg = 0;
        --pt;
      }
    } else if (--pt < t_begin) {
      pt = t_end - 1;
      ++pg;
    }
  };
  if (n_it > 0) copy_step(smem);
  wait_vmcnt0();
  __syncthreads();

  int ct_row = t_end - 1;  // row step being computed
  int ct_g = 0;            // and its query head
  // one step on stage PAR (a compile-time constant, so that every LDS
  // address of the step is a per-lane base plus an immediate)
  auto step = [&](int it, auto par) {
    constexpr int PAR = decltype(par)::value;
    const char* qt = smem + PAR * STAGE;
    const char* dt = qt + QR * T::ROWP;
    const float* ls = reinterpret_cast<const float*>(qt + 2 * QR * T::ROWP);
    const float* dd = ls + QR;
    const int q0 = ct_row * QR;
    if (HEADS_INNER) {
      if (++ct_g == G) {
        ct_g = 0;
        --ct_row;
      }
    } else if (--ct_row < t_begin) {
      ct_row = t_end - 1;
    }
    if (it + 1 < n_it) copy_step(smem + (1 - PAR) * STAGE);

    // Products on rows 32 half .. +31 of the step: C row 8(i/4) + 4h + i%4
    // reads tile row row_slot of it, so register i holds row
    // 32 half + 16(i/8) + 8h + i%8 and the column is the lane's key.
    bf16x8 op[4];  // P or dS operands, k-steps of 16 rows
    // S = Q K^T (P waves) or dP = dO V^T (dS waves) for both halves,
    // products alternating between the two accumulators
    f32x16 sp[2] = {f32x16{}, f32x16{}};
    {
      const char* at = pw ? qt : dt;
      lds_pipeline<2 * NSTEP, 4>(
          [&](int i) {
            return row_operand<D>(at, 32 * (i & 1) + arow, h, i >> 1);
          },
          [&](int i, bf16x8 a) {
            sp[i & 1] = mfma32x32x16(a, kv[i >> 1], sp[i & 1]);
          });
    }
    if (pw) {
      // every score of the step visible: all rows in range, all keys in
      // range, and the first row sees the workgroup's last key
      const bool full = q0 + QR <= Nq && keys_in &&
                        (!CAUSAL || kfirst + 127 <= q0 + off) &&
                        (!BAND || (kfirst + 127 <= q0 + off + wr &&
                                   kfirst >= q0 + QR - 1 + off - wl));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float lsv[16];
        row_stats(ls + 32 * half, h, lsv);
        f32x16 p;
        if (full) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            p[i] = exp2_fast(fmaf(sp[half][i], c2, -lsv[i]));
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = q0 + 32 * half + 16 * (i >> 3) + 8 * h + (i & 7);
            bool vis = row < Nq && key < Nk;
            if (CAUSAL) vis = vis && key <= row + off;
            if (BAND)
              vis = vis && key <= row + off + wr && key >= row + off - wl;
            // rows that see no key have lse = -inf; their P is 0
            const float e = exp2_fast(fmaf(sp[half][i], c2, -lsv[i]));
            p[i] = vis && lsv[i] != -INFINITY ? e : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<f32x4*>(xw + (4 * half + e) * 256 + 4 * lane) =
              f32x4{p[4 * e], p[4 * e + 1], p[4 * e + 2], p[4 * e + 3]};
        op[2 * half] = pack_operand(p, 0);
        op[2 * half + 1] = pack_operand(p, 1);
      }
    }
    __syncthreads();  // P of the step visible to the dS waves
    if (!pw) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float ddv[16];
        row_stats(dd + 32 * half, h, ddv);
        f32x16 ds;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4 p = *reinterpret_cast<const f32x4*>(
              xw + (4 * half + e) * 256 + 4 * lane);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            ds[4 * e + u] = p[u] * (sp[half][4 * e + u] - ddv[4 * e + u]);
        }
        op[2 * half] = pack_operand(ds, 0);
        op[2 * half + 1] = pack_operand(ds, 1);
      }
    }
    // dV^T += dO^T P (P waves), dK^T += Q^T dS (dS waves); rows = head
    // dims of tile ct; product i: k-step i / NTILE, tile i % NTILE
    {
      const char* at = pw ? dt : qt;
      lds_pipeline<4 * NTILE, 4>(
          [&](int i) { return col_operand<D>(at, i % NTILE, i / NTILE); },
          [&](int i, bf16x8 a) {
            acc[i % NTILE] = mfma32x32x16(a, op[i / NTILE], acc[i % NTILE]);
          });
    }
    wait_vmcnt0();  // this wave's copies for the next step have landed
    __syncthreads();
  };
  int it = 0;
  for (; it + 2 <= n_it; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    step(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < n_it) step(it, std::integral_constant<int, 0>{});

  // epilogue: lane holds dV^T or dK^T rows 8(i/4) + 4h + i%4 of tile ct
  // (head dims), column = its key
  if (key < Nk) {
    const int64_t base = ((int64_t)bh * Nk + key) * D;
    const float sc = pw ? 1.f : scale;
    void* out = pw ? dv : dk;
#pragma unroll
    for (int ct = 0; ct < NTILE; ++ct) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int c = 32 * ct + 8 * gg + 4 * h;
        const f32x16& a = acc[ct];
        if (OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + base + c) =
              f32x4{a[4 * gg] * sc, a[4 * gg + 1] * sc, a[4 * gg + 2] * sc,
                    a[4 * gg + 3] * sc};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + base + c) =
              u32x2{pack_bf16x2(a[4 * gg] * sc, a[4 * gg + 1] * sc),
                    pack_bf16x2(a[4 * gg + 2] * sc, a[4 * gg + 3] * sc)};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int D, int MODE, bool OUT_F32>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ dvec, const float* __restrict__ lse2,
    void* __restrict__ dq, int Hq, int Hkv, int Nq, int Nk, float c2,
    float scale, int n_qblk, int wl, int wr) {
  constexpr bool CAUSAL = MODE == kCausal;
  constexpr bool BAND = MODE == kBand;
  using T = Tiles<D>;
  constexpr int NSTEP = T::NSTEP, NTILE = T::NTILE;
  constexpr int KR = 64;  // keys per step
  using Dma = TileDma<D>;
  constexpr int STAGE = 2 * KR * T::ROWP;  // [K tile | V tile]
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63;
  // wave index, uniform (so buffer resources and LDS bases of copies stay
  // in scalar registers instead of going through per-lane loops)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, col = lane & 31;

  // work item: (b, kv head, Q block of 128, head in group); causal: late
  // rows (more keys) first
  const int item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int G = Hq / Hkv;
  const int gq = item % G;
  const int t1 = item / G;
  const int jq = t1 % n_qblk;
  const int bh = t1 / n_qblk;
  const int qblk = MODE != kNone ? (n_qblk - 1 - jq) : jq;
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int hq = hkv * G + gq;
  const int off = Nk - Nq;
  const int64_t qhead = (int64_t)(b * Hq + hq) * Nq;
  const int qfirst = qblk * 128;
  const int qrow = qfirst + wave * 32 + col;  // this lane's query row
  const bool row_ok = qrow < Nq;

  // Q^T and dO^T as B operands: lane (col, h) holds row [16t + 8h .. +7]
  bf16x8 qf[NSTEP], df[NSTEP];
  {
    const uint16_t* qp = q + (qhead + (row_ok ? qrow : 0)) * D + 8 * h;
    const uint16_t* dp = dout + (qhead + (row_ok ? qrow : 0)) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      qf[t] = __builtin_bit_cast(bf16x8, row_ok ? ldg16(qp + 16 * t)
                                                : u32x4{0u, 0u, 0u, 0u});
      df[t] = __builtin_bit_cast(bf16x8, row_ok ? ldg16(dp + 16 * t)
                                                : u32x4{0u, 0u, 0u, 0u});
    }
  }
  const float l2 = row_ok ? lse2[qhead + qrow] : -INFINITY;
  const float dval = row_ok ? dvec[qhead + qrow] : 0.f;
  f32x16 acc[NTILE];  // dQ: rows 8(i/4) + 4h + i%4 (query), column = dim
#pragma unroll
  for (int i = 0; i < NTILE; ++i) acc[i] = f32x16{};

  const int64_t kvbase = (int64_t)bh * Nk * D;
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, qfirst + 128 + off);
  // band: keys from the first row's lower bound to the last row's upper one
  int j0 = 0;
  if (BAND) {
    kv_end = min(Nk, min(qfirst + 128, Nq) + off + wr);
    j0 = max(0, qfirst + off - wl) / KR;
  }
  const int nblk = kv_end > 0 ? (kv_end + KR - 1) / KR : 0;
  const int arow = row_slot(col);
  // this lane's last (band: and first) visible key
  const int lim = CAUSAL ? min(Nk - 1, qrow + off)
                  : BAND ? min(Nk - 1, qrow + off + wr)
                         : Nk - 1;
  const int lo = BAND ? qrow + off - wl : 0;
  // rows all in range (then every row sees key 0 or more)
  const bool rows_in = qfirst + 128 <= Nq;
  const char* kh = reinterpret_cast<const char*>(k + kvbase);
  const char* vh = reinterpret_cast<const char*>(v + kvbase);

  // copies of one step: 2 * NI tile instructions spread over the 4 waves
  // (instruction i = wave + 4 m: tile i / NI, part i % NI, the same part
  // modulo the swizzle period for every m)
  static_assert((2 * Dma::NI) % 4 == 0, "copy split");
  const uint32_t loff = Dma::lane_off(wave);
  auto copy_step = [&](char* dst, int k0) {
#pragma unroll
    for (int m = 0; m < 2 * Dma::NI / 4; ++m) {
      const int i = wave + 4 * m;
      const bool second = i >= Dma::NI;
      Dma::issue(dst + (second ? KR * T::ROWP : 0), second ? vh : kh, Nk, k0,
                 i % Dma::NI, loff);
    }
  };
  if (nblk > j0) copy_step(smem, j0 * KR);
  wait_vmcnt0();
  __syncthreads();

  // one step on stage PAR (compile-time, so LDS addresses are a per-lane
  // base plus an immediate)
  auto step = [&](int j, auto par) {
    constexpr int PAR = decltype(par)::value;
    const char* kt = smem + PAR * STAGE;
    const char* vt = kt + KR * T::ROWP;
    const int k0 = j * KR;
    if (j + 1 < nblk) copy_step(smem + (1 - PAR) * STAGE, k0 + KR);
    // every score of the step visible: keys in range, rows in range, and
    // the workgroup's first row sees the step's last key
    const bool full = k0 + KR <= Nk && rows_in &&
                      (!CAUSAL || k0 + KR - 1 <= qfirst + off) &&
                      (!BAND || (k0 + KR - 1 <= qfirst + off + wr &&
                                 k0 >= qfirst + 127 + off - wl));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // S^T = K Q^T, dP^T = V dO^T for keys 32 half + row_slot(row):
      // register i holds key 32 half + 16(i/8) + 8h + i%8, column = query;
      // products alternate between the two accumulators
      f32x16 sp[2] = {f32x16{}, f32x16{}};
      lds_pipeline<2 * NSTEP, 4>(
          [&](int i) {
            return row_operand<D>((i & 1) ? vt : kt, 32 * half + arow, h,
                                  i >> 1);
          },
          [&](int i, bf16x8 a) {
            sp[i & 1] = mfma32x32x16(a, (i & 1) ? df[i >> 1] : qf[i >> 1],
                                     sp[i & 1]);
          });
      f32x16 ds;
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ds[i] = exp2_fast(fmaf(sp[0][i], c2, -l2)) * (sp[1][i] - dval);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * half + 16 * (i >> 3) + 8 * h + (i & 7);
          const bool vis = row_ok && key <= lim && (!BAND || key >= lo) &&
                           l2 != -INFINITY;
          const float p = vis ? exp2_fast(fmaf(sp[0][i], c2, -l2)) : 0.f;
          ds[i] = p * (sp[1][i] - dval);
        }
      }
      // dQ += dS K: A = dS (row = query, k = keys 8h + 0..7 of k-step ks),
      // B = K read transposed (k = key, column = head dim); product i:
      // k-step i / NTILE, tile i % NTILE
      const bf16x8 a2[2] = {pack_operand(ds, 0), pack_operand(ds, 1)};
      lds_pipeline<2 * NTILE, 4>(
          [&](int i) {
            return col_operand<D>(kt, i % NTILE, 2 * half + i / NTILE);
          },
          [&](int i, bf16x8 b2) {
            acc[i % NTILE] = mfma32x32x16(a2[i / NTILE], b2, acc[i % NTILE]);
          });
    }
    wait_vmcnt0();  // this wave's copies for the next step have landed
    __syncthreads();
  };
  int j = j0;
  for (; j + 2 <= nblk; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    step(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < nblk) step(j, std::integral_constant<int, 0>{});

  // epilogue: lane holds dQ rows 8(i/4) + 4h + i%4 of the wave's 32 rows,
  // column 32 ct + col
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = qfirst + wave * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (r < Nq) {
#pragma unroll
      for (int ct = 0; ct < NTILE; ++ct) {
        const int64_t idx = (qhead + r) * D + 32 * ct + col;
        const float x = acc[ct][i] * scale;
        if (OUT_F32)
          static_cast<float*>(dq)[idx] = x;
        else
          static_cast<uint16_t*>(dq)[idx] =
              (uint16_t)(pack_bf16x2(x, 0.f) & 0xFFFFu);
      }
    }
  }
}

template <int D, int MODE, bool OUT_F32>
hipError_t launch_bwd(const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, const Shape& s,
                      const MaskBounds& mb, void* workspace,
                      hipStream_t stream) {
  const long long rows = (long long)s.B * s.Hq * s.Nq;
  float* dvec = static_cast<float*>(workspace);
  float* lse2 = dvec + rows;
  const float c2 = s.scale * kLog2e;
  {
    const long long threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>),
                       dim3((unsigned)((threads + NT - 1) / NT)), dim3(NT), 0,
                       stream, static_cast<const uint16_t*>(o),
                       static_cast<const uint16_t*>(dout), lse, dvec, lse2,
                       rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kblk = (s.Nk + 127) / 128;
    const long long items = (long long)s.B * s.Hkv * n_kblk;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, MODE, OUT_F32>),
                       dim3((unsigned)items), dim3(NT2), 0, stream,
                       static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), dvec, lse2, dk, dv,
                       s.Hq, s.Hkv, s.Nq, s.Nk, c2, s.scale, n_kblk, mb.wl,
                       mb.wr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qblk = (s.Nq + 127) / 128;
  const long long items = (long long)s.B * s.Hq * n_qblk;
  hipLaunchKernelGGL((bwd_dq_kernel<D, MODE, OUT_F32>),
                     dim3((unsigned)items), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dout), dvec, lse2, dq, s.Hq,
                     s.Hkv, s.Nq, s.Nk, c2, s.scale, n_qblk, mb.wl, mb.wr);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv, const Shape& s,
                        bool out_f32, void* ws, hipStream_t stream) {
  const MaskBounds mb = mask_bounds(s);
#define FA_MODE(M_)                                                          \
  return out_f32 ? launch_bwd<D, M_, true>(q, k, v, o, lse, dout, dq, dk, dv, \
                                           s, mb, ws, stream)                \
                 : launch_bwd<D, M_, false>(q, k, v, o, lse, dout, dq, dk,   \
                                            dv, s, mb, ws, stream);
  if (mb.kind == 0) { FA_MODE(kNone) }
  if (mb.kind == 1) { FA_MODE(kCausal) }
  FA_MODE(kBand)
#undef FA_MODE
}

}  // namespace

size_t backward_workspace_bytes(long long rows) {
  return (size_t)rows * 2 * sizeof(float);  // D and lse2 per query row
}

hipError_t launch_backward(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, const Shape& s,
                           bool out_f32, void* workspace, hipStream_t stream) {
  if (s.d == 128)
    return launch_bwd_d<128>(q, k, v, o, lse, dout, dq, dk, dv, s, out_f32,
                             workspace, stream);
  if (s.d == 64)
    return launch_bwd_d<64>(q, k, v, o, lse, dout, dq, dk, dv, s, out_f32,
                            workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

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
// * bwd_dkdv_kernel: one workgroup per (batch, KV head, 128 keys), 4 waves
//   of 32 keys.  K and V of the wave's keys stay in registers as matrix-core
//   operands; the Q / dO tiles of 32 query rows of every query head of the
//   group stream through LDS.  Per tile: S = Q K^T and dP = dO V^T
//   (v_mfma_f32_32x32x16_bf16, lane = one key, 16 query rows), P and dS in
//   registers, then dV^T += dO^T P and dK^T += Q^T dS with P and dS as the
//   B operands as they are (the query rows are read in an order, bits 2 and
//   3 of the row index swapped, that makes a lane's score registers 8
//   consecutive query rows) and dO^T, Q^T read with the transposing LDS
//   read ds_read_b64_tr_b16.
// * bwd_dq_kernel: one workgroup per (batch, query head, 128 query rows),
//   4 waves of 32 rows, Q and dO in registers; K / V tiles of 64 keys
//   stream through LDS.  Per tile: S^T = K Q^T and dP^T = V dO^T (lane = one
//   query row, 16 keys, key order swapped the same way), dS^T in registers,
//   then dQ += dS K with dS as the A operand as it is and K read
//   transposed.
// Tiles are staged through LDS in row-major order with rows padded by 16
// bytes.  Tails read as zeros and are masked.
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
  static constexpr int ROWP = 2 * D + 16;  // padded LDS row (bytes)
  static constexpr int NSTEP = D / 16;     // k-steps over the head dim
  static constexpr int NTILE = D / 32;     // 32-column tiles of the head dim
};

// Copies rows [r0, r0 + R) of a [N, D] bf16 matrix into LDS (padded rows);
// rows at or past N are zeros.  All NT threads take part.
template <int D, int R>
__device__ __forceinline__ void stage_rows(char* dst, const uint16_t* src,
                                           int r0, int N) {
  using T = Tiles<D>;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = threadIdx.x; i < R * CPR; i += NT) {
    const int r = i / CPR, c = i % CPR;
    const int row = r0 + r;
    const u32x4 x = row < N ? ldg16(src + (int64_t)row * D + 8 * c)
                            : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(dst + r * T::ROWP + 16 * c) = x;
  }
}

// A / B operand (8 bf16) of lane (row or column `lr` = lane % 32, half h)
// for k-step t of a tile row: head dims 16t + 8h .. +7 of LDS row `row`.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char* tile, int row,
                                              int h, int t) {
  using T = Tiles<D>;
  return *reinterpret_cast<const bf16x8*>(tile + row * T::ROWP + 32 * t +
                                          16 * h);
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
  const int col = 32 * ct + 16 * (lg & 1) + 4 * (lp & 3);
  const char* a0 = tile + row * T::ROWP + 2 * col;
  const i16x4 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_char*)a0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((lds_char*)(a0 + 4 * T::ROWP)));
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
// Register prefetch of the next pair of row tiles (R rows each, R = one
// wave's lanes: Q and dO, or K and V) and, with STATS, the lse2 and D
// values of the rows; stored to an LDS buffer laid out as [first tile |
// second tile | lse2[R] | D[R]] after the current step's products.  The
// loads go through buffer resources spanning one head, so rows past its
// end read as zeros.
template <int D, int R, bool STATS>
struct TilePrefetch {
  using T = Tiles<D>;
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int N = 2 * R * CPR / NT;      // chunks per thread
  static constexpr int BYTES = 2 * R * T::ROWP + (STATS ? 2 * R * 4 : 0);
  static_assert(N * NT == 2 * R * CPR && N % 2 == 0 && R == 64, "tile split");
  u32x4 x[N];
  float st;

  // ra, rb: the two tiles' heads (rows of D bf16)
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t ra,
                                       __amdgpu_buffer_rsrc_t rb, int r0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = threadIdx.x + NT * (j % (N / 2));
      const int r = i / CPR, c = i % CPR;
      x[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     j < N / 2 ? ra : rb, (r0 + r) * (2 * D) + 16 * c, 0, 0));
    }
  }
  // rl, rv: lse2 and D of the head; waves 0 and 1 fetch one each (a
  // wave-uniform choice)
  __device__ __forceinline__ void load_stats(__amdgpu_buffer_rsrc_t rl,
                                             __amdgpu_buffer_rsrc_t rv,
                                             int r0) {
    if (threadIdx.x < R)
      st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rl, (r0 + threadIdx.x) * 4, 0, 0));
    else if (threadIdx.x < 2 * R)
      st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rv, (r0 + threadIdx.x - R) * 4, 0, 0));
  }
  __device__ __forceinline__ void store(char* buf) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = threadIdx.x + NT * (j % (N / 2));
      const int r = i / CPR, c = i % CPR;
      *reinterpret_cast<u32x4*>(buf + (j < N / 2 ? 0 : R * T::ROWP) +
                                r * T::ROWP + 16 * c) = x[j];
    }
    if (STATS && threadIdx.x < 2 * R)
      reinterpret_cast<float*>(buf + 2 * R * T::ROWP)[threadIdx.x] = st;
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

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NT, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ dvec, const float* __restrict__ lse2,
    void* __restrict__ dk, void* __restrict__ dv, int Hq, int Hkv, int Nq,
    int Nk, float c2, float scale, int n_kblk) {
  using T = Tiles<D>;
  constexpr int NSTEP = T::NSTEP, NTILE = T::NTILE;
  constexpr int QR = 64;  // query rows per step
  using Pf = TilePrefetch<D, QR, true>;
  __shared__ __attribute__((aligned(16))) char smem[2 * Pf::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;

  // work item: (b, kv head, key block of 128); causal: early keys (more
  // query rows to visit) first
  const int item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int kblk = item % n_kblk;
  const int bh = item / n_kblk;  // b * Hkv + hkv
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int G = Hq / Hkv;
  const int off = Nk - Nq;
  const int kfirst = kblk * 128;
  const int key = kfirst + wave * 32 + col;  // this lane's key

  // K and V of the wave's keys as B operands: lane (col, h) holds
  // [key][16t + 8h .. +7]
  const uint16_t* kh = k + (int64_t)bh * Nk * D;
  const uint16_t* vh = v + (int64_t)bh * Nk * D;
  bf16x8 kf[NSTEP], vf[NSTEP];
#pragma unroll
  for (int t = 0; t < NSTEP; ++t) {
    const bool ok = key < Nk;
    kf[t] = __builtin_bit_cast(bf16x8, ok ? ldg16(kh + (int64_t)key * D + 16 * t + 8 * h)
                                          : u32x4{0u, 0u, 0u, 0u});
    vf[t] = __builtin_bit_cast(bf16x8, ok ? ldg16(vh + (int64_t)key * D + 16 * t + 8 * h)
                                          : u32x4{0u, 0u, 0u, 0u});
  }
  f32x16 dkt[NTILE], dvt[NTILE];
#pragma unroll
  for (int i = 0; i < NTILE; ++i) {
    dkt[i] = f32x16{};
    dvt[i] = f32x16{};
  }

  // query rows that can see a key of this workgroup (causal: rows i with
  // i + off >= its first key), in steps of QR rows, for each of the G query
  // heads of the group
  const int t_begin = CAUSAL ? max(0, kfirst - off) / QR : 0;
  const int t_end = (Nq + QR - 1) / QR;
  const int n_it = G * (t_end - t_begin);
  const bool keys_in = kfirst + 128 <= Nk;
  const int arow = row_slot(col);  // tile row read for operand row col
  const uint32_t head_bytes = (uint32_t)Nq * (2 * D);

  // (g, t): query head within the group and row step of the next prefetch
  int pg = 0, pt = t_begin;
  Pf pf;
  auto prefetch = [&]() {
    const int64_t qh = (int64_t)(b * Hq + hkv * G + pg) * Nq;
    pf.load(buffer_rsrc(q + qh * D, head_bytes),
            buffer_rsrc(dout + qh * D, head_bytes), pt * QR);
    pf.load_stats(buffer_rsrc(lse2 + qh, (uint32_t)Nq * 4),
                  buffer_rsrc(dvec + qh, (uint32_t)Nq * 4), pt * QR);
    if (++pt == t_end) {
      pt = t_begin;
      ++pg;
    }
  };
  if (n_it > 0) {
    prefetch();
    pf.store(smem);
  }
  __syncthreads();

  int ct_row = t_begin;  // row step being computed
  for (int it = 0; it < n_it; ++it) {
    const char* buf = smem + (it & 1) * Pf::BYTES;
    const char* qt = buf;
    const char* dt = buf + QR * T::ROWP;
    const float* ls = reinterpret_cast<const float*>(buf + 2 * QR * T::ROWP);
    const float* dd = ls + QR;
    const int q0 = ct_row * QR;
    if (++ct_row == t_end) ct_row = t_begin;
    if (it + 1 < n_it) prefetch();
    // every score of the step visible: all rows in range, all keys in
    // range, and the first row sees the workgroup's last key
    const bool full = q0 + QR <= Nq && keys_in &&
                      (!CAUSAL || kfirst + 127 <= q0 + off);

    bf16x8 pop[4], sop[4];  // P and dS operands, k-steps of 16 rows
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // S = Q K^T and dP = dO V^T for rows 32 half .. +31: C row
      // 8(i/4) + 4h + i%4 reads tile row row_slot of it, i.e. register i
      // holds row 32 half + 16(i/8) + 8h + i%8, column = key
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < NSTEP; ++t) {
        s = mfma32x32x16(row_operand<D>(qt, 32 * half + arow, h, t), kf[t], s);
        dp = mfma32x32x16(row_operand<D>(dt, 32 * half + arow, h, t), vf[t],
                          dp);
      }
      float lsv[16], ddv[16];
      row_stats(ls + 32 * half, h, lsv);
      row_stats(dd + 32 * half, h, ddv);
      f32x16 p, ds;
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = exp2_fast(fmaf(s[i], c2, -lsv[i]));
          ds[i] = p[i] * (dp[i] - ddv[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = q0 + 32 * half + 16 * (i >> 3) + 8 * h + (i & 7);
          bool vis = row < Nq && key < Nk;
          if (CAUSAL) vis = vis && key <= row + off;
          // rows that see no key have lse = -inf; their P is 0
          const float e = exp2_fast(fmaf(s[i], c2, -lsv[i]));
          p[i] = vis && lsv[i] != -INFINITY ? e : 0.f;
          ds[i] = p[i] * (dp[i] - ddv[i]);
        }
      }
      pop[2 * half] = pack_operand(p, 0);
      pop[2 * half + 1] = pack_operand(p, 1);
      sop[2 * half] = pack_operand(ds, 0);
      sop[2 * half + 1] = pack_operand(ds, 1);
    }
    // dV^T += dO^T P, dK^T += Q^T dS (rows = head dims of tile ct)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int ct = 0; ct < NTILE; ++ct) {
        dvt[ct] = mfma32x32x16(col_operand<D>(dt, ct, ks), pop[ks], dvt[ct]);
        dkt[ct] = mfma32x32x16(col_operand<D>(qt, ct, ks), sop[ks], dkt[ct]);
      }
    }
    if (it + 1 < n_it) pf.store(smem + ((it + 1) & 1) * Pf::BYTES);
    __syncthreads();
  }

  // epilogue: lane holds dK^T / dV^T rows 8(i/4) + 4h + i%4 of tile ct
  // (head dims), column = its key
  if (key < Nk) {
    const int64_t base = ((int64_t)bh * Nk + key) * D;
#pragma unroll
    for (int ct = 0; ct < NTILE; ++ct) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int c = 32 * ct + 8 * gg + 4 * h;
        const f32x16& a = dkt[ct];
        const f32x16& w = dvt[ct];
        if (OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(dk) + base + c) =
              f32x4{a[4 * gg] * scale, a[4 * gg + 1] * scale,
                    a[4 * gg + 2] * scale, a[4 * gg + 3] * scale};
          *reinterpret_cast<f32x4*>(static_cast<float*>(dv) + base + c) =
              f32x4{w[4 * gg], w[4 * gg + 1], w[4 * gg + 2], w[4 * gg + 3]};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dk) + base + c) =
              u32x2{pack_bf16x2(a[4 * gg] * scale, a[4 * gg + 1] * scale),
                    pack_bf16x2(a[4 * gg + 2] * scale, a[4 * gg + 3] * scale)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dv) + base + c) =
              u32x2{pack_bf16x2(w[4 * gg], w[4 * gg + 1]),
                    pack_bf16x2(w[4 * gg + 2], w[4 * gg + 3])};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ dvec, const float* __restrict__ lse2,
    void* __restrict__ dq, int Hq, int Hkv, int Nq, int Nk, float c2,
    float scale, int n_qblk) {
  using T = Tiles<D>;
  constexpr int NSTEP = T::NSTEP, NTILE = T::NTILE;
  constexpr int KR = 64;  // keys per step
  using Pf = TilePrefetch<D, KR, false>;
  __shared__ __attribute__((aligned(16))) char smem[2 * Pf::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;

  // work item: (b, kv head, Q block of 128, head in group); causal: late
  // rows (more keys) first
  const int item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int G = Hq / Hkv;
  const int gq = item % G;
  const int t1 = item / G;
  const int jq = t1 % n_qblk;
  const int bh = t1 / n_qblk;
  const int qblk = CAUSAL ? (n_qblk - 1 - jq) : jq;
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
  const int nblk = kv_end > 0 ? (kv_end + KR - 1) / KR : 0;
  const int arow = row_slot(col);
  // this lane's last visible key
  const int lim = CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1;
  // rows all in range (then every row sees key 0 or more)
  const bool rows_in = qfirst + 128 <= Nq;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + kvbase, (uint32_t)Nk * (2 * D));
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(v + kvbase, (uint32_t)Nk * (2 * D));

  Pf pf;
  if (nblk > 0) {
    pf.load(rk, rv, 0);
    pf.store(smem);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const char* buf = smem + (j & 1) * Pf::BYTES;
    const char* kt = buf;
    const char* vt = buf + KR * T::ROWP;
    const int k0 = j * KR;
    if (j + 1 < nblk) pf.load(rk, rv, k0 + KR);
    // every score of the step visible: keys in range, rows in range, and
    // the workgroup's first row sees the step's last key
    const bool full = k0 + KR <= Nk && rows_in &&
                      (!CAUSAL || k0 + KR - 1 <= qfirst + off);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // S^T = K Q^T, dP^T = V dO^T for keys 32 half + row_slot(row):
      // register i holds key 32 half + 16(i/8) + 8h + i%8, column = query
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < NSTEP; ++t) {
        s = mfma32x32x16(row_operand<D>(kt, 32 * half + arow, h, t), qf[t],
                         s);
        dp = mfma32x32x16(row_operand<D>(vt, 32 * half + arow, h, t), df[t],
                          dp);
      }
      f32x16 ds;
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ds[i] = exp2_fast(fmaf(s[i], c2, -l2)) * (dp[i] - dval);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * half + 16 * (i >> 3) + 8 * h + (i & 7);
          const bool vis = row_ok && key <= lim && l2 != -INFINITY;
          const float p = vis ? exp2_fast(fmaf(s[i], c2, -l2)) : 0.f;
          ds[i] = p * (dp[i] - dval);
        }
      }
      // dQ += dS K: A = dS (row = query, k = keys 8h + 0..7 of k-step ks),
      // B = K read transposed (k = key, column = head dim)
      const bf16x8 a0 = pack_operand(ds, 0), a1 = pack_operand(ds, 1);
#pragma unroll
      for (int ct = 0; ct < NTILE; ++ct) {
        acc[ct] = mfma32x32x16(a0, col_operand<D>(kt, ct, 2 * half), acc[ct]);
        acc[ct] =
            mfma32x32x16(a1, col_operand<D>(kt, ct, 2 * half + 1), acc[ct]);
      }
    }
    if (j + 1 < nblk) pf.store(smem + ((j + 1) & 1) * Pf::BYTES);
    __syncthreads();
  }

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

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_bwd(const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, const Shape& s,
                      void* workspace, hipStream_t stream) {
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
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, OUT_F32>),
                       dim3((unsigned)items), dim3(NT), 0, stream,
                       static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), dvec, lse2, dk, dv,
                       s.Hq, s.Hkv, s.Nq, s.Nk, c2, s.scale, n_kblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qblk = (s.Nq + 127) / 128;
  const long long items = (long long)s.B * s.Hq * n_qblk;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, OUT_F32>),
                     dim3((unsigned)items), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dout), dvec, lse2, dq, s.Hq,
                     s.Hkv, s.Nq, s.Nk, c2, s.scale, n_qblk);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(long long rows) {
  return (size_t)rows * 2 * sizeof(float);  // D and lse2 per query row
}

hipError_t launch_backward(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, const Shape& s,
                           bool out_f32, void* workspace, hipStream_t stream) {
  const bool c = s.causal != 0;
#define FA_DISPATCH(D_)                                                       \
  if (s.d == D_) {                                                            \
    if (c)                                                                    \
      return out_f32 ? launch_bwd<D_, true, true>(q, k, v, o, lse, dout, dq,  \
                                                  dk, dv, s, workspace, stream) \
                     : launch_bwd<D_, true, false>(q, k, v, o, lse, dout, dq, \
                                                   dk, dv, s, workspace,      \
                                                   stream);                   \
    return out_f32 ? launch_bwd<D_, false, true>(q, k, v, o, lse, dout, dq,   \
                                                 dk, dv, s, workspace, stream) \
                   : launch_bwd<D_, false, false>(q, k, v, o, lse, dout, dq,  \
                                                  dk, dv, s, workspace,       \
                                                  stream);                    \
  }
  FA_DISPATCH(128)
  FA_DISPATCH(64)
#undef FA_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace fa

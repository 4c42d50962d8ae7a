// Block statistics for PISA: centroids, value sums, H_j, Hbar and M_j.
//
// PISA summary (gist.science), section 2: "Core algorithm" (centroid kbar_j,
// value sum, H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n}, Hbar = mean of H_j),
// "Covariance-aware routing" (M_j = ||H_j - Hbar||_2, Frobenius reading) and
// "Hardware implementation" (computed before the attention stages).
//
// bf16 path: H_j = K_j^T V_j - kbar_j^T sigma_j, with K_j^T V_j on bf16 MFMA
// (products of bf16 values are exact in the fp32 accumulator).  Pass 1 streams
// K and V once and writes one fp32 partial sum of H_j per group of
// kStatsGroup blocks; a fixed-order fp64 reduction gives Hbar; pass 2 streams K
// and V again, recomputes each H_j and writes M_j (and H_j when asked).  No
// atomics: results are bitwise reproducible.
//
// fp32 path: plain fp32 VALU arithmetic with centred keys; H_j is kept in a
// buffer, reduced to Hbar, then M_j is read off the buffer.
#include "common.hpp"
#include "launch.hpp"

namespace pisa {
namespace {

template <int D, int BLK>
struct SCfg {
  static constexpr int NT = 256;
  static constexpr int ROW = BLK + 8;                 // LDS row (tokens) of K^T / V^T, padded
  static constexpr int SUB = (BLK / 8) * (D / 8);     // 8x8 sub-tiles per tensor
  static constexpr int PER_T = (2 * SUB + NT - 1) / NT;
  static constexpr int TM = (D == 128) ? 2 : 1;       // 32x32 output tiles per wave, per dim
  static_assert(2 * D <= NT, "column sums use one thread per column");
};

// STORE: pass 2 also writes the optional H_j (fp32) and H_j^T (bf16) outputs;
// without them pass 2 fits 256 registers and runs two workgroups per CU.
template <int D, int BLK, bool PASS2, bool STORE>
__global__ __launch_bounds__(256, (PASS2 && STORE) ? 1 : 2) void stats_bf16_kernel(
    const bf16* __restrict__ K, const bf16* __restrict__ V, int nb, float* __restrict__ centroid,
    float* __restrict__ vsum, float* __restrict__ partial, const float* __restrict__ hbar_frag,
    float* __restrict__ M, float* __restrict__ Hout, bf16* __restrict__ pk_cen,
    bf16* __restrict__ pk_vsum, bf16* __restrict__ Ht, const int32_t* __restrict__ lens,
    int heads) {
  using C = SCfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) bf16 Kt[D * C::ROW];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * C::ROW];
  __shared__ float s_k[D];
  __shared__ float s_v[D];
  __shared__ float s_red[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q32 = lane & 31, hh = lane >> 5;
  const int ngrp = (nb + kStatsGroup - 1) / kStatsGroup;
  const int bh = blockIdx.x / ngrp, grp = blockIdx.x - bh * ngrp;
  const int j0 = grp * kStatsGroup;
  const int j1 = min(nb, j0 + kStatsGroup);
  const size_t L = (size_t)nb * BLK;
  const bf16* Kh = K + (size_t)bh * L * D;
  const bf16* Vh = V + (size_t)bh * L * D;
  const int mt0 = (w >> 1) * C::TM, nt0 = (w & 1) * C::TM;
  const int Lv = valid_len(lens, bh, heads, (int)L);      // tokens past Lv are not counted

  f32x16 acc[C::TM][C::TM];
#pragma unroll
  for (int a = 0; a < C::TM; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b) acc[a][b] = f32x16{};

  // pass 2: this lane's Hbar entries, stored by the reduction in fragment order
  // (4 consecutive floats per (tile, row group)); re-read per block from L2
  // rather than held in 64 registers for the whole loop
  const float* hbf = PASS2 ? hbar_frag + (size_t)bh * D * D + (size_t)w * C::TM * C::TM * 1024 + 4 * lane
                           : nullptr;

  u32x4 regs[C::PER_T][8];
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < C::PER_T; ++u) {
      const int p = tid + u * C::NT;
      if (p < 2 * C::SUB) {
        const bf16* X = ((p < C::SUB) ? Kh : Vh) + (size_t)j * BLK * D;
        const int q = p % C::SUB;
        const int g = q % (BLK / 8), c = q / (BLK / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) regs[u][e] = ld16(X + (8 * g + e) * D + 8 * c);
      }
    }
  };
  auto lstore = [&](int nj) {
#pragma unroll
    for (int u = 0; u < C::PER_T; ++u) {
      const int p = tid + u * C::NT;
      if (p < 2 * C::SUB) {
        bf16* Xt = (p < C::SUB) ? Kt : Vt;
        const int q = p % C::SUB;
        const int g = q % (BLK / 8), c = q / (BLK / 8);
        // tokens 8 g + e at or past the block's valid count are stored as zeros
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * g + e >= nj) regs[u][e] = u32x4{0u, 0u, 0u, 0u};
        u32x4 col[8];
        transpose8x8(regs[u], col);
#pragma unroll
        for (int i = 0; i < 8; ++i) st16(Xt + (8 * c + i) * C::ROW + 8 * g, col[i]);
      }
    }
  };

  gload(j0);
  for (int j = j0; j < j1; ++j) {
    const int nj = block_count(Lv, j, BLK);
    __syncthreads();
    lstore(nj);
    __syncthreads();
    if (j + 1 < j1) gload(j + 1);

    // centroid (mean of keys) and value sum, one thread per column
    if (tid < 2 * D) {
      const bf16* rp = (tid < D) ? (Kt + tid * C::ROW) : (Vt + (tid - D) * C::ROW);
      float s = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < BLK / 8; ++c8) {
        const bf16x8 v = as_bf16x8(ld16(rp + 8 * c8));
#pragma unroll
        for (int e = 0; e < 8; ++e) s += (float)v[e];
      }
      const size_t prow = ((size_t)bh * ((nb + BLK - 1) / BLK * BLK) + j) * D;
      if (tid < D) {
        const float kbar = (nj == BLK) ? s * (1.f / BLK) : (nj > 0 ? s / (float)nj : 0.f);
        s_k[tid] = kbar;
        if (!PASS2) {
          centroid[((size_t)bh * nb + j) * D + tid] = kbar;
          if (pk_cen) pk_cen[prow + tid] = (bf16)kbar;
        }
      } else {
        s_v[tid - D] = s;
        if (!PASS2) {
          vsum[((size_t)bh * nb + j) * D + (tid - D)] = s;
          if (pk_vsum) pk_vsum[prow + (tid - D)] = (bf16)s;
        }
      }
    }

    // K_j^T V_j on MFMA: A = K^T rows (key dim), B = V^T rows (value dim), k = tokens
    if (PASS2) {
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b) acc[a][b] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < BLK / 16; ++ks) {
      bf16x8 A[C::TM], Bv[C::TM];
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
        A[a] = as_bf16x8(ld16(Kt + (32 * (mt0 + a) + q32) * C::ROW + 16 * ks + 8 * hh));
#pragma unroll
      for (int b = 0; b < C::TM; ++b)
        Bv[b] = as_bf16x8(ld16(Vt + (32 * (nt0 + b) + q32) * C::ROW + 16 * ks + 8 * hh));
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b) acc[a][b] = mfma32(A[a], Bv[b], acc[a][b]);
    }
    __syncthreads();

    // H_j = K_j^T V_j - kbar_j^T sigma_j
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
      for (int b = 0; b < C::TM; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ra = 32 * (mt0 + a) + 8 * (r / 4) + 4 * hh + (r % 4);
          const int cb = 32 * (nt0 + b) + q32;
          acc[a][b][r] -= s_k[ra] * s_v[cb];
        }

    if (PASS2) {
      float sq = 0.f;
      float* Hj = (STORE && Hout) ? Hout + ((size_t)bh * nb + j) * D * D : nullptr;
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 h4 = *reinterpret_cast<const f32x4*>(hbf + ((a * C::TM + b) * 4 + g) * 256);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int r = 4 * g + rr;
              const float x = acc[a][b][r];
              const float dlt = x - h4[rr];
              sq += dlt * dlt;
              if (Hj) Hj[(32 * (mt0 + a) + 8 * (r / 4) + 4 * hh + (r % 4)) * D + 32 * (nt0 + b) + q32] = x;
            }
          }
      if (STORE && Ht) {
        // H_j^T in bf16: row = value dim, 4 consecutive key-dim columns per store
        bf16* Hj = Ht + ((size_t)bh * nb + j) * D * D;
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
#pragma unroll
          for (int b = 0; b < C::TM; ++b)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x16& x = acc[a][b];
              const u32x2 v = {pack2(x[4 * g4], x[4 * g4 + 1]), pack2(x[4 * g4 + 2], x[4 * g4 + 3])};
              st8(Hj + (size_t)(32 * (nt0 + b) + q32) * D + 32 * (mt0 + a) + 8 * g4 + 4 * hh, v);
            }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
      if (lane == 0) s_red[w] = sq;
      __syncthreads();
      if (tid == 0) M[(size_t)bh * nb + j] = nj > 0 ? sqrtf(s_red[0] + s_red[1] + s_red[2] + s_red[3]) : 0.f;
    }
  }

  if (!PASS2) {
    float* P = partial + ((size_t)bh * ngrp + grp) * D * D;
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
      for (int b = 0; b < C::TM; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          P[(32 * (mt0 + a) + 8 * (r / 4) + 4 * hh + (r % 4)) * D + 32 * (nt0 + b) + q32] = acc[a][b][r];
  }
}

// Hbar[bh][e] = (1/nb) sum_g parts[bh][g][e], summed in fp64 in group order.
// With a bf16 pack: also writes Hbar^T in bf16 and zeroes the padding rows
// (nb .. nbp) of the packed centroids and value sums.
__global__ __launch_bounds__(256) void hbar_reduce_kernel(const float* __restrict__ parts, int ngrp,
                                                          int nb, int D, int total,
                                                          float* __restrict__ hbar,
                                                          bf16* __restrict__ pk_hbart,
                                                          bf16* __restrict__ pk_cen,
                                                          bf16* __restrict__ pk_vsum, int nbp,
                                                          const int32_t* __restrict__ lens,
                                                          int heads, int BLK,
                                                          float* __restrict__ hbar_frag) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int DD = D * D;
  if (t < total) {
    const int bh = t / DD, e = t - bh * DD;
    const float* p = parts + (size_t)bh * ngrp * DD + e;
    // loads of 8 groups in flight, summed in group order (fixed, reproducible)
    double s = 0.0;
    int g = 0;
    for (; g + 8 <= ngrp; g += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = p[(size_t)(g + u) * DD];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += (double)x[u];
    }
    for (; g < ngrp; ++g) s += (double)p[(size_t)g * DD];
    // mean over the non-empty blocks (all nb without lengths)
    const int nne = (valid_len(lens, bh, heads, nb * BLK) + BLK - 1) / BLK;
    const float v = nne > 0 ? (float)(s / nne) : 0.f;
    hbar[t] = v;
    if (hbar_frag) {
      // fragment order of the statistics kernel's pass 2: wave w = 2 (row tile / TM) +
      // (column tile / TM) holds tiles (a, b); lane q32 + 32 hh holds rows
      // 32 mt + 8 g + 4 hh + rr of column 32 nt + q32; 4 rows rr are contiguous
      const int TM = (D == 128) ? 2 : 1;
      const int row = e / D, col = e - (e / D) * D;
      const int mt = row >> 5, rem = row & 31, nt = col >> 5;
      const int wv = 2 * (mt / TM) + nt / TM, a = mt % TM, b = nt % TM;
      const int g = rem >> 3, hh = (rem >> 2) & 1, rr = rem & 3, ln = (col & 31) + 32 * hh;
      hbar_frag[(size_t)bh * DD + ((((wv * TM + a) * TM + b) * 4 + g) * 64 + ln) * 4 + rr] = v;
    }
    if (pk_hbart) {
      const int a = e / D, c = e - a * D;
      pk_hbart[(size_t)bh * DD + (size_t)c * D + a] = (bf16)v;
    }
  }
  if (pk_cen && nbp > nb) {
    const int per = (nbp - nb) * D;
    const int npad = (total / DD) * per;
    for (int u = t; u < npad; u += gridDim.x * 256) {
      const int bh = u / per, r = u - bh * per;
      const size_t o = ((size_t)bh * nbp + nb) * D + r;
      pk_cen[o] = (bf16)0.f;
      pk_vsum[o] = (bf16)0.f;
    }
  }
}

// ---------------------------------------------------------------- fp32 path

// one workgroup per (bh, block j): centroid, value sum and H_j with centred keys
template <int D>
__global__ __launch_bounds__(256) void stats_f32_block_kernel(
    const float* __restrict__ K, const float* __restrict__ V, int nb, int BLK,
    float* __restrict__ centroid, float* __restrict__ vsum, float* __restrict__ Hbuf,
    const int32_t* __restrict__ lens, int heads) {
  constexpr int NT = 256, CH = 32, PER = D * D / NT;
  __shared__ float kc[CH][D];
  __shared__ float vc[CH][D];
  __shared__ float s_k[D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / nb, j = blockIdx.x - bh * nb;
  const float* Kb = K + ((size_t)bh * nb + j) * BLK * D;
  const float* Vb = V + ((size_t)bh * nb + j) * BLK * D;
  const int nj = block_count(valid_len(lens, bh, heads, nb * BLK), j, BLK);   // valid tokens
  if (tid < D) {
    float sk = 0.f, sv = 0.f;
    for (int n = 0; n < nj; ++n) {
      sk += Kb[(size_t)n * D + tid];
      sv += Vb[(size_t)n * D + tid];
    }
    const float kbar = nj > 0 ? sk / nj : 0.f;
    s_k[tid] = kbar;
    centroid[((size_t)bh * nb + j) * D + tid] = kbar;
    vsum[((size_t)bh * nb + j) * D + tid] = sv;
  }
  __syncthreads();
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = 0.f;
  for (int n0 = 0; n0 < BLK; n0 += CH) {
    for (int q = tid; q < CH * D; q += NT) {
      const int n = q / D, c = q % D;
      const bool ok = n0 + n < nj;
      kc[n][c] = ok ? Kb[(size_t)(n0 + n) * D + c] - s_k[c] : 0.f;
      vc[n][c] = ok ? Vb[(size_t)(n0 + n) * D + c] : 0.f;
    }
    __syncthreads();
    for (int n = 0; n < CH; ++n)
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + u * NT;
        acc[u] += kc[n][e / D] * vc[n][e % D];
      }
    __syncthreads();
  }
  float* Hj = Hbuf + ((size_t)bh * nb + j) * D * D;
#pragma unroll
  for (int u = 0; u < PER; ++u) Hj[tid + u * NT] = acc[u];
}

// M_j = ||H_j - Hbar||_F, one workgroup per (bh, j), fixed reduction order
template <int D>
__global__ __launch_bounds__(256) void frob_kernel(const float* __restrict__ Hbuf,
                                                   const float* __restrict__ hbar, int nb,
                                                   float* __restrict__ M, const int32_t* lens,
                                                   int heads, int BLK) {
  __shared__ float s_red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x / nb;
  const float* Hj = Hbuf + (size_t)blockIdx.x * D * D;
  const float* hb = hbar + (size_t)bh * D * D;
  float sq = 0.f;
  for (int e = tid; e < D * D; e += 256) {
    const float dlt = Hj[e] - hb[e];
    sq += dlt * dlt;
  }
  for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
  if (lane == 0) s_red[w] = sq;
  __syncthreads();
  const int j = blockIdx.x - bh * nb;
  const bool empty = block_count(valid_len(lens, bh, heads, nb * BLK), j, BLK) == 0;
  if (tid == 0) M[blockIdx.x] = empty ? 0.f : sqrtf(s_red[0] + s_red[1] + s_red[2] + s_red[3]);
}

// ---- spectral reading of M_j = ||H_j - Hbar||_2: the largest singular value
//
// One workgroup per block.  A = H_j - Hbar is staged in LDS (rows padded to
// D + 4 floats, so the row reads of A v are conflict-free 16-byte reads and the
// column reads of A^T u conflict-free 4-byte reads).  kLanczos steps of plain
// Lanczos on A^T A from a fixed start vector give a tridiagonal T whose largest
// eigenvalue approximates sigma_max^2 from below; without reorthogonalisation
// the extreme eigenvalue still converges (lost orthogonality only repeats
// converged values).  Wave 0 then finds lambda_max(T) by multisection on Sturm
// counts in fp64 (64 points per round, 6 rounds: 65^6 > 7e10), and
// M_j = sqrt(lambda_max).
// Reductions run in a fixed order, so the result is bitwise reproducible.
constexpr int kLanczos = 24;

template <int NT>
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

template <int D>
__global__ __launch_bounds__(256) void spectral_kernel(const float* __restrict__ H,
                                                       const float* __restrict__ hbar, int nb,
                                                       float* __restrict__ M, const int32_t* lens,
                                                       int heads, int BLK) {
  constexpr int NT = 256, LD = D + 4, NH = NT / D, CW = D / NH;
  __shared__ __attribute__((aligned(16))) float A[D * LD];
  __shared__ __attribute__((aligned(16))) float v[D];
  __shared__ float vp[D], u[D], part[NT], red[NT / 64];
  __shared__ float s_al[kLanczos], s_be[kLanczos];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x, bh = blk / nb;
  if (block_count(valid_len(lens, bh, heads, nb * BLK), blk - bh * nb, BLK) == 0) {
    if (tid == 0) M[blk] = 0.f;                   // empty block: never routed
    return;
  }
  const float* Hj = H + (size_t)blk * D * D;
  const float* Hb = hbar + (size_t)bh * D * D;
  for (int e = 4 * tid; e < D * D; e += 4 * NT) {
    const f32x4 h = *reinterpret_cast<const f32x4*>(Hj + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(Hb + e);
    *reinterpret_cast<f32x4*>(&A[(e / D) * LD + e % D]) = h - b;
  }
  const int r = tid % D, h = tid / D;            // row (or column) and which slice of it
  float x0 = 0.f;
  if (tid < D) x0 = 1.f + (float)((unsigned)tid * 2654435761u % 1024u) * (1.f / 1024.f);
  const float n0 = block_sum<NT>(x0 * x0, red);
  if (tid < D) {
    v[tid] = x0 / sqrtf(n0);
    vp[tid] = 0.f;
  }
  __syncthreads();
  float beta = 0.f;
  int kk = 0;
  for (int it = 0; it < kLanczos; ++it) {
    // u = A v: thread (r, h) sums columns h*CW .. h*CW + CW - 1 of row r
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};             // four independent FMA chains
    {
      const float* Ar = &A[r * LD + h * CW];
      const float* vv = &v[h * CW];
#pragma unroll
      for (int c = 0; c < CW; c += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(Ar + c);
        const f32x4 b = *reinterpret_cast<const f32x4*>(vv + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc4[e] = fmaf(a[e], b[e], acc4[e]);
      }
    }
    part[tid] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    __syncthreads();
    if (tid < D) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NH; ++q) t += part[q * D + tid];
      u[tid] = t;
    }
    __syncthreads();
    // w = A^T u: thread (c = r, h) sums rows h*CW .. h*CW + CW - 1 of column c
    acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int rr = h * CW; rr < h * CW + CW; rr += 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc4[e] = fmaf(A[(rr + e) * LD + r], u[rr + e], acc4[e]);
    }
    part[tid] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    __syncthreads();
    float w = 0.f, vc = 0.f;
    if (tid < D) {
#pragma unroll
      for (int q = 0; q < NH; ++q) w += part[q * D + tid];
      vc = v[tid];
    }
    const float alpha = block_sum<NT>(vc * w, red);
    if (tid < D) w = w - alpha * vc - beta * vp[tid];
    const float bnew = sqrtf(block_sum<NT>(w * w, red));
    if (tid == 0) {
      s_al[it] = alpha;
      s_be[it] = bnew;
    }
    kk = it + 1;
    if (!(bnew > 1e-6f * fabsf(alpha))) break;      // invariant subspace (or A = 0)
    if (tid < D) {
      vp[tid] = vc;
      v[tid] = w / bnew;
    }
    beta = bnew;
    __syncthreads();
  }
  __syncthreads();
  if (tid < 64) {
    // lambda_max of the kk x kk tridiagonal (diag s_al, off-diag s_be) by
    // multisection: count(x) = number of eigenvalues below x = number of
    // negative pivots of T - x I; lanes with count < kk lie below lambda_max.
    const int lane = tid;
    double hi = 0.0;
    for (int i = 0; i < kk; ++i) {
      double g = fabs((double)s_al[i]);
      if (i > 0) g += fabs((double)s_be[i - 1]);
      if (i + 1 < kk) g += fabs((double)s_be[i]);
      hi = fmax(hi, g);
    }
    double lo = 0.0;                               // A^T A is positive semidefinite
    for (int round = 0; round < 6; ++round) {
      const double step = (hi - lo) / 65.0;
      const double x = lo + step * (lane + 1);
      int cnt = 0;
      double dd = 1.0;
      for (int i = 0; i < kk; ++i) {
        const double b2 = (i > 0) ? (double)s_be[i - 1] * (double)s_be[i - 1] : 0.0;
        dd = ((double)s_al[i] - x) - (i > 0 ? b2 / dd : 0.0);
        if (dd == 0.0) dd = -1e-300;
        cnt += dd < 0.0;
      }
      const unsigned long long below = __ballot(cnt < kk);
      if (below == 0ull) {
        hi = lo + step;
      } else {
        const int l = 63 - __clzll(below);
        const double nlo = lo + step * (l + 1);
        hi = (l == 63) ? hi : lo + step * (l + 2);
        lo = nlo;
      }
    }
    if (lane == 0) M[blk] = (float)sqrt(0.5 * (lo + hi));
  }
}

template <int D>
hipError_t launch_spectral(const float* H, const float* hbar, int bh, int nb, float* M,
                           const StatsArgs& a) {
  hipLaunchKernelGGL((spectral_kernel<D>), dim3(bh * nb), dim3(256), 0, a.stream, H, hbar, nb, M,
                     a.lens, a.heads, a.BLK);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t stats_bf16_t(const StatsArgs& a) {
  const int ngrp = (a.nb + kStatsGroup - 1) / kStatsGroup;
  const int nbp = (a.nb + BLK - 1) / BLK * BLK;
  float* parts = static_cast<float*>(a.ws);
  bf16* pk = static_cast<bf16*>(a.packed);
  bf16* pk_cen = pk;
  bf16* pk_vsum = pk ? pk + (size_t)a.bh * nbp * D : nullptr;
  bf16* pk_hbart = pk ? pk + (size_t)2 * a.bh * nbp * D : nullptr;
  const int grid = a.bh * ngrp;
  float* frag = parts + (size_t)a.bh * ngrp * D * D;     // Hbar in pass 2's fragment order
  hipLaunchKernelGGL((stats_bf16_kernel<D, BLK, false, false>), dim3(grid), dim3(256), 0, a.stream,
                     (const bf16*)a.K, (const bf16*)a.V, a.nb, a.centroid, a.vsum, parts,
                     (const float*)nullptr, (float*)nullptr, (float*)nullptr, pk_cen, pk_vsum,
                     (bf16*)nullptr, a.lens, a.heads);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int total = a.bh * D * D;
  hipLaunchKernelGGL(hbar_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, a.stream,
                     (const float*)parts, ngrp, a.nb, D, total, a.hbar, pk_hbart, pk_cen, pk_vsum,
                     nbp, a.lens, a.heads, BLK, frag);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  auto pass2 = (a.H || a.ht) ? stats_bf16_kernel<D, BLK, true, true> : stats_bf16_kernel<D, BLK, true, false>;
  hipLaunchKernelGGL(pass2, dim3(grid), dim3(256), 0, a.stream,
                     (const bf16*)a.K, (const bf16*)a.V, a.nb, (float*)nullptr, (float*)nullptr,
                     (float*)nullptr, (const float*)frag, a.M, a.H, (bf16*)nullptr,
                     (bf16*)nullptr, static_cast<bf16*>(a.ht), a.lens, a.heads);
  err = hipGetLastError();
  if (err != hipSuccess || !a.spectral) return err;
  return launch_spectral<D>(a.H, a.hbar, a.bh, a.nb, a.M, a);
}

template <int D>
hipError_t stats_f32_t(const StatsArgs& a) {
  float* Hbuf = a.H ? a.H : static_cast<float*>(a.ws);
  const int grid = a.bh * a.nb;
  hipLaunchKernelGGL((stats_f32_block_kernel<D>), dim3(grid), dim3(256), 0, a.stream,
                     (const float*)a.K, (const float*)a.V, a.nb, a.BLK, a.centroid, a.vsum, Hbuf,
                     a.lens, a.heads);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int total = a.bh * D * D;
  hipLaunchKernelGGL(hbar_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, a.stream,
                     (const float*)Hbuf, a.nb, a.nb, D, total, a.hbar, (bf16*)nullptr,
                     (bf16*)nullptr, (bf16*)nullptr, a.nb, a.lens, a.heads, a.BLK, (float*)nullptr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.spectral) return launch_spectral<D>(Hbuf, a.hbar, a.bh, a.nb, a.M, a);
  hipLaunchKernelGGL((frob_kernel<D>), dim3(grid), dim3(256), 0, a.stream, (const float*)Hbuf,
                     (const float*)a.hbar, a.nb, a.M, a.lens, a.heads, a.BLK);
  return hipGetLastError();
}

}  // namespace

size_t stats_workspace_bf16(int bh, int nb, int D) {
  // per-group partial sums of H_j, then Hbar in pass 2's fragment order
  const size_t ngrp = (size_t)(nb + kStatsGroup - 1) / kStatsGroup;
  return (size_t)bh * (ngrp + 1) * D * D * sizeof(float);
}

size_t stats_packed_bytes(int bh, int nb, int D, int BLK) {
  const size_t nbp = (size_t)(nb + BLK - 1) / BLK * BLK;
  return (size_t)bh * (2 * nbp * D + (size_t)D * D) * sizeof(bf16);
}

size_t stats_workspace_f32(int bh, int nb, int D) {
  return (size_t)bh * nb * D * D * sizeof(float);
}

hipError_t launch_stats_bf16(const StatsArgs& a) {
  if (a.D == 128 && a.BLK == 64) return stats_bf16_t<128, 64>(a);
  if (a.D == 128 && a.BLK == 128) return stats_bf16_t<128, 128>(a);
  if (a.D == 64 && a.BLK == 64) return stats_bf16_t<64, 64>(a);
  if (a.D == 64 && a.BLK == 128) return stats_bf16_t<64, 128>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_stats_f32(const StatsArgs& a) {
  if (a.D == 128) return stats_f32_t<128>(a);
  if (a.D == 64) return stats_f32_t<64>(a);
  return hipErrorInvalidValue;
}

}  // namespace pisa

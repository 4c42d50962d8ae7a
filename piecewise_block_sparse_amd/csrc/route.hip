// Covariance-aware top-k routing (PISA summary, gist.science, section 2,
// "Covariance-aware routing": the block score combines the attention score
// with M_j = ||H_j - Hbar||).  Score of query block i and KV block j:
//
//     score_ij = scale * qbar_i . kbar_j + lambda * M_j     (float64)
//
// qbar_i is the mean query of block i.  The sum of bf16 (or fp32) values in
// float64 is exact for these block sizes, so qbar_i carries no rounding; the
// dot products are float64 FMAs.  S_i = the k highest scores, ties to the lower
// j, written in ascending order.
//
// One workgroup = 2 waves = 2 query blocks of one head.  Each wave pools its
// block's queries with 16-byte loads, the workgroup stages 32-centroid tiles
// through LDS for the scores, and each wave sorts its row's block ids with a
// bitonic network in LDS (score descending, id ascending; padding last).
#include "common.hpp"
#include "launch.hpp"

namespace pisa {
namespace {

constexpr int kRows = 2;       // query blocks per workgroup (one wave each)
constexpr int kCT = 32;        // centroids per LDS tile

template <typename T>
struct Load8;
template <>
struct Load8<bf16> {
  __device__ static void get(const bf16* p, double (&x)[8]) {
    const bf16x8 v = as_bf16x8(ld16(p));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (double)(float)v[e];
  }
};
template <>
struct Load8<float> {
  __device__ static void get(const float* p, double (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = (double)a[e];
      x[4 + e] = (double)b[e];
    }
  }
};

__device__ __forceinline__ bool before(int ia, int ib, const double* sc, int nb) {
  if (ia >= nb) return (ib >= nb) && (ia < ib);
  if (ib >= nb) return true;
  const double a = sc[ia], b = sc[ib];
  return (a > b) || (a == b && ia < ib);
}

template <int D, typename T>
__global__ __launch_bounds__(64 * kRows) void route_kernel(const T* __restrict__ Q,
                                                            const float* __restrict__ centroid,
                                                            const float* __restrict__ M, int nb,
                                                            int BLK, int nbp, int k, double scale,
                                                            double lam, int32_t* __restrict__ idx) {
  __shared__ double s_q[kRows][D];
  __shared__ float s_c[kCT][D + 1];
  __shared__ double s_sc[kRows][kMaxBlocks];
  __shared__ short s_ord[kRows][kMaxBlocks];
  __shared__ unsigned s_sel[kRows][kMaxBlocks / 32];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nrb = (nb + kRows - 1) / kRows;
  const int bh = blockIdx.x / nrb;
  const int i = (blockIdx.x - bh * nrb) * kRows + w;   // this wave's query block
  const bool active = i < nb;
  const size_t L = (size_t)nb * BLK;

  // ---- pool: qbar_i = (1/BLK) sum of the block's queries, exact in fp64
  {
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;            // rows per wave instruction
    const int c = lane % CPR, rs = lane / CPR;
    double x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active) {
      const T* qb = Q + ((size_t)bh * L + (size_t)i * BLK) * D + 8 * c;
      for (int r = rs; r < BLK; r += RPI) {
        double y[8];
        Load8<T>::get(qb + (size_t)r * D, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += y[e];
      }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += __shfl_xor(x[e], off);
    if (rs == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_q[w][8 * c + e] = x[e] / BLK;
  }

  // ---- scores against every block centroid
  const float* cen = centroid + (size_t)bh * nb * D;
  const float* Mh = M + (size_t)bh * nb;
  for (int j0 = 0; j0 < nb; j0 += kCT) {
    __syncthreads();
    for (int q = tid; q < kCT * D; q += 64 * kRows) {
      const int r = q / D, c = q % D;
      s_c[r][c] = (j0 + r < nb) ? cen[(size_t)(j0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    const int jj = lane % kCT, half = lane / kCT;    // two lanes per centroid, half the dims each
    double dot = 0.0;
#pragma unroll 8
    for (int a = half * (D / 2); a < (half + 1) * (D / 2); ++a)
      dot = fma(s_q[w][a], (double)s_c[jj][a], dot);
    dot += __shfl_xor(dot, kCT);
    const int j = j0 + jj;
    if (half == 0 && j < nb) s_sc[w][j] = scale * dot + lam * (double)Mh[j];
  }
  for (int t = lane; t < nbp; t += 64) s_ord[w][t] = (short)t;
  for (int t = lane; t < nbp / 32; t += 64) s_sel[w][t] = 0u;
  __syncthreads();

  // ---- bitonic sort of this row's ids: "before" = higher score, then lower id
  const double* sc = s_sc[w];
  short* ord = s_ord[w];
  for (int size = 2; size <= nbp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = lane; t < nbp / 2; t += 64) {
        const int a = 2 * t - (t & (stride - 1));
        const int b = a + stride;
        const int ia = ord[a], ib = ord[b];
        const bool asc = (a & size) == 0;
        const bool swap = asc ? before(ib, ia, sc, nb) : before(ia, ib, sc, nb);
        if (swap) {
          ord[a] = (short)ib;
          ord[b] = (short)ia;
        }
      }
      __syncthreads();
    }
  }

  // ---- the first k ids, written in ascending order
  for (int t = lane; t < k; t += 64) {
    const int j = ord[t];
    atomicOr(&s_sel[w][j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (!active) return;
  int32_t* out = idx + ((size_t)bh * nb + i) * k;
  const int nw = nbp / 32;                                   // <= 64 words
  const unsigned word = (lane < nw) ? s_sel[w][lane] : 0u;
  int cnt = __popc(word), pre = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(pre, off);
    if (lane >= off) pre += y;
  }
  int pos = pre - cnt;
  unsigned wv = word;
  while (wv) {
    const int b = __ffs(wv) - 1;
    out[pos++] = 32 * lane + b;
    wv &= wv - 1;
  }
}

template <int D, typename T>
hipError_t route_t(const RouteArgs& a) {
  int nbp = 64;
  while (nbp < a.nb) nbp <<= 1;
  const int nrb = (a.nb + kRows - 1) / kRows;
  hipLaunchKernelGGL((route_kernel<D, T>), dim3(a.bh * nrb), dim3(64 * kRows), 0, a.stream,
                     (const T*)a.Q, a.centroid, a.M, a.nb, a.BLK, nbp, a.k, a.scale, a.lam, a.idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_bf16(const RouteArgs& a) {
  if (a.D == 128) return route_t<128, bf16>(a);
  if (a.D == 64) return route_t<64, bf16>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_route_f32(const RouteArgs& a) {
  if (a.D == 128) return route_t<128, float>(a);
  if (a.D == 64) return route_t<64, float>(a);
  return hipErrorInvalidValue;
}

}  // namespace pisa

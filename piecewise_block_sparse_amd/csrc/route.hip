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
// One workgroup = 4 waves = 4 query blocks of one head.  Each wave pools its
// block's queries with fully unrolled 16-byte loads (the HBM-bound part), the
// workgroup stages 32-centroid tiles through LDS for the scores, and each
// wave sorts its row's block ids with a bitonic network in LDS (score
// descending, id ascending; padding last).  LDS is sized to the padded block
// count, so small nb keeps many workgroups resident.
#include "common.hpp"
#include "launch.hpp"

namespace pisa {
namespace {

constexpr int kRows = 4;       // query blocks per workgroup (one wave each)
constexpr int kCT = 32;        // centroids per LDS tile

template <typename T>
struct Chunk8;
template <>
struct Chunk8<bf16> {
  typedef u32x4 raw;
  __device__ static raw load(const bf16* p) { return ld16(p); }
  __device__ static void add(double (&x)[8], const raw& r) {
    const bf16x8 v = as_bf16x8(r);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += (double)(float)v[e];
  }
};
template <>
struct Chunk8<float> {
  struct raw { f32x4 a, b; };
  __device__ static raw load(const float* p) {
    return raw{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
  }
  __device__ static void add(double (&x)[8], const raw& r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] += (double)r.a[e];
      x[4 + e] += (double)r.b[e];
    }
  }
};

__device__ __forceinline__ bool before(int ia, int ib, const double* sc, int nb) {
  if (ia >= nb) return (ib >= nb) && (ia < ib);
  if (ib >= nb) return true;
  const double a = sc[ia], b = sc[ib];
  return (a > b) || (a == b && ia < ib);
}

// dynamic LDS layout (bytes): q[kRows][D] f64 | c[kCT][D+1] f32 | sc[kRows][nbp] f64 |
// ord[kRows][nbp] i16 | sel[kRows][nbp/32] u32
template <int D>
__host__ __device__ constexpr size_t route_lds_bytes(int nbp) {
  return (size_t)kRows * D * 8 + (size_t)kCT * (D + 1) * 4 + (size_t)kRows * nbp * 8 +
         (size_t)kRows * nbp * 2 + (size_t)kRows * (nbp / 32) * 4;
}

template <int D, int BLK, typename T>
__global__ __launch_bounds__(64 * kRows) void route_kernel(const T* __restrict__ Q,
                                                            const float* __restrict__ centroid,
                                                            const float* __restrict__ M, int nb,
                                                            int nbp, int k, double scale,
                                                            double lam, int32_t* __restrict__ idx) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* s_q = reinterpret_cast<double*>(smem);
  float* s_c = reinterpret_cast<float*>(s_q + kRows * D);
  double* s_sc = reinterpret_cast<double*>(s_c + kCT * (D + 1));
  short* s_ord = reinterpret_cast<short*>(s_sc + kRows * nbp);
  unsigned* s_sel = reinterpret_cast<unsigned*>(s_ord + kRows * nbp);

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
    constexpr int NR = BLK / RPI;            // rows per lane
    constexpr int BATCH = 8;
    static_assert(NR % BATCH == 0, "pooling batches");
    const int c = lane % CPR, rs = lane / CPR;
    double x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active) {
      const T* qb = Q + ((size_t)bh * L + (size_t)i * BLK + rs) * D + 8 * c;
#pragma unroll
      for (int r0 = 0; r0 < NR; r0 += BATCH) {
        typename Chunk8<T>::raw v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) v[u] = Chunk8<T>::load(qb + (size_t)(r0 + u) * RPI * D);
#pragma unroll
        for (int u = 0; u < BATCH; ++u) Chunk8<T>::add(x, v[u]);
      }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += __shfl_xor(x[e], off);
    if (rs == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_q[w * D + 8 * c + e] = x[e] * (1.0 / BLK);
  }

  // ---- scores against every block centroid
  const float* cen = centroid + (size_t)bh * nb * D;
  const float* Mh = M + (size_t)bh * nb;
  double* sc = s_sc + w * nbp;
  for (int j0 = 0; j0 < nb; j0 += kCT) {
    __syncthreads();
    for (int q = tid; q < kCT * (D / 4); q += 64 * kRows) {
      const int r = q / (D / 4), c4 = q % (D / 4);
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (j0 + r < nb) v = *reinterpret_cast<const f32x4*>(cen + (size_t)(j0 + r) * D + 4 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s_c[r * (D + 1) + 4 * c4 + e] = v[e];
    }
    __syncthreads();
    const int jj = lane % kCT, half = lane / kCT;    // two lanes per centroid, half the dims each
    const double* qv = s_q + w * D + half * (D / 2);
    const float* cv = s_c + jj * (D + 1) + half * (D / 2);
    double d0 = 0.0, d1 = 0.0;
#pragma unroll
    for (int a = 0; a < D / 2; a += 2) {
      d0 = fma(qv[a], (double)cv[a], d0);
      d1 = fma(qv[a + 1], (double)cv[a + 1], d1);
    }
    double dot = d0 + d1;
    dot += __shfl_xor(dot, kCT);
    const int j = j0 + jj;
    if (half == 0 && j < nb) sc[j] = scale * dot + lam * (double)Mh[j];
  }
  short* ord = s_ord + w * nbp;
  unsigned* sel = s_sel + w * (nbp / 32);
  for (int t = lane; t < nbp; t += 64) ord[t] = (short)t;
  for (int t = lane; t < nbp / 32; t += 64) sel[t] = 0u;
  __syncthreads();

  // ---- bitonic sort of this row's ids: "before" = higher score, then lower id
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
    atomicOr(&sel[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (!active) return;
  int32_t* out = idx + ((size_t)bh * nb + i) * k;
  const int nw = nbp / 32;                                   // <= 64 words
  const unsigned word = (lane < nw) ? sel[lane] : 0u;
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

template <int D, int BLK, typename T>
hipError_t route_t(const RouteArgs& a) {
  int nbp = 64;
  while (nbp < a.nb) nbp <<= 1;
  const size_t lds = route_lds_bytes<D>(nbp);
  auto kern = route_kernel<D, BLK, T>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int nrb = (a.nb + kRows - 1) / kRows;
  hipLaunchKernelGGL(kern, dim3(a.bh * nrb), dim3(64 * kRows), lds, a.stream, (const T*)a.Q,
                     a.centroid, a.M, a.nb, nbp, a.k, a.scale, a.lam, a.idx);
  return hipGetLastError();
}

template <typename T>
hipError_t route_dispatch(const RouteArgs& a) {
  if (a.D == 128 && a.BLK == 64) return route_t<128, 64, T>(a);
  if (a.D == 128 && a.BLK == 128) return route_t<128, 128, T>(a);
  if (a.D == 64 && a.BLK == 64) return route_t<64, 64, T>(a);
  if (a.D == 64 && a.BLK == 128) return route_t<64, 128, T>(a);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route_bf16(const RouteArgs& a) { return route_dispatch<bf16>(a); }
hipError_t launch_route_f32(const RouteArgs& a) { return route_dispatch<float>(a); }

}  // namespace pisa

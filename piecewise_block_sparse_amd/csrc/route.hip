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
// One workgroup = R waves = R query blocks of one head (R = 8 when there are at
// least 256 blocks to score, else 4; each centroid is read from L2 once per
// workgroup, so more rows per workgroup means fewer re-reads of it).  Each wave pools its
// block's queries with fully unrolled 16-byte loads (the HBM-bound part); for
// the scores each thread owns one centroid and forms its dot products with all
// R pooled queries (broadcast LDS reads); each wave then selects its row's
// top k with a radix select over order-preserving 64-bit keys (ties at the
// threshold resolved to the lower block ids), stopping as soon as the keys
// still in play are exactly the ones it has left to take.  LDS is sized to the padded
// block count, so small nb keeps many workgroups resident.
//
// With valid lengths, block i pools its n_i valid queries, only the non-empty
// blocks (a prefix: j < ceil(len / BLK)) are candidates, a row with fewer than
// k candidates ends in -1, and an empty query block gets an all -1 row.
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace pisa {
namespace {


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

// dynamic LDS layout (bytes): q[R][D] f64 | sc[R][nbp] f64 |
// hist[R][256] u32 | sel[R][nbp/32] u32
template <int D, int R>
__host__ __device__ constexpr size_t route_lds_bytes(int nbp) {
  return (size_t)R * D * 8 + (size_t)R * nbp * 8 + (size_t)R * 256 * 4 +
         (size_t)R * (nbp / 32) * 4;
}

template <int D, int BLK, typename T, int kRows>
__global__ __launch_bounds__(64 * kRows) void route_kernel(const T* __restrict__ Q,
                                                            const float* __restrict__ centroid,
                                                            const float* __restrict__ M, int nb,
                                                            int nbp, int k, double scale,
                                                            double lam, int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ lens,
                                                            int heads) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* s_q = reinterpret_cast<double*>(smem);
  double* s_sc = s_q + kRows * D;
  unsigned* s_hist = reinterpret_cast<unsigned*>(s_sc + kRows * nbp);
  unsigned* s_sel = s_hist + kRows * 256;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nrb = (nb + kRows - 1) / kRows;
  const int bh = blockIdx.x / nrb;
  const int i = (blockIdx.x - bh * nrb) * kRows + w;   // this wave's query block
  const bool active = i < nb;
  const size_t L = (size_t)nb * BLK;
  const int Lv = valid_len(lens, bh, heads, (int)L);
  const int nne = (Lv + BLK - 1) / BLK;                // non-empty blocks: j < nne
  const int ni = block_count(Lv, i, BLK);              // valid queries of block i

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
        for (int u = 0; u < BATCH; ++u)
          if (rs + (r0 + u) * RPI < ni) Chunk8<T>::add(x, v[u]);   // padding rows never enter
      }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += __shfl_xor(x[e], off);
    const double inv = (ni == BLK) ? 1.0 / BLK : 1.0 / (double)(ni > 0 ? ni : 1);
    if (rs == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_q[w * D + 8 * c + e] = x[e] * inv;
  }

  // ---- scores against every block centroid: thread t owns centroid j0 + t
  // and all kRows pooled queries (read as LDS broadcasts), fp64 FMAs
  __syncthreads();
  const float* cen = centroid + (size_t)bh * nb * D;
  const float* Mh = M + (size_t)bh * nb;
  for (int j0 = 0; j0 < nb; j0 += 64 * kRows) {
    const int j = j0 + tid;
    if (j < nb) {
      const float* cj = cen + (size_t)j * D;
      double acc[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r] = 0.0;
      // the centroid row in batches of eight 16-byte loads in flight (the
      // scoring waits on L2 latency, not on the FMAs)
      for (int a0 = 0; a0 < D; a0 += 32) {
        f32x4 kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = *reinterpret_cast<const f32x4*>(cj + a0 + 4 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            const double* q = s_q + r * D + a0 + 4 * u;
            acc[r] = fma(q[0], (double)kv[u][0], acc[r]);
            acc[r] = fma(q[1], (double)kv[u][1], acc[r]);
            acc[r] = fma(q[2], (double)kv[u][2], acc[r]);
            acc[r] = fma(q[3], (double)kv[u][3], acc[r]);
          }
      }
      const double mj = lam * (double)Mh[j];
#pragma unroll
      for (int r = 0; r < kRows; ++r) s_sc[r * nbp + j] = fma(scale, acc[r], mj);
    }
  }
  double* sc = s_sc + w * nbp;
  unsigned* hist = s_hist + w * 256;
  unsigned* sel = s_sel + w * (nbp / 32);
  for (int t = lane; t < nbp / 32; t += 64) sel[t] = 0u;
  __syncthreads();

  // ---- top-k of this wave's row (ties to the lower block ids)
  const int kk = (ni > 0) ? min(k, nne) : 0;            // blocks this row can hold
  select_top_k(sc, hist, sel, nbp / 64, nne, kk, lane);

  // ---- the selected ids, written in ascending order
  if (!active) return;
  write_ids_ascending(sel, nbp / 32, kk, k, idx + ((size_t)bh * nb + i) * k, lane);
}

template <int D, int BLK, typename T, int R>
hipError_t route_launch(const RouteArgs& a, int nbp) {
  const size_t lds = route_lds_bytes<D, R>(nbp);
  auto kern = route_kernel<D, BLK, T, R>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int nrb = (a.nb + R - 1) / R;
  hipLaunchKernelGGL(kern, dim3(a.bh * nrb), dim3(64 * R), lds, a.stream, (const T*)a.Q,
                     a.centroid, a.M, a.nb, nbp, a.k, a.scale, a.lam, a.idx, a.lens, a.heads);
  return hipGetLastError();
}

template <int D, int BLK, typename T>
hipError_t route_t(const RouteArgs& a) {
  int nbp = 64;
  while (nbp < a.nb) nbp <<= 1;
  return a.nb >= 256 ? route_launch<D, BLK, T, 8>(a, nbp) : route_launch<D, BLK, T, 4>(a, nbp);
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

// Covariance-aware top-k routing (PISA summary, gist.science, section 2,
// "Covariance-aware routing": the block score combines the attention score
// with M_j = ||H_j - Hbar||).  Score of query block i and KV block j:
//
//     score_ij = scale * qbar_i . kbar_j + lambda * M_j     (float64)
//
// qbar_i is the mean query of block i.  The sum of bf16 (or fp32) values in
// float64 is exact for these block sizes, so qbar_i carries no rounding.  The
// dot product is a chain of fp64 FMAs over the head dimension in the order
// d = 16 t + 4 g + s for t, then s, then g (t < D / 16, s, g < 4), then
// scale * dot + lambda * M_j as one more FMA; the in-kernel routing of the
// attention kernel uses the same chain, so both select the same blocks.
// S_i = the k highest scores, ties to the lower j, written in ascending order.
//
// One workgroup = R waves = R query blocks of one head (R = 8 when there are
// at least 256 blocks to score, else 4).  Workgroups are placed so that each
// XCD takes a contiguous range of them: the query blocks of one head then share
// that XCD's L2 copy of the head's centroids.  Three phases:
//   pool   each wave sums its block's queries with fully unrolled 16-byte
//          loads (the HBM-bound part) into a qbar row in LDS;
//   score  the R x nb scores on fp64 MFMA (A = the qbar rows, B = 16
//          centroids per tile, read with 16-byte loads): 16x16x4 for eight
//          rows (A rows 8..15 zero), four 4x4x4 blocks per instruction for
//          four rows (no padding).  Both compute each output as the chain of
//          four FMAs over k in order, so the tiles reproduce the FMA chain
//          above exactly; each wave runs two tiles side by side, sharing every
//          A fragment read.
//          (The fp64 FMAs of a thread-per-centroid loop would read every qbar
//          value from LDS once per FMA as a broadcast, which made the LDS port
//          the bound of this phase.)
//   select each wave takes its row's top k over order-preserving 64-bit keys:
//          the k-th largest key is found bit by bit with ballot counts, from
//          the highest bit in which the keys differ, stopping as soon as
//          exactly k keys lie at or above the prefix (ties at the threshold
//          resolved to the lower block ids).
//
// With valid lengths, block i pools its n_i valid queries, only the non-empty
// blocks (a prefix: j < ceil(len / BLK)) are candidates, a row with fewer than
// k candidates ends in -1, and an empty query block gets an all -1 row.
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace pisa {
namespace {


// The queries are read once: their loads carry the non-temporal hint, so the
// Q stream does not push the head's centroids (read by every row group) out of
// L2 (video-DiT-L: 80-82 us against 86-87 us with plain loads).
template <typename T>
struct Chunk8;
template <>
struct Chunk8<bf16> {
  typedef u32x4 raw;
  __device__ static raw load(const bf16* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
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
    return raw{__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
               __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4))};
  }
  __device__ static void add(double (&x)[8], const raw& r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] += (double)r.a[e];
      x[4 + e] += (double)r.b[e];
    }
  }
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

// D[16x16] += A[16x4] B[4x16] in fp64, each output the chain of four FMAs over
// k in order.  Lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]; register
// r of the result holds D[l / 16 + 4 r][l % 16].
__device__ __forceinline__ f64x4 mfma_f64_16x16(double a, double b, const f64x4& c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// Four independent 4x4x4 fp64 products per instruction (blocks b = 0..3),
// each output the chain of four FMAs over k in order: lane 16 k + 4 b + i
// holds A_b[i][k], lane 16 k + 4 b + j holds B_b[k][j], and the result lane
// 16 i + 4 b + j holds D_b[i][j].
__device__ __forceinline__ double mfma_f64_4x4(double a, double b, double c) {
  return __builtin_amdgcn_mfma_f64_4x4x4f64(a, b, c, 0, 0, 0);
}

// qbar rows are padded by two doubles (16 bytes) so that the rows a fragment
// read touches start in different banks
template <int D>
__host__ __device__ constexpr int qbar_stride() { return D + 2; }

// dynamic LDS layout (bytes): qbar [R][D + 2] f64 | scores [R][nbp] f64 |
// sel [R][nbp / 32] u32
template <int D>
__host__ __device__ constexpr size_t route_lds_bytes(int R, int nbp) {
  return (size_t)R * qbar_stride<D>() * 8 + (size_t)R * nbp * 8 + (size_t)R * (nbp / 32) * 4;
}

// A operand of 16-wide chunk t for a lane whose k index is kq: qbar[row][16 t
// + 4 kq + s] for s = 0..3 (two 16-byte LDS reads)
template <int D>
__device__ __forceinline__ void qbar_frag(const double* s_q, int row, int kq, int t, double (&a)[4]) {
  const double* p = s_q + row * qbar_stride<D>() + 16 * t + 4 * kq;
#pragma unroll
  for (int s = 0; s < 4; ++s) a[s] = p[s];
}

template <int D, int BLK, typename T, int R>
__global__ __launch_bounds__(64 * R) void route_kernel(const T* __restrict__ Q,
                                                        const float* __restrict__ centroid,
                                                        const float* __restrict__ M, int nb, int nbp,
                                                        int k, double scale, double lam,
                                                        int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ lens, int heads) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int QS = qbar_stride<D>();
  constexpr int NT = D / 16;                             // 16-wide chunks of the head dimension
  double* s_q = reinterpret_cast<double*>(smem);
  double* s_sc = s_q + R * QS;
  unsigned* s_sel = reinterpret_cast<unsigned*>(s_sc + R * nbp);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ngr = (nb + R - 1) / R;                      // row groups per (batch, head)
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / ngr, i0 = (item - bh * ngr) * R;
  const int i = i0 + w;                                  // this wave's query block
  const bool active = i < nb;
  const size_t L = (size_t)nb * BLK;
  const int Lv = valid_len(lens, bh, heads, (int)L);
  const int nne = (Lv + BLK - 1) / BLK;                  // non-empty blocks: j < nne
  const int ni = active ? block_count(Lv, i, BLK) : 0;   // valid queries of block i

  // ---- pool: qbar_i = (1 / n_i) sum of the block's valid queries, exact in fp64
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
      for (int e = 0; e < 8; ++e) s_q[w * QS + 8 * c + e] = x[e] * inv;
  }
  for (int t = tid; t < R * (nbp / 32); t += 64 * R) s_sel[t] = 0u;
  __syncthreads();

  // ---- score, on fp64 MFMA.  Every MFMA (t, s) contracts k (the lane's
  // quarter, lane / 16) with d = 16 t + 4 k + s, so every score gets the FMA
  // chain in the order stated at the top.  Each wave runs two tiles side by
  // side, sharing each A fragment read.
  const int kq = lane >> 4;
  const float* cen = centroid + (size_t)bh * nb * D;
  const float* Mh = M + (size_t)bh * nb;
  if constexpr (R == 8) {
    // 16x16x4 tiles of 16 centroids; A rows 8..15 are zero (measured faster
    // for eight rows than 4x4x4 blocks without padding)
    const int col = lane & 15;
    const int ntile = nbp / 16;                           // even: nbp >= 64
#pragma unroll 1
    for (int n0 = 2 * w; n0 < ntile; n0 += 2 * R) {
      const int ja = 16 * n0 + col, jb = ja + 16;
      const bool va = ja < nb, vb = jb < nb;
      const float* ca = cen + (size_t)(va ? ja : 0) * D + 4 * kq;
      const float* cb = cen + (size_t)(vb ? jb : 0) * D + 4 * kq;
      f64x4 acc_a = {0.0, 0.0, 0.0, 0.0}, acc_b = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 xa = va ? *reinterpret_cast<const f32x4*>(ca + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 xb = vb ? *reinterpret_cast<const f32x4*>(cb + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
        double a[4] = {0.0, 0.0, 0.0, 0.0};
        if (col < R) qbar_frag<D>(s_q, col, kq, t, a);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc_a = mfma_f64_16x16(a[s], (double)xa[s], acc_a);
          acc_b = mfma_f64_16x16(a[s], (double)xb[s], acc_b);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = kq + 4 * r;
        if (row < R) {
          if (va) s_sc[row * nbp + ja] = fma(scale, acc_a[r], lam * (double)Mh[ja]);
          if (vb) s_sc[row * nbp + jb] = fma(scale, acc_b[r], lam * (double)Mh[jb]);
        }
      }
    }
  } else {
    // four rows: 4x4x4 blocks, block b taking centroids 4 b .. 4 b + 3 of a
    // 16-centroid tile (no padding)
    static_assert(R == 4, "route rows per workgroup: 4 or 8");
    const int blk = (lane & 15) >> 2, i4 = lane & 3;
    const int ntile = nbp / 16;
#pragma unroll 1
    for (int n0 = 2 * w; n0 < ntile; n0 += 2 * R) {
      const int ja = 16 * n0 + 4 * blk + i4, jb = ja + 16;   // B and result centroids of the lane
      const bool va = ja < nb, vb = jb < nb;
      const float* ca = cen + (size_t)(va ? ja : 0) * D + 4 * kq;
      const float* cb = cen + (size_t)(vb ? jb : 0) * D + 4 * kq;
      double acc_a = 0.0, acc_b = 0.0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 xa = va ? *reinterpret_cast<const f32x4*>(ca + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 xb = vb ? *reinterpret_cast<const f32x4*>(cb + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
        double a[4];
        qbar_frag<D>(s_q, i4, kq, t, a);                     // A row of the lane: i4
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc_a = mfma_f64_4x4(a[s], (double)xa[s], acc_a);
          acc_b = mfma_f64_4x4(a[s], (double)xb[s], acc_b);
        }
      }
      // result lane 16 i + 4 b + j: row i = kq, centroid 4 b + j of the tile
      if (va) s_sc[kq * nbp + ja] = fma(scale, acc_a, lam * (double)Mh[ja]);
      if (vb) s_sc[kq * nbp + jb] = fma(scale, acc_b, lam * (double)Mh[jb]);
    }
  }
  double* sc = s_sc + w * nbp;
  unsigned* sel = s_sel + w * (nbp / 32);
  __syncthreads();

  // ---- top-k of this wave's row (ties to the lower block ids)
  const int kk = (ni > 0) ? min(k, nne) : 0;            // blocks this row can hold
  select_top_k(sc, sel, nbp / 64, nne, kk, lane);

  // ---- the selected ids, written in ascending order
  if (!active) return;
  write_ids_ascending(sel, nbp / 32, kk, k, idx + ((size_t)bh * nb + i) * k, lane);
}

template <int D, int BLK, typename T, int R>
hipError_t route_launch(const RouteArgs& a, int nbp) {
  const size_t lds = route_lds_bytes<D>(R, nbp);
  auto kern = route_kernel<D, BLK, T, R>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int ngr = (a.nb + R - 1) / R;
  hipLaunchKernelGGL(kern, dim3(a.bh * ngr), dim3(64 * R), lds, a.stream, (const T*)a.Q,
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

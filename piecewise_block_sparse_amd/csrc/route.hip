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

// Ordering of one wave's LDS accesses among its own lanes (each row's histogram
// and selection bitmap belong to one wave, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp64 score -> unsigned key with the same order (larger score, larger key);
// -0.0 becomes +0.0 first so that equal scores give equal keys
__device__ __forceinline__ unsigned long long order_key(double x) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x + 0.0);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
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
#pragma unroll 4
      for (int a = 0; a < D; a += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(cj + a);
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const double* q = s_q + r * D + a;
          acc[r] = fma(q[0], (double)kv[0], acc[r]);
          acc[r] = fma(q[1], (double)kv[1], acc[r]);
          acc[r] = fma(q[2], (double)kv[2], acc[r]);
          acc[r] = fma(q[3], (double)kv[3], acc[r]);
        }
      }
      const double mj = lam * (double)Mh[j];
#pragma unroll
      for (int r = 0; r < kRows; ++r) s_sc[r * nbp + j] = scale * acc[r] + mj;
    }
  }
  double* sc = s_sc + w * nbp;
  unsigned* hist = s_hist + w * 256;
  unsigned* sel = s_sel + w * (nbp / 32);
  for (int t = lane; t < nbp / 32; t += 64) sel[t] = 0u;
  __syncthreads();

  // ---- top-k by radix select on the order-preserving 64-bit keys, one row
  // per wave.  Lane l owns candidates j = l + 64 u.  Each pass histograms the
  // next 8-bit digit of the candidates still in play, finds the digit value d*
  // holding the k-th largest, selects the candidates above it and keeps those
  // equal to it in play.  After the last pass the ones left tie exactly with
  // the k-th largest score; the lowest block ids among them fill the rest.
  const int nu = nbp / 64;                                // candidates per lane (<= 32)
  unsigned inplay = 0u, chosen = 0u;
  for (int u = 0; u < nu; ++u)
    if (lane + 64 * u < nne) inplay |= 1u << u;
  const int kk = (ni > 0) ? min(k, nne) : 0;            // blocks this row can hold
  int krem = kk;
  // Digits above the highest bit in which the candidates' keys differ are the
  // same for all of them (on these scores: the sign and most of the exponent),
  // so those passes would split nothing: start below them.
  int top_pass = 0;
  {
    unsigned long long kand = ~0ull, kor = 0ull;
    for (int u = 0; u < nu; ++u)
      if ((inplay >> u) & 1u) {
        const unsigned long long key = order_key(sc[lane + 64 * u]);
        kand &= key;
        kor |= key;
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned alo = __shfl_xor((unsigned)kand, off), ahi = __shfl_xor((unsigned)(kand >> 32), off);
      const unsigned olo = __shfl_xor((unsigned)kor, off), ohi = __shfl_xor((unsigned)(kor >> 32), off);
      kand &= ((unsigned long long)ahi << 32) | alo;
      kor |= ((unsigned long long)ohi << 32) | olo;
    }
    const unsigned long long diff = kor & ~kand;          // bits that differ somewhere
    if (diff != 0ull) top_pass = (63 - __clzll((long long)diff)) / 8;
  }
  for (int pass = top_pass; pass >= 0; --pass) {
    // every candidate still in play is needed: take them all and stop early
    int ip = __popc(inplay);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ip += __shfl_xor(ip, off);
    if (ip == krem) {
      chosen |= inplay;
      inplay = 0u;
      krem = 0;
      break;
    }
    const int shift = 8 * pass;
    for (int b = lane; b < 256; b += 64) hist[b] = 0u;
    wave_sync();
    for (int u = 0; u < nu; ++u)
      if ((inplay >> u) & 1u) atomicAdd(&hist[(order_key(sc[lane + 64 * u]) >> shift) & 255u], 1u);
    wave_sync();
    // this lane holds histogram bins 4l .. 4l + 3
    unsigned h[4], own = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = hist[4 * lane + e];
      own += h[e];
    }
    // exclusive suffix sum over lanes: above = sum of `own` over lanes > this lane
    unsigned above;
    {
      unsigned incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_down(incl, off);
        if (lane + off < 64) incl += y;
      }
      above = incl - own;
    }
    int dstar = -1;
    unsigned cnt_above = 0u;
    {
      unsigned acc = above;                               // count of bins > 4l + 3
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (dstar < 0 && acc < (unsigned)krem && acc + h[e] >= (unsigned)krem) {
          dstar = 4 * lane + e;
          cnt_above = acc;
        }
        acc += h[e];
      }
    }
    const unsigned long long who = __ballot(dstar >= 0);
    if (who == 0ull) {                                    // krem == 0: nothing left to pick
      dstar = 256;
      cnt_above = 0u;
    } else {
      const int src = __ffsll(who) - 1;
      dstar = __shfl(dstar, src);
      cnt_above = __shfl(cnt_above, src);
    }
    krem -= (int)cnt_above;
    for (int u = 0; u < nu; ++u)
      if ((inplay >> u) & 1u) {
        const int dg = (int)((order_key(sc[lane + 64 * u]) >> shift) & 255u);
        if (dg > dstar) {
          chosen |= 1u << u;
          inplay &= ~(1u << u);
        } else if (dg < dstar) {
          inplay &= ~(1u << u);
        }
      }
    wave_sync();
  }
  // exact ties with the k-th largest: lowest block ids first
  for (int u = 0; u < nu && krem > 0; ++u) {
    const bool tie = (inplay >> u) & 1u;
    const unsigned long long m = __ballot(tie);
    const int before_me = __popcll(m & ((1ull << lane) - 1));
    if (tie && before_me < krem) chosen |= 1u << u;
    krem -= min(krem, __popcll(m));
  }
  for (int u = 0; u < nu; ++u)
    if ((chosen >> u) & 1u) atomicOr(&sel[(lane + 64 * u) >> 5], 1u << ((lane + 64 * u) & 31));
  wave_sync();

  // ---- the selected ids, written in ascending order
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
  for (int e = kk + lane; e < k; e += 64) out[e] = -1;   // fewer candidates than k
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

// Piecewise block-sparse attention for float32 inputs: the precision path.
//
// Same three stages and the same online-softmax bookkeeping as the bf16 MFMA
// kernel (PISA summary, gist.science, section 2, "Core algorithm" and
// "Hardware implementation"; keep-or-drop from the block-sparse notes,
// section 3.3), but every operand stays float32 and every product is a VALU
// FMA, so nothing is rounded to a narrower type.  One thread per query row,
// one workgroup per query block; keys, values, centroids and Hbar rows are
// staged through LDS in chunks of CH rows.
#include "common.hpp"
#include "launch.hpp"

namespace pisa {
namespace {

constexpr int CH = 16;

template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ idx, int kmax, const float* __restrict__ centroid,
    const float* __restrict__ vsum, const float* __restrict__ hbar, const float* __restrict__ H,
    int approx, int order, float scale, float* __restrict__ O, int nb, int BLK,
    const int32_t* __restrict__ lens, int heads) {
  __shared__ float kt[CH][D];
  __shared__ float vt[CH][D];
  __shared__ unsigned bits[kMaxBlocks / 32];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / nb, i = blockIdx.x - bh * nb;
  const size_t L = (size_t)nb * BLK;
  const float* Kh = K + (size_t)bh * L * D;
  const float* Vh = V + (size_t)bh * L * D;
  const int32_t* row = idx + ((size_t)bh * nb + i) * kmax;
  // valid tokens: blocks j < nne are non-empty; this block holds ni queries
  const int Lv = valid_len(lens, bh, heads, (int)L);
  const int nne = (Lv + BLK - 1) / BLK;
  const int ni = block_count(Lv, i, BLK);

  for (int e = tid; e < (nb + 31) / 32; e += BLK) bits[e] = 0u;
  __syncthreads();
  for (int e = tid; e < kmax; e += BLK) {
    const int j = row[e];
    if (j >= 0 && j < nne) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();

  float q[D], acc[D];
  const float* qrow = Q + ((size_t)bh * L + (size_t)i * BLK + tid) * D;
  const bool live = tid < ni;                       // padding queries: a zero row
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = live ? qrow[c] : 0.f;
    acc[c] = 0.f;
  }
  const float c2 = scale * kLog2e;
  float m = -1e30f, l = 0.f, asum = 0.f;

  // one chunk of CH keys (or centroids) staged in kt / vt
  auto consume = [&](bool stage2, int jbase, int nvalid) {
    float cntw[CH];                                 // stage 2: tokens of each centroid's block
#pragma unroll
    for (int n = 0; n < CH; ++n) cntw[n] = (float)block_count(Lv, jbase + n, BLK);
    float lg[CH];
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < CH; ++n) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(q[c], kt[n][c], s);
      float x = s * c2;
      if (n >= nvalid) x = -INFINITY;
      if (stage2) {
        const int j = jbase + n;
        if (j >= nne || ((bits[j >> 5] >> (j & 31)) & 1u)) x = -INFINITY;
      }
      lg[n] = x;
      mx = fmaxf(mx, x);
    }
    const float mnew = fmaxf(m, mx);
    const float corr = exp2f(m - mnew);
    m = mnew;
    float ps = 0.f, pw = 0.f;
#pragma unroll
    for (int n = 0; n < CH; ++n) {
      lg[n] = exp2f(lg[n] - mnew);
      ps += lg[n];
      pw += cntw[n] * lg[n];
    }
    if (stage2) {
      l = l * corr + pw;                            // each block weighs its n_j tokens
      asum = asum * corr + ps;
    } else {
      l = l * corr + ps;
    }
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float x = acc[c] * corr;
#pragma unroll
      for (int n = 0; n < CH; ++n) x = fmaf(lg[n], vt[n][c], x);
      acc[c] = x;
    }
  };

  // stage 1: exact keys of the selected blocks, ascending, each once (S_i is
  // a set: an id repeated in the idx row counts once)
  for (int j = 0; j < nne; ++j) {
    if (!((bits[j >> 5] >> (j & 31)) & 1u)) continue;
    const int nj = block_count(Lv, j, BLK);
    for (int n0 = 0; n0 < BLK; n0 += CH) {
      const int nv = min(max(nj - n0, 0), CH);       // keys of this chunk inside the sequence
      __syncthreads();
      for (int t = tid; t < CH * D; t += BLK) {
        const int n = t / D, c = t % D;
        kt[n][c] = n < nv ? Kh[((size_t)j * BLK + n0 + n) * D + c] : 0.f;
        vt[n][c] = n < nv ? Vh[((size_t)j * BLK + n0 + n) * D + c] : 0.f;
      }
      __syncthreads();
      consume(false, 0, nv);
    }
  }

  if (approx) {
    // stage 2: zeroth-order term of every block outside S_i
    const float* cen = centroid + (size_t)bh * nb * D;
    const float* vs = vsum + (size_t)bh * nb * D;
    for (int j0 = 0; j0 < nb; j0 += CH) {
      __syncthreads();
      for (int t = tid; t < CH * D; t += BLK) {
        const int n = t / D, c = t % D;
        const bool ok = j0 + n < nb;
        kt[n][c] = ok ? cen[(size_t)(j0 + n) * D + c] : 0.f;
        vt[n][c] = ok ? vs[(size_t)(j0 + n) * D + c] : 0.f;
      }
      __syncthreads();
      consume(true, j0, min(CH, nb - j0));
    }
  }
  // acc += f * (q G) for a d x d matrix G (row = key dim), rows staged CH at a time
  auto add_qG = [&](const float* G, float f) {
    for (int r0 = 0; r0 < D; r0 += CH) {
      __syncthreads();
      for (int t = tid; t < CH * D; t += BLK) kt[t / D][t % D] = G[(size_t)(r0 + t / D) * D + t % D];
      __syncthreads();
#pragma unroll
      for (int n = 0; n < CH; ++n) {
        const float fq = f * q[r0 + n];
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(fq, kt[n][c], acc[c]);
      }
    }
  };
  if (approx && order == kOrderMixed) {
    // stage 3: acc += scale * asum * (q Hbar)
    add_qG(hbar + (size_t)bh * D * D, scale * asum);
  }
  if (approx && order == kOrderFirst) {
    // per-block first order: acc += scale * alpha_j * (q H_j) for every j outside S_i,
    // alpha_j = e^{q kbar_j} against the running max (the same shift as every term)
    const float* cen = centroid + (size_t)bh * nb * D;
    for (int j = 0; j < nne; ++j) {
      if ((bits[j >> 5] >> (j & 31)) & 1u) continue;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(q[c], cen[(size_t)j * D + c], s);
      add_qG(H + ((size_t)bh * nb + j) * D * D, scale * exp2f(s * c2 - m));
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* orow = O + ((size_t)bh * L + (size_t)i * BLK + tid) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) orow[c] = live ? acc[c] * inv : 0.f;
}

template <int D>
hipError_t attn_f32_t(const AttnArgs& a) {
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3(a.bh * a.nb), dim3(a.BLK), 0, a.stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, a.idx, a.kmax,
                     a.centroid, a.vsum, a.hbar, a.H, a.approx, a.order, a.scale, (float*)a.O,
                     a.nb, a.BLK, a.lens, a.heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a) {
  if (a.D == 128) return attn_f32_t<128>(a);
  if (a.D == 64) return attn_f32_t<64>(a);
  return hipErrorInvalidValue;
}

}  // namespace pisa

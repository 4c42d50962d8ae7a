// Fused piecewise block-sparse attention, bf16 storage, gfx950 MFMA.
//
// Method: PISA summary (gist.science), section 2, "Core algorithm" and
// "Hardware implementation": one online softmax per query row whose
// numerator and denominator receive (1) exact terms of the selected KV blocks,
// (2) one zeroth-order term per unselected block, alpha = e^{q kbar_j} times the
// block value sum (weight `block` in the denominator), and (3) the global
// first-order correction (q Hbar) * sum alpha.  Keep-or-drop (block-sparse
// notes, section 3.3) runs stage 1 only.
//
// Work decomposition: one workgroup per (batch*head, query block); BLK/32
// waves, each owning 32 query rows.  Everything is computed transposed so
// that a lane owns one query row:
//   S^T[key][query]  = K_tile . Q^T      (A = K rows from LDS, B = Q fragments in VGPRs)
//   O^T[d][query]   += V_tile^T . P^T    (A = V^T rows from LDS, B = P straight from S^T)
// The 32x32x16 result layout gives lane l the 16 keys {8(r/4) + 4(l/32) + r%4}
// of query l%32, so the row max needs one cross-lane step (lane l ^ 32) and the
// rescale of O^T is lane-local.  The V tile is stored transposed in LDS with
// each 16-key slab permuted (keys 0-3, 8-11, 4-7, 12-15) so that a lane's P
// registers feed the next MFMA's B operand without any shuffle.
#include "common.hpp"
#include "launch.hpp"

namespace pisa {
namespace {

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;          // waves per workgroup
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int KS = D / 16;            // MFMA k-steps over the head dim
  static constexpr int MT = D / 32;            // 32-row tiles of O^T
  static constexpr int KROW = D + 8;           // LDS row (elements) of the K tile, padded
  static constexpr int VROW = BLK + 8;         // LDS row of the V^T tile, padded
  static constexpr int K_ELEMS = BLK * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr int LDS_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int K_PER_T = BLK * D / 8 / NT;        // 16-byte K chunks per thread
  static constexpr int VSUB = (BLK / 8) * (D / 8);        // 8x8 sub-tiles of V
  static_assert(BLK * D / 8 % NT == 0, "K tile split");
  static_assert(VSUB <= NT, "one V sub-tile per thread");
  static_assert(D * KROW <= LDS_ELEMS, "Hbar^T fits in the tile buffers");
};

// physical slot (0..15) inside a 16-key slab of V^T holding logical key e of
// a thread's 8-key group h2: groups are {4 h2 + 0..3, 8 + 4 h2 + 0..3}
__device__ __forceinline__ int slab_key(int h2, int e) {
  return (e < 4) ? (4 * h2 + e) : (8 + 4 * h2 + (e - 4));
}

template <int D, int BLK>
struct TileRegs {
  u32x4 k[Cfg<D, BLK>::K_PER_T];
  u32x4 v[8];
};

// global -> registers: one KV block (BLK tokens) of one head
template <int D, int BLK>
__device__ __forceinline__ void load_kv(TileRegs<D, BLK>& t, const bf16* Kb, const bf16* Vb, int tid) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int u = 0; u < C::K_PER_T; ++u) {
    const int q = tid + u * C::NT;
    const int r = q / (D / 8), c = q % (D / 8);
    t.k[u] = ld16(Kb + r * D + c * 8);
  }
  if (tid < C::VSUB) {
    const int g = tid % (BLK / 8), c = tid / (BLK / 8);
    const int s = g >> 1, h2 = g & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) t.v[e] = ld16(Vb + (16 * s + slab_key(h2, e)) * D + c * 8);
  }
}

// registers -> LDS: K row-major, V transposed with permuted slabs
template <int D, int BLK>
__device__ __forceinline__ void store_kv(const TileRegs<D, BLK>& t, bf16* Ks, bf16* Vt, int tid) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int u = 0; u < C::K_PER_T; ++u) {
    const int q = tid + u * C::NT;
    const int r = q / (D / 8), c = q % (D / 8);
    st16(Ks + r * C::KROW + c * 8, t.k[u]);
  }
  if (tid < C::VSUB) {
    const int g = tid % (BLK / 8), c = tid / (BLK / 8);
    const int s = g >> 1, h2 = g & 1;
    u32x4 col[8];
    transpose8x8(t.v, col);
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(Vt + (8 * c + i) * C::VROW + 16 * s + 8 * h2, col[i]);
  }
}

// fp32 centroid / value-sum tile (BLK consecutive blocks starting at j0) ->
// bf16 LDS in the same layouts as a KV tile; rows past nb are zero.
template <int D, int BLK>
__device__ __forceinline__ void stage_centroids(const float* cen, const float* vs, int j0, int nb,
                                                bf16* Ks, bf16* Vt, int tid) {
  using C = Cfg<D, BLK>;
  for (int q = tid; q < BLK * (D / 4); q += C::NT) {
    const int r = q / (D / 4), c4 = q % (D / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j0 + r < nb) v = *reinterpret_cast<const f32x4*>(cen + (size_t)(j0 + r) * D + c4 * 4);
    u32x2 p = {pack2(v[0], v[1]), pack2(v[2], v[3])};
    st8(Ks + r * C::KROW + c4 * 4, p);
  }
  for (int p = tid; p < C::VSUB; p += C::NT) {
    const int g = p % (BLK / 8), c = p / (BLK / 8);
    const int s = g >> 1, h2 = g & 1;
    f32x4 lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = j0 + 16 * s + slab_key(h2, e);
      if (r < nb) {
        lo[e] = *reinterpret_cast<const f32x4*>(vs + (size_t)r * D + 8 * c);
        hi[e] = *reinterpret_cast<const f32x4*>(vs + (size_t)r * D + 8 * c + 4);
      } else {
        lo[e] = hi[e] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 col;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const float a = (i < 4) ? lo[2 * q2][i] : hi[2 * q2][i - 4];
        const float b = (i < 4) ? lo[2 * q2 + 1][i] : hi[2 * q2 + 1][i - 4];
        col[q2] = pack2(a, b);
      }
      st16(Vt + (8 * c + i) * C::VROW + 16 * s + 8 * h2, col);
    }
  }
}

// Hbar [d_k][d_v] fp32 -> LDS Hbar^T [d_v][d_k] bf16, row stride KROW
template <int D, int BLK>
__device__ __forceinline__ void stage_hbar_t(const float* hb, bf16* Ht, int tid) {
  using C = Cfg<D, BLK>;
  for (int p = tid; p < (D / 8) * (D / 8); p += C::NT) {
    const int g = p % (D / 8), c = p / (D / 8);   // rows 8g.., cols 8c..
    f32x4 lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = *reinterpret_cast<const f32x4*>(hb + (size_t)(8 * g + e) * D + 8 * c);
      hi[e] = *reinterpret_cast<const f32x4*>(hb + (size_t)(8 * g + e) * D + 8 * c + 4);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 col;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const float a = (i < 4) ? lo[2 * q2][i] : hi[2 * q2][i - 4];
        const float b = (i < 4) ? lo[2 * q2 + 1][i] : hi[2 * q2 + 1][i - 4];
        col[q2] = pack2(a, b);
      }
      st16(Ht + (8 * c + i) * C::KROW + 8 * g, col);
    }
  }
}

// Online-softmax state of one lane (one query row, half of each key tile).
template <int D>
struct RowState {
  f32x16 acc[D / 32];
  float m;      // running max, log2 domain (logit * scale * log2 e)
  float l;      // this lane's share of the denominator
  float a;      // this lane's share of sum over U_i of alpha (same scaling as acc)
};

// The running max is only raised when a row's new maximum exceeds it by more
// than kTau (log2 units); until then the weights exp2(x - m) stay below 2^kTau.
// Any m gives the same N / D, so this only saves rescales of acc.
constexpr float kTau = 8.f;

// exp2 weights of one 64-key chunk -> bf16 MFMA B operands (pf) and the sum of
// the same bf16-rounded weights.  Each pair is packed into its own 32-bit value
// and summed from that value with v_dot2 against (1, 1) before the four pairs
// of a slab are assembled into the 128-bit operand.
__device__ __forceinline__ float weights_bf16(const f32x16 (&s)[2], float c2, float nm,
                                              u32x4 (&pf)[4]) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  float sum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float p0 = fast_exp2(fmaf(s[kt][2 * q], c2, nm));
      const float p1 = fast_exp2(fmaf(s[kt][2 * q + 1], c2, nm));
      const bf16x2 pr = {(bf16)p0, (bf16)p1};
      sum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum, false);
      pf[2 * kt + q / 4][q % 4] = __builtin_bit_cast(unsigned, pr);
    }
  return sum;
}

// One 64-key chunk of the LDS tile: S^T, softmax update, O^T += V^T P^T.
// STAGE2: the keys are block centroids (values = block value sums); entries
// whose block is in S_i or past nb are masked, and each weight counts `block`
// times in the denominator.  The denominator sums the same bf16-rounded
// weights that the MFMA multiplies into the numerator.
template <int D, int BLK, bool STAGE2>
__device__ __forceinline__ void chunk(RowState<D>& st, const bf16x8 (&qf)[D / 16], const bf16* Ks,
                                      const bf16* Vt, int ch, float c2, int q32, int hh,
                                      const unsigned* bits, int jbase, int nb) {
  using C = Cfg<D, BLK>;
  f32x16 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    s[kt] = f32x16{};
    const bf16* krow = Ks + (64 * ch + 32 * kt + q32) * C::KROW + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s[kt] = mfma32(as_bf16x8(ld16(krow + 16 * ks)), qf[ks], s[kt]);
  }
  if (STAGE2) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jbase + 64 * ch + 32 * kt + 8 * (r / 4) + 4 * hh + (r % 4);
        const bool masked = (j >= nb) || ((bits[j >> 5] >> (j & 31)) & 1u);
        s[kt][r] = masked ? -INFINITY : s[kt][r];
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
  if (__any(mx > st.m + kTau)) {
    const float mnew = fmaxf(st.m, mx);
    const float corr = fast_exp2(st.m - mnew);
    st.m = mnew;
    st.l *= corr;
    st.a *= corr;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) st.acc[mt] *= corr;
  }
  u32x4 pf[4];
  const float ps = weights_bf16(s, c2, -st.m, pf);
  if (STAGE2) {
    st.l += (float)BLK * ps;
    st.a += ps;
  } else {
    st.l += ps;
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    const bf16* vrow = Vt + (32 * mt + q32) * C::VROW + 64 * ch + 8 * hh;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      st.acc[mt] = mfma32(as_bf16x8(ld16(vrow + 16 * sl)), as_bf16x8(pf[sl]), st.acc[mt]);
  }
}

__device__ __forceinline__ int next_valid(const int32_t* row, int e, int kmax, int nb) {
  while (e < kmax) {
    const int j = row[e];
    if (j >= 0 && j < nb) break;
    ++e;
  }
  return e;
}

// Kernel arguments: fp32 statistics, plus (optionally) their bf16 packs written
// by the statistics pass: centroids and value sums [nbp][D] per head (nbp = nb
// rounded up to BLK, padding rows zero) and Hbar^T [D][D] per head.
struct AttnPtrs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  const int32_t* idx;
  const float* centroid;
  const float* vsum;
  const float* hbar;
  const bf16* pk_cen;
  const bf16* pk_vsum;
  const bf16* pk_hbart;
  bf16* O;
};

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK) void attn_bf16_kernel(AttnPtrs p, int kmax, int approx,
                                                            float scale, int nb) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) bf16 lds[C::LDS_ELEMS];
  __shared__ unsigned bits[kMaxBlocks / 32];
  bf16* Ks = lds;
  bf16* Vt = lds + C::K_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q32 = lane & 31, hh = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nb, i = logical - bh * nb;
  const size_t L = (size_t)nb * BLK;
  const int nbp = (nb + BLK - 1) / BLK * BLK;
  const bf16* Kh = p.K + (size_t)bh * L * D;
  const bf16* Vh = p.V + (size_t)bh * L * D;
  const int32_t* row = p.idx + ((size_t)bh * nb + i) * kmax;
  const bool packed = approx && p.pk_cen != nullptr;

  if (approx) {
    for (int e = tid; e < (nb + 31) / 32; e += C::NT) bits[e] = 0u;
    __syncthreads();
    for (int e = tid; e < kmax; e += C::NT) {
      const int j = row[e];
      if (j >= 0 && j < nb) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
  }

  // this lane's query row as 16-byte B-operand fragments (d = 16 ks + 8 hh + 0..7)
  bf16x8 qf[C::KS];
  {
    const bf16* qrow = p.Q + ((size_t)bh * L + (size_t)i * BLK + 32 * w + q32) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }
  RowState<D> st;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) st.acc[mt] = f32x16{};
  st.m = -1e30f;
  st.l = 0.f;
  st.a = 0.f;
  const float c2 = scale * kLog2e;

  // ---- stages 1 and 2 as one register-prefetched stream of tiles: the exact
  // blocks of S_i, then (PISA mode, packed statistics) the centroid / value-sum
  // tiles, which have exactly the layout of a K / V block.
  const int ntile = packed ? nbp / BLK : 0;
  int e = next_valid(row, 0, kmax, nb), t = 0;
  auto next_tile = [&](int& kind, int& id) {
    if (e < kmax) {
      kind = 0;
      id = row[e];
      e = next_valid(row, e + 1, kmax, nb);
    } else if (t < ntile) {
      kind = 1;
      id = t++;
    } else {
      kind = -1;
    }
  };
  TileRegs<D, BLK> regs;
  auto load = [&](int kind, int id) {
    if (kind == 0)
      load_kv<D, BLK>(regs, Kh + (size_t)id * BLK * D, Vh + (size_t)id * BLK * D, tid);
    else
      load_kv<D, BLK>(regs, p.pk_cen + ((size_t)bh * nbp + (size_t)id * BLK) * D,
                      p.pk_vsum + ((size_t)bh * nbp + (size_t)id * BLK) * D, tid);
  };
  int kind, id;
  next_tile(kind, id);
  if (kind >= 0) load(kind, id);
  while (kind >= 0) {
    __syncthreads();
    store_kv<D, BLK>(regs, Ks, Vt, tid);
    __syncthreads();
    int kind_n, id_n;
    next_tile(kind_n, id_n);
    if (kind_n >= 0) load(kind_n, id_n);
    if (kind == 0) {
#pragma unroll
      for (int ch = 0; ch < BLK / 64; ++ch)
        chunk<D, BLK, false>(st, qf, Ks, Vt, ch, c2, q32, hh, bits, 0, nb);
    } else {
#pragma unroll
      for (int ch = 0; ch < BLK / 64; ++ch)
        chunk<D, BLK, true>(st, qf, Ks, Vt, ch, c2, q32, hh, bits, id * BLK, nb);
    }
    kind = kind_n;
    id = id_n;
  }

  if (approx) {
    if (!packed) {
      // ---- stage 2 from the fp32 statistics (converted while staging)
      const float* cen = p.centroid + (size_t)bh * nb * D;
      const float* vs = p.vsum + (size_t)bh * nb * D;
      for (int j0 = 0; j0 < nb; j0 += BLK) {
        __syncthreads();
        stage_centroids<D, BLK>(cen, vs, j0, nb, Ks, Vt, tid);
        __syncthreads();
#pragma unroll
        for (int ch = 0; ch < BLK / 64; ++ch)
          chunk<D, BLK, true>(st, qf, Ks, Vt, ch, c2, q32, hh, bits, j0, nb);
      }
    }
    // ---- stage 3: global first-order correction, acc += scale * (q Hbar) * sum alpha
    const float atot = st.a + __shfl_xor(st.a, 32);
    const float f = scale * atot;
    if (packed) {
      // A operand (Hbar^T rows) straight from the bf16 pack, two d-tiles at a time
      const bf16* hb = p.pk_hbart + ((size_t)bh * D + q32) * D + 8 * hh;
#pragma unroll
      for (int m0 = 0; m0 < C::MT; m0 += 2) {
        constexpr int NM = (C::MT >= 2) ? 2 : 1;
        u32x4 ha[NM][C::KS];
#pragma unroll
        for (int u = 0; u < NM; ++u)
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) ha[u][ks] = ld16(hb + (size_t)(32 * (m0 + u)) * D + 16 * ks);
#pragma unroll
        for (int u = 0; u < NM; ++u) {
          f32x16 hq = f32x16{};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) hq = mfma32(as_bf16x8(ha[u][ks]), qf[ks], hq);
          st.acc[m0 + u] += f * hq;
        }
      }
    } else {
      __syncthreads();
      stage_hbar_t<D, BLK>(p.hbar + (size_t)bh * D * D, lds, tid);
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        f32x16 hq = f32x16{};
        const bf16* hrow = lds + (32 * mt + q32) * C::KROW + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) hq = mfma32(as_bf16x8(ld16(hrow + 16 * ks)), qf[ks], hq);
        st.acc[mt] += f * hq;
      }
    }
  }

  // ---- epilogue: o = N / D (0 when nothing was attended in keep-or-drop)
  const float ltot = st.l + __shfl_xor(st.l, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  bf16* orow = p.O + ((size_t)bh * L + (size_t)i * BLK + 32 * w + q32) * D;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x16& a = st.acc[mt];
      u32x2 pk = {pack2(a[4 * g4] * inv, a[4 * g4 + 1] * inv), pack2(a[4 * g4 + 2] * inv, a[4 * g4 + 3] * inv)};
      st8(orow + 32 * mt + 8 * g4 + 4 * hh, pk);
    }
}

template <int D, int BLK>
hipError_t launch_t(const AttnArgs& a) {
  using C = Cfg<D, BLK>;
  const int grid = a.bh * a.nb;
  const int nbp = (a.nb + BLK - 1) / BLK * BLK;
  const bf16* pk = static_cast<const bf16*>(a.packed);
  AttnPtrs p{(const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, a.idx, a.centroid, a.vsum,
             a.hbar, pk, pk ? pk + (size_t)a.bh * nbp * D : nullptr,
             pk ? pk + (size_t)2 * a.bh * nbp * D : nullptr, (bf16*)a.O};
  hipLaunchKernelGGL((attn_bf16_kernel<D, BLK>), dim3(grid), dim3(C::NT), 0, a.stream, p, a.kmax,
                     a.approx, a.scale, a.nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a) {
  if (a.D == 128 && a.BLK == 64) return launch_t<128, 64>(a);
  if (a.D == 128 && a.BLK == 128) return launch_t<128, 128>(a);
  if (a.D == 64 && a.BLK == 64) return launch_t<64, 64>(a);
  if (a.D == 64 && a.BLK == 128) return launch_t<64, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace pisa

// Block statistics for PISA: centroids, value sums, H_j, Hbar and M_j.
//
// PISA summary (gist.science), section 2: "Core algorithm" (centroid kbar_j,
// value sum, H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n}, Hbar = mean of H_j),
// "Covariance-aware routing" (M_j = ||H_j - Hbar||_2, Frobenius reading) and
// "Hardware implementation" (computed before the attention stages).
//
// bf16 path: H_j = K_j^T V_j - kbar_j^T sigma_j, with K_j^T V_j on bf16 MFMA
// (products of bf16 values are exact in the fp32 accumulator).  Pass 1 streams
// K and V once and writes one fp32 partial sum of H_j per workgroup range of
// blocks; a fixed-order fp64 reduction gives Hbar; pass 2 streams K
// and V again, recomputes each H_j and writes M_j (and H_j when asked).  No
// atomics: results are bitwise reproducible.
//
// fp32 path: plain fp32 VALU arithmetic with centred keys; H_j is kept in a
// buffer, reduced to Hbar, then M_j is read off the buffer.
#include "common.hpp"
#include "launch.hpp"
#include "lds_stream.hpp"

namespace pisa {
namespace {

// Streaming configuration: 32-token chunks of K and V through a four-stage
// LDS ring (the layout of lds_stream.hpp), four waves, each owning TM x TM
// 32x32 tiles of the d x d product.
template <int D_, int BLK_>
struct SCfg {
  static constexpr int D = D_, BLK = BLK_;
  static constexpr int NW = 4, NT = 64 * NW;
  static constexpr int CK = 32;                       // tokens per chunk
  static constexpr int CPB = BLK / CK;                // chunks per block
  static constexpr int NSL = CK / 16;                 // 16-token MFMA k-steps per chunk
  static constexpr int RB = 2 * D, CPR = D / 8, SUBB = CK * RB, STB = 2 * SUBB;
  static constexpr int NDMA = STB / 1024, DPW = NDMA / NW, RPD = 1024 / RB;
  // ring stages: four 16 KB stages (d = 128) at two workgroups per CU, for
  // both block sizes (64-token blocks measured 15% faster this way than at
  // three workgroups per CU with three stages and 8-block ranges: the longer
  // ranges halve the pass-1 partial sums written and re-read)
  static constexpr int NS = 4;
  static constexpr int TM = (D == 128) ? 2 : 1;       // 32x32 output tiles per wave, per dim
  // blocks per workgroup range: at most PMAX (the pass-1 register window of
  // per-block outputs), at least PMIN, else enough for one round of GT
  // workgroups (two per CU on 256 CUs)
  static constexpr int PMAX = 24;
  static constexpr int PMIN = 4;
  static constexpr int GT = 512;
  static_assert(BLK % CK == 0 && NDMA % NW == 0 && DPW % 2 == 0, "chunking");
};

// Ranges per head (bf16 path): enough workgroups for one round of GT (b*h*R
// <= GT), ranges of at most PMAX blocks and, where the head allows, at least
// PMIN.  Depends on the shape only, so results are reproducible.
template <int D, int BLK>
int stats_ranges(int bh, int nb) {
  using C = SCfg<D, BLK>;
  long long r = C::GT / bh;                                  // one round of GT workgroups
  const long long rmin = (nb + C::PMAX - 1) / C::PMAX;       // the window holds PMAX blocks
  const long long rmax = nb / C::PMIN > 0 ? nb / C::PMIN : 1;
  if (r > rmax) r = rmax;
  if (r < rmin) r = rmin;
  if (r < 1) r = 1;
  return (int)r;
}

// Sum of the 8 bf16 values of a fragment, added to acc (v_dot2 against 1;
// the pairs are taken from the bf16 view of the fragment).
__device__ __forceinline__ float frag_sum(const u32x4& f, float acc) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  const bf16x8 v = as_bf16x8(f);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

// Work split.  Each head's nb blocks are dealt in R near-equal contiguous
// ranges, one per workgroup: range r covers blocks r*nb/R .. (r+1)*nb/R - 1
// (stats_ranges picks R so that the b*h*R workgroups fill one round on a
// 256-CU MI355X and a range holds at most PMAX blocks).  Pass 1 writes the
// range's sum of H_j to partial slot bh*R + r; the reduction sums a head's R
// slots in order (a fixed order: bitwise reproducible).  Pass 2 walks its range
// backwards, last block first: the blocks pass 1 read last are the ones most
// likely still held by the memory-side cache.
//
// Per 16-token slab every wave reads its K^T and V fragments with transposing
// LDS reads (both operands index tokens the same way), accumulates K_j^T V_j
// on MFMA and the column sums of K and V from the same fragments (lanes l and
// l + 32 hold the two halves of a column's tokens).  At the end of a block the
// sums give kbar_j and sigma_j, and H_j = K_j^T V_j - kbar_j^T sigma_j.
// STORE: pass 2 also writes the optional H_j (fp32) and H_j^T (bf16) outputs.
template <int D, int BLK, bool PASS2, bool STORE>
__global__ __launch_bounds__(256, 2) void stats_bf16_kernel(
    const bf16* __restrict__ K, const bf16* __restrict__ V, int nb, int R,
    float* __restrict__ centroid, float* __restrict__ vsum, float* __restrict__ partial,
    const float* __restrict__ hbar_frag, float* __restrict__ M, float* __restrict__ Hout,
    bf16* __restrict__ pk_cen, bf16* __restrict__ pk_vsum, bf16* __restrict__ Ht,
    const int32_t* __restrict__ lens, int heads) {
  using C = SCfg<D, BLK>;
  constexpr int TM = C::TM, PM = C::PMAX;
  __shared__ __attribute__((aligned(1024))) char ring[C::NS * C::STB];
  __shared__ float s_kv[C::NW][2][TM * 32];              // per wave: its kbar and sigma entries
  __shared__ float s_sq[PM][C::NW];                       // per block and wave: part of ||H_j - Hbar||^2

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q32 = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.x / R, rg = blockIdx.x - bh * R;
  // (scalars: the copies take their global base from scalar registers)
  const int j0 = __builtin_amdgcn_readfirstlane((int)((long long)rg * nb / R));
  const int j1 = __builtin_amdgcn_readfirstlane((int)((long long)(rg + 1) * nb / R));
  const int ng = j1 - j0;                                 // 1 .. PMAX blocks
  // block at walk position u (pass 2 walks backwards)
  auto block_at = [&](int u) { return PASS2 ? j1 - 1 - u : j0 + u; };
  const size_t L = (size_t)nb * BLK;
  const int mt0 = (w >> 1) * TM, nt0 = (w & 1) * TM;
  const bool kout = nt0 == 0, vout = mt0 == 0;            // waves that write centroid / value sum
  const int Lv = valid_len(lens, bh, heads, (int)L);      // tokens past Lv are not counted

  f32x16 acc[TM][TM];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x16{};

  // pass 2: this lane's Hbar entries (stored by the reduction in fragment
  // order: 4 consecutive floats per tile and row group), held for the whole
  // range; loaded before the ring starts so no wait for them lands in the loop
  f32x4 hb[TM][TM][4];
  if (PASS2) {
    const float* hbf = hbar_frag + (size_t)bh * D * D + (size_t)w * TM * TM * 1024 + 4 * lane;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          hb[a][b][g] = *reinterpret_cast<const f32x4*>(hbf + ((a * TM + b) * 4 + g) * 256);
  }

  const DmaOff<C> loff = dma_lane_offsets<C>(w, lane);
  const int ws = __builtin_amdgcn_readfirstlane(w);        // wave index as a scalar
  int ao[TM][2], bo[TM][2];                               // this wave's tiles' read offsets
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ao[a][h] = tr_lane_offset<C>(lane, mt0 + a, h);
      bo[a][h] = tr_lane_offset<C>(lane, nt0 + a, h) + C::SUBB;
    }
  const unsigned ring_m0 = (unsigned)(uintptr_t)(lvoid*)ring;
  const int nch = ng * C::CPB;
  const char* Kb = reinterpret_cast<const char*>(K + (size_t)bh * L * D);
  const char* Vb = reinterpret_cast<const char*>(V + (size_t)bh * L * D);
  auto issue = [&](int u) {                 // copy chunk u into stage u % NS
    const size_t off = ((size_t)block_at(u / C::CPB) * BLK + (size_t)(u % C::CPB) * C::CK) * C::RB;
    dma_stage<C>(Kb + off, Vb + off, ring_m0 + (unsigned)((u % C::NS) * C::STB), ws, loff);
  };
  for (int u = 0; u < C::NS - 1 && u < nch; ++u) issue(u);
  wait_vm0();   // the first chunks and the Hbar entries; no compiler-placed waits in the loop

  float ks[TM], vs[TM];                    // this lane's half of the block's column sums
#pragma unroll
  for (int a = 0; a < TM; ++a) ks[a] = vs[a] = 0.f;
  // Per-block outputs are written after the loop: stores count in vmcnt with
  // the copies, so a store issued between copies would hold up every later
  // wait for a chunk.  Pass 1 keeps the lane's centroid / value-sum entries of
  // the range's blocks in a window shifted by one block at each block end
  // (entry PM - 1 is the newest); pass 2 keeps M_j in LDS.
  float ocen[TM][PM], ovs[TM][PM];

  for (int t = 0; t < nch; ++t) {
    // chunk t: wait for it (chunks t + 1 .. t + NS - 2 may be in flight),
    // publish it, and refill the stage read in the previous step
    wait_groups<C>(min(C::NS - 2, nch - 1 - t));
    __syncthreads();
    if (t + C::NS - 1 < nch) issue(t + C::NS - 1);
    const int u = t / C::CPB, j = block_at(u), tb = (t % C::CPB) * C::CK;
    const int nj = block_count(Lv, j, BLK);
    char* stage = ring + (t % C::NS) * C::STB;
    if (nj < tb + C::CK) {
      // tokens at or past the block's valid count are stored as zeros
      const int r0 = max(nj - tb, 0);
      for (int e = tid; e < 2 * (C::CK - r0) * C::CPR; e += C::NT) {
        const int half = e / ((C::CK - r0) * C::CPR), q = e % ((C::CK - r0) * C::CPR);
        st16(stage + half * C::SUBB + (r0 + q / C::CPR) * C::RB + 16 * (q % C::CPR),
             u32x4{0u, 0u, 0u, 0u});
      }
      __syncthreads();
    }
#pragma unroll
    for (int sl = 0; sl < C::NSL; ++sl) {
      u32x4 fa[TM], fb[TM];
#pragma unroll
      for (int a = 0; a < TM; ++a) fa[a] = tr_read<C>(stage, sl, ao[a][0], ao[a][1]);
#pragma unroll
      for (int b = 0; b < TM; ++b) fb[b] = tr_read<C>(stage, sl, bo[b][0], bo[b][1]);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma32(as_bf16x8(fa[a]), as_bf16x8(fb[b]), acc[a][b]);
#pragma unroll
      for (int a = 0; a < TM; ++a) ks[a] = frag_sum(fa[a], ks[a]);
#pragma unroll
      for (int b = 0; b < TM; ++b) vs[b] = frag_sum(fb[b], vs[b]);
    }
    if (t % C::CPB != C::CPB - 1) continue;

    // ---- end of block j: centroid (mean of keys) and value sum
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const float sk = ks[a] + __shfl_xor(ks[a], 32);
      const float sv = vs[a] + __shfl_xor(vs[a], 32);
      ks[a] = vs[a] = 0.f;
      const float kbar = (nj == BLK) ? sk * (1.f / BLK) : (nj > 0 ? sk / (float)nj : 0.f);
      if (hh == 0) {
        s_kv[w][0][32 * a + q32] = kbar;
        s_kv[w][1][32 * a + q32] = sv;
      }
      if (!PASS2) {
#pragma unroll
        for (int g = 0; g + 1 < PM; ++g) {
          ocen[a][g] = ocen[a][g + 1];
          ovs[a][g] = ovs[a][g + 1];
        }
        ocen[a][PM - 1] = kbar;
        ovs[a][PM - 1] = sv;
      }
    }
    // every wave summed its own rows and columns, so the exchange stays
    // inside the wave: no workgroup barrier at the end of a block
    wave_sync();

    // H_j = K_j^T V_j - kbar_j^T sigma_j (pass 1: summed over the range)
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ra = 32 * a + 8 * (r / 4) + 4 * hh + (r % 4);
          acc[a][b][r] -= s_kv[w][0][ra] * s_kv[w][1][32 * b + q32];
        }
    wave_sync();                            // reads done before the next block's writes

    if (PASS2) {
      float sq = 0.f;
      float* Hj = (STORE && Hout) ? Hout + ((size_t)bh * nb + j) * D * D : nullptr;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int r = 4 * g + rr;
              const float xv = acc[a][b][r];
              const float dlt = xv - hb[a][b][g][rr];
              sq += dlt * dlt;
              if (Hj) Hj[(32 * (mt0 + a) + 8 * (r / 4) + 4 * hh + (r % 4)) * D + 32 * (nt0 + b) + q32] = xv;
            }
      if (STORE && Ht) {
        // H_j^T in bf16: row = value dim, 4 consecutive key-dim columns per store
        bf16* Hjt = Ht + ((size_t)bh * nb + j) * D * D;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x16& xa = acc[a][b];
              const u32x2 v = {pack2(xa[4 * g4], xa[4 * g4 + 1]), pack2(xa[4 * g4 + 2], xa[4 * g4 + 3])};
              st8(Hjt + (size_t)(32 * (nt0 + b) + q32) * D + 32 * (mt0 + a) + 8 * g4 + 4 * hh, v);
            }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
      if (lane == 0) s_sq[u][w] = (nj > 0) ? sq : -1.f;        // -1: empty block
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = f32x16{};
    }
  }

  // ---- the range's per-block outputs (the loop ends with a full wait)
  if (PASS2) {
    __syncthreads();
    if (tid < ng) {
      const float* q = s_sq[tid];
      M[(size_t)bh * nb + block_at(tid)] = q[0] < 0.f ? 0.f : sqrtf(q[0] + q[1] + q[2] + q[3]);
    }
  } else {
    const size_t nbp = (size_t)(nb + BLK - 1) / BLK * BLK;
#pragma unroll
    for (int g = 0; g < PM; ++g) {
      const int jj = j0 + g - (PM - ng);                   // block of window entry g
      if (g < PM - ng || hh != 0) continue;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        if (kout) {
          const int dk = 32 * (mt0 + a) + q32;
          centroid[((size_t)bh * nb + jj) * D + dk] = ocen[a][g];
          if (pk_cen) pk_cen[((size_t)bh * nbp + jj) * D + dk] = (bf16)ocen[a][g];
        }
        if (vout) {
          const int dv = 32 * (nt0 + a) + q32;
          vsum[((size_t)bh * nb + jj) * D + dv] = ovs[a][g];
          if (pk_vsum) pk_vsum[((size_t)bh * nbp + jj) * D + dv] = (bf16)ovs[a][g];
        }
      }
    }
    float* P = partial + (size_t)blockIdx.x * D * D;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          P[(32 * (mt0 + a) + 8 * (r / 4) + 4 * hh + (r % 4)) * D + 32 * (nt0 + b) + q32] = acc[a][b][r];
  }
}

// Hbar[bh] = (1 / n) sum of head bh's R partial sums (slots bh*R .. bh*R +
// R - 1: the ranges of the bf16 statistics kernel, or the fp32 path's one
// matrix per block with R = nb), n = the non-empty blocks (all nb without
// lengths), summed in fp64 in slot order (fixed, reproducible).  One
// workgroup per 32x32 tile of one head; each thread sums 4 adjacent entries of
// a tile row with 16-byte loads.  The tile is then staged in LDS so that the
// other layouts are written with whole rows too: Hbar in the fragment order of
// pass 2 (a tile is one contiguous 4 KB region there) and, with a bf16 pack,
// Hbar^T in bf16.  The pack's padding rows (nb .. nbp) of the centroids and
// value sums are zeroed here as well.
template <int D>
__global__ __launch_bounds__(256) void hbar_reduce_kernel(const float* __restrict__ parts, int ngrp,
                                                          int nb, float* __restrict__ hbar,
                                                          bf16* __restrict__ pk_hbart,
                                                          bf16* __restrict__ pk_cen,
                                                          bf16* __restrict__ pk_vsum, int nbp,
                                                          const int32_t* __restrict__ lens,
                                                          int heads, int BLK,
                                                          float* __restrict__ hbar_frag) {
  constexpr int TT = D / 32, DD = D * D;
  __shared__ float tile[32][33];
  const int bh = blockIdx.x / (TT * TT), tix = blockIdx.x - bh * (TT * TT);
  const int mt = tix / TT, nt = tix - mt * TT;
  const int t = threadIdx.x, r = t >> 3, c0 = (t & 7) * 4;
  const size_t e0 = (size_t)(32 * mt + r) * D + 32 * nt + c0;
  const float* p = parts + (size_t)bh * ngrp * DD + e0;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  int g = 0;
  for (; g + 4 <= ngrp; g += 4) {
    f32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const f32x4*>(p + (size_t)(g + u) * DD);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] += (double)x[u][q];
  }
  for (; g < ngrp; ++g) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p + (size_t)g * DD);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += (double)x[q];
  }
  const int nne = (valid_len(lens, bh, heads, nb * BLK) + BLK - 1) / BLK;
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = nne > 0 ? (float)(s[q] / nne) : 0.f;
  *reinterpret_cast<f32x4*>(hbar + (size_t)bh * DD + e0) = v;
  if (hbar_frag || pk_hbart) {
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[r][c0 + q] = v[q];
    __syncthreads();
    if (hbar_frag) {
      // pass 2's order: wave w = 2 (row tile / TM) + (column tile / TM) holds
      // tiles (a, b); within a tile, lane ln = col + 32 hh holds rows
      // 8 g + 4 hh + rr (rr = 0 .. 3 contiguous), at ((g * 64 + ln) * 4 + rr)
      constexpr int TM = (D == 128) ? 2 : 1;
      const int wv = 2 * (mt / TM) + nt / TM, a = mt % TM, b = nt % TM;
      float* fr = hbar_frag + (size_t)bh * DD + (size_t)((wv * TM + a) * TM + b) * 1024;
      const int fg = t >> 6, ln = t & 63, hh = ln >> 5, col = ln & 31;
      f32x4 o;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) o[rr] = tile[8 * fg + 4 * hh + rr][col];
      *reinterpret_cast<f32x4*>(fr + 4 * t) = o;
    }
    if (pk_hbart) {
      // Hbar^T: row 32 nt + rt holds column 32 nt + rt of the tile
      const int rt = t >> 3, cc = (t & 7) * 4;
      const u32x2 pk = {pack2(tile[cc][rt], tile[cc + 1][rt]), pack2(tile[cc + 2][rt], tile[cc + 3][rt])};
      st8(pk_hbart + (size_t)bh * DD + (size_t)(32 * nt + rt) * D + 32 * mt + cc, pk);
    }
  }
  if (pk_cen && nbp > nb) {
    // sizes in 64 bits: b*h*(nbp - nb)*d can pass 2^31 for large head counts
    const size_t pad = (size_t)(nbp - nb) * D;
    const size_t npad = (size_t)(gridDim.x / (TT * TT)) * pad;
    for (size_t u = (size_t)blockIdx.x * 256 + t; u < npad; u += (size_t)gridDim.x * 256) {
      const size_t b2 = u / pad, rr = u - b2 * pad;
      const size_t o = (b2 * nbp + nb) * D + rr;
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
// One workgroup per block, A = H_j - Hbar held in registers: thread (tr, tc)
// owns the 8 x 8 tile of rows 8 tr .. 8 tr + 7 and columns 8 tc .. 8 tc + 7
// (D / 8 tiles a side; D = 128: four waves, a tile row per 16 lanes; D = 64:
// one wave, a tile row per 8 lanes).  kLanczos steps of plain Lanczos on
// A^T A from a fixed start vector give a tridiagonal T whose largest
// eigenvalue approximates sigma_max^2 from below; without reorthogonalisation
// the extreme eigenvalue still converges (lost orthogonality only repeats
// converged values).  Per step, u = A v sums each tile row across its lanes
// (DPP), w = A^T u sums each tile column across the wave's rows and then
// across the waves (one LDS exchange, double-buffered: one barrier per step);
// every thread then holds u for its tile's rows and v, w for its tile's
// columns, so the dot products need no further exchange.  All threads then
// find lambda_max(T) by multisection on Sturm counts in fp64 (one point per
// thread and round: 4 rounds of 256 points, or 6 of 64 for d = 64), and
// M_j = sqrt(lambda_max).  Every sum runs in a fixed order, so the result is
// bitwise reproducible.
constexpr int kLanczos = 24;

// x + x of another lane, by DPP within rows of 16 lanes (the permutations are
// involutions, so both lanes of a pair form the same sum)
template <int CTRL>
__device__ __forceinline__ float dpp_pair_sum(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over a tile row: the NL consecutive lanes (NL = 8 or 16) holding it
template <int NL>
__device__ __forceinline__ float tile_row_sum(float x) {
  x = dpp_pair_sum<0xB1>(x);                       // quad_perm [1,0,3,2]: lane ^ 1
  x = dpp_pair_sum<0x4E>(x);                       // quad_perm [2,3,0,1]: lane ^ 2
  x = dpp_pair_sum<0x141>(x);                      // row_half_mirror: the other quad of 8
  if (NL == 16) x = dpp_pair_sum<0x140>(x);        // row_mirror: the other 8 of 16
  return x;
}

// sum over the lanes l ^ m for every m the mask covers above NL (the wave's
// tile rows that share this lane's tile column)
template <int NL>
__device__ __forceinline__ float tile_col_sum_wave(float x) {
  if (NL == 8) x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 16);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);   // lanes l and l ^ 32: same order
}

template <int D>
__global__ __launch_bounds__(D * D / 64, 4) void spectral_kernel(const float* __restrict__ H,
                                                              const float* __restrict__ hbar, int nb,
                                                              float* __restrict__ M,
                                                              const int32_t* lens, int heads,
                                                              int BLK) {
  constexpr int T = D / 8, NT = T * T, NWV = NT / 64, NL = (T < 16) ? T : 16;
  __shared__ float xch[2][NWV][D];                 // per-wave column partials of A^T u
  __shared__ float s_al[kLanczos], s_be[kLanczos];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tr = tid / T, tc = tid % T;
  const int blk = blockIdx.x, bh = blk / nb;
  if (block_count(valid_len(lens, bh, heads, nb * BLK), blk - bh * nb, BLK) == 0) {
    if (tid == 0) M[blk] = 0.f;                   // empty block: never routed
    return;
  }
  const float* Hj = H + (size_t)blk * D * D + (size_t)(8 * tr) * D + 8 * tc;
  const float* Hb = hbar + (size_t)bh * D * D + (size_t)(8 * tr) * D + 8 * tc;
  float A[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 h = *reinterpret_cast<const f32x4*>(Hj + r * D + 4 * hf);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Hb + r * D + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) A[r][4 * hf + e] = h[e] - b[e];
    }
  // start vector on this tile's columns
  float v[8], vp[8];
  float n0 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = 1.f + (float)((unsigned)(8 * tc + e) * 2654435761u % 1024u) * (1.f / 1024.f);
    n0 = fmaf(v[e], v[e], n0);
    vp[e] = 0.f;
  }
  n0 = tile_row_sum<NL>(n0);
  const float inv0 = 1.f / sqrtf(n0);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= inv0;
  float beta = 0.f;
  int kk = 0;
  for (int it = 0; it < kLanczos; ++it) {
    // u = A v on this tile's rows
    float u[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) t = fmaf(A[r][e], v[e], t);
      u[r] = tile_row_sum<NL>(t);
    }
    // w = A^T u on this tile's columns: this wave's rows, then all waves
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) t = fmaf(A[r][e], u[r], t);
      w[e] = tile_col_sum_wave<NL>(t);
    }
    if constexpr (NWV > 1) {
      float* x = xch[it & 1][wv];
      if (lane < T)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * tc + e] = w[e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = xch[it & 1][0][8 * tc + e];
#pragma unroll
        for (int q = 1; q < NWV; ++q) t += xch[it & 1][q][8 * tc + e];
        w[e] = t;
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(v[e], w[e], dot);
    const float alpha = tile_row_sum<NL>(dot);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w[e] = w[e] - alpha * v[e] - beta * vp[e];
      ss = fmaf(w[e], w[e], ss);
    }
    const float bnew = sqrtf(tile_row_sum<NL>(ss));
    if (tid == 0) {
      s_al[it] = alpha;
      s_be[it] = bnew;
    }
    kk = it + 1;
    if (!(bnew > 1e-6f * fabsf(alpha))) break;      // invariant subspace (or A = 0); uniform
    const float ib = 1.f / bnew;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vp[e] = v[e];
      v[e] = w[e] * ib;
    }
    beta = bnew;
  }
  __syncthreads();
  // lambda_max of the kk x kk tridiagonal (diag s_al, off-diag s_be) by
  // multisection over all NT threads: count(x) = number of eigenvalues below x
  // = number of negative pivots of T - x I, nondecreasing in x, so the points
  // with count < kk (below lambda_max) form a prefix; the interval shrinks to
  // the gap after its last point.  (NT + 1)^rounds > 4e9 either way.
  constexpr int ROUNDS = (NT >= 256) ? 4 : 6;
  __shared__ unsigned long long s_below[2][NWV];
  double hi = 0.0;
  for (int i = 0; i < kk; ++i) {
    double g = fabs((double)s_al[i]);
    if (i > 0) g += fabs((double)s_be[i - 1]);
    if (i + 1 < kk) g += fabs((double)s_be[i]);
    hi = fmax(hi, g);
  }
  double lo = 0.0;                                 // A^T A is positive semidefinite
  for (int round = 0; round < ROUNDS; ++round) {
    const double step = (hi - lo) / (double)(NT + 1);
    const double x = lo + step * (tid + 1);
    int cnt = 0;
    double dd = 1.0;
    for (int i = 0; i < kk; ++i) {
      const double b2 = (i > 0) ? (double)s_be[i - 1] * (double)s_be[i - 1] : 0.0;
      dd = ((double)s_al[i] - x) - (i > 0 ? b2 / dd : 0.0);
      if (dd == 0.0) dd = -1e-300;
      cnt += dd < 0.0;
    }
    const unsigned long long below = __ballot(cnt < kk);
    int l = -1;                                    // last point below lambda_max
    if constexpr (NWV > 1) {
      if (lane == 0) s_below[round & 1][wv] = below;
      __syncthreads();
      for (int q = NWV - 1; q >= 0 && l < 0; --q) {
        const unsigned long long m = s_below[round & 1][q];
        if (m != 0ull) l = 64 * q + 63 - __clzll(m);
      }
    } else {
      if (below != 0ull) l = 63 - __clzll(below);
    }
    if (l < 0) {
      hi = lo + step;
    } else {
      const double nlo = lo + step * (l + 1);
      hi = (l == NT - 1) ? hi : lo + step * (l + 2);
      lo = nlo;
    }
  }
  if (tid == 0) M[blk] = (float)sqrt(0.5 * (lo + hi));
}

template <int D>
hipError_t launch_spectral(const float* H, const float* hbar, int bh, int nb, float* M,
                           const StatsArgs& a) {
  hipLaunchKernelGGL((spectral_kernel<D>), dim3(bh * nb), dim3(D * D / 64), 0, a.stream, H, hbar, nb,
                     M, a.lens, a.heads, a.BLK);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t stats_bf16_t(const StatsArgs& a) {
  const int R = stats_ranges<D, BLK>(a.bh, a.nb);
  const int grid = a.bh * R;
  const int nbp = (a.nb + BLK - 1) / BLK * BLK;
  float* parts = static_cast<float*>(a.ws);
  bf16* pk = static_cast<bf16*>(a.packed);
  bf16* pk_cen = pk;
  bf16* pk_vsum = pk ? pk + (size_t)a.bh * nbp * D : nullptr;
  bf16* pk_hbart = pk ? pk + (size_t)2 * a.bh * nbp * D : nullptr;
  float* frag = parts + (size_t)grid * D * D;             // Hbar in pass 2's fragment order
  hipLaunchKernelGGL((stats_bf16_kernel<D, BLK, false, false>), dim3(grid), dim3(256), 0, a.stream,
                     (const bf16*)a.K, (const bf16*)a.V, a.nb, R, a.centroid, a.vsum, parts,
                     (const float*)nullptr, (float*)nullptr, (float*)nullptr, pk_cen, pk_vsum,
                     (bf16*)nullptr, a.lens, a.heads);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(hbar_reduce_kernel<D>, dim3(a.bh * (D / 32) * (D / 32)), dim3(256), 0, a.stream,
                     (const float*)parts, R, a.nb, a.hbar, pk_hbart, pk_cen, pk_vsum, nbp,
                     a.lens, a.heads, BLK, frag);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  auto pass2 = (a.H || a.ht) ? stats_bf16_kernel<D, BLK, true, true> : stats_bf16_kernel<D, BLK, true, false>;
  hipLaunchKernelGGL(pass2, dim3(grid), dim3(256), 0, a.stream,
                     (const bf16*)a.K, (const bf16*)a.V, a.nb, R, (float*)nullptr, (float*)nullptr,
                     (float*)nullptr, (const float*)frag, a.M, a.H, (bf16*)nullptr, (bf16*)nullptr,
                     static_cast<bf16*>(a.ht), a.lens, a.heads);
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
  hipLaunchKernelGGL(hbar_reduce_kernel<D>, dim3(a.bh * (D / 32) * (D / 32)), dim3(256), 0, a.stream,
                     (const float*)Hbuf, a.nb, a.nb, a.hbar, (bf16*)nullptr, (bf16*)nullptr,
                     (bf16*)nullptr, a.nb, a.lens, a.heads, a.BLK, (float*)nullptr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.spectral) return launch_spectral<D>(Hbuf, a.hbar, a.bh, a.nb, a.M, a);
  hipLaunchKernelGGL((frob_kernel<D>), dim3(grid), dim3(256), 0, a.stream, (const float*)Hbuf,
                     (const float*)a.hbar, a.nb, a.M, a.lens, a.heads, a.BLK);
  return hipGetLastError();
}

}  // namespace

size_t stats_workspace_bf16(int bh, int nb, int D, int BLK) {
  // one partial sum of H_j per range (b*h*R), then Hbar per head in pass 2's
  // fragment order
  int R = 0;
  if (D == 128 && BLK == 64) R = stats_ranges<128, 64>(bh, nb);
  else if (D == 128 && BLK == 128) R = stats_ranges<128, 128>(bh, nb);
  else if (D == 64 && BLK == 64) R = stats_ranges<64, 64>(bh, nb);
  else if (D == 64 && BLK == 128) R = stats_ranges<64, 128>(bh, nb);
  else return 0;
  return (size_t)bh * (R + 1) * D * D * sizeof(float);
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

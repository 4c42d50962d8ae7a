// Top-k selection of one row of fp64 scores by one wave, shared by the route
// kernel and the attention kernel's in-kernel routing.
//
// Radix select over order-preserving 64-bit keys of the scores.  Lane l owns
// candidates j = l + 64 u.  Each pass histograms the next 8-bit digit of the
// candidates still in play, finds the digit value d* holding the k-th largest,
// selects the candidates above it and keeps those equal to it in play.  After
// the last pass the ones left tie exactly with the k-th largest score; the
// lowest block ids among them fill the rest.  -0.0 is folded into +0.0 first so
// that equal scores give equal keys.
#pragma once

#include "common.hpp"

namespace pisa {

// Wave-wide scans and reductions on DPP row shifts (within rows of 16 lanes)
// plus three or four readlanes across the rows, instead of LDS permutes: each
// step costs a few cycles rather than an LDS round trip.  The whole wave must
// be active.
template <int N>
__device__ __forceinline__ unsigned dpp_row_shr(unsigned x, unsigned fill) {
  // row_shr:N; a lane with no source lane in its row gets `fill`
  return (unsigned)__builtin_amdgcn_update_dpp((int)fill, (int)x, 0x110 + N, 0xF, 0xF, false);
}

// inclusive prefix sum over lanes 0 .. lane
__device__ __forceinline__ unsigned wave_prefix_sum(unsigned x, int lane) {
  x += dpp_row_shr<1>(x, 0u);
  x += dpp_row_shr<2>(x, 0u);
  x += dpp_row_shr<4>(x, 0u);
  x += dpp_row_shr<8>(x, 0u);
  const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)x, 15);
  const unsigned r1 = (unsigned)__builtin_amdgcn_readlane((int)x, 31);
  const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)x, 47);
  const int row = lane >> 4;
  return x + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// AND and OR of x over the wave (uniform results)
__device__ __forceinline__ unsigned wave_and(unsigned x) {
  x &= dpp_row_shr<1>(x, ~0u);
  x &= dpp_row_shr<2>(x, ~0u);
  x &= dpp_row_shr<4>(x, ~0u);
  x &= dpp_row_shr<8>(x, ~0u);
  return (unsigned)__builtin_amdgcn_readlane((int)x, 15) & (unsigned)__builtin_amdgcn_readlane((int)x, 31) &
         (unsigned)__builtin_amdgcn_readlane((int)x, 47) & (unsigned)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ unsigned wave_or(unsigned x) {
  x |= dpp_row_shr<1>(x, 0u);
  x |= dpp_row_shr<2>(x, 0u);
  x |= dpp_row_shr<4>(x, 0u);
  x |= dpp_row_shr<8>(x, 0u);
  return (unsigned)__builtin_amdgcn_readlane((int)x, 15) | (unsigned)__builtin_amdgcn_readlane((int)x, 31) |
         (unsigned)__builtin_amdgcn_readlane((int)x, 47) | (unsigned)__builtin_amdgcn_readlane((int)x, 63);
}

// fp64 score -> unsigned key with the same order (larger score, larger key)
__device__ __forceinline__ unsigned long long order_key(double x) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x + 0.0);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// One wave selects the kk largest of sc[0 .. nne) (LDS, nu = ceil(columns / 64)
// <= 32 per lane, ties to the lower index) and sets their bits in sel (LDS,
// zeroed beforehand and ordered before this call).  hist: 256 words of LDS
// owned by this wave.  kk <= nne.  Ends with the wave's writes to sel visible
// to the wave.
__device__ inline void select_top_k(const double* sc, unsigned* hist, unsigned* sel, int nu,
                                    int nne, int kk, int lane) {
  unsigned inplay = 0u, chosen = 0u;
  for (int u = 0; u < nu; ++u)
    if (lane + 64 * u < nne) inplay |= 1u << u;
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
    kand = ((unsigned long long)wave_and((unsigned)(kand >> 32)) << 32) | wave_and((unsigned)kand);
    kor = ((unsigned long long)wave_or((unsigned)(kor >> 32)) << 32) | wave_or((unsigned)kor);
    const unsigned long long diff = kor & ~kand;          // bits that differ somewhere
    if (diff != 0ull) top_pass = (63 - __clzll((long long)diff)) / 8;
  }
  for (int pass = top_pass; pass >= 0; --pass) {
    // every candidate still in play is needed: take them all and stop early
    int ip = 0;
    for (int u = 0; u < nu; ++u) ip += __popcll(__ballot((inplay >> u) & 1u));
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
      const unsigned incl = wave_prefix_sum(own, lane);  // over lanes <= this one
      above = (unsigned)__builtin_amdgcn_readlane((int)incl, 63) - incl;
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
      const int src = __ffsll(who) - 1;                  // uniform
      dstar = __builtin_amdgcn_readlane(dstar, src);
      cnt_above = (unsigned)__builtin_amdgcn_readlane((int)cnt_above, src);
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

}

// The ids set in sel (nw <= 64 words), ascending, into out[0 .. kk), then -1
// up to out[k - 1]; sel holds exactly kk bits.  One wave.
__device__ inline void write_ids_ascending(const unsigned* sel, int nw, int kk, int k, int32_t* out,
                                           int lane) {
  const unsigned word = (lane < nw) ? sel[lane] : 0u;
  const int cnt = __popc(word);
  int pos = (int)wave_prefix_sum((unsigned)cnt, lane) - cnt;
  unsigned wv = word;
  while (wv && pos < k) {
    const int b = __ffs(wv) - 1;
    out[pos++] = 32 * lane + b;
    wv &= wv - 1;
  }
  for (int e = kk + lane; e < k; e += 64) out[e] = -1;   // fewer candidates than k
}

}  // namespace pisa

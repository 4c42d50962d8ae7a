// Top-k selection of one row of fp64 scores by one wave, shared by the route
// kernel and the attention kernel's in-kernel routing.
//
// Threshold search over order-preserving 64-bit keys of the scores.  Lane l
// owns candidates j = l + 64 u.  -0.0 is folded into +0.0 first so that equal
// scores give equal keys.
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
// zeroed beforehand and ordered before this call).  kk <= nne.  Ends with the
// wave's writes to sel visible to the wave.
//
// The threshold T (the kk-th largest key) is found bit by bit from the highest
// bit in which the keys differ: a bit is kept when at least kk keys are >= the
// prefix with that bit set.  Counts are ballots of 64-bit compares, so a step
// costs a few instructions and no LDS traffic.  As soon as exactly kk keys are
// >= the prefix, those are the answer; otherwise the keys > T are taken and
// the keys == T fill the rest, lowest ids first.  The first eight keys of each
// lane stay in registers; beyond that (more than 512 candidates) they are
// re-read from LDS at each step.
__device__ inline void select_top_k(const double* sc, unsigned* sel, int nu, int nne, int kk,
                                    int lane) {
  constexpr int NRK = 8;                                 // keys held in registers per lane
  unsigned valid = 0u;
  for (int u = 0; u < nu; ++u)
    if (lane + 64 * u < nne) valid |= 1u << u;
  unsigned long long kr[NRK];
#pragma unroll
  for (int u = 0; u < NRK; ++u)
    kr[u] = (u < nu && ((valid >> u) & 1u)) ? order_key(sc[lane + 64 * u]) : 0ull;
  auto key = [&](int u) { return order_key(sc[lane + 64 * u]); };   // u >= NRK
  // number of candidates with key >= t (uniform)
  auto count_ge = [&](unsigned long long t) {
    int c = 0;
#pragma unroll
    for (int u = 0; u < NRK; ++u)
      if (u < nu) c += __popcll(__ballot(((valid >> u) & 1u) && kr[u] >= t));
    for (int u = NRK; u < nu; ++u) c += __popcll(__ballot(((valid >> u) & 1u) && key(u) >= t));
    return c;
  };
  unsigned chosen = 0u;
  if (kk >= nne) {
    chosen = valid;                                      // every candidate
  } else if (kk > 0) {
    unsigned long long kand = ~0ull, kor = 0ull;
#pragma unroll
    for (int u = 0; u < NRK; ++u)
      if (u < nu && ((valid >> u) & 1u)) {
        kand &= kr[u];
        kor |= kr[u];
      }
    for (int u = NRK; u < nu; ++u)
      if ((valid >> u) & 1u) {
        const unsigned long long x = key(u);
        kand &= x;
        kor |= x;
      }
    kand = ((unsigned long long)wave_and((unsigned)(kand >> 32)) << 32) | wave_and((unsigned)kand);
    kor = ((unsigned long long)wave_or((unsigned)(kor >> 32)) << 32) | wave_or((unsigned)kor);
    const unsigned long long diff = kor & ~kand;          // bits that differ somewhere
    unsigned long long t = kand;                          // all keys equal: T is that key
    bool exact = false;
    if (diff != 0ull) {
      const int top = 63 - __clzll((long long)diff);
      t = (top == 63) ? 0ull : (kand & ~((2ull << top) - 1ull));   // the common prefix
      for (int b = top; b >= 0; --b) {
        const unsigned long long cand = t | (1ull << b);
        const int c = count_ge(cand);
        if (c >= kk) t = cand;
        if (c == kk) {
          exact = true;
          break;
        }
      }
    }
    // keys above T (with `exact`, keys >= T: exactly kk of them)
    int taken = 0;
#pragma unroll
    for (int u = 0; u < NRK; ++u)
      if (u < nu && ((valid >> u) & 1u) && (exact ? kr[u] >= t : kr[u] > t)) chosen |= 1u << u;
    for (int u = NRK; u < nu; ++u)
      if ((valid >> u) & 1u) {
        const unsigned long long x = key(u);
        if (exact ? x >= t : x > t) chosen |= 1u << u;
      }
    if (!exact) {
      for (int u = 0; u < nu; ++u) taken += __popcll(__ballot((chosen >> u) & 1u));
      // exact ties with the kk-th largest: lowest block ids first
      int krem = kk - taken;
      auto take_ties = [&](int u, bool tie) {
        const unsigned long long m = __ballot(tie);
        const int before_me = __popcll(m & ((1ull << lane) - 1));
        if (tie && before_me < krem) chosen |= 1u << u;
        krem -= min(krem, __popcll(m));
      };
#pragma unroll
      for (int u = 0; u < NRK; ++u)
        if (u < nu && krem > 0) take_ties(u, ((valid >> u) & 1u) && kr[u] == t);
      for (int u = NRK; u < nu && krem > 0; ++u) take_ties(u, ((valid >> u) & 1u) && key(u) == t);
    }
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

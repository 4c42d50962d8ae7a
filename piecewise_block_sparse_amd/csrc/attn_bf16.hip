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
// waves, each owning 32 query rows.  With 64-token blocks a workgroup takes
// two neighbouring query blocks (four waves): their chunk stream is the union
// of the two routed lists, in ascending block order, and each wave computes
// only the blocks of its own query block, so every row sees the same sequence
// of terms as alone, while each chunk copied to LDS serves four waves and the
// register budget allows three waves per SIMD.  Everything is computed
// transposed so that a lane owns one query row:
//   S^T[key][query]  = K_chunk . Q^T      (A = K rows from LDS, B = Q fragments in VGPRs)
//   O^T[d][query]   += V_chunk^T . P^T    (A = V read transposed from LDS, B = P from S^T)
// The 32x32x16 result layout gives lane l the 16 keys {8(r/4) + 4(l/32) + r%4}
// of query l%32, so the row max needs one cross-lane step (lane l ^ 32) and the
// rescale of O^T is lane-local.
//
// Memory pipeline: keys and values stream in chunks of CK tokens through a
// ring of two LDS stages.  Each chunk is copied global -> LDS by the waves'
// global_load_lds_dwordx4 (no registers, no staging ALU), row-major, with the
// 16-byte slots of row r XOR-swizzled by swz(r) so that the K reads (16 rows,
// one column each) and the transposing V reads (ds_read_b64_tr_b16: 4 rows x
// 32 columns) are both free of bank conflicts.  The V read of each 4-key group
// picks the keys that the lane's P registers hold, so P feeds the MFMA as is.
// PISA's zeroth-order sweep streams the bf16 centroid / value-sum pack through
// the same ring (a centroid chunk has the layout of a K / V chunk), gathering
// only the rows of blocks that some query row of the workgroup leaves
// unselected.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "lds_stream.hpp"
#include "topk.hpp"

namespace pisa {
namespace {

typedef __attribute__((address_space(1))) void gvoid;

// QB_: query blocks per workgroup.  With 64-token blocks two neighbouring
// query blocks share one workgroup (QB = 2): the chunk stream is the union of
// their routed KV blocks, and each wave computes only the blocks routed to its
// own query block.  Four waves then share every chunk copied to LDS, as with
// 128-token blocks.
template <int D_, int BLK_, int CK_, int QB_ = 1>
struct Cfg {
  static constexpr int D = D_, BLK = BLK_, CK = CK_, QB = QB_;
  static constexpr int WPQ = BLK / 32;           // waves per query block
  static constexpr int NW = QB * WPQ;            // waves per workgroup
  static constexpr int NT = 64 * NW;             // threads
  static constexpr int RB = 2 * D;               // bytes per row
  static constexpr int CPR = D / 8;              // 16-byte slots per row
  static constexpr int SUBB = CK * RB;           // bytes of one K (or V) chunk
  static constexpr int STB = 2 * SUBB;           // bytes of one stage: K chunk, then V chunk
  static constexpr int LDSB = 2 * STB;           // two stages
  static constexpr int KS = D / 16;              // MFMA k-steps over the head dim
  static constexpr int MT = D / 32;              // 32-row tiles of O^T
  static constexpr int NKT = CK / 32;            // S^T tiles per chunk
  static constexpr int NSL = CK / 16;            // 16-key slabs per chunk
  static constexpr int NDMA = STB / 1024;        // 1 KB wave copies per stage
  static constexpr int DPW = NDMA / NW;          // ... per wave
  static constexpr int RPD = 1024 / RB;          // rows per 1 KB copy
  // waves per SIMD the register budget is sized for: three (<= 168 VGPRs)
  // for d = 128 with 128 query rows per workgroup and 32-key chunks (three
  // 4-wave groups per CU, 41 KB of LDS each); two otherwise
  static constexpr int MINB = (D == 128 && QB * BLK == 128 && CK == 32) ? 3 : 2;
  static_assert(QB == 1 || (QB == 2 && BLK == 64), "query-block pairs are for 64-token blocks");
  static_assert(NDMA % NW == 0, "copies split evenly over waves");
  static_assert(DPW % 2 == 0, "per-wave copies: half K, half V");
  static_assert(D * RB <= LDSB && (D / 2) * RB <= STB, "Hbar^T (fallback) halves fit the stages");
  static_assert(BLK % CK == 0 && CK % 32 == 0, "chunking");
  // per-block first order: H_j^T (D rows) streams as HP ring chunks of RP rows
  static constexpr int RP = (2 * CK < D) ? 2 * CK : D;
  static constexpr int HP = D / RP;
  static_assert(HP <= 2, "Hbar^T streams in at most two parts");
};

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
// Any m gives the same N / D, so this only saves rescales of acc.  The weights
// of a tile are computed against the current m first; only if a lane's sum
// reaches 2^kTau (which it does whenever one weight exceeds 2^kTau, and on
// inf / NaN) is the row max formed and the tile redone, so the common path has
// no max reduction and no cross-lane wait before the exponentials.
constexpr float kTau = 8.f;
constexpr float kSumCap = 256.f;     // 2^kTau

// Lanes l and l ^ 32 hold the two halves of one query row.  permlane32_swap of
// x with itself gives every lane the pair (x[l % 32], x[l % 32 + 32]), so the
// row total / max is formed in the same order in both halves.
__device__ __forceinline__ float row_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Per-lane LDS byte offsets, fixed for the whole kernel.  The swizzle is an
// XOR on the 16-byte slot, so one lane's offsets differ only in XORed slot
// bits, and each is one XOR away from a single base:
//   K row 32 kt + q32 (kt added as an immediate), columns 16 ks + 8 hh ..:
//     k0 ^ 32 ks (column 16 ks adds 2 ks to the slot, whose low bit is hh);
//   transposing V read of tile mt: rows 0..7 of the slab at v0 ^ 64 mt,
//     rows 8..15 at that ^ 32, plus 8 RB (swz(r + 8) = swz(r) ^ 2 for both
//     head dims).
// Holding two offsets instead of sixteen leaves the compiler registers to read
// fragments further ahead of their MFMAs (measured 0.5-1.9% faster calls).
template <class C>
struct Offsets {
  int k0;
  int v0;
};

template <class C>
__device__ __forceinline__ Offsets<C> make_offsets(int lane) {
  Offsets<C> o;
  const int q32 = lane & 31, hh = lane >> 5;
  o.k0 = q32 * C::RB + ((hh ^ swz<C::D>(q32)) << 4);
  o.v0 = tr_lane_offset<C>(lane, 0, 0);
  return o;
}

template <class C>
__device__ __forceinline__ int koff_of(const Offsets<C>& o, int ks) {
  return o.k0 ^ (32 * ks);
}

// A operand of O^T += V^T P^T for 16-key slab sl and d-tile mt; its key order
// within the slab is the one the lane's P registers hold.
template <class C>
__device__ __forceinline__ u32x4 v_frag(const char* vst, int sl, int mt, const Offsets<C>& off) {
  const int t0 = off.v0 ^ (64 * mt);
  return tr_read<C>(vst + 8 * C::RB, sl, t0 - 8 * C::RB, t0 ^ 32);
}

// exp2 weights -> bf16 MFMA B operands, and the sum of the same bf16 weights.
// Each pair is packed into its own 32-bit value and summed from that value
// with v_dot2 against (1, 1), alternating between two partial sums so that the
// chain the rescale test waits for is half as long.
template <int NKT>
__device__ __forceinline__ float weights_bf16(const f32x16 (&s)[NKT], float c2, float nm,
                                              u32x4 (&pf)[2 * NKT]) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  float sum[2] = {0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float p0 = fast_exp2(fmaf(s[kt][2 * q], c2, nm));
      const float p1 = fast_exp2(fmaf(s[kt][2 * q + 1], c2, nm));
      const bf16x2 pr = {(bf16)p0, (bf16)p1};
      sum[q & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum[q & 1], false);
      pf[2 * kt + q / 4][q % 4] = __builtin_bit_cast(unsigned, pr);
    }
  return sum[0] + sum[1];
}

// S^T of the chunk in `stage` (K rows) against this wave's queries.  PRE:
// all K fragments of a tile are read before its MFMA chain (two-wave register
// budget); otherwise through a window of three fragments.
template <class C, bool PRE>
__device__ __forceinline__ void s_tiles(f32x16 (&s)[C::NKT], const bf16x8 (&qf)[C::KS],
                                        const char* stage, const Offsets<C>& off) {
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt) {
    s[kt] = f32x16{};
    if constexpr (PRE) {
      u32x4 kf[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) kf[ks] = ld16(stage + kt * 32 * C::RB + koff_of<C>(off, ks));
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) s[kt] = mfma32(as_bf16x8(kf[ks]), qf[ks], s[kt]);
    } else {
      // a window of three fragments: each K read goes out three MFMAs ahead of
      // its use, and the scheduling fences keep that order (the compiler alone
      // placed them two ahead; three measured 0.5-3% faster calls, four the same)
      constexpr int W = 3;
      u32x4 kf[W];
#pragma unroll
      for (int ks = 0; ks < W; ++ks) kf[ks] = ld16(stage + kt * 32 * C::RB + koff_of<C>(off, ks));
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        s[kt] = mfma32(as_bf16x8(kf[ks % W]), qf[ks], s[kt]);
        if (ks + W < C::KS) kf[ks % W] = ld16(stage + kt * 32 * C::RB + koff_of<C>(off, ks + W));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Logits of keys that do not take part -> -inf.  STAGE2: positions of the
// stage-2 list that this query block does not take (bit jbase + key set in
// `bits`: a block of its S_i, or the list's padding); stage 1: keys past the
// sequence's end (key of register r: 32 kt + 8 (r / 4) + 4 hh + r % 4).
template <class C, bool STAGE2>
__device__ __forceinline__ void mask_keys(f32x16 (&s)[C::NKT], int hh, const unsigned* bits,
                                          int jbase, int kvalid) {
  if (STAGE2) {
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
      const unsigned wbits = bits[(jbase >> 5) + kt] >> (4 * hh);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((wbits >> (8 * (r / 4) + (r % 4))) & 1u) s[kt][r] = -INFINITY;
    }
  } else if (kvalid < C::CK) {
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kt + 8 * (r / 4) + 4 * hh + (r % 4) >= kvalid) s[kt][r] = -INFINITY;
  }
}

// Weights of one chunk's logits into the online softmax: bf16 B operands in
// pf, the running max raised (and acc, l, a rescaled) only when needed, and
// the chunk's share added to l (and, STAGE2, to a).  In stage 2 each weight
// counts BLK times in the denominator; the block at chunk position jpart (if
// >= 0) holds BLK - wmiss tokens, so its weight counts that many times.
template <class C, bool STAGE2>
__device__ __forceinline__ void softmax_update(RowState<C::D>& st, const f32x16 (&s)[C::NKT],
                                               float c2, int hh, u32x4 (&pf)[C::NSL],
                                               int jpart = -1, float wmiss = 0.f) {
  float ps = weights_bf16<C::NKT>(s, c2, -st.m, pf);
  if (__any(!(ps < kSumCap))) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = row_max(mx) * c2;
    if (__any(mx > st.m + kTau)) {
      const float mnew = fmaxf(st.m, mx);
      const float corr = fast_exp2(st.m - mnew);
      st.m = mnew;
      st.l *= corr;
      st.a *= corr;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) st.acc[mt] *= corr;
      ps = weights_bf16<C::NKT>(s, c2, -st.m, pf);
    }
  }
  if (STAGE2) {
    st.l += (float)C::BLK * ps;
    st.a += ps;
    if (jpart >= 0) {
      // the ragged block weighs n_j = BLK - wmiss: take back wmiss times its
      // (bf16) weight, recomputed exactly as weights_bf16 formed it
      float sl = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kt + 8 * (r / 4) + 4 * hh + (r % 4) == jpart) sl = s[kt][r];
      st.l -= wmiss * (float)(bf16)fast_exp2(fmaf(sl, c2, -st.m));
    }
  } else {
    st.l += ps;
  }
}

// All V fragments of a chunk (A operands of O^T += V^T P^T)
template <class C>
__device__ __forceinline__ void v_frags(u32x4 (&vf)[C::NSL][C::MT], const char* vst,
                                        const Offsets<C>& off) {
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int sl = 0; sl < C::NSL; ++sl) vf[sl][mt] = v_frag<C>(vst, sl, mt, off);
}

template <class C>
__device__ __forceinline__ void pv_frags(RowState<C::D>& st, const u32x4 (&vf)[C::NSL][C::MT],
                                         const u32x4 (&pf)[C::NSL]) {
#pragma unroll
  for (int sl = 0; sl < C::NSL; ++sl)
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      st.acc[mt] = mfma32(as_bf16x8(vf[sl][mt]), as_bf16x8(pf[sl]), st.acc[mt]);
}

// One CK-key chunk from a stage: S^T, softmax update, O^T += V^T P^T.
// With the two-wave register budget and 32-key chunks (PRE) every LDS
// fragment is read well before its MFMA; the three-wave budget (and 64-key
// chunks) leave room for a window of three fragments each for K and V.
template <class C, bool STAGE2>
__device__ __forceinline__ void chunk(RowState<C::D>& st, const bf16x8 (&qf)[C::KS],
                                      const char* stage, const Offsets<C>& off, float c2, int hh,
                                      const unsigned* bits, int jbase, int kvalid = C::CK,
                                      int jpart = -1, float wmiss = 0.f) {
  constexpr bool PRE = C::MINB == 2 && C::CK == 32;
  const char* vst = stage + C::SUBB;
  f32x16 s[C::NKT];
  s_tiles<C, PRE>(s, qf, stage, off);
  u32x4 vf[C::NSL][C::MT];
  if constexpr (PRE) v_frags<C>(vf, vst, off);
  mask_keys<C, STAGE2>(s, hh, bits, jbase, kvalid);
  u32x4 pf[C::NSL];
  // without PRE: the first VW V fragments are read before the softmax, so
  // their latency hides under the exponentials, then each read goes out VW
  // MFMAs ahead of its use (fenced like the K window; measured 0.7-1.3%
  // faster calls, four fragments the same)
  constexpr int VW = 3, NF = C::MT * C::NSL;
  u32x4 vw[VW];
  if constexpr (!PRE) {
#pragma unroll
    for (int f = 0; f < VW; ++f) vw[f] = v_frag<C>(vst, f % C::NSL, f / C::NSL, off);
    __builtin_amdgcn_sched_barrier(0);   // issued in the wait for the last S^T MFMA
  }
  softmax_update<C, STAGE2>(st, s, c2, hh, pf, jpart, wmiss);
  if constexpr (PRE) {
    pv_frags<C>(st, vf, pf);
  } else {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mt = f / C::NSL, sl = f % C::NSL;
      st.acc[mt] = mfma32(as_bf16x8(vw[f % VW]), as_bf16x8(pf[sl]), st.acc[mt]);
      if (f + VW < NF) vw[f % VW] = v_frag<C>(vst, (f + VW) % C::NSL, (f + VW) / C::NSL, off);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// First-order term of one unselected block j (per-block order): the stage
// holds RP rows (value dims part * RP ..) of H_j^T in the K-chunk layout.
//   alpha = exp2(c2 * q . kbar_j - m)  (q . kbar_j by v_dot2 over the lane's half
//           of q and of the bf16 centroid, summed with the partner lane),
//   acc[d] += scale * alpha * (q H_j)[d]  for the RP value dims of this part,
// with q H_j as MFMAs: A = H_j^T rows from LDS, B = the query fragments.
// alpha uses the current running max, as every other term added now.
template <class C>
__device__ __forceinline__ void first_order_part(RowState<C::D>& st, const bf16x8 (&qf)[C::KS],
                                                 const char* stage, const Offsets<C>& off,
                                                 float c2, float scale, const bf16* cen_j,
                                                 int part, int hh) {
  constexpr int MTP = C::RP / 32;                     // 32-row tiles per part
  // bf16 -> fp32 by placing the 16 bits high (exact), then fp32 FMAs.  (v_dot2
  // on 32-bit lanes of a bit-cast 128-bit vector is miscompiled to read one
  // register pair for every lane.)
  float dot = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const u32x4 kc = ld16(cen_j + 16 * ks + 8 * hh);
    const u32x4 qq = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot = fmaf(__uint_as_float(qq[e] << 16), __uint_as_float(kc[e] << 16), dot);
      dot = fmaf(__uint_as_float(qq[e] & 0xffff0000u), __uint_as_float(kc[e] & 0xffff0000u), dot);
    }
  }
  const float f = scale * fast_exp2(row_sum(dot) * c2 - st.m);
  f32x16 hq[MTP];
#pragma unroll
  for (int mtl = 0; mtl < MTP; ++mtl) {
    hq[mtl] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      hq[mtl] = mfma32(as_bf16x8(ld16(stage + mtl * 32 * C::RB + koff_of<C>(off, ks))), qf[ks], hq[mtl]);
  }
  // acc tile mt belongs to part mt / MTP; the other parts' tiles get a zero factor
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) st.acc[mt] += (mt / MTP == part ? f : 0.f) * hq[mt % MTP];
}

// The lane's query fragments times f, rounded to bf16: the B operands of the
// global first-order term, so that term accumulates straight into the output
// tiles (no temporary tile).
template <class C>
__device__ __forceinline__ void scale_frags(bf16x8 (&qf)[C::KS], float f) {
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)qf[ks][e] * f);
}

// Global first-order term, part PART: the stage holds RP rows (value dims
// PART * RP ..) of Hbar^T in the K-chunk layout; acc[d] += (q Hbar)[d] f for
// those dims as MFMAs into the output tiles (A = Hbar^T rows from LDS, B = the
// query fragments already scaled by f).
template <class C, int PART>
__device__ __forceinline__ void hbar_part(RowState<C::D>& st, const bf16x8 (&fq)[C::KS],
                                          const char* stage, const Offsets<C>& off) {
  constexpr int MTP = C::RP / 32;                     // 32-row tiles per part
#pragma unroll
  for (int mtl = 0; mtl < MTP; ++mtl) {
    if constexpr (PART * MTP + MTP <= C::MT) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        st.acc[PART * MTP + mtl] = mfma32(as_bf16x8(ld16(stage + mtl * 32 * C::RB + koff_of<C>(off, ks))), fq[ks],
                                          st.acc[PART * MTP + mtl]);
    }
  }
}

// Stage-2 copy of CK gathered rows: row r of the stage's centroid half is row
// rows[r] of the bf16 centroid pack gC, and the same row of the value-sum
// pack gS fills the other half.  The pieces and lane slots are those of
// dma_stage (wave w copies pieces w H .. w H + H - 1 of each half, H = DPW / 2),
// with the row's global offset taken per lane from its id instead of from its
// position, and M0 set per piece since the pieces are no longer contiguous in
// global memory.  The lane's row within its piece and its swizzled slot are
// read back from its dma_stage offset o.v[u] = row * RB + 16 * slot (RB a power
// of two above 16 * slot), so no other per-lane value stays live for this.
template <class C>
__device__ __forceinline__ void dma_rows(const char* gC, const char* gS, const short* rows,
                                         unsigned stage_m0, int w, const DmaOff<C>& o) {
  constexpr int H = C::DPW / 2;
  static_assert((C::RB & (C::RB - 1)) == 0 && C::RPD * C::RB == 1024, "rows are a power of two bytes");
#pragma unroll
  for (int u = 0; u < H; ++u) {
    // an opaque copy: what is derived from it is recomputed at each call
    // instead of being hoisted out of the chunk loop and held in registers
    unsigned ov = o.v[u];
    asm volatile("" : "+v"(ov));
    const int r = (w * H + u) * C::RPD + (int)(ov / C::RB);   // row of the chunk
    const unsigned voff = (unsigned)rows[r] * C::RB + (ov & (C::RB - 1));
    const unsigned m0c = stage_m0 + (unsigned)(w * H + u) * 1024u;
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, %4"
        :
        : "s"(m0c), "s"(m0c + (unsigned)C::SUBB), "v"(voff), "s"(gC), "s"(gS)
        : "memory", "m0");
  }
}

// fp32 statistics -> bf16 chunk of CK centroids / value sums in the stage
// layout (used when no bf16 pack was supplied): row r of the chunk is block
// rows[r] (an id at or past nb gives a zero row).
template <class C>
__device__ __forceinline__ void stage_centroids(const float* cen, const float* vs, const short* rows,
                                                int nb, char* stage, int tid) {
  for (int q = tid; q < 2 * C::CK * C::CPR; q += C::NT) {
    const bool isv = q >= C::CK * C::CPR;
    const int qq = isv ? q - C::CK * C::CPR : q;
    const int r = qq / C::CPR, c = qq % C::CPR;
    const int j = rows[r];
    const float* src = (isv ? vs : cen) + (size_t)j * C::D + 8 * c;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
    if (j < nb) {
      lo = *reinterpret_cast<const f32x4*>(src);
      hi = *reinterpret_cast<const f32x4*>(src + 4);
    }
    const u32x4 v = {pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
    st16(stage + (isv ? C::SUBB : 0) + r * C::RB + ((c ^ swz<C::D>(r)) << 4), v);
  }
}

// fp32 Hbar [d_k][d_v] -> bf16 Hbar^T [d_v][d_k] rows in the K layout; rows
// below D/2 go to stage 0, the others to stage 1
template <class C>
__device__ __forceinline__ void stage_hbar_t(const float* hb, char* s0, char* s1, int tid) {
  for (int q = tid; q < C::D * C::CPR; q += C::NT) {
    const int r = q / C::CPR, c = q % C::CPR;   // row = d_v, columns d_k = 8c .. 8c+7
    unsigned w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pack2(hb[(size_t)(8 * c + 2 * e) * C::D + r], hb[(size_t)(8 * c + 2 * e + 1) * C::D + r]);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    char* dst = (r < C::D / 2) ? s0 + r * C::RB : s1 + (r - C::D / 2) * C::RB;
    st16(dst + ((c ^ swz<C::D>(r)) << 4), v);
  }
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
  const bf16* ht;        // H_j^T per block, bf16 [bh][nb][D][D] (per-block first order)
  bf16* O;
  const float* M;        // in-kernel routing: M_j [bh][nb]
  int32_t* idx_out;      // in-kernel routing: the selection written out (nullable)
  float* part;           // split work items: partial states, one slot per (item, part)
  int* nparts;           // split work items: parts of each item (written by part 0)
};

// Split work items: an item (the query block(s) of one workgroup) whose exact
// list holds more than `cap` blocks runs as up to `pmax` parts on separate
// workgroups, each over a contiguous share of the exact chunks (part 0 also
// runs stages 2 and 3).  A part leaves its unnormalised state in a slot:
// acc [QB*BLK][D] | m [QB*BLK] (log2 units) | l [QB*BLK], all fp32.
struct SplitIn {
  int cap;
  int pmax;
  int items;
};

constexpr int kSplitMaxParts = 32;                     // parts per split item, at most

template <class C>
__host__ __device__ constexpr size_t split_slot_floats() {
  return ((size_t)C::QB * C::BLK * (C::D + 2) + 63) / 64 * 64;
}

// In-kernel routing (workgroup-local copy of the route kernel's selection):
// rk blocks per query block, score = rscale * qbar . kbar_j + rlam * M_j in fp64.
struct RouteIn {
  int rk;
  double rscale;
  double rlam;
};

constexpr int kBitWords = (kMaxBlocks + 128) / 32;
constexpr int kIdMask = 0xfff;                  // block id bits of a list entry (ids < 4096)
static_assert(kMaxBlocks <= kIdMask + 1, "block ids fit below the pair flags");

// The lane's query row (32 wq + q32 of block qblk) as MFMA B-operand fragments;
// padding queries (row >= ni) are zero rows.
template <class C, bool VL>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[C::KS], const bf16* Q, int bh, size_t L,
                                             int qblk, int wq, int q32, int hh, int ni) {
  const bf16* qrow = Q + ((size_t)bh * L + (size_t)qblk * C::BLK + 32 * wq + q32) * C::D + 8 * hh;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  if ((VL || C::QB == 2) && 32 * wq + q32 >= ni)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

// VL: sequences have valid lengths (lens); without, the length code compiles away.
// FO: the per-block first order (its stage lives only in these instantiations,
// so the other modes keep their register budget).
// FR: the workgroup routes its own query blocks (pooled query, fp64 scores
// against every centroid, top-k) instead of reading idx; the selection is the
// route kernel's, bit for bit.
// NP: the approximate modes without the bf16 statistics pack: stages 2 and 3
// convert the fp32 statistics while staging them (an instantiation of its own,
// so that the other instantiations carry none of its registers).
// SP: split work items (see SplitIn).  XCD x (workgroups w with w % 8 == x)
// owns items x*c .. x*c + c - 1 (c = ceil(items / 8)) and runs, in dispatch
// order, parts 1 .. pmax - 1 of all of them, then their parts 0: the parts of
// one item are c workgroups apart (different CUs), the parts that an item does
// not need exit at once, and the extra parts of heavy items start first.
template <class C, bool VL, bool FO, bool FR = false, bool NP = false, bool SP = false>
__global__ __launch_bounds__(C::NT, C::MINB) void attn_bf16_kernel(AttnPtrs p, int kmax, int approx,
                                                             int order, float scale, int nb,
                                                             const int32_t* lens, int heads,
                                                             RouteIn ri, SplitIn si) {
  constexpr int D = C::D, BLK = C::BLK, CK = C::CK;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDSB];
  constexpr int QB = C::QB;
  static_assert(QB == 1 || !FO, "the per-block first order runs one query block per workgroup");
  __shared__ unsigned bits[QB][kBitWords];
  static_assert(!(FR && FO), "in-kernel routing runs with the other orders");
  static_assert(!FR || QB * BLK * C::RB <= C::LDSB, "in-kernel routing stages the query rows in the ring");
  __shared__ unsigned exb[QB][kBitWords];               // exact blocks (a set: duplicates count once)
  __shared__ short s_list[kMaxBlocks];                 // exact block ids of S_i, in order;
                                                       // then (per-block first order) U_i.
                                                       // Pairs: the union, ascending, with
                                                       // bit 12 + q set if query block q
                                                       // routes the block
  // stage 2: the blocks that some live query block of the item leaves
  // unselected, ascending, then id 0 up to a whole chunk; s_umask[q] bit p set
  // when position p does not take part for query block q (a block of its S_i,
  // or past the list's end); s_rag: the position of the ragged last block
  __shared__ short s_ulist[kMaxBlocks];
  __shared__ unsigned s_umask[QB][kBitWords];
  __shared__ int s_cnt[3];
  __shared__ int s_rag;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q32 = lane & 31, hh = lane >> 5;
  static_assert(!SP || (!FO && !FR), "split work items run the idx-driven orders other than the per-block first order");
  const int ngrp = (nb + QB - 1) / QB;                 // items per (batch, head)
  int item, part = 0;
  if constexpr (SP) {
    const int nitems = si.items, c = (nitems + 7) / 8;
    const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3;
    const int grp = sl / c;
    item = xcd * c + (sl - grp * c);
    part = (grp + 1) % si.pmax;
    if (item >= nitems) return;                         // (grid padding)
  } else {
    item = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int bh = item / ngrp, i0 = (item - bh * ngrp) * QB;
  // this wave: query block i0 + qb, rows 32 wq .. (qb as a scalar, so that
  // branches on the wave's query block are uniform)
  const int qb = __builtin_amdgcn_readfirstlane(w / C::WPQ), wq = w - qb * C::WPQ;
  const int i = i0 + qb;
  const bool qvalid = i < nb;                          // (odd nb: the last pair has one block)
  const size_t L = (size_t)nb * BLK;
  const int nbp = (nb + BLK - 1) / BLK * BLK;
  const bf16* Kh = p.K + (size_t)bh * L * D;
  const bf16* Vh = p.V + (size_t)bh * L * D;
  const bool packed = approx && !NP;
  static_assert(!(NP && FO), "the per-block first order streams the pack");
  // valid tokens: blocks j < nne are non-empty; query block i holds ni queries
  const int Lv = VL ? valid_len(lens, bh, heads, (int)L) : (int)L;
  const int nne = VL ? (Lv + BLK - 1) / BLK : nb;
  const int ni = !qvalid ? 0 : (VL ? block_count(Lv, i, BLK) : BLK);
  // the workgroup's query blocks past the sequence (or past nb) have no work
  int nlive = 0;
#pragma unroll
  for (int q = 0; q < QB; ++q)
    nlive += (i0 + q < nb) && (!VL || block_count(Lv, i0 + q, BLK) > 0);
  if (nlive == 0) {
    // query blocks past the sequence: their rows are 0
    if (SP && part > 0) return;
    if (SP && tid == 0) p.nparts[item] = 1;
    for (int q = 0; q < QB; ++q) {
      if (i0 + q >= nb) break;
      bf16* ob = p.O + ((size_t)bh * L + (size_t)(i0 + q) * BLK) * D;
      for (int e = tid; e < BLK * D / 8; e += C::NT) st16(ob + 8 * e, u32x4{0u, 0u, 0u, 0u});
      if (FR && p.idx_out)
        for (int e = tid; e < ri.rk; e += C::NT) p.idx_out[((size_t)bh * nb + i0 + q) * ri.rk + e] = -1;
    }
    return;
  }
  const bool alive = ni > 0;                           // wave-uniform
  const bool first = FO && approx && order == kOrderFirst && packed && p.ht != nullptr;
  // this lane's query row as 16-byte B-operand fragments (d = 16 ks + 8 hh + 0..7);
  // with in-kernel routing they are loaded first, as the pooling reads them too
  bf16x8 qf[C::KS];
  if constexpr (FR) load_q_frags<C, VL>(qf, p.Q, bh, L, qvalid ? i : i0, wq, q32, hh, ni);

  if constexpr (FR) {
    // ---- in-kernel routing.  LDS (the ring, idle until the chunk stream
    // starts): first the query rows, staged for pooling over the whole ring;
    // then qbar [QB][D] f64 | pooling partials [QB][WPQ][D] f64, then the
    // scores [QB][ncol] f64 in their place (the launcher checks that the
    // scores fit).
    double* s_qbar = reinterpret_cast<double*>(lds);
    double* s_part = s_qbar + QB * D;
    double* s_sc = s_qbar + QB * D;
    const int ncol = (nb + 63) / 64 * 64;
    for (int e = tid; e < kBitWords; e += C::NT) {
      const int lo = 32 * e;
      unsigned pad = 0u;                                 // padding and empty blocks: j >= nne
      if (lo + 32 > nne) pad = (lo >= nne) ? ~0u : (~0u << (nne - lo));
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        bits[q][e] = pad;
        exb[q][e] = 0u;
      }
    }
    // pooled query of block i: exact fp64 sums of its ni valid queries.  The
    // query rows, already in registers as MFMA fragments (padding queries are
    // zero rows), are staged row-major in the ring; the waves of each query
    // block then sum its columns with 16-byte LDS reads and times 1 / ni below.
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      st16(lds + (size_t)(qb * BLK + 32 * wq + q32) * C::RB + 32 * ks + 16 * hh,
           __builtin_bit_cast(u32x4, qf[ks]));
    __syncthreads();
    {
      constexpr int CPR = D / 8, TPQ = 64 * C::WPQ, RPI = TPQ / CPR, NR = BLK / RPI;
      const int tq = tid - qb * TPQ, c = tq % CPR, rs = tq / CPR;
      double x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int n = 0; n < NR; ++n) {
        const bf16x8 v = as_bf16x8(ld16(lds + (size_t)(qb * BLK + rs + n * RPI) * C::RB + 16 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += (double)(float)v[e];
      }
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += __shfl_xor(x[e], o);
      __syncthreads();                                   // staged rows read before the partials
      if (lane < CPR)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_part[(qb * C::WPQ + wq) * D + 8 * c + e] = x[e];
    }
    __syncthreads();
    for (int e = tid; e < QB * D; e += C::NT) {
      const int q = e / D;
      double sum = 0.0;
#pragma unroll
      for (int u = 0; u < C::WPQ; ++u) sum += s_part[(q * C::WPQ + u) * D + (e - q * D)];
      const int nq = (i0 + q < nb) ? (VL ? block_count(Lv, i0 + q, BLK) : BLK) : 0;
      s_qbar[e] = sum * ((nq == BLK) ? 1.0 / BLK : 1.0 / (double)(nq > 0 ? nq : 1));
    }
    __syncthreads();
    // scores of the candidates j < nne against the QB pooled queries: one
    // fp64 FMA chain over d in the route kernel's order (within each 16-wide
    // chunk of the head dimension: d = 16 t + 4 g + s for s, then g), then
    // scale * dot + lambda * M_j as one FMA: the route kernel's arithmetic, so
    // both select the same blocks
    {
      const float* cen = p.centroid + (size_t)bh * nb * D;
      const float* Mh = p.M + (size_t)bh * nb;
      for (int j = tid; j < nne; j += C::NT) {
        const float* cj = cen + (size_t)j * D;
        double acc[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) acc[q] = 0.0;
        // the centroid row in 16-byte loads, eight in flight for query-block
        // pairs (with one query block per workgroup eight make the compiler
        // spill the main loop, so that case reads four at a time)
        constexpr int CH = (QB == 2) ? 2 : 1;            // 16-wide chunks per batch
        auto batch = [&](int a0) {
          f32x4 kv[4 * CH];
#pragma unroll
          for (int u = 0; u < 4 * CH; ++u) kv[u] = *reinterpret_cast<const f32x4*>(cj + a0 + 4 * u);
#pragma unroll
          for (int h = 0; h < CH; ++h)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
              for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int q = 0; q < QB; ++q)
                  acc[q] = fma(s_qbar[q * D + a0 + 16 * h + 4 * g + s], (double)kv[4 * h + g][s], acc[q]);
        };
        if constexpr (QB == 2) {
          for (int a0 = 0; a0 < D; a0 += 16 * CH) batch(a0);
        } else {
#pragma unroll 1
          for (int a0 = 0; a0 < D; a0 += 16 * CH) batch(a0);   // one batch at a time: no spills
        }
        const double mj = ri.rlam * (double)Mh[j];
#pragma unroll
        for (int q = 0; q < QB; ++q) s_sc[q * ncol + j] = fma(ri.rscale, acc[q], mj);
      }
    }
    __syncthreads();
    // top-k of each query block by its first wave; the ids go out when asked
    if (wq == 0 && qvalid) {
      const int kk = (ni > 0) ? min(ri.rk, nne) : 0;
      select_top_k(s_sc + qb * ncol, exb[qb], ncol / 64, nne, kk, lane);
      if (p.idx_out) write_ids_ascending(exb[qb], ncol / 32, kk, ri.rk, p.idx_out + ((size_t)bh * nb + i) * ri.rk, lane);
    }
    __syncthreads();
    for (int e = tid; e < nbp / 32; e += C::NT)
#pragma unroll
      for (int q = 0; q < QB; ++q) bits[q][e] |= exb[q][e];
    __syncthreads();
  }
  if (!FR) {
    // bits[q]: bit j set when block j is exact for query block i0 + q (in its
    // S_i) or padding (j >= nne); exb[q]: the exact blocks alone
    for (int e = tid; e < nbp / 32; e += C::NT) {
      const int lo = 32 * e;
      unsigned pad = 0u;                                 // padding and empty blocks: j >= nne
      if (lo + 32 > nne) pad = (lo >= nne) ? ~0u : (~0u << (nne - lo));
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        bits[q][e] = pad;
        exb[q][e] = 0u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (i0 + q >= nb) break;
      const int32_t* rq = p.idx + ((size_t)bh * nb + i0 + q) * kmax;
      for (int e = tid; e < kmax; e += C::NT) {
        const int j = rq[e];
        if (j >= 0 && j < nne) {
          atomicOr(&bits[q][j >> 5], 1u << (j & 31));
          atomicOr(&exb[q][j >> 5], 1u << (j & 31));
        }
      }
    }
    __syncthreads();
  }

  // this lane's query row as 16-byte B-operand fragments (d = 16 ks + 8 hh + 0..7)
  if constexpr (!FR) load_q_frags<C, VL>(qf, p.Q, bh, L, qvalid ? i : i0, wq, q32, hh, ni);
  const Offsets<C> off = make_offsets<C>(lane);
  const DmaOff<C> loff = dma_lane_offsets<C>(w, lane);
  RowState<D> st;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) st.acc[mt] = f32x16{};
  st.m = -1e30f;
  st.l = 0.f;
  st.a = 0.f;
  const float c2 = scale * kLog2e;

  // ---- the chunk stream: CK-token chunks of the exact blocks of S_i (in idx
  // order), then (approximate modes with a pack) the compacted stage-2 list,
  // CK gathered centroid / value-sum rows per chunk.  Both lists are built in
  // LDS once, in ascending block order.
  constexpr int SPB = BLK / CK;                          // chunks per KV block
  if (w == 0) {
    int cnt = 0;
    {
      // the exact blocks (pairs: the union of the two rows), ascending, from
      // the bitmaps (lane = bitmap word: nbp <= 2048)
      const unsigned a = (lane < nbp / 32) ? exb[0][lane] : 0u;
      const unsigned b = (QB == 2 && lane < nbp / 32) ? exb[QB - 1][lane] : 0u;
      const unsigned u = a | b;
      const int n = __popc(u);
      int pre = n;                                       // inclusive prefix over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(pre, o);
        if (lane >= o) pre += y;
      }
      int pos = pre - n;
      for (unsigned r = u; r; r &= r - 1) {
        const int bit = __ffs(r) - 1;
        s_list[pos++] = (short)((32 * lane + bit) | (((a >> bit) & 1u) << 12) | (((b >> bit) & 1u) << 13));
      }
      cnt = __shfl(pre, 63);
    }
    // stage 2 (approximate modes): the blocks that a live query block of the
    // item leaves unselected, compacted in ascending order, so the sweep
    // multiplies no column that every one of its rows masks; per query block,
    // the positions it does not take (its exact blocks, the list's padding)
    int ccnt = 0;                                        // stage-2 chunks
    if (lane == 0) s_rag = -1;
    if (approx) {
      const int jr = (VL && Lv % BLK != 0) ? nne - 1 : -1;   // the ragged last block
      unsigned live = 0u;
#pragma unroll
      for (int q = 0; q < QB; ++q)
        if (i0 + q < nb && (!VL || block_count(Lv, i0 + q, BLK) > 0)) live |= 1u << q;
      for (int e = lane; e < kBitWords; e += 64)
#pragma unroll
        for (int q = 0; q < QB; ++q) s_umask[q][e] = 0u;
      wave_sync();
      int n = 0;
      for (int j0 = 0; j0 < nbp; j0 += 64) {
        const int j = j0 + lane;
        unsigned skip = 0u;                              // bit q: query block q does not take j
        bool u = false;
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const bool ex = j >= nbp || !((live >> q) & 1u) || ((bits[q][j >> 5] >> (j & 31)) & 1u);
          if (ex) skip |= 1u << q;
          else u = true;
        }
        const unsigned long long m = __ballot(u);
        if (u) {
          const int pos = n + __popcll(m & ((1ull << lane) - 1));
          s_ulist[pos] = (short)j;
#pragma unroll
          for (int q = 0; q < QB; ++q)
            if ((skip >> q) & 1u) atomicOr(&s_umask[q][pos >> 5], 1u << (pos & 31));
          if (j == jr) s_rag = pos;
        }
        n += __popcll(m);
      }
      ccnt = (n + CK - 1) / CK;
      for (int pos = n + lane; pos < ccnt * CK; pos += 64) {
        s_ulist[pos] = 0;                                // a valid row, masked for every query block
#pragma unroll
        for (int q = 0; q < QB; ++q) atomicOr(&s_umask[q][pos >> 5], 1u << (pos & 31));
      }
    }
    int ucnt = 0;
    if (first) {
      // unselected blocks (bit clear), ascending, after the exact ids
      for (int c0 = 0; c0 < nb; c0 += 64) {
        const int j = c0 + lane;
        const bool u = j < nb && !((bits[0][j >> 5] >> (j & 31)) & 1u);
        const unsigned long long m = __ballot(u);
        // exact ids plus U_i fill at most nb <= kMaxBlocks slots (more only for
        // an idx row with duplicate ids, whose excess is dropped)
        const int slot = cnt + ucnt + __popcll(m & ((1ull << lane) - 1));
        if (u && slot < kMaxBlocks) s_list[slot] = (short)j;
        ucnt = min(ucnt + __popcll(m), kMaxBlocks - cnt);
      }
    }
    if (lane == 0) {
      s_cnt[0] = cnt;
      s_cnt[1] = ccnt;
      s_cnt[2] = ucnt;
    }
  }
  __syncthreads();
  const int ncnt = s_cnt[0];
  // split items: this part's share [ex0, ex0 + nex) of the exact chunks; parts
  // past the item's count have nothing to do; only part 0 runs stages 2 and 3
  int nparts = 1, ex0 = 0, nexp = ncnt * SPB;
  if constexpr (SP) {
    nparts = min(si.pmax, max(1, (ncnt + si.cap - 1) / si.cap));
    if (part >= nparts) return;
    if (part == 0 && tid == 0) p.nparts[item] = nparts;
    ex0 = (int)((long long)ncnt * SPB * part / nparts);
    nexp = (int)((long long)ncnt * SPB * (part + 1) / nparts) - ex0;
  }
  const bool tail = !SP || part == 0;                  // this workgroup runs stages 2 and 3
  // mixed order with the bf16 pack: Hbar^T streams as HP ring chunks after stage 2
  const int nhb = (tail && packed && order == kOrderMixed) ? C::HP : 0;
  const int nex = nexp, ncen = nex + (tail && packed ? s_cnt[1] : 0), nhbe = ncen + nhb, ntot = nhbe + s_cnt[2] * C::HP;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const unsigned lds_m0 = (unsigned)(uintptr_t)(lvoid*)lds;
  const char* Kb = reinterpret_cast<const char*>(Kh);
  const char* Vb = reinterpret_cast<const char*>(Vh);
  const char* Cb = packed ? reinterpret_cast<const char*>(p.pk_cen + (size_t)bh * nbp * D) : nullptr;
  const char* Sb = packed ? reinterpret_cast<const char*>(p.pk_vsum + (size_t)bh * nbp * D) : nullptr;
  const char* Hb = first ? reinterpret_cast<const char*>(p.ht + (size_t)bh * nb * D * D) : nullptr;
  const char* Hbt = nhb ? reinterpret_cast<const char*>(p.pk_hbart + (size_t)bh * D * D) : nullptr;
  // copy chunk t into stage t & 1
  // copy chunk t into stage t & 1; returns an exact chunk's list entry (block id
  // and pair membership bits, wave-uniform), 0 otherwise
  auto issue = [&](int t, int raw = -1) {
    const unsigned m0 = lds_m0 + (unsigned)((t & 1) * C::STB);
    int entry = 0;
    if (t < nex) {
      const int u = t + ex0;                              // exact chunk u of the item
      entry = __builtin_amdgcn_readfirstlane(raw >= 0 ? raw : (int)s_list[u / SPB]);
      const int j = entry & kIdMask;
      const size_t off = ((size_t)j * BLK + (size_t)(u % SPB) * CK) * C::RB;
      dma_stage<C>(Kb + off, Vb + off, m0, ws, loff);
    } else if (t < ncen) {
      // stage-2 chunk t - nex: CK gathered rows of the compacted list
      dma_rows<C>(Cb, Sb, s_ulist + (t - nex) * CK, m0, ws, loff);
    } else if (t < nhbe) {
      // rows part * RP .. of Hbar^T (same layout as the H_j^T parts below)
      const char* g = Hbt + (size_t)(t - ncen) * C::RP * C::RB;
      dma_stage<C>(g, (2 * CK <= D) ? g + CK * C::RB : g, m0, ws, loff);
    } else {
      // rows part * RP .. of H_j^T; with RP = D < 2 CK the second half repeats them
      const int hc = t - nhbe;
      const int j = __builtin_amdgcn_readfirstlane((int)s_list[ncnt + hc / C::HP]);
      const char* g = Hb + ((size_t)j * D + (size_t)(hc % C::HP) * C::RP) * C::RB;
      dma_stage<C>(g, (2 * CK <= D) ? g + CK * C::RB : g, m0, ws, loff);
    }
    return entry;
  };
  // the list entry of the next chunk to compute: read once, when its copy is
  // issued, and carried to its step in a scalar register
  int entry = ntot > 0 ? issue(0) : 0;
  // the list entry of exact chunk 1, read ahead: step t reads chunk t + 2's entry
  // after its barrier, for the copy that step t + 1 issues
  int raw_next = (nex > 1) ? (int)(unsigned short)s_list[(1 + ex0) / SPB] : 0;
  // keys of exact chunk u inside the sequence (fewer only in a ragged last block)
  auto keys_of = [&](int u) {
    return VL ? min(max(block_count(Lv, (int)s_list[u / SPB] & kIdMask, BLK) - (u % SPB) * CK, 0), CK) : CK;
  };
  int t = 0;
  // stream chunk t sits in stage t & 1, passed as `stage`; it is exact chunk
  // u = t + ex0 of the item
  auto exact_step = [&](int t, char* stage) {
    const int cur = entry;
    wait_vm0();
    __syncthreads();
    if (t + 1 < ntot) entry = issue(t + 1, t + 1 < nex ? raw_next : -1);
    if (t + 2 < nex) raw_next = (int)(unsigned short)s_list[(t + 2 + ex0) / SPB];
    const int u = t + ex0;
    const int kv = keys_of(u);
    if (VL && kv < CK) {
      // padding values must not reach the MFMA (0 * NaN): zero those V rows
      char* vz = stage + C::SUBB;
      for (int e = tid; e < (CK - kv) * C::CPR; e += C::NT)
        st16(vz + (kv + e / C::CPR) * C::RB + 16 * (e % C::CPR), u32x4{0u, 0u, 0u, 0u});
      __syncthreads();
    }
    // pairs: only the waves of a query block that routes this block compute it
    const bool mine = QB == 1 || (alive && ((cur >> (12 + qb)) & 1));
    if (mine) chunk<C, false>(st, qf, stage, off, c2, hh, bits[qb], 0, kv);
  };
  // stage 1, two exact chunks per trip (t even), so each stage's offset is a
  // constant that folds into the LDS reads' immediate offsets
  for (; t + 1 < nex; t += 2) {
    exact_step(t, lds);
    exact_step(t + 1, lds + C::STB);
  }
  if (t < nex) exact_step(t++, lds);
  // stage 2: the ragged last block (if any) weighs its n_j tokens
  const int jrag = (VL && Lv % BLK != 0) ? nne - 1 : -1;
  const float wmiss = (float)(BLK - (Lv - jrag * BLK));
  const int prag = VL ? s_rag : -1;         // its position in the stage-2 list (-1: absent)
  for (; t < ncen; ++t) {                   // stage 2: centroid / value-sum chunks
    wait_vm0();
    __syncthreads();
    if (t + 1 < ntot) issue(t + 1);
    const int pos0 = (t - nex) * CK;
    const int jp = (VL && prag >= pos0 && prag < pos0 + CK) ? prag - pos0 : -1;
    if (alive) chunk<C, true>(st, qf, lds + (t & 1) * C::STB, off, c2, hh, s_umask[qb], pos0, CK, jp, wmiss);
  }
  if (FO) {
    for (; t < ntot; ++t) {                 // per-block first order: H_j^T parts
      wait_vm0();
      __syncthreads();
      if (t + 1 < ntot) issue(t + 1);
      const int hc = t - nhbe;
      const int j = (int)s_list[ncnt + hc / C::HP];
      first_order_part<C>(st, qf, lds + (t & 1) * C::STB, off, c2, scale,
                          p.pk_cen + ((size_t)bh * nbp + j) * D, hc % C::HP, hh);
    }
  }

  if (approx && tail) {
    if (!packed) {
      // ---- stage 2 from the fp32 statistics (converted while staging)
      const float* cen = p.centroid + (size_t)bh * nb * D;
      const float* vs = p.vsum + (size_t)bh * nb * D;
      const int nch = s_cnt[1];
      for (int pos0 = 0; pos0 < nch * CK; pos0 += CK) {
        __syncthreads();
        stage_centroids<C>(cen, vs, s_ulist + pos0, nb, lds, tid);
        __syncthreads();
        const int jp = (VL && prag >= pos0 && prag < pos0 + CK) ? prag - pos0 : -1;
        if (alive) chunk<C, true>(st, qf, lds, off, c2, hh, s_umask[qb], pos0, CK, jp, wmiss);
      }
    }
  }
  if (approx && tail && order == kOrderMixed) {
    // ---- stage 3: global first-order correction, acc += scale * (q Hbar) * sum alpha
    // (sum alpha is complete once stage 2 is done; m does not move from here on)
    // the query fragments are not read again: scale them by f in place
    scale_frags<C>(qf, scale * row_sum(st.a));
    if (packed) {
      // the Hbar^T parts (HP <= 2), streamed through the ring behind the
      // centroid chunks; each part owns compile-time accumulator tiles
      if (t < nhbe) {
        wait_vm0();
        __syncthreads();
        if (t + 1 < ntot) issue(t + 1);
        if (alive) hbar_part<C, 0>(st, qf, lds + (t & 1) * C::STB, off);
        ++t;
      }
      if constexpr (C::HP > 1) {
        if (t < nhbe) {
          wait_vm0();
          __syncthreads();
          if (t + 1 < ntot) issue(t + 1);
          if (alive) hbar_part<C, 1>(st, qf, lds + (t & 1) * C::STB, off);
          ++t;
        }
      }
    } else {
      __syncthreads();
      stage_hbar_t<C>(p.hbar + (size_t)bh * D * D, lds, lds + C::STB, tid);
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const char* base = (mt < C::MT / 2) ? lds + 32 * mt * C::RB : lds + C::STB + 32 * (mt - C::MT / 2) * C::RB;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) st.acc[mt] = mfma32(as_bf16x8(ld16(base + koff_of<C>(off, ks))), qf[ks], st.acc[mt]);
      }
    }
  }

  // ---- epilogue: o = N / D (0 when nothing was attended in keep-or-drop)
  const float ltot = row_sum(st.l);
  if constexpr (SP) {
    if (nparts > 1) {
      // an unnormalised partial state; the merge kernel forms o
      if (!qvalid) return;
      const int row = qb * BLK + 32 * wq + q32;
      float* slot = p.part + ((size_t)item * si.pmax + part) * split_slot_floats<C>();
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& a = st.acc[mt];
          *reinterpret_cast<f32x4*>(slot + (size_t)row * D + 32 * mt + 8 * g4 + 4 * hh) =
              f32x4{a[4 * g4], a[4 * g4 + 1], a[4 * g4 + 2], a[4 * g4 + 3]};
        }
      if (hh == 0) {
        slot[(size_t)QB * BLK * D + row] = st.m;
        slot[(size_t)QB * BLK * D + QB * BLK + row] = ltot;
      }
      return;
    }
  }
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (!qvalid) return;                                  // (odd nb: no second query block)
  const bool live = 32 * wq + q32 < ni;                 // padding query rows are written 0
  bf16* orow = p.O + ((size_t)bh * L + (size_t)i * BLK + 32 * wq + q32) * D;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x16& a = st.acc[mt];
      u32x2 pk = {pack2(a[4 * g4] * inv, a[4 * g4 + 1] * inv), pack2(a[4 * g4 + 2] * inv, a[4 * g4 + 3] * inv)};
      if (!live) pk = u32x2{0u, 0u};
      st8(orow + 32 * mt + 8 * g4 + 4 * hh, pk);
    }
}

// Split items: o = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over the
// item's parts (M = max_p m_p; the states of different parts are relative to
// their own running maxima), 0 where the weights sum to 0 (keep-or-drop with
// nothing attended) and for padding queries.  One workgroup per item; items
// that ran as one part were written by the attention kernel.
template <class C, bool VL>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ part,
                                                          const int* __restrict__ nparts, int pmax,
                                                          bf16* __restrict__ O, int nb,
                                                          const int32_t* __restrict__ lens, int heads) {
  constexpr int D = C::D, BLK = C::BLK, QB = C::QB, R = QB * BLK;
  constexpr size_t SF = split_slot_floats<C>();
  __shared__ float s_w[kSplitMaxParts][R];             // per part and row: 2^(m_p - M) / den
  const int item = blockIdx.x;
  const int np = nparts[item];
  if (np <= 1) return;
  const int ngrp = (nb + QB - 1) / QB;
  const int bh = item / ngrp, i0 = (item - bh * ngrp) * QB;
  const size_t L = (size_t)nb * BLK;
  const int Lv = VL ? valid_len(lens, bh, heads, (int)L) : (int)L;
  const float* base = part + (size_t)item * pmax * SF;
  // the rows' weights, once
  for (int row = threadIdx.x; row < R; row += 256) {
    const int q = row / BLK, tok = (i0 + q) * BLK + (row - q * BLK);
    float mx = -INFINITY;
    for (int pp = 0; pp < np; ++pp) mx = fmaxf(mx, base[pp * SF + (size_t)R * D + row]);
    float den = 0.f;
    for (int pp = 0; pp < np; ++pp) {
      const float wgt = fast_exp2(base[pp * SF + (size_t)R * D + row] - mx);
      s_w[pp][row] = wgt;
      den += wgt * base[pp * SF + (size_t)R * D + R + row];
    }
    const float inv = (i0 + q < nb && tok < Lv && den > 0.f) ? 1.f / den : 0.f;
    for (int pp = 0; pp < np; ++pp) s_w[pp][row] *= inv;
  }
  __syncthreads();
  // o = sum_p w_p acc_p, 16 bytes per thread and step, parts four loads at a time
  for (int e = threadIdx.x; e < R * D / 4; e += 256) {
    const int row = e / (D / 4), c = 4 * (e - row * (D / 4));
    const int q = row / BLK;
    if (i0 + q >= nb) continue;                         // (odd nb: no second query block)
    const float* a0 = base + (size_t)row * D + c;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    int pp = 0;
    for (; pp + 4 <= np; pp += 4) {
      f32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const f32x4*>(a0 + (pp + u) * SF);
#pragma unroll
      for (int u = 0; u < 4; ++u) num += s_w[pp + u][row] * x[u];
    }
    for (; pp < np; ++pp) num += s_w[pp][row] * *reinterpret_cast<const f32x4*>(a0 + pp * SF);
    const u32x2 pk = {pack2(num[0], num[1]), pack2(num[2], num[3])};
    st8(O + ((size_t)bh * L + (size_t)(i0 + q) * BLK + (row - q * BLK)) * D + c, pk);
  }
}

// In-kernel routing keeps the pooled queries and the score rows in the ring's
// LDS.
template <class C>
constexpr bool fused_route_fits(int nb) {
  const int ncol = (nb + 63) / 64 * 64;
  return nb <= kMaxBlocks &&
         (size_t)C::QB * (C::D * 8 + ncol * 8) <= (size_t)C::LDSB &&
         (size_t)C::QB * (C::D * 8 + C::WPQ * C::D * 8) <= (size_t)C::LDSB;
}

// FR_: this configuration also serves in-kernel routing (the ones the
// per-block first order alone uses do not)
// parts per split item and workspace bytes (nparts array, then the slots)
template <class C>
int split_pmax(int nb, int kmax, int cap) {
  const int most = min(nb, C::QB * kmax);               // exact blocks an item can hold
  return cap > 0 ? min(kSplitMaxParts, max(1, (most + cap - 1) / cap)) : 1;
}
template <class C>
size_t split_ws_bytes(int bh, int nb, int kmax, int cap) {
  const size_t items = (size_t)bh * ((nb + C::QB - 1) / C::QB);
  return (items * sizeof(int) + 255) / 256 * 256 +
         items * split_pmax<C>(nb, kmax, cap) * split_slot_floats<C>() * sizeof(float);
}

template <class C, bool FR_ = true>
hipError_t launch_t(const AttnArgs& a) {
  const int items = a.bh * ((a.nb + C::QB - 1) / C::QB);
  const int nbp = (a.nb + C::BLK - 1) / C::BLK * C::BLK;
  const bf16* pk = static_cast<const bf16*>(a.packed);
  AttnPtrs p{(const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, a.idx, a.centroid, a.vsum,
             a.hbar, pk, pk ? pk + (size_t)a.bh * nbp * C::D : nullptr,
             pk ? pk + (size_t)2 * a.bh * nbp * C::D : nullptr, (const bf16*)a.ht, (bf16*)a.O,
             a.M, a.idx_out, nullptr, nullptr};
  const RouteIn ri{a.route_k, a.route_scale, a.route_lam};
  const bool fo = a.approx && a.order == kOrderFirst;
  const bool fr = a.route_k > 0;
  const bool np = a.approx && pk == nullptr;           // approximate modes without the pack
  const bool vl = a.lens != nullptr;
  SplitIn si{0, 1, items};
  int grid = items;
  if (a.split_cap > 0) {
    if (fo || fr) return hipErrorInvalidValue;
    si = SplitIn{a.split_cap, split_pmax<C>(a.nb, a.kmax, a.split_cap), items};
    grid = (items + 7) / 8 * 8 * si.pmax;
    p.nparts = static_cast<int*>(a.split_ws);
    p.part = reinterpret_cast<float*>(static_cast<char*>(a.split_ws) +
                                      ((size_t)items * sizeof(int) + 255) / 256 * 256);
  }
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), 0, a.stream, p, a.kmax, a.approx, a.order,
                       a.scale, a.nb, a.lens, a.heads, ri, si);
    return hipGetLastError();
  };
  if (a.split_cap > 0) {
    if constexpr (!FR_) return hipErrorInvalidValue;   // (configurations of the per-block first order)
    hipError_t e;
    if (np) e = vl ? go(attn_bf16_kernel<C, true, false, false, true, true>) : go(attn_bf16_kernel<C, false, false, false, true, true>);
    else e = vl ? go(attn_bf16_kernel<C, true, false, false, false, true>) : go(attn_bf16_kernel<C, false, false, false, false, true>);
    if (e != hipSuccess || si.pmax == 1) return e;
    auto merge = vl ? split_merge_kernel<C, true> : split_merge_kernel<C, false>;
    hipLaunchKernelGGL(merge, dim3(items), dim3(256), 0, a.stream, (const float*)p.part,
                       (const int*)p.nparts, si.pmax, (bf16*)a.O, a.nb, a.lens, a.heads);
    return hipGetLastError();
  }
  if (fr) {
    if constexpr (FR_) {
      if (fo || !fused_route_fits<C>(a.nb)) return hipErrorInvalidValue;
      if (np) return vl ? go(attn_bf16_kernel<C, true, false, true, true>) : go(attn_bf16_kernel<C, false, false, true, true>);
      return vl ? go(attn_bf16_kernel<C, true, false, true>) : go(attn_bf16_kernel<C, false, false, true>);
    } else {
      return hipErrorInvalidValue;
    }
  } else if constexpr (C::QB == 1) {
    if (fo) {
      if (np) return hipErrorInvalidValue;      // the per-block first order needs the pack
      return vl ? go(attn_bf16_kernel<C, true, true>) : go(attn_bf16_kernel<C, false, true>);
    }
    if (np) return vl ? go(attn_bf16_kernel<C, true, false, false, true>) : go(attn_bf16_kernel<C, false, false, false, true>);
    return vl ? go(attn_bf16_kernel<C, true, false>) : go(attn_bf16_kernel<C, false, false>);
  } else {
    if (fo) return hipErrorInvalidValue;        // the launcher sends this order to QB = 1
    if (np) return vl ? go(attn_bf16_kernel<C, true, false, false, true>) : go(attn_bf16_kernel<C, false, false, false, true>);
    return vl ? go(attn_bf16_kernel<C, true, false>) : go(attn_bf16_kernel<C, false, false>);
  }
}

}  // namespace

int fused_route_max_blocks(int D, int BLK) {
  int best = 0;
  for (int nb = 1; nb <= kMaxBlocks; ++nb) {
    bool ok = false;
    if (D == 128 && BLK == 64) ok = fused_route_fits<Cfg<128, 64, 32, 2>>(nb);
    if (D == 128 && BLK == 128) ok = fused_route_fits<Cfg<128, 128, 32>>(nb);
    if (D == 64 && BLK == 64) ok = fused_route_fits<Cfg<64, 64, 32, 2>>(nb);
    if (D == 64 && BLK == 128) ok = fused_route_fits<Cfg<64, 128, 64>>(nb);
    if (ok) best = nb;
  }
  return best;
}

namespace {
int fused_route_resident_query(int D, int BLK);

template <class C>
int resident_of(const void* kern) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, C::NT, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per_cu * cus;
}
}  // namespace

int fused_route_items(int D, int BLK, int bh, int nb) {
  const int qb = (BLK == 64) ? 2 : 1;                   // query blocks per workgroup (see launch_attn_bf16)
  (void)D;
  return bh * ((nb + qb - 1) / qb);
}

int fused_route_resident(int D, int BLK) {
  // answered once per device and configuration (the occupancy of a kernel
  // on a device does not change)
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][4];
  const int cfg = (D == 128 ? 0 : 2) + (BLK == 64 ? 0 : 1);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kDevs) {
    const int c = cache[dev][cfg].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  const int r = fused_route_resident_query(D, BLK);
  if (r > 0 && dev >= 0 && dev < kDevs) cache[dev][cfg].store(r, std::memory_order_relaxed);
  return r;
}

namespace {
int fused_route_resident_query(int D, int BLK) {
  // the in-kernel routing instantiations launch_t picks (without valid lengths
  // and with the bf16 pack; the others hold as many workgroups per CU)
  if (D == 128 && BLK == 64)
    return resident_of<Cfg<128, 64, 32, 2>>((const void*)attn_bf16_kernel<Cfg<128, 64, 32, 2>, false, false, true>);
  if (D == 128 && BLK == 128)
    return resident_of<Cfg<128, 128, 32>>((const void*)attn_bf16_kernel<Cfg<128, 128, 32>, false, false, true>);
  if (D == 64 && BLK == 64)
    return resident_of<Cfg<64, 64, 32, 2>>((const void*)attn_bf16_kernel<Cfg<64, 64, 32, 2>, false, false, true>);
  if (D == 64 && BLK == 128)
    return resident_of<Cfg<64, 128, 64>>((const void*)attn_bf16_kernel<Cfg<64, 128, 64>, false, false, true>);
  return 0;
}
}  // namespace

size_t attn_split_workspace(int D, int BLK, int bh, int nb, int kmax, int cap) {
  // the configurations launch_attn_bf16 picks for the orders other than the per-block first
  if (D == 128 && BLK == 64) return split_ws_bytes<Cfg<128, 64, 32, 2>>(bh, nb, kmax, cap);
  if (D == 128 && BLK == 128) return split_ws_bytes<Cfg<128, 128, 32>>(bh, nb, kmax, cap);
  if (D == 64 && BLK == 64) return split_ws_bytes<Cfg<64, 64, 32, 2>>(bh, nb, kmax, cap);
  if (D == 64 && BLK == 128) return split_ws_bytes<Cfg<64, 128, 64>>(bh, nb, kmax, cap);
  return 0;
}

hipError_t launch_attn_bf16(const AttnArgs& a) {
  // 64-token blocks: query blocks in pairs, except for the per-block first order
  const bool fo = a.approx && a.order == kOrderFirst;
  if (a.D == 128 && a.BLK == 64)
    return fo ? launch_t<Cfg<128, 64, 32>, false>(a) : launch_t<Cfg<128, 64, 32, 2>>(a);
  if (a.D == 128 && a.BLK == 128) {
    // the per-block first order streams whole 128-row H_j^T matrices: 64-key chunks
    if (fo) return launch_t<Cfg<128, 128, 64>, false>(a);
    return launch_t<Cfg<128, 128, 32>>(a);
  }
  if (a.D == 64 && a.BLK == 64)
    return fo ? launch_t<Cfg<64, 64, 32>, false>(a) : launch_t<Cfg<64, 64, 32, 2>>(a);
  if (a.D == 64 && a.BLK == 128) return launch_t<Cfg<64, 128, 64>>(a);
  return hipErrorInvalidValue;
}

}  // namespace pisa

// Forward of alpha-entmax attention: a histogram kernel and a refinement/output kernel.
//
// Stages (AdaSplash-2 pages, AdaSplash-2 (zh) §2, AdaSplash-2 (ja) §2, AdaSplash-2 (es) §2):
//   1. k_hist -- histogram pass: every valid key block streams through once; each lane
//      keeps an online max and a B-bin histogram of its scores on the anchored grid
//      (bins [m/B, (m+1)/B), window = the B cells ending with the max's cell); a window
//      that slides up drops the cells that fall off. tau_h, the root of the B-bin
//      problem (counts at lower bin edges), satisfies tau* - 1/B < tau_h <= tau*
//      (Proposition 1). The same pass marks the 32-key sub-blocks that hold a score at
//      most two bins below the running window (every score that can exceed the
//      bracket's lower end lies in one of them) and records each marked sub-block's
//      largest score per 32-row chunk.
//   2. k_refine_out -- refinement passes: a safeguarded hybrid root solver on
//      f(tau) = sum_j [x_j - tau]_+^kappa - 1 in the bracket [tau_h, tau_h + 1/B]:
//      Halley (alpha <= 1.5), Newton (1.5 < alpha <= 2), secant (alpha > 2, started by
//      false position on the bracket ends), bisection whenever a step leaves the bracket
//      (AdaSplash-2 (zh) §2.2, AdaSplash-2 (ja) §2.2). Each pass visits only the marked
//      sub-blocks whose recorded maximum exceeds the evaluation point. Then the output
//      pass: p = [x - tau]_+^kappa, o = P V, o~ = G V / sum G with g = [x - tau]_+^(kappa-1),
//      and the exact block mask (bit-packed, 32 blocks per word; AdaSplash-2 (zh) §2.3).
//
// MI355X decomposition. Scores are computed transposed (keys x queries) on 32x32 MFMA
// tiles so that a lane owns one query (two lanes per query, 16 keys each per tile): the
// histogram of a query is private to its lane (its own LDS column, no contention), and
// P and G come out already in the B-operand layout of the PV product. K and V are read
// from fragment-major copies, so each operand load of a wave is one contiguous run.
// The histogram kernel streams K for 256 query rows that share one KV head (8 waves) and
// keeps its register count low enough for four waves per SIMD, so one wave's MFMA latency
// hides under the others' VALU work; the refinement/output kernel has a data-dependent
// cost per wave and runs in small work groups of 4 waves for balance. When the score
// scale (alpha-1) * scale is a power of two it is folded into Q (exact), and the offset
// each pass subtracts from the scores (the histogram window base, or tau) enters the
// score product as its initial accumulator.
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "solver.hpp"

namespace entmax {


// Waves per histogram work group and the waves per SIMD the register budget allows: eight
// 32-row waves at head_dim 64 (four per SIMD in bf16, 128 registers); four at head_dim 128
// in bf16, where a wave needs more than 128 registers, so that three groups (three waves per
// SIMD) share a CU instead of one eight-wave group.
template <typename T, int D>
constexpr int hist_waves() { return (D == 128 && sizeof(T) == 2) ? 4 : (D == 64 && sizeof(T) == 2) ? ENTMAX_HIST_WAVES64 : 8; }
template <typename T, int D>
constexpr int hist_occ() { return (D == 64 && sizeof(T) == 2) ? ENTMAX_HIST_OCC64 : (D == 128 && sizeof(T) == 2) ? 3 : 2; }
// Histogram cells per wave in LDS: 18 rows of 64 lane columns (4608 B), enough for the
// B + 2 cells of every supported B (B <= 16); the row of a cell is the second byte of its
// LDS address, so the wave's histogram lies at a fixed multiple of 4608 B.
constexpr int HIST_ROWS = 18;
constexpr uint32_t HIST_WAVE_BYTES = HIST_ROWS * 64 * 4;

// Count 16 scores of a tile: cell = trunc(y) saturated at 0 goes straight into the second byte
// of the lane's address register (an SDWA conversion that keeps the other bytes: lane * 4 in
// the first byte, zero above), and the wave's histogram offset is the instruction's immediate.
// One conversion and one LDS add per score; cells of any y in [0, 18) stay inside the wave's
// rows, y < 1 (and NaN) lands in the discard cell 0.
// Four address registers (all lane * 4 in the first byte) take the conversions in turn, so
// four conversions go out back to back before their four adds instead of one conversion
// waiting for the previous add's address.
struct CountRegs {
  uint32_t a0, a1, a2, a3;
};
template <uint32_t OFF>
__device__ __forceinline__ void count16(const f32x16& a, CountRegs& r, uint32_t one) {
#define ENTMAX_CV(d, i) "v_cvt_u32_f32_sdwa %" #d ", %" #i " dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD\n"
#define ENTMAX_AD(d) "ds_add_u32 %" #d ", %4 offset:%21\n"
#define ENTMAX_Q(i0, i1, i2, i3) ENTMAX_CV(0, i0) ENTMAX_CV(1, i1) ENTMAX_CV(2, i2) ENTMAX_CV(3, i3) \
                                 ENTMAX_AD(0) ENTMAX_AD(1) ENTMAX_AD(2) ENTMAX_AD(3)
  asm volatile(ENTMAX_Q(5, 6, 7, 8) ENTMAX_Q(9, 10, 11, 12) ENTMAX_Q(13, 14, 15, 16) ENTMAX_Q(17, 18, 19, 20)
               : "+v"(r.a0), "+v"(r.a1), "+v"(r.a2), "+v"(r.a3)
               : "v"(one), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
                 "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
                 "v"(a[14]), "v"(a[15]), "i"(OFF)
               : "memory");
#undef ENTMAX_Q
#undef ENTMAX_AD
#undef ENTMAX_CV
}
// both tiles of a step into the histogram of wave w (w < HW)
template <int HW>
__device__ __forceinline__ void count_pair(int w, const f32x16& a0, const f32x16& a1, CountRegs& ad, uint32_t one) {
#define ENTMAX_CASE(k)                                      \
  case k:                                                   \
    if constexpr (k < HW) {                                 \
      count16<k * HIST_WAVE_BYTES>(a0, ad, one);            \
      count16<k * HIST_WAVE_BYTES>(a1, ad, one);            \
    }                                                       \
    break;
  switch (w) { ENTMAX_CASE(0) ENTMAX_CASE(1) ENTMAX_CASE(2) ENTMAX_CASE(3)
               ENTMAX_CASE(4) ENTMAX_CASE(5) ENTMAX_CASE(6) ENTMAX_CASE(7) }
#undef ENTMAX_CASE
}

constexpr int ALPHA2_POINTS = 2;   // evaluation points per refinement pass at alpha = 2 (2 beat 3 and 4)
constexpr int OUT_WAVES = 4;

// ================================================================================ k_hist
template <typename T, int D, int MODE, bool QS, bool BIAS>
__global__ __launch_bounds__((64 * hist_waves<T, D>()), (hist_occ<T, D>())) void k_hist(FwdParams p) {
  using Ops = KvOps<T, D>;
  constexpr int DS = Ops::DS;
  extern __shared__ uint32_t lds[];
  int unit, rank;
  if (!wgmap_get(p.map, blockIdx.x, unit, rank)) return;   // whole work group

  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int nsub = p.G / p.GP;
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int rg = p.causal ? (p.RG - 1 - rank / nsub) : (rank / nsub);
  const int gsub = rank % nsub;
  constexpr int HW = hist_waves<T, D>();
  const int per = HW / p.GP;                   // waves per head
  const int head = kvh * p.G + gsub * p.GP + w / per;
  const int row0 = rg * p.RH + (w % per) * 32; // this wave's 32 rows
  const int n = p.n, B = p.B;                  // histogram window of B cells + 2 trash cells per lane
  const bool valid_rows = row0 < n;
  const int qrow = row0 + c;
  const size_t bh = (size_t)(bi * p.hq + head);

  const T* Q = reinterpret_cast<const T*>(p.q) + bh * n * D;
  const T* Kf = reinterpret_cast<const T*>(p.kf) + ((size_t)(bi * p.hkv + kvh) * n) * D;
  // position bias of this head on the x*B scale: x*B gains -cmB |i - j|
  const float cmB = BIAS ? p.slopes[head] * (p.alpha - 1.0f) * (float)B : 0.0f;
  static_assert(HW <= 8, "histogram offsets are written for at most eight waves");
  uint32_t* hist = lds + w * (HIST_ROWS * 64);  // [B + 2][64] of this wave (in an 18-row slot)
  for (int i = lane; i < (B + 2) * 64; i += 64) hist[i] = 0;
  float* dmx = p.dmax + dmax_row(p, bh, row0 >> 5);
  float* wx_out = p.wmax + (bh * p.nkb + (row0 >> 5)) * p.NW32;

  // clear the block-mask words of this work group's tiles (k_refine_out ORs bits in)
  {
    const int tiles_per_head = p.RH / p.Br;
    const int total = p.GP * tiles_per_head * p.W;
    for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
      const int wi = idx % p.W, t = (idx / p.W) % tiles_per_head, hs = idx / (p.W * tiles_per_head);
      const int trow0 = rg * p.RH + t * p.Br;
      if (trow0 >= n) continue;
      const int hg = kvh * p.G + gsub * p.GP + hs;
      p.mask[((size_t)(bi * p.hq + hg) * p.Tr + trow0 / p.Br) * p.W + wi] = 0u;
    }
  }
  if (!valid_rows) return;                     // no barrier follows: the wave may leave
  const int kb_end = p.causal ? min(p.nkb, (row0 + 31) / 32 + 1) : p.nkb;

  Frag<T> qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) load_frag(qf[s], Q + (size_t)qrow * D + 16 * s + 8 * h);
  // x * B = cB * s exactly (B is a power of two). When cB is itself a power of two it is
  // folded into Q (exact scaling), and the score tile is x * B directly. Either way a tile
  // is held as x * B - base (base: the window's offset below).
  const float cB = QS ? 1.0f : p.cx * (float)B;
  if constexpr (QS) {
    const float qsc = p.cx * (float)B;
#pragma unroll
    for (int s = 0; s < DS; ++s) scale_frag(qf[s], qsc);
  }

  // Window of a lane: bins Tt-B+1 .. Tt of its running max cell Tt, held in cells 1..B
  // (cell j <-> bin base + j with base = Tt - B); cell 0 takes every lower score, and
  // cell B+1 the lane's max when rounding of x*B - base lands exactly on B+1. A score's
  // cell is cvt_u32(x*B - base): the conversion saturates negative values to 0.
  // With the scale folded into Q the offset -base enters the score product as its
  // initial accumulator, so a score costs a conversion, an address and an LDS add.
  //
  // Two sub-blocks per step: both tiles update the running max first, then all their
  // scores are counted against the updated window. This is exact: a score that would
  // have been counted under the older window but lies below the newer one is exactly a
  // score the window slide would drop later.
  float mB = -INFINITY;   // running max of x*B over this lane's scores
  int Tt = 0;             // its cell floor(mB): top of the lane's window
  int base = -B;          // Tt - B
  bool have = false;
  f32x16 negb;            // -base in every register (initial accumulator)
#pragma unroll
  for (int r = 0; r < 16; ++r) negb[r] = (float)B;
  float dreg = -INFINITY; // lane j < 32 keeps the chunk max of sub-block 32*word + j
  unsigned long long n_cand = 0;

  Frag<T> kf[DS], kf2[DS];
  // Sub-blocks go by aligned pairs (2m, 2m + 1) from the last pair down to the first: under
  // the causal mask the keys next to the diagonal come first, so with a position bias (and
  // in any recency-weighted data) the running max settles early and the far, lower tiles
  // find the window already in place (fewer slides, fewer active tiles).
  const int last_pair = (kb_end - 1) >> 1;
  // K fragments through a buffer resource: a fixed lane offset and a scalar sub-block offset
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kf, (uint32_t)((size_t)n * D * sizeof(T)));
  Ops::load_k_buf(kf, krs, 2 * last_pair, lane);
  Ops::load_k_buf(kf2, krs, min(2 * last_pair + 1, kb_end - 1), lane);
  // x * B - base of sub-block kbb (with the head's position bias). Keys after the query
  // under the causal mask are -inf, and so are keys past the last one without it (the
  // second tile of the last pair when the sub-block count is odd). At head_dim 64 the score
  // products mask keys above the row limit ml on the tiles that reach past it (one rule, no
  // branch per step); at head_dim 128 the limit's register would spill, so they mask the
  // causal keys and the loop sets a tile past the last key to -inf.
  constexpr bool UM = D == 64;
  const int ml = UM ? (p.causal ? qrow : n - 1) : qrow, ml0 = UM ? (p.causal ? row0 : n - 1) : row0;
  const bool mc = UM || p.causal;
  auto tile = [&](const Frag<T> (&kc)[DS], int kbb) -> f32x16 {
    if constexpr (BIAS) {
      const float d0 = (float)(qrow - 32 * kbb - 4 * h);
      if constexpr (QS)
        return Ops::scores(kc, qf, kbb, ml0, ml, h, mc, bias16<-1>(-(float)base, cmB, d0, p.causal));
      f32x16 a = Ops::scores(kc, qf, kbb, ml0, ml, h, mc);
      scale_add_bias16<-1>(a, cB, -(float)base, cmB, d0, p.causal);
      return a;
    } else {
      if constexpr (QS) return Ops::scores(kc, qf, kbb, ml0, ml, h, mc, negb);
      f32x16 a = Ops::scores(kc, qf, kbb, ml0, ml, h, mc);
      const float nb = -(float)base;
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = fmaf(cB, a[r], nb);
      return a;
    }
  };
  const uint32_t l4 = 4u * (uint32_t)lane;
  CountRegs cad{l4, l4, l4, l4};              // LDS addresses of counts: cell in the second byte
  const uint32_t one = 1u;
  for (int kb = 2 * last_pair; kb >= 0; kb -= 2) {
    // The second tile of the last pair may lie past the last valid sub-block: every one of its
    // keys is then masked to -inf, and its loads past the end of K read zeros through the
    // buffer bounds.
    f32x16 acc0 = tile(kf, kb);
    f32x16 acc1 = tile(kf2, kb + 1);
    if constexpr (!UM) {
      if (kb + 1 >= kb_end) {
        asm volatile("" ::: "memory");   // a branch taken once per wave at most: keep it one
#pragma unroll
        for (int r = 0; r < 16; ++r) acc1[r] = -INFINITY;
      }
    }
    // the next pair (every pair below the last one is whole); loaded on every step, the
    // first pair again at the end, so the waits at the next step count a fixed number of loads
    Ops::load_k_buf(kf, krs, max(kb - 2, 0), lane);
    Ops::load_k_buf(kf2, krs, max(kb - 1, 0), lane);
    const float bF = (float)base;
    const float t0 = max16(acc0) + bF;   // largest x*B of each tile
    const float t1 = max16(acc1) + bF;
    const float nmB = fmaxf(mB, fmaxf(t0, t1));
    const bool fin = nmB > -INFINITY;
    const int Tfl = cvt_floor(nmB);
    const int Tn = fin ? Tfl : Tt;
    // a tile is active for a lane when one of its scores lies at most two bins below
    // the lane's window
    const float thrB = (float)(Tn - B - 1);
    const bool act0 = fin && t0 >= thrB;
    const bool act1 = fin && t1 >= thrB;
    const uint64_t b0 = ballot(act0), b1 = ballot(act1);
    if ((b0 | b1) != 0) {
      // largest x*B of the 32 rows in each sub-block, kept by lane (sub-block mod 32)
      float cm0, cm1;
      pair_max_dpp(t0, t1, cm0, cm1);
      if (b0) write_lane(dreg, cm0, kb & 31);
      if (b1) write_lane(dreg, cm1, (kb + 1) & 31);
      const bool act = act0 || act1;
      // slide a window up: cell k takes cell k + shift, the top cells start empty
      const bool slide = act && (!have || Tn > Tt) && p.tau_init == 0;
      if (ballot(slide) != 0) {
        const int shift = slide ? (have ? Tn - Tt : B + 1) : 0;
        for (int k = 1; k <= B; ++k) {
          if (slide) {
            const int from = k + shift;
            hist[k * 64 + lane] = from <= B ? hist[from * 64 + lane] : 0u;
          }
        }
        const int nbase = slide ? Tn - B : base;
        const float corr = (float)(nbase - base);  // small integers
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc0[r] -= corr;
          acc1[r] -= corr;
          negb[r] = (float)(-nbase);
        }
        base = nbase;
      }
      if (act) {
        mB = nmB;
        Tt = Tn;
        have = true;
      }
      // count every score of both tiles (lanes with no active tile land in cell 0)
      if (p.tau_init == 0) count_pair<HW>(w, acc0, acc1, cad, one);
    }
    // flush a finished word of chunk maxima and its own maximum (-inf: no candidate in the
    // word; pairs never straddle a word, which is complete once its lowest sub-block,
    // kb == 0 mod 32, is done)
    if ((kb & 31) == 0) {
      float wm, wm_hi;
      pair_max_dpp(dreg, dreg, wm, wm_hi);   // lanes 32..63 of dreg stay -inf
      if (lane == 0) wx_out[kb >> 5] = wm;
      if (p.stats) n_cand += __builtin_popcountll(ballot(dreg != -INFINITY));   // a candidate's maximum is finite
      if (lane < 32 && kb + lane < kb_end) dmx[kb + lane] = dreg;
      dreg = -INFINITY;
    }
  }

  // merge the two half-wave histograms of each query and solve the B-bin problem
  const int To = xor32i(Tt);
  const bool ho = xor32i(have ? 1 : 0) != 0;
  const int Tf = (have && ho) ? max(Tt, To) : (have ? Tt : To);
  int cnt[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int mine = 0;
    if (k < B) {
      const int bin = Tf - B + 1 + k;
      if (have && bin >= Tt - B + 1 && bin <= Tt) mine = (int)hist[(bin - base) * 64 + lane];
    }
    cnt[k] = mine + xor32i(mine);
  }
  // the refinement gets tau_h and the row max; in bracket mode it starts from the row max
  // alone, the test output tau_h is then its lower end x_max - 1 and the counts are 0
  const float xmax = fmaxf(mB, xor32f(mB)) / (float)B;
  const float tau_h = p.tau_init == 0 ? tau_from_counts<MODE>(cnt, Tf, B, p.kappa) : xmax - 1.0f;
  if (h == 0) {
    const size_t row = bh * n + qrow;
    float start = tau_h;   // alpha = 1.5: the spread-count root (other alpha start from tau_h itself)
    if constexpr (MODE == 2)
      if (p.tau_init == 0) start = tau_spread_start(cnt, Tf, B, tau_h);
    p.tauh_ws[row] = make_float4(tau_h, xmax, start, 0.0f);
    if (p.tau_h) p.tau_h[row] = tau_h;
    if (p.hist) {
      int32_t* dst = p.hist + row * B;
      for (int k = 0; k < 16; ++k)
        if (k < B) dst[k] = p.tau_init == 0 ? cnt[k] : 0;
    }
  }
  if (p.stats && lane == 0) {
    atomicAdd(&p.stats[20], (unsigned long long)kb_end);
    atomicAdd(&p.stats[23], n_cand);
  }
}

// ================================================================================ k_refine_out
// Work groups of OUT_WAVES waves over consecutive 32-row chunks of one query head, one
// chunk per wave; a wave's cost depends on its rows' candidates and passes, so small
// groups keep the machine balanced.
template <typename T, int D, int MODE, bool QS, bool BIAS>
__global__ __launch_bounds__(64 * OUT_WAVES, 2) void k_refine_out(FwdParams p) {
  using Ops = KvOps<T, D>;
  constexpr int DS = Ops::DS, DC = Ops::DC;
  int unit, rank;
  if (!wgmap_get(p.map2, blockIdx.x, unit, rank)) return;   // whole work group
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int head = kvh * p.G + rank % p.G;
  const int ngrp = (p.nkb + OUT_WAVES - 1) / OUT_WAVES;
  const int grp = p.causal ? (ngrp - 1 - rank / p.G) : (rank / p.G);
  const int chunk = grp * OUT_WAVES + w;
  if (chunk >= p.nkb) return;            // no barrier follows: the wave may leave
  const int row0 = chunk * 32;
  const int n = p.n, B = p.B;
  const int qrow = row0 + c;
  const size_t bh = (size_t)(bi * p.hq + head);
  const int kb_end = p.causal ? min(p.nkb, (row0 + 31) / 32 + 1) : p.nkb;
  const int nwords = (kb_end + 31) >> 5;

  const T* Q = reinterpret_cast<const T*>(p.q) + bh * n * D;
  const T* Kf = reinterpret_cast<const T*>(p.kf) + ((size_t)(bi * p.hkv + kvh) * n) * D;
  const T* Vf = reinterpret_cast<const T*>(p.vf) + ((size_t)(bi * p.hkv + kvh) * n) * D;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kf, (uint32_t)((size_t)n * D * sizeof(T)));
  const float* dmx = p.dmax + dmax_row(p, bh, chunk);
  const float* wmx = p.wmax + (bh * p.nkb + chunk) * p.NW32;

  Frag<T> qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) load_frag(qf[s], Q + (size_t)qrow * D + 16 * s + 8 * h);
  // with QS the score scale is a power of two folded into Q (exact) and -tau enters the
  // score product as its initial accumulator, so the tile holds x - tau directly
  if constexpr (QS) {
#pragma unroll
    for (int s = 0; s < DS; ++s) scale_frag(qf[s], p.cx);
  }
  const float cx = p.cx;
  // solver state: the bracket from tau_h (or the plain bracket below the row max)
  const float nv = p.causal ? (float)(qrow + 1) : (float)n;
  // (alpha = 2: several evaluation points per pass, see MultiState)
  using State = std::conditional_t<MODE == 1, MultiState<ALPHA2_POINTS>, RowState>;
  const float4 hm = p.tauh_ws[bh * n + qrow];   // (tau_h, x_max, start)
  State st;
  if (p.tau_init != 0) st = State::from_max(hm.y, nv, p.alpha);
  else if constexpr (MODE == 0) st = State::from_hist_bounded(hm.x, B, hm.y, nv, p.alpha);
  else if constexpr (MODE == 2) st = State::from_hist_at(hm.x, B, hm.z);
  else st = State::from_hist(hm.x, B);
  float& tau = st.tau;

  // The chunk's sub-block maxima and word maxima are staged once in this wave's part of LDS
  // (sub-block maxima as bf16 rounded up, so a walk never skips a sub-block it needs), so the
  // walks below read them from LDS: reads of the maxima from global memory would share the
  // vector-memory wait counter with the K fragments in flight, and every wait for a maximum
  // would also wait for the prefetched K.
  extern __shared__ __align__(16) uint8_t out_lds[];
  uint16_t* const ldmax = reinterpret_cast<uint16_t*>(out_lds + (size_t)w * p.out_lds_wave);
  float* const lwmax = reinterpret_cast<float*>(out_lds + (size_t)w * p.out_lds_wave + p.out_lds_wmax);
  if (!p.dense) {
    for (int i = lane; i < kb_end; i += 64) {
      const uint32_t bits = __float_as_uint(dmx[i]);
      // bf16 rounded towards +inf: truncation raises a negative value; a positive value with
      // dropped bits goes one step up (-inf and +inf stay)
      const uint32_t up = ((bits >> 31) == 0 && (bits & 0xFFFFu) != 0) ? 1u : 0u;
      ldmax[i] = (uint16_t)((bits >> 16) + up);
    }
    for (int i = lane; i < nwords; i += 64) lwmax[i] = wmx[i];
    // (only this wave reads its part, and a wave's LDS accesses complete in order)
    __builtin_amdgcn_wave_barrier();
  }
  // Walk over the sub-blocks a pass needs: those whose recorded chunk maximum exceeds the
  // threshold (non-candidates hold -inf). Words of 32 sub-blocks are screened 64 at a time
  // through their maxima (one LDS read per lane), so a pass reads the chunk maxima of the
  // words it needs only.
  struct Walk {
    int g;          // group of 64 words being walked
    uint64_t nm;    // its needed words not yet started
    int wi;         // current word
    uint32_t word;  // its needed sub-blocks not yet taken
  };
  auto walk_next = [&](Walk& wk, float thr) -> int {
    if (p.dense) return ++wk.wi < kb_end ? wk.wi : -1;   // ablation: every valid sub-block
    while (wk.word == 0) {
      while (wk.nm == 0) {
        if (64 * (++wk.g) >= nwords) return -1;
        const int wl = 64 * wk.g + lane;
        const float wm = wl < nwords ? lwmax[wl] : -INFINITY;
        wk.nm = ballot(wm > thr);
      }
      wk.wi = 64 * wk.g + __builtin_ctzll(wk.nm);
      wk.nm &= wk.nm - 1;
      const int kbl = wk.wi * 32 + (lane & 31);
      const float dv = kbl < kb_end ? __uint_as_float((uint32_t)ldmax[kbl] << 16) : -INFINITY;
      wk.word = (uint32_t)ballot(dv > thr);
    }
    const int kb = wk.wi * 32 + __builtin_ctz(wk.word);
    wk.word &= wk.word - 1;
    return kb;
  };
  f32x16 negt;
  // position bias of this head on the x-scale: x gains -cm |i - j|
  const float cm = BIAS ? p.slopes[head] * (p.alpha - 1.0f) : 0.0f;
  auto tile = [&](const Frag<T> (&kc)[DS], int kb) -> f32x16 {   // x - tau; -inf if masked
    if constexpr (BIAS) {
      const float d0 = (float)(qrow - 32 * kb - 4 * h);
      if constexpr (QS)
        return Ops::scores(kc, qf, kb, row0, qrow, h, p.causal, bias16<-1>(-tau, cm, d0, p.causal));
      f32x16 acc = Ops::scores(kc, qf, kb, row0, qrow, h, p.causal);
      scale_add_bias16<-1>(acc, cx, -tau, cm, d0, p.causal);
      return acc;
    } else if constexpr (QS) {
      return Ops::scores(kc, qf, kb, row0, qrow, h, p.causal, negt);
    } else {
      f32x16 acc = Ops::scores(kc, qf, kb, row0, qrow, h, p.causal);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = fmaf(cx, acc[r], -tau);
      return acc;
    }
  };

  // ---------------------------------------------------------------- refinement passes
  // per-row sums: v0 = sum d^kappa, v1 = sum d^(kappa-1), v2 = support size (alpha 1.5, 2)
  // or sum d^(kappa-2), v3 = sum (x - hi)_+^kappa (secant start), v4 = smallest positive
  // gap x - tau (alpha 1.5, 2)
  const float kappa = p.kappa, alpha = p.alpha;
  const bool secant = alpha > 2.0f;
  int npass = 0;
  unsigned long long n_ref = 0;
  Frag<T> kf[DS], kf1[DS], kf2[DS];
  while (npass < p.max_iters) {
    if (ballot(!st.done) == 0) break;
    const bool first = (npass == 0);
    const float thr = wave_min(st.done ? INFINITY : tau) * (float)B;
#pragma unroll
    for (int r = 0; r < 16; ++r) negt[r] = -tau;
    PassSums sums;
    MultiSums<ALPHA2_POINTS> msums;
    const float thi = st.hi - st.tau;    // secant start: f at the bracket's upper end
    Walk wk{-1, 0ull, -1, 0u};
    // a visit: the scores of sub-block kbv against this pass's evaluation points
    auto visit = [&](const Frag<T> (&kc)[DS], int kbv) {
      ++n_ref;
      const f32x16 t = tile(kc, kbv);
      if constexpr (MODE == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) msums.add(t[r], st.off);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sums.add<MODE>(t[r], thi, secant && first, kappa);
      }
    };
    // The K fragments of the next KPF sub-blocks are in flight while one is scored (a visit
    // is short next to the latency of a load from beyond the L2). Three register slots used
    // in turn, the loop unrolled by three so that no fragment is moved between slots.
    // Every stage issues its load (sub-block 0 stands in once the walk has ended), so each
    // slot's fragments are a fixed number of loads behind the newest and the compiler's wait
    // before a visit covers that slot only.
    int kb0 = walk_next(wk, thr);
    int kb1 = kb0 >= 0 ? walk_next(wk, thr) : -1;
    Ops::load_k_buf(kf, krs, max(kb0, 0), lane);
    Ops::load_k_buf(kf1, krs, max(kb1, 0), lane);
    while (kb0 >= 0) {
      int kb2 = kb1 >= 0 ? walk_next(wk, thr) : -1;
      Ops::load_k_buf(kf2, krs, max(kb2, 0), lane);
      visit(kf, kb0);
      if (kb1 < 0) break;
      kb0 = kb2 >= 0 ? walk_next(wk, thr) : -1;
      Ops::load_k_buf(kf, krs, max(kb0, 0), lane);
      visit(kf1, kb1);
      if (kb2 < 0) break;
      kb1 = kb0 >= 0 ? walk_next(wk, thr) : -1;
      Ops::load_k_buf(kf1, krs, max(kb1, 0), lane);
      visit(kf2, kb2);
    }
    ++npass;
    if constexpr (MODE == 1) {
      float Ft[ALPHA2_POINTS];
      int Nt[ALPHA2_POINTS];
#pragma unroll
      for (int k = 0; k < ALPHA2_POINTS; ++k) {
        Ft[k] = msums.F[k] + xor32f(msums.F[k]);
        Nt[k] = msums.N[k] + xor32i(msums.N[k]);
      }
      if (!st.done) st.update(Ft, Nt, npass, p.tol);
    } else {
      // combine the two half-lanes of a row
      float tot[5];
      tot[0] = sums.F0 + xor32f(sums.F0);
      tot[1] = sums.F1 + xor32f(sums.F1);
      if constexpr (MODE == 0) {
        tot[2] = sums.F2 + xor32f(sums.F2);
        tot[4] = INFINITY;
      } else {
        tot[2] = (float)(sums.cnt + xor32i(sums.cnt));
        const uint32_t mb = min(sums.mrelb, (uint32_t)xor32i((int)sums.mrelb));
        tot[4] = mb < 0x7F800000u ? __uint_as_float(mb) : INFINITY;
      }
      tot[3] = sums.Fh + xor32f(sums.Fh);
      if (!st.done) st.template update<MODE>(tot, npass, first, thi, kappa, alpha, p.tol);
    }
  }

  // ---------------------------------------------------------------- output pass
  f32x16 oacc[DC], gacc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    oacc[dc] = f32x16{};
    gacc[dc] = f32x16{};
  }
  float sg = 0.f;
  const float othr = wave_min(tau) * (float)B;
#pragma unroll
  for (int r = 0; r < 16; ++r) negt[r] = -tau;
  unsigned long long n_out = 0;
  // exact mask bits of this wave, OR-ed into the tile's words one word at a time
  uint32_t* mrow = p.mask + (bh * p.Tr + row0 / p.Br) * p.W;
  const int bc_shift = p.Bc == 32 ? 0 : (p.Bc == 64 ? 1 : 2);   // sub-blocks per key block: 1, 2, 4
  int mw = -1;
  uint32_t mbits = 0;
  {
    // head_dim 64: the next sub-block's V is loaded with its K (most visited sub-blocks hold
    // a weight), so the P.V product does not wait for it
    constexpr bool VPRE = D == 64;
    Frag<T> vn[VPRE ? DC : 1][2];
    // V fragments of sub-block kbv through a buffer resource (fixed lane offset, scalar
    // sub-block offset), like K
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(Vf, (uint32_t)((size_t)n * D * sizeof(T)));
    auto load_v = [&](Frag<T> (&dst)[VPRE ? DC : 1][2], int kbv) {
      const uint32_t soff = (uint32_t)kbv * (uint32_t)(DC * 1024 * sizeof(T));
#pragma unroll
      for (int dc = 0; dc < (VPRE ? DC : 1); ++dc)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t voff = (uint32_t)((dc * 2 + m) * 512 + lane * 8) * (uint32_t)sizeof(T);
          if constexpr (sizeof(T) == 2) {
            dst[dc][m].v = __builtin_bit_cast(bf16x8, buffer_load16(vrs, voff, soff));
          } else {
            dst[dc][m].a = __builtin_bit_cast(f32x4, buffer_load16(vrs, voff, soff));
            dst[dc][m].b = __builtin_bit_cast(f32x4, buffer_load16(vrs, voff + 16, soff));
          }
        }
    };
    Walk wk{-1, 0ull, -1, 0u};
    int kb = walk_next(wk, othr);
    // head_dim 64: the next sub-block's fragments are loaded on every visit (sub-block 0
    // once the walk has ended), so a visit's waits do not drain them. (At head_dim 128 the
    // same form measured slower: 16K output pass +17%.)
    if constexpr (VPRE) {
      Ops::load_k_buf(kf, krs, max(kb, 0), lane);
      load_v(vn, max(kb, 0));
    } else if (kb >= 0) {
      Ops::load_k(kf, Kf, kb, c, h);
    }
    while (kb >= 0) {
      Frag<T> kc[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) kc[s] = kf[s];
      Frag<T> vc[VPRE ? DC : 1][2];
      if constexpr (VPRE) {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
          for (int m = 0; m < 2; ++m) vc[dc][m] = vn[dc][m];
      }
      const int kn = walk_next(wk, othr);
      if constexpr (VPRE) {
        Ops::load_k_buf(kf, krs, max(kn, 0), lane);
        load_v(vn, max(kn, 0));
      } else if (kn >= 0) {
        Ops::load_k(kf, Kf, kn, c, h);
      }
      const f32x16 t = tile(kc, kb);
      f32x16 pw, gw;
      float mx = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dm = relu_raw(t[r]);
        pw[r] = Weight<MODE>::p(dm, kappa);
        gw[r] = Weight<MODE>::g(dm, kappa);
        sg += gw[r];
        mx = fmaxf(mx, dm);
      }
      if (p.dense || ballot(mx > 0.f) != 0) {
        ++n_out;
        const int J = kb >> bc_shift;            // key block of this sub-block
        if ((J >> 5) != mw) {
          if (mw >= 0 && lane == 0) atomicOr(mrow + mw, mbits);
          mw = J >> 5;
          mbits = 0;
        }
        mbits |= 1u << (J & 31);
        Frag<T> vf[DC][2];
        if constexpr (VPRE) {
#pragma unroll
          for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int m = 0; m < 2; ++m) vf[dc][m] = vc[dc][m];
        } else {
          const T* vp = Vf + (size_t)kb * (DC * 1024);
#pragma unroll
          for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int m = 0; m < 2; ++m) load_frag(vf[dc][m], vp + (dc * 2 + m) * 512 + lane * 8);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          Frag<T> pf, gf;
          acc_frag(pf, pw, m);
          acc_frag(gf, gw, m);
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            mma16(oacc[dc], vf[dc][m], pf);
            mma16(gacc[dc], vf[dc][m], gf);
          }
        }
      }
      kb = kn;
    }
  }
  if (mw >= 0 && lane == 0) atomicOr(mrow + mw, mbits);

  {
    const float sgt = sg + xor32f(sg);
    const float inv = sgt > 0.f ? 1.0f / sgt : 0.f;
    const size_t row = bh * n + qrow;
    float* orow = p.o + row * D;
    float* arow = p.aux + row * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dc + 8 * g4 + 4 * h;
        const f32x16& oa = oacc[dc];
        const f32x16& ga = gacc[dc];
        store4(orow + d0, oa[4 * g4 + 0], oa[4 * g4 + 1], oa[4 * g4 + 2], oa[4 * g4 + 3]);
        store4(arow + d0, ga[4 * g4 + 0] * inv, ga[4 * g4 + 1] * inv, ga[4 * g4 + 2] * inv,
               ga[4 * g4 + 3] * inv);
      }
    if (h == 0) p.tau[row] = tau;
  }
  if (p.stats) {
    {
      // rows by refinement passes (rows that hit the cap go to max_iters + 1; 16 and more
      // passes share the last bucket)
      for (int ps = 1; ps <= min(p.max_iters + 1, 16); ++ps) {
        const int rp = min(st.done ? st.rowpass : p.max_iters + 1, 16);
        const int cntp = __popcll(ballot(h == 0 && rp == ps));
        if (lane == 0 && cntp) atomicAdd(&p.stats[ps], (unsigned long long)cntp);
      }
    }
    if (lane == 0) {
      atomicAdd(&p.stats[21], n_ref);
      atomicAdd(&p.stats[22], n_out);
    }
  }
}

template <typename T, int D>
static void (*hist_kernel(bool qs, bool bias, int mode))(FwdParams) {
  if (bias) {
    if (qs) return mode == 1 ? k_hist<T, D, 1, true, true> : mode == 2 ? k_hist<T, D, 2, true, true>
                                                                     : k_hist<T, D, 0, true, true>;
    return mode == 1 ? k_hist<T, D, 1, false, true> : mode == 2 ? k_hist<T, D, 2, false, true>
                                                                : k_hist<T, D, 0, false, true>;
  }
  if (qs) return mode == 1 ? k_hist<T, D, 1, true, false> : mode == 2 ? k_hist<T, D, 2, true, false>
                                                                    : k_hist<T, D, 0, true, false>;
  return mode == 1 ? k_hist<T, D, 1, false, false> : mode == 2 ? k_hist<T, D, 2, false, false>
                                                               : k_hist<T, D, 0, false, false>;
}

template <typename T, int D>
static void (*out_kernel(bool qs, bool bias, int mode))(FwdParams) {
  if (bias) {
    if (qs)
      return mode == 1 ? k_refine_out<T, D, 1, true, true> : mode == 2 ? k_refine_out<T, D, 2, true, true>
                                                                       : k_refine_out<T, D, 0, true, true>;
    return mode == 1 ? k_refine_out<T, D, 1, false, true> : mode == 2 ? k_refine_out<T, D, 2, false, true>
                                                                      : k_refine_out<T, D, 0, false, true>;
  }
  if (qs)
    return mode == 1 ? k_refine_out<T, D, 1, true, false> : mode == 2 ? k_refine_out<T, D, 2, true, false>
                                                                      : k_refine_out<T, D, 0, true, false>;
  return mode == 1 ? k_refine_out<T, D, 1, false, false> : mode == 2 ? k_refine_out<T, D, 2, false, false>
                                                                     : k_refine_out<T, D, 0, false, false>;
}

static size_t fwd_lds_bytes(int waves) { return (size_t)waves * HIST_WAVE_BYTES; }

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams& p, int mode, hipStream_t s) {
  const size_t lds = fwd_lds_bytes(hist_waves<T, D>());
  // the work decomposition (rows per head and work group) is sized for this group shape
  if (p.RH != (hist_waves<T, D>() / p.GP) * 32) return hipErrorInvalidConfiguration;
  const int grid = wgmap_grid(p.map);
  const int grid2 = wgmap_grid(p.map2);
  if (grid == 0) return hipSuccess;
  // fold the score scale into Q when it is an exact power of two
  const float cB = p.cx * (float)p.B;
  int ex = 0;
  const bool qs = std::frexp(cB, &ex) == 0.5f && ex >= -8 && ex <= 8;
  const bool bias = p.slopes != nullptr;
  void (*hist_fn)(FwdParams) = hist_kernel<T, D>(qs, bias, mode);
  hipError_t e = hipFuncSetAttribute((const void*)hist_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  prof_begin("entmax_fwd_hist", s);
  hipLaunchKernelGGL(hist_fn, dim3(grid), dim3(64 * hist_waves<T, D>()), lds, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // (at head_dim 128 the extra accumulator block of the folded form would spill)
  void (*out_fn)(FwdParams) = out_kernel<T, D>(qs && D == 64, bias, mode);
  const size_t out_lds = (size_t)OUT_WAVES * p.out_lds_wave;
  if (out_lds > 160 * 1024) return hipErrorInvalidConfiguration;
  e = hipFuncSetAttribute((const void*)out_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)out_lds);
  if (e != hipSuccess) return e;
  prof_begin("entmax_fwd_refine_out", s);
  hipLaunchKernelGGL(out_fn, dim3(grid2), dim3(64 * OUT_WAVES), out_lds, s, p);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_fwd_t<__bf16, 64>(p, mode, s) : launch_fwd_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_fwd_t<float, 64>(p, mode, s) : launch_fwd_t<float, 128>(p, mode, s);
}

}  // namespace entmax

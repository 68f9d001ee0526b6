// Forward of alpha-entmax attention: one fused kernel per group of query rows.
//
// Stages (AdaSplash-2 pages, page 1 section 2, page 3 section 2, page 5 section 2):
//   1. histogram pass: every valid key block streams through once; each lane keeps
//      an online max and a B-bin histogram of its scores on the anchored grid
//      (bins [m/B, (m+1)/B), window = the B cells ending with the max's cell); a
//      window that slides up drops the cells that fall off. tau_h, the root of the
//      B-bin problem (counts at lower bin edges), satisfies tau* - 1/B < tau_h <= tau*
//      (Proposition 1). The same pass marks the 32-key sub-blocks that hold a score
//      within two bins below the running window: every score that can exceed the
//      bracket's lower end lies in one of them.
//   2. refinement passes over the marked sub-blocks only: a safeguarded hybrid root
//      solver on f(tau) = sum_j [x_j - tau]_+^kappa - 1 from tau_h with bracket
//      [tau_h, tau_h + 1/B]: Halley (alpha <= 1.5), Newton (1.5 < alpha <= 2), secant
//      (alpha > 2, started by false position on the bracket ends), bisection whenever a
//      step leaves the bracket (page 1 section 2.2, page 3 section 2.2).
//   3. output pass over the marked sub-blocks: p = [x - tau]_+^kappa, o = P V,
//      o~ = G V / sum G with g = [x - tau]_+^(kappa-1), and the exact block mask
//      (bit-packed, 32 blocks per word; page 1 section 2.3). Sub-blocks without a
//      non-zero weight skip the PV products.
//
// Work decomposition (MI355X): a work group is 4 waves over up to 256 query rows that
// share one KV head (GQA heads of a group, or consecutive row blocks of one head), so
// the streamed K blocks are shared through L1/L2; each wave owns QW = 32*QC rows.
// Scores are computed transposed (keys x queries) on 32x32 MFMA tiles so that a lane
// owns one query (two lanes per query, 16 keys each per tile): the histogram state of a
// query is private to its lane (its own LDS column, no atomic contention), and P and G
// come out already in the B-operand layout of the PV product (V is read from its
// permuted transpose).
#include "common.hpp"
#include "kernels.hpp"

namespace entmax {

namespace {

// tau_h from merged counts c[0..B-1] (bin k has lower edge l_k = (T - B + 1 + k)/B).
// Works relative to l_top = T/B with u_k = l_k - l_top = (k - B + 1)/B exactly.
template <int MODE>
__device__ float tau_from_counts(const int (&cnt)[16], int T, int B, float kappa) {
  const float invB = 1.0f / (float)B;
  const float ltop = (float)T * invB;
  float v = -1.0f;
  if constexpr (MODE == 1) {
    // sum_k c_k (u_k - v)_+ = 1: scan bins from the top, v = (S1 - 1)/S0
    float S0 = 0.f, S1 = 0.f;
    bool found = false;
#pragma unroll
    for (int kk = 15; kk >= 0; --kk) {
      if (kk < B && !found) {
        const int k = kk;
        const float u = (float)(k - B + 1) * invB;
        S0 += (float)cnt[k];
        S1 += (float)cnt[k] * u;
        if (S0 > 0.f) {
          const float vv = (S1 - 1.0f) / S0;
          const float lower = (k > 0) ? u - invB : -INFINITY;
          if (vv >= lower) {
            v = vv;
            found = true;
          }
        }
      }
    }
  } else if constexpr (MODE == 2) {
    // sum_k c_k (u_k - v)_+^2 = 1 on the top bins: v = mu - sqrt((1 - sum c (u - mu)^2)/S0)
    float S0 = 0.f, S1 = 0.f, S2 = 0.f;
    bool found = false;
#pragma unroll
    for (int kk = 15; kk >= 0; --kk) {
      if (kk < B && !found) {
        const int k = kk;
        const float u = (float)(k - B + 1) * invB;
        const float cf = (float)cnt[k];
        S0 += cf;
        S1 += cf * u;
        S2 += cf * u * u;
        if (S0 > 0.f) {
          const float mu = S1 / S0;
          const float ss = fmaxf(S2 - S1 * mu, 0.f);
          const float vv = mu - sqrtf(fmaxf(1.0f - ss, 0.f) / S0);
          const float lower = (k > 0) ? u - invB : -INFINITY;
          if (vv >= lower) {
            v = vv;
            found = true;
          }
        }
      }
    }
  } else {
    // any kappa: bisection on [-1, 0]; keep the end where the B-bin mass is >= 1
    float lo = -1.0f, hi = 0.0f;
    for (int it = 0; it < 32; ++it) {
      const float mid = 0.5f * (lo + hi);
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < B && cnt[k] > 0) {
          const float t = (float)(k - B + 1) * invB - mid;
          if (t > 0.f) s += (float)cnt[k] * exp2f(kappa * log2f(t));
        }
      }
      if (s >= 1.0f) lo = mid; else hi = mid;
    }
    v = lo;
  }
  return ltop + v;
}

}  // namespace

template <typename T, int D, int QC, int MODE>
__global__ __launch_bounds__(256, 1) void k_fwd(FwdParams p) {
  constexpr int DS = D / 16;   // contraction chunks over the head dimension
  constexpr int DC = D / 32;   // 32-wide output chunks of the head dimension
  constexpr int QW = 32 * QC;
  extern __shared__ uint32_t lds[];

  int unit, rank;
  if (!wgmap_get(p.map, blockIdx.x, unit, rank)) return;   // whole work group

  const int lane = lane_id(), c = lane & 31, h = lane >> 5, w = wave_id();
  const int nsub = p.G / p.GP;                 // head subgroups per KV head
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int rg = p.causal ? (p.RG - 1 - rank / nsub) : (rank / nsub);
  const int gsub = rank % nsub;
  const int per = 4 / p.GP;                    // waves per head
  const int head = kvh * p.G + gsub * p.GP + w / per;
  const int row0 = rg * p.RH + (w % per) * QW;
  const int n = p.n, B = p.B;

  const T* Q = reinterpret_cast<const T*>(p.q) + ((size_t)(bi * p.hq + head) * n) * D;
  const T* K = reinterpret_cast<const T*>(p.k) + ((size_t)(bi * p.hkv + kvh) * n) * D;
  const T* Vt = reinterpret_cast<const T*>(p.vt) + ((size_t)(bi * p.hkv + kvh) * D) * n;

  uint32_t* hist = lds + (w * QC * B) * 64;                   // [QC][B][64]
  uint32_t* cand = lds + 4 * QC * B * 64 + w * p.NW32;        // [NW32]
  uint32_t* exact = lds + 4 * QC * B * 64 + 4 * p.NW32 + w * QC * p.NW32;  // [QC][NW32]

  for (int i = lane; i < QC * B * 64; i += 64) hist[i] = 0;
  for (int i = lane; i < p.NW32; i += 64) cand[i] = 0;
  for (int i = lane; i < QC * p.NW32; i += 64) exact[i] = 0;

  bool cvalid[QC];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) cvalid[qc] = (row0 + 32 * qc) < n;
  const int row_end = min(row0 + QW, n);        // rows of this wave: [row0, row_end)
  const int kb_end = (row0 >= n) ? 0 : (p.causal ? min(p.nkb, (row_end - 1) / 32 + 1) : p.nkb);

  // Q fragments (B operand of S^T = K Q^T): lane (c, h) holds row row0+32qc+c, d = 16s+8h..+7
  Frag<T> qf[QC][DS];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc)
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (cvalid[qc]) load_frag(qf[qc][s], Q + (size_t)(row0 + 32 * qc + c) * D + 16 * s + 8 * h);
      else zero_frag(qf[qc][s]);
    }

  const float cx = p.cx;
  const float cB = cx * (float)B;              // x * B = cB * s exactly (B is a power of two)

  // ---------------------------------------------------------------- 1. histogram pass
  float mB[QC];     // running max of x*B over this lane's scores
  int Tt[QC];       // floor(mB): top cell of the window
  bool have[QC];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    mB[qc] = -INFINITY;
    Tt[qc] = 0;
    have[qc] = false;
  }
  uint32_t cword = 0;
  unsigned long long n_sweep = 0;

  Frag<T> kf[DS];
  if (kb_end > 0) {
#pragma unroll
    for (int s = 0; s < DS; ++s) load_frag(kf[s], K + (size_t)(c) * D + 16 * s + 8 * h);
  }
  for (int kb = 0; kb < kb_end; ++kb) {
    Frag<T> kc[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) kc[s] = kf[s];
    if (kb + 1 < kb_end) {
#pragma unroll
      for (int s = 0; s < DS; ++s) load_frag(kf[s], K + (size_t)((kb + 1) * 32 + c) * D + 16 * s + 8 * h);
    }
    f32x16 acc[QC];
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      acc[qc] = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) mma16(acc[qc], kc[s], qf[qc][s]);
    }
    bool act[QC];
    float tmB[QC];
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      act[qc] = false;
      tmB[qc] = -INFINITY;
      if (!cvalid[qc]) continue;
      const int qrow = row0 + 32 * qc + c;
      if (p.causal && kb * 32 + 31 > row0 + 32 * qc) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + acc_row(r, h) > qrow) acc[qc][r] = -INFINITY;
      }
      tmB[qc] = cB * max16(acc[qc]);
      const float nmB = fmaxf(mB[qc], tmB[qc]);
      if (nmB > -INFINITY) {
        const int Tn = (int)floorf(nmB);
        act[qc] = tmB[qc] >= (float)(Tn - B - 1);
      }
    }
    bool anyact = false;
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) anyact = anyact || act[qc];
    if (ballot(anyact) != 0) {
      cword |= 1u << (kb & 31);
      ++n_sweep;
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        if (!cvalid[qc]) continue;
        const float nmB = fmaxf(mB[qc], tmB[qc]);
        const int Tn = act[qc] ? (int)floorf(nmB) : Tt[qc];
        // slide the window up: clear the cells of bins Tt+1 .. Tn (they reuse dropped slots)
        const int nz = (have[qc] && act[qc]) ? min(Tn - Tt[qc], B) : 0;
        uint32_t* col = hist + (qc * B) * 64 + lane;
        for (int z = 0; ballot(z < nz) != 0; ++z)
          if (z < nz) col[((Tt[qc] + 1 + z) & (B - 1)) * 64] = 0;
        if (act[qc]) {
          mB[qc] = nmB;
          Tt[qc] = Tn;
          have[qc] = true;
          const float low = (float)(Tn - B + 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float xb = cB * acc[qc][r];
            if (xb >= low) {
              const int t = (int)floorf(xb);
              atomicAdd(&col[(t & (B - 1)) * 64], 1u);
            }
          }
        }
      }
    }
    if ((kb & 31) == 31 || kb == kb_end - 1) {
      if (lane == 0) cand[kb >> 5] = cword;
      cword = 0;
    }
  }

  // merge the two half-wave histograms of each query and solve the B-bin problem
  float tau[QC], lo[QC], hi[QC];
  const float hB = 1.0f / (float)B;
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    const int To = xor32i(Tt[qc]);
    const bool ho = xor32i(have[qc] ? 1 : 0) != 0;
    const int Tf = (have[qc] && ho) ? max(Tt[qc], To) : (have[qc] ? Tt[qc] : To);
    int cnt[16];
    const uint32_t* col = hist + (qc * B) * 64 + lane;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      int mine = 0;
      if (k < B) {
        const int bin = Tf - B + 1 + k;
        if (have[qc] && bin >= Tt[qc] - B + 1 && bin <= Tt[qc]) mine = (int)col[(bin & (B - 1)) * 64];
      }
      cnt[k] = mine + xor32i(mine);
    }
    tau[qc] = tau_from_counts<MODE>(cnt, Tf, B, p.kappa);
    lo[qc] = tau[qc];
    hi[qc] = tau[qc] + hB;
    if (cvalid[qc] && h == 0) {
      const size_t row = (size_t)(bi * p.hq + head) * n + row0 + 32 * qc + c;
      if (p.tau_h) p.tau_h[row] = tau[qc];
      if (p.hist) {
        int32_t* dst = p.hist + row * B;
        for (int k = 0; k < 16; ++k)
          if (k < B) dst[k] = cnt[k];
      }
    }
  }

  // ---------------------------------------------------------------- 2. refinement passes
  // candidate sub-block iterator over this wave's bits (wave-uniform)
  auto next_cand = [&](int from) -> int {
    int wi = from >> 5;
    if (wi >= p.NW32) return -1;
    uint32_t word = uniform_u32(cand[wi]) & (~0u << (from & 31));
    while (word == 0) {
      if (++wi >= p.NW32) return -1;
      word = uniform_u32(cand[wi]);
    }
    return (wi << 5) + __builtin_ctz(word);
  };
  int ncand = 0;
  for (int i = 0; i < p.NW32; ++i) ncand += __builtin_popcount(uniform_u32(cand[i]));

  const float kappa = p.kappa, alpha = p.alpha;
  bool done[QC];
  int rowpass[QC];
  float tprev[QC], fprev[QC];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    done[qc] = !cvalid[qc];
    rowpass[qc] = 0;
    tprev[qc] = 0.f;
    fprev[qc] = 0.f;
  }
  const bool secant = alpha > 2.0f;
  int npass = 0;
  while (npass < p.max_iters) {
    bool pending = false;
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) pending = pending || !done[qc];
    if (ballot(pending) == 0) break;
    const bool first = (npass == 0);
    float F0[QC], F1[QC], F2[QC], Fh[QC];
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) F0[qc] = F1[qc] = F2[qc] = Fh[qc] = 0.f;
    int kb = next_cand(0);
    if (kb >= 0) {
#pragma unroll
      for (int s = 0; s < DS; ++s) load_frag(kf[s], K + (size_t)(kb * 32 + c) * D + 16 * s + 8 * h);
    }
    while (kb >= 0) {
      Frag<T> kc[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) kc[s] = kf[s];
      const int kn = next_cand(kb + 1);
      if (kn >= 0) {
#pragma unroll
        for (int s = 0; s < DS; ++s) load_frag(kf[s], K + (size_t)(kn * 32 + c) * D + 16 * s + 8 * h);
      }
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        if (!cvalid[qc]) continue;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < DS; ++s) mma16(acc, kc[s], qf[qc][s]);
        const int qrow = row0 + 32 * qc + c;
        const bool diag = p.causal && kb * 32 + 31 > row0 + 32 * qc;
        const float tq = tau[qc], th = hi[qc];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool valid = !diag || (kb * 32 + acc_row(r, h) <= qrow);
          const float x = cx * acc[r];
          const float t = valid ? (x - tq) : -1.0f;
          if (t > 0.f) {
            if constexpr (MODE == 2) {
              F0[qc] += t * t;
              F1[qc] += t;
              F2[qc] += 1.0f;
            } else if constexpr (MODE == 1) {
              F0[qc] += t;
              F1[qc] += 1.0f;
            } else {
              const float lt = log2f(t);
              F0[qc] += exp2f(kappa * lt);
              F1[qc] += exp2f((kappa - 1.0f) * lt);
              F2[qc] += exp2f((kappa - 2.0f) * lt);
            }
          }
          if constexpr (MODE == 0) {
            if (secant && first) {
              const float u = valid ? (x - th) : -1.0f;
              if (u > 0.f) Fh[qc] += exp2f(kappa * log2f(u));
            }
          }
        }
      }
      kb = kn;
    }
    ++npass;
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      F0[qc] += xor32f(F0[qc]);
      F1[qc] += xor32f(F1[qc]);
      F2[qc] += xor32f(F2[qc]);
      Fh[qc] += xor32f(Fh[qc]);
      if (done[qc]) continue;
      const float f = F0[qc] - 1.0f;
      const float t0 = tau[qc];
      if (f >= 0.f) lo[qc] = t0; else hi[qc] = t0;
      if (first && f < 0.f) lo[qc] = t0 - hB;   // rounding lost the histogram bound
      float tn;
      if (alpha <= 1.5f) {
        const float fp = -kappa * F1[qc];
        const float fpp = kappa * (kappa - 1.0f) * F2[qc];
        tn = t0 - 2.0f * f * fp / (2.0f * fp * fp - f * fpp);
      } else if (alpha <= 2.0f) {
        const float fp = -kappa * F1[qc];
        tn = t0 - f / fp;
      } else {
        if (first) {
          const float th = t0 + hB;
          const float fh = Fh[qc] - 1.0f;
          if (fh >= 0.f) lo[qc] = th; else hi[qc] = fminf(hi[qc], th);
          tn = t0 - f * (th - t0) / (fh - f);
        } else {
          tn = t0 - f * (t0 - tprev[qc]) / (f - fprev[qc]);
        }
        tprev[qc] = t0;
        fprev[qc] = f;
      }
      // converged when the solver's own step is below tolerance (tested before the
      // bracket check: a vanishing step lands on a bracket end and must not be
      // replaced by a bisection jump); otherwise keep the step inside (lo, hi)
      const float tabs = p.tol * fmaxf(1.0f, fabsf(t0));
      if (fabsf(tn - t0) <= tabs) {
        done[qc] = true;
        rowpass[qc] = npass;
        tn = fminf(fmaxf(tn, lo[qc]), hi[qc]);
      } else {
        if (!(tn > lo[qc] && tn < hi[qc])) tn = 0.5f * (lo[qc] + hi[qc]);
        if (hi[qc] - lo[qc] <= tabs) {
          done[qc] = true;
          rowpass[qc] = npass;
        }
      }
      tau[qc] = tn;
    }
  }

  // ---------------------------------------------------------------- 3. output pass
  f32x16 oacc[QC][DC], gacc[QC][DC];
  float sg[QC];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    sg[qc] = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      oacc[qc][dc] = f32x16{};
      gacc[qc][dc] = f32x16{};
    }
  }
  unsigned long long n_out = 0;
  {
    int kb = next_cand(0);
    if (kb >= 0) {
#pragma unroll
      for (int s = 0; s < DS; ++s) load_frag(kf[s], K + (size_t)(kb * 32 + c) * D + 16 * s + 8 * h);
    }
    while (kb >= 0) {
      Frag<T> kc[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) kc[s] = kf[s];
      const int kn = next_cand(kb + 1);
      if (kn >= 0) {
#pragma unroll
        for (int s = 0; s < DS; ++s) load_frag(kf[s], K + (size_t)(kn * 32 + c) * D + 16 * s + 8 * h);
      }
      f32x16 pacc[QC], gw[QC];
      bool nzq[QC];
      bool anynz = false;
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        nzq[qc] = false;
        pacc[qc] = f32x16{};
        gw[qc] = f32x16{};
        if (!cvalid[qc]) continue;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < DS; ++s) mma16(acc, kc[s], qf[qc][s]);
        const int qrow = row0 + 32 * qc + c;
        const bool diag = p.causal && kb * 32 + 31 > row0 + 32 * qc;
        const float tq = tau[qc];
        bool any = false;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool valid = !diag || (kb * 32 + acc_row(r, h) <= qrow);
          const float t = valid ? (cx * acc[r] - tq) : -1.0f;
          const float dm = fmaxf(t, 0.f);
          pacc[qc][r] = Weight<MODE>::p(dm, kappa);
          gw[qc][r] = Weight<MODE>::g(t > 0.f ? dm : 0.f, kappa);
          sg[qc] += gw[qc][r];
          any = any || (t > 0.f);
        }
        nzq[qc] = ballot(any) != 0;
        anynz = anynz || nzq[qc];
      }
      if (anynz) {
        ++n_out;
#pragma unroll
        for (int qc = 0; qc < QC; ++qc)
          if (nzq[qc] && lane == 0) exact[qc * p.NW32 + (kb >> 5)] |= 1u << (kb & 31);
        Frag<T> vf[DC][2];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            load_frag(vf[dc][m], Vt + (size_t)(32 * dc + c) * n + kb * 32 + 16 * m + 8 * h);
#pragma unroll
        for (int qc = 0; qc < QC; ++qc) {
          if (!nzq[qc]) continue;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            Frag<T> pf, gf;
            acc_frag(pf, pacc[qc], m);
            acc_frag(gf, gw[qc], m);
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
              mma16(oacc[qc][dc], vf[dc][m], pf);
              mma16(gacc[qc][dc], vf[dc][m], gf);
            }
          }
        }
      }
      kb = kn;
    }
  }

  // ---------------------------------------------------------------- outputs of this wave
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    if (!cvalid[qc]) continue;
    const float sgt = sg[qc] + xor32f(sg[qc]);
    const float inv = sgt > 0.f ? 1.0f / sgt : 0.f;
    const size_t row = (size_t)(bi * p.hq + head) * n + row0 + 32 * qc + c;
    float* orow = p.o + row * D;
    float* arow = p.aux + row * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dc + 8 * g4 + 4 * h;
        const f32x16& oa = oacc[qc][dc];
        const f32x16& ga = gacc[qc][dc];
        store4(orow + d0, oa[4 * g4 + 0], oa[4 * g4 + 1], oa[4 * g4 + 2], oa[4 * g4 + 3]);
        store4(arow + d0, ga[4 * g4 + 0] * inv, ga[4 * g4 + 1] * inv, ga[4 * g4 + 2] * inv,
               ga[4 * g4 + 3] * inv);
      }
    if (h == 0) p.tau[row] = tau[qc];
  }
  if (p.stats) {
    // rows by refinement passes (rows that hit the cap go to max_iters + 1)
    for (int ps = 1; ps <= p.max_iters + 1; ++ps) {
      int cntp = 0;
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        const int rp = done[qc] ? rowpass[qc] : p.max_iters + 1;
        cntp += __popcll(ballot(cvalid[qc] && h == 0 && rp == ps));
      }
      if (lane == 0 && cntp) atomicAdd(&p.stats[ps], (unsigned long long)cntp);
    }
    if (lane == 0) {
      atomicAdd(&p.stats[20], (unsigned long long)kb_end * QC);
      atomicAdd(&p.stats[21], (unsigned long long)ncand * npass * QC);
      atomicAdd(&p.stats[22], n_out * QC);
    }
  }
  (void)n_sweep;

  // ---------------------------------------------------------------- block mask of the tiles
  __syncthreads();
  const int tiles_per_head = p.RH / p.Br;
  const int KW = p.Bc / 32;                    // sub-blocks per key block
  const int QCB = p.Br / 32;                   // 32-row chunks per tile
  const int total = p.GP * tiles_per_head * p.W;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int wi = idx % p.W;
    const int t = (idx / p.W) % tiles_per_head;
    const int hs = idx / (p.W * tiles_per_head);
    const int trow0 = rg * p.RH + t * p.Br;
    if (trow0 >= n) continue;
    uint32_t word = 0;
    for (int bit = 0; bit < 32; ++bit) {
      const int J = wi * 32 + bit;
      if (J >= p.Tc) break;
      uint32_t any = 0;
      for (int u = 0; u < KW && !any; ++u) {
        const int kbi = J * KW + u;
        if ((kbi >> 5) >= p.NW32) break;
        for (int ch = 0; ch < QCB && !any; ++ch) {
          const int chunk = t * QCB + ch;       // 32-row chunk within this head's rows
          const int ww = hs * per + chunk / QC; // wave holding it
          const int qq = chunk % QC;
          const uint32_t* ex = lds + 4 * QC * B * 64 + 4 * p.NW32 + ww * QC * p.NW32 + qq * p.NW32;
          any |= (ex[kbi >> 5] >> (kbi & 31)) & 1u;
        }
      }
      word |= any << bit;
    }
    const int hg = kvh * p.G + gsub * p.GP + hs;
    const int I = trow0 / p.Br;
    p.mask[((size_t)(bi * p.hq + hg) * p.Tr + I) * p.W + wi] = word;
  }
}

template <typename T, int D, int QC>
static hipError_t launch_fwd_t(const FwdParams& p, int mode, hipStream_t s) {
  const size_t lds = (size_t)(4 * QC * p.B * 64 + 4 * p.NW32 + 4 * QC * p.NW32) * sizeof(uint32_t);
  const int grid = wgmap_grid(p.map);
  if (grid == 0) return hipSuccess;
  if (mode == 1) hipLaunchKernelGGL((k_fwd<T, D, QC, 1>), dim3(grid), dim3(256), lds, s, p);
  else if (mode == 2) hipLaunchKernelGGL((k_fwd<T, D, QC, 2>), dim3(grid), dim3(256), lds, s, p);
  else hipLaunchKernelGGL((k_fwd<T, D, QC, 0>), dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (dtype == 1) {
    if (D == 64) return launch_fwd_t<__bf16, 64, 2>(p, mode, s);
    return launch_fwd_t<__bf16, 128, 1>(p, mode, s);
  }
  if (D == 64) return launch_fwd_t<float, 64, 2>(p, mode, s);
  return launch_fwd_t<float, 128, 1>(p, mode, s);
}

}  // namespace entmax

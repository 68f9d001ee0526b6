// The per-row threshold solver shared by the prefill and decode forwards (AdaSplash-2
// pages, AdaSplash-2 (zh) §2.1-2.2, AdaSplash-2 (ja) §2.1-2.2): tau_h from the B-bin histogram
// (Proposition 1: tau* - 1/B < tau_h <= tau*), then a safeguarded hybrid root solver on
// f(tau) = sum_j [x_j - tau]_+^kappa - 1 -- Halley (alpha <= 1.5), Newton (1.5 < alpha <= 2),
// secant started by false position (alpha > 2), bisection whenever a step leaves the
// bracket. A pass over a row's scores accumulates PassSums; RowState::update takes the
// row's totals and moves tau.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace entmax {

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


// Start of the refinement at alpha = 1.5. The root t_s of the B-bin problem with each count
// spread evenly over its bin instead of placed at the lower edge, sum_k c_k E[(U_k - t)_+^2] = 1
// with U_k uniform on bin k, lies in [tau_h, tau_h + 1/B] like tau* (the lower-edge and
// upper-edge versions of the same problem bracket it) and tracks tau* closely when the
// scores crowd a few bins. The solver certifies a root only from below (f >= 0), so the
// start is a quarter bin under it, and never under the fixed start tau_h + 1/(4B):
// max(tau_h + 1/(4B), t_s - 1/(4B)). (fp64 emulation on sampled rows, sub-blocks visited
// per row over all passes: 128K layer 71 -> 55, 16K at 95% block sparsity 42 -> 27, 4K at
// 60% 61 -> 50, 4K at 90% 10.2 -> 9.7; denser rows visit more: 16K at 60% +6%, 4K at 0%
// +23%.) t_s comes from two Newton steps from tau_h: the function is convex and decreasing
// and positive at tau_h, so the steps rise monotonically towards the root without passing
// it. Relative to l_top = T/B, bin k spans [u_k, u_k + h) with u_k = (k - B + 1)/B exactly.
__device__ __forceinline__ float tau_spread_start(const int (&cnt)[16], int T, int B, float tau_h) {
  const float h = 1.0f / (float)B;
  const float ltop = (float)T * h;
  const float inv3h = (float)B / 3.0f;
  float v = tau_h - ltop;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    float F = -1.0f, Dv = 0.0f;   // f and -f' / 2 at v
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < B) {
        const float u = (float)(k - B + 1) * h;
        const float a = fmaxf(u - v, 0.0f), b = fmaxf(u + h - v, 0.0f);
        const float cf = (float)cnt[k];
        F = fmaf(cf * inv3h, b * b * b - a * a * a, F);
        Dv = fmaf(cf * 0.5f * (float)B, b * b - a * a, Dv);
      }
    }
    if (Dv > 0.0f && F > 0.0f) v += F / (2.0f * Dv);
  }
  return fmaxf(tau_h + 0.25f * h, ltop + v - 0.25f * h);
}

// Per-score sums of one pass at the evaluation point tau, fed with tt = x - tau:
// F0 = sum d^kappa, F1 = sum d^(kappa-1), F2 = sum d^(kappa-2) (general alpha), cnt = |support|
// and mrelb = bits of the smallest positive gap (alpha 1.5, 2; positive floats order like
// their bits), Fh = sum (x - hi)_+^kappa on the first pass of the secant (thi = hi - tau).
struct PassSums {
  float F0 = 0.f, F1 = 0.f, F2 = 0.f, Fh = 0.f;
  int cnt = 0;
  uint32_t mrelb = 0xFFFFFFFFu;

  template <int MODE>
  __device__ __forceinline__ void add(float tt, float thi, bool sec_first, float kappa) {
    if constexpr (MODE == 2) {
      const float dm = relu_raw(tt);
      F0 = fmaf(dm, dm, F0);
      F1 += dm;
      cnt += (tt > 0.f) ? 1 : 0;
      mrelb = min(mrelb, __float_as_uint(tt));
    } else if constexpr (MODE == 1) {
      F0 += relu_raw(tt);
      cnt += (tt > 0.f) ? 1 : 0;
      mrelb = min(mrelb, __float_as_uint(tt));
    } else {
      const bool in = tt > 0.f;
      const float lt = log2f(in ? tt : 1.0f);
      F0 += in ? exp2f(kappa * lt) : 0.f;
      F1 += in ? exp2f((kappa - 1.0f) * lt) : 0.f;
      F2 += in ? exp2f((kappa - 2.0f) * lt) : 0.f;
      if (sec_first) {
        const float u = tt - thi;      // x - hi
        Fh += u > 0.f ? exp2f(kappa * log2f(u)) : 0.f;
      }
    }
  }
};

// General alpha has no exact-support test: a row stops once |sum p - 1| <= FTOL0 at the
// evaluated tau. Where f is steep (alpha > 2 with a wide support of small weights, such as
// all scores equal), a step that is small in tau can still leave sum p well away from 1.
// Where f is flat the same mass error means a larger error in tau (about |f| / |f'| with
// |f'| = kappa F1; a single-key support at alpha = 16 has |f'| = 1/15), so the test is
// |f| <= FTOL0 min(1, kappa F1): both sum p and tau end within about FTOL0 of their targets.
constexpr float FTOL0 = 1e-4f;

// Solver state of one row: bracket [lo, hi] holding tau*, the evaluation point tau, the
// previous secant iterate, and whether (after how many passes) the row has converged.
struct RowState {
  float lo, hi, tau;
  float tprev = 0.f, fprev = 0.f;
  bool done = false;
  int rowpass = 0;

  // Bracket [tau_h, tau_h + 1/B] (with a margin of 1/(16B) below tau_h for fp32 rounding of
  // the B-bin solve); the first evaluation is a quarter of the way into it. Starting above
  // tau_h leaves out the sub-blocks whose scores all lie in the bottom quarter, and on the
  // workloads' rows it also takes fewer passes than starting at tau_h.
  __device__ __forceinline__ static RowState from_hist(float tau_h, int B) {
    const float hB = 1.0f / (float)B;
    RowState s;
    s.lo = tau_h - 0.0625f * hB;
    s.hi = tau_h + hB;
    s.tau = tau_h + 0.25f * hB;
    return s;
  }
  // the same bracket, started at a given point (alpha = 1.5: tau_spread_start)
  __device__ __forceinline__ static RowState from_hist_at(float tau_h, int B, float start) {
    RowState s = from_hist(tau_h, B);
    s.tau = fminf(fmaxf(start, s.lo), s.hi);
    return s;
  }
  // General alpha: the histogram bracket narrowed by the plain bounds below (which hold
  // for any row), started a quarter of the way into it. With many nearly equal scores at
  // alpha > 2 the root lies within a tiny fraction of 1/B below x_max and f is steep
  // there; the upper bound then sits at (all scores equal: exactly on) the root, while
  // tau_h + 1/B would leave the first evaluations above every score, where f = -1 carries
  // no slope for the secant.
  __device__ __forceinline__ static RowState from_hist_bounded(float tau_h, int B, float xmax, float nvalid,
                                                               float alpha) {
    RowState s = from_hist(tau_h, B);
    s.hi = fminf(s.hi, xmax - exp2f((1.0f - alpha) * log2f(nvalid)));
    s.lo = fminf(fmaxf(s.lo, xmax - 1.0f), s.hi);
    s.tau = fminf(fmaxf(tau_h + 0.25f * (s.hi - tau_h), s.lo), s.hi);
    return s;
  }
  // the plain bracket [x_max - 1, x_max - n_valid^(1-alpha)], started at its lower end
  // (upper end: at that tau each of the n_valid weights is at most 1/n_valid)
  __device__ __forceinline__ static RowState from_max(float xmax, float nvalid, float alpha) {
    RowState s;
    s.lo = xmax - 1.0f;
    s.hi = xmax - exp2f((1.0f - alpha) * log2f(nvalid));
    s.tau = s.lo;
    return s;
  }

  // One solver step from a pass's row totals: tot[0] = F0, tot[1] = F1, tot[2] = |support|
  // (alpha 1.5, 2) or F2, tot[3] = Fh, tot[4] = smallest positive gap (alpha 1.5, 2) or inf.
  // npass counts the passes done, including this one; thi = hi - tau of the first pass.
  template <int MODE>
  __device__ __forceinline__ void update(const float (&tot)[5], int npass, bool first, float thi, float kappa,
                                         float alpha, float tol) {
    const float f = tot[0] - 1.0f;
    const float t0 = tau;
    if (f >= 0.f) lo = t0; else hi = t0;
    if constexpr (MODE == 0) {
      if (fabsf(f) <= FTOL0 * fminf(1.0f, kappa * tot[1])) {   // tau stays at the evaluated point
        done = true;
        rowpass = npass;
        return;
      }
    }
    // alpha in {1.5, 2}: the root of the equation restricted to the support {x > t0}
    // is exact when it keeps that support (it lies at or above t0 and no further than
    // the support's smallest gap): then stop without a confirming pass
    if constexpr (MODE == 1 || MODE == 2) {
      const float cntS = tot[2];
      if (cntS > 0.f && f >= 0.f) {
        float u;
        if constexpr (MODE == 2) {
          const float disc = tot[1] * tot[1] - cntS * f;
          u = disc >= 0.f ? f / (tot[1] + sqrtf(disc)) : INFINITY;
        } else {
          u = f / cntS;
        }
        if (u <= tot[4]) {
          tau = t0 + u;
          done = true;
          rowpass = npass;
          return;
        }
      }
    }
    float tn;
    if constexpr (MODE == 2) {
      // Halley on f = sum d^2 - 1: f' = -2 sum d, f'' = 2 |support|
      const float fp = -2.0f * tot[1];
      const float fpp = 2.0f * tot[2];
      tn = t0 - 2.0f * f * fp / (2.0f * fp * fp - f * fpp);
    } else if constexpr (MODE == 1) {
      tn = tot[2] > 0.f ? t0 + f / tot[2] : 0.5f * (lo + hi);   // Newton, f' = -|support|
    } else {
      const float fp = -kappa * tot[1];
      if (alpha <= 1.5f) {
        const float fpp = kappa * (kappa - 1.0f) * tot[2];
        tn = t0 - 2.0f * f * fp / (2.0f * fp * fp - f * fpp);
      } else if (alpha <= 2.0f) {
        tn = t0 - f / fp;
      } else {
        if (first) {
          const float th = t0 + thi;   // the bracket's upper end at the start of the pass
          const float fh = tot[3] - 1.0f;
          // the upper end already meets the test (its slope is not summed; with a support
          // of weights at most 1, F1 >= 1 there when kappa < 1, so kappa bounds kappa F1)
          if (fabsf(fh) <= FTOL0 * fminf(1.0f, kappa)) {
            tau = th;
            done = true;
            rowpass = npass;
            return;
          }
          if (fh >= 0.f) lo = fmaxf(lo, th); else hi = fminf(hi, th);
          tn = t0 - f * (th - t0) / (fh - f);
        } else {
          tn = t0 - f * (t0 - tprev) / (f - fprev);
        }
        tprev = t0;
        fprev = f;
      }
    }
    if constexpr (MODE == 0) {
      // no exact test at general alpha: besides |f| <= FTOL0 above, a row ends only when
      // fp32 can no longer move tau (a stalled step, or a bracket one ulp wide)
      if (!(tn > lo && tn < hi)) tn = 0.5f * (lo + hi);
      if (tn == t0 || tn <= lo || tn >= hi) {
        done = true;
        rowpass = npass;
      }
      tau = tn;
      return;
    }
    // converged when the solver's own step is below tolerance (tested before the
    // bracket check: a vanishing step lands on a bracket end and must not be
    // replaced by a bisection jump); otherwise keep the step inside (lo, hi)
    const float tabs = tol * fmaxf(1.0f, fabsf(t0));
    if (fabsf(tn - t0) <= tabs) {
      done = true;
      rowpass = npass;
      tn = fminf(fmaxf(tn, lo), hi);
    } else {
      if (!(tn > lo && tn < hi)) tn = 0.5f * (lo + hi);
      if (hi - lo <= tabs) {
        done = true;
        rowpass = npass;
      }
    }
    tau = tn;
  }
};


// alpha = 2 in the forward's refinement: f(tau) = sum (x - tau)_+ - 1 is piecewise linear
// and convex, and Newton from below (the pages' solver for 1.5 < alpha <= 2) shrinks the
// error only about by half per pass when many scores sit just below the root. A pass costs
// one sweep over the candidate keys whatever is evaluated on them, so each pass here
// evaluates f and the support count at NP points at once: the Newton point from the best
// lower end (at or below the root) and NP - 1 points between it and the chord root through
// the bracket ends (at or above the root, by convexity). The bracket then shrinks to the
// two points around the root, and the next Newton point starts from its lower end. The
// root is exact when no score lies between the lower end and the next point above it and
// the Newton step stays inside that gap (the support does not change on it).
template <int NP>
struct MultiState {
  float lo, hi;          // bracket: f(lo) >= 0 > f(hi) (f at the initial ends may be unknown)
  float flo = 0.f, fhi = 0.f;
  int nlo = 0;           // support count at lo (0: f(lo) unknown)
  bool fhi_known = false;
  float tau;             // lowest evaluation point of the next pass; the root once done
  float off[NP];         // evaluation points tau + off[k], off[0] = 0
  bool done = false;
  int rowpass = 0;

  __device__ __forceinline__ void spread(float t0, float top) {
    tau = t0;
#pragma unroll
    for (int k = 0; k < NP; ++k) off[k] = (top - t0) * (float)k / (float)NP;
  }
  // histogram start: bracket [tau_h - 1/(16B), tau_h + 1/B], first points close above tau_h
  // (at alpha = 2 tau_h is within a few hundredths of a bin of the root on the workloads)
  __device__ __forceinline__ static MultiState from_hist(float tau_h, int B) {
    const float hB = 1.0f / (float)B;
    MultiState s;
    s.lo = tau_h - 0.0625f * hB;
    s.hi = tau_h + hB;
    s.tau = tau_h + 0.02f * hB;
    // first-pass points above the start, in units of 1/B (set on the workloads' rows)
    const float first[4] = {0.0f, 0.03f, 0.08f, 0.23f};
    const float first2[2] = {0.0f, 0.02f};
#pragma unroll
    for (int k = 0; k < NP; ++k) s.off[k] = (NP == 2 ? first2[k] : first[k < 4 ? k : 3]) * hB;
    return s;
  }
  __device__ __forceinline__ static MultiState from_max(float xmax, float nvalid, float alpha) {
    MultiState s;
    s.lo = xmax - 1.0f;
    s.hi = xmax - exp2f((1.0f - alpha) * log2f(nvalid));
    s.spread(s.lo, s.hi);
    return s;
  }

  // F[k] = sum (x - tau - off[k])_+ and N[k] = support count at point k, over the row
  __device__ __forceinline__ void update(const float (&F)[NP], const int (&N)[NP], int npass, float tol) {
    int klo = -1;
#pragma unroll
    for (int k = 0; k < NP; ++k)
      if (F[k] - 1.0f >= 0.0f) klo = k;          // f decreases: a prefix of the points
    // the values at points klo and klo + 1, picked with constant indices (selects, so the
    // arrays stay in registers)
    float off_lo = 0.f, f_lo = 0.f, off_nx = 0.f, f_nx = 0.f;
    int n_lo = 0, n_nx = -1;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      if (k == klo) { off_lo = off[k]; f_lo = F[k] - 1.0f; n_lo = N[k]; }
      if (k == klo + 1) { off_nx = off[k]; f_nx = F[k] - 1.0f; n_nx = N[k]; }
    }
    if (klo >= 0) {
      lo = tau + off_lo;
      flo = f_lo;
      nlo = n_lo;
    }
    int nnext = -1;
    float tnext = hi;
    if (klo + 1 < NP) {
      tnext = tau + off_nx;
      hi = tnext;
      fhi = f_nx;
      fhi_known = true;
      nnext = n_nx;
    }
    const float tabs = tol * fmaxf(1.0f, fabsf(lo));
    if (nlo > 0) {
      const float u = flo / (float)nlo;
      // exact: the support is the same at lo and at the next point, and the root lies before it
      if (nnext == nlo && lo + u <= tnext) {
        tau = lo + u;
        done = true;
        rowpass = npass;
        return;
      }
      const float t0 = fminf(lo + u, hi);        // Newton from the lower end: at or below the root
      float top = fhi_known ? lo + flo * (hi - lo) / (flo - fhi) : hi;   // chord: at or above
      top = fminf(fmaxf(top, t0), hi);
      if (top - t0 <= tabs || hi - lo <= tabs) {
        tau = t0;
        done = true;
        rowpass = npass;
        return;
      }
      spread(t0, top);
    } else {
      // no point with f >= 0 yet: the root lies in [lo, lowest point); spread over it
      if (hi - lo <= tabs) {
        tau = lo;
        done = true;
        rowpass = npass;
        return;
      }
      spread(lo, hi);
    }
  }
};

template <int NP>
struct MultiSums {
  float F[NP];
  int N[NP];
  __device__ __forceinline__ MultiSums() {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      F[k] = 0.f;
      N[k] = 0;
    }
  }
  // tt = x - tau (the lowest point)
  __device__ __forceinline__ void add(float tt, const float (&off)[NP]) {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const float d = k == 0 ? tt : tt - off[k];
      F[k] += relu_raw(d);
      N[k] += d > 0.f ? 1 : 0;
    }
  }
};

}  // namespace entmax

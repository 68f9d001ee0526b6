// DashAttention forward, stages 1 and 2 (DashAttention page, Italian summary,
// "Metodologia"), on the primitives of the alpha-entmax attention kernels.
//
//   k_dash_route -- stage 1: one work group per (batch, KV head, 64-row query tile). For
//      each query head of the group a wave scores its 32 rows against the chunk summaries
//      on the matrix cores (transposed tiles: lane = query, registers = chunks; a row
//      spans at most 256 chunks, eight 32-chunk tiles held in registers), finds the
//      alpha-entmax threshold with the safeguarded hybrid solver of the attention forward
//      (same RowState, started from the plain bracket below the row max: a routing row is
//      short, so the histogram stage would not pay), and adds its weights / G into an LDS
//      accumulator. Then the group average goes to HBM chunk-major (a chunk's 32 rows of a
//      wave are one 128-byte run) and the tile's chunk-mask words are formed by ballots.
//   k_dash_attn -- stage 2: one work group per (query head, 64-row tile), a wave per 32
//      rows. It walks the diagonal chunk's 32-key sub-blocks, then the chunks set in the
//      tile's mask word by word (a chunk none of the wave's rows routes is skipped after
//      one coalesced read of the weights), with an online softmax: the row max and the
//      sum of exponentials are per lane (lane = query), so rescaling the output
//      accumulators is a per-lane multiply. The routing prior enters each score of a
//      chunk as the per-row constant sigma log2 wbar (scores in base-2 units).
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "solver.hpp"

namespace entmax {

constexpr int DASH_NB = 8;      // 32-chunk tiles a routing row may span (n_chunks <= 256)
constexpr int DASH_WAVES = 2;   // a 64-row query tile per work group, 32 rows per wave

// ================================================================================ stage 1
template <typename T, int D, int MODE>
__global__ __launch_bounds__(64 * DASH_WAVES) void k_dash_route(DashParams p) {
  constexpr int DS = D / 16;
  extern __shared__ float wsum[];               // [DASH_WAVES][Wc * 16][64]
  __shared__ uint32_t mwords[DASH_WAVES][DASH_NB];
  const int U = p.b * p.hkv;
  const int bid = blockIdx.x;
  if (bid >= U * p.Tr) return;                  // whole work group
  const int t = p.Tr - 1 - bid / U;             // tiles with the most chunks first
  const int unit = bid % U;
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int qrow = t * 64 + w * 32 + c;
  const int m = (t * 64) / p.C;                 // every row of the tile routes chunks 0 .. m-1
  const int nb = (m + 31) >> 5;
  float* wl = wsum + (size_t)w * p.Wc * 1024;
  for (int i = 0; i < nb * 16; ++i) wl[i * 64 + lane] = 0.f;
  const float invG = 1.0f / (float)p.G;
  const float kappa = p.kappa, alpha = p.alpha;
  const bool secant = alpha > 2.0f;
  const T* Ks = reinterpret_cast<const T*>(p.ks) + (size_t)unit * p.nc * D;

  for (int g = 0; g < p.G; ++g) {
    const size_t bh = (size_t)bi * p.hq + kvh * p.G + g;
    float tau = 0.f;
    if (m > 0) {
      const T* Q = reinterpret_cast<const T*>(p.q) + bh * p.n * D;
      Frag<T> qf[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) load_frag(qf[s], Q + (size_t)qrow * D + 16 * s + 8 * h);
      // x = (alpha - 1) gamma scale q . ksum; chunks >= m are -inf
      f32x16 x[DASH_NB];
      float xmax = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < DASH_NB; ++jb) {
        x[jb] = f32x16{};
        if (jb < nb) {
          const int ch = 32 * jb + c;
          Frag<T> kf[DS];
#pragma unroll
          for (int s = 0; s < DS; ++s) {
            if (ch < m) load_frag(kf[s], Ks + (size_t)ch * D + 16 * s + 8 * h);
            else zero_frag(kf[s]);
          }
          f32x16 acc = f32x16{};
#pragma unroll
          for (int s = 0; s < DS; ++s) mma16(acc, kf[s], qf[s]);
#pragma unroll
          for (int r = 0; r < 16; ++r) x[jb][r] = (32 * jb + acc_row(r, h) < m) ? p.cx * acc[r] : -INFINITY;
          xmax = fmaxf(xmax, max16(x[jb]));
        }
      }
      xmax = fmaxf(xmax, xor32f(xmax));
      RowState st = RowState::from_max(xmax, (float)m, alpha);
      for (int npass = 0; npass < p.max_iters;) {
        if (ballot(!st.done) == 0) break;
        const bool first = npass == 0;
        const float thi = st.hi - st.tau;
        PassSums sums;
#pragma unroll
        for (int jb = 0; jb < DASH_NB; ++jb)
          if (jb < nb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sums.add<MODE>(x[jb][r] - st.tau, thi, secant && first, kappa);
          }
        ++npass;
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
      tau = st.tau;
#pragma unroll
      for (int jb = 0; jb < DASH_NB; ++jb)
        if (jb < nb) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            wl[(jb * 16 + r) * 64 + lane] += Weight<MODE>::p(fmaxf(x[jb][r] - tau, 0.f), kappa) * invG;
        }
    }
    if (p.rtau && h == 0) p.rtau[bh * p.n + qrow] = tau;
  }

  // group average to HBM (zeros past chunk m - 1) and the tile's mask words
  float* rw = p.rw + (size_t)unit * p.nc * p.n;
  for (int jb = 0; jb < p.Wc; ++jb) {
    uint32_t word = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int cr = 32 * jb + acc_row(r, h);
      const float val = jb < nb ? wl[(jb * 16 + r) * 64 + lane] : 0.f;
      if (cr < p.nc) rw[(size_t)cr * p.n + qrow] = val;
      const uint64_t bl = ballot(val > 0.f);
      if ((uint32_t)bl) word |= 1u << acc_row(r, 0);
      if ((uint32_t)(bl >> 32)) word |= 1u << acc_row(r, 1);
    }
    if (lane == 0) mwords[w][jb] = word;
  }
  __syncthreads();
  if (w == 0 && lane < p.Wc) {
    uint32_t word = 0;
#pragma unroll
    for (int v = 0; v < DASH_WAVES; ++v) word |= mwords[v][lane];
    p.cmask[((size_t)unit * p.Tr + t) * p.Wc + lane] = word;
  }
}

// ================================================================================ stage 2
// waves per SIMD the stage-2 register budget is held to (bf16: two, so one wave's exponentials
// overlap the other's matrix products; fp32 operands would spill at two)
template <typename T>
constexpr int dash_attn_occ() { return sizeof(T) == 2 ? 2 : 1; }

template <typename T, int D>
__global__ __launch_bounds__((64 * DASH_WAVES), (dash_attn_occ<T>())) void k_dash_attn(DashParams p) {
  using Ops = KvOps<T, D>;
  constexpr int DS = D / 16, DC = D / 32;
  const int U = p.b * p.hkv;
  const int per_tile = U * p.G;
  const int bid = blockIdx.x;
  if (bid >= per_tile * p.Tr) return;           // whole work group
  const int t = p.Tr - 1 - bid / per_tile;      // longest rows first
  const int rem = bid % per_tile;
  const int unit = rem / p.G;
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const size_t bh = (size_t)bi * p.hq + kvh * p.G + rem % p.G;
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int row0 = t * 64 + w * 32;
  const int qrow = row0 + c;
  const int n = p.n;
  const int spc = p.C / 32;                     // 32-key sub-blocks per chunk
  const int md = (t * 64) / p.C;                // the diagonal chunk

  const T* Q = reinterpret_cast<const T*>(p.q) + bh * n * D;
  const T* Kf = reinterpret_cast<const T*>(p.kf) + (size_t)unit * n * D;
  const T* Vf = reinterpret_cast<const T*>(p.vf) + (size_t)unit * n * D;
  const float* wcol = p.rw + (size_t)unit * p.nc * n + qrow;   // + chunk * n
  const uint32_t* mw = p.cmask + ((size_t)unit * p.Tr + t) * p.Wc;
  Frag<T> qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) load_frag(qf[s], Q + (size_t)qrow * D + 16 * s + 8 * h);

  // the walk: the diagonal run of sub-blocks, then one run per routed chunk. The weights of
  // the next chunk in the mask are read one chunk ahead, so their latency hides under the
  // current chunk's products.
  int kb = md * spc, kb_end = row0 / 32 + 1;
  float bias = 0.f;                              // base-2 prior of the current run
  int wi = 0;
  uint32_t word = uniform_u32(mw[0]);
  int ch_next = -1;
  float wv_next = 0.f;
  auto fetch_next = [&]() {
    while (word == 0) {
      if (++wi >= p.Wc) {
        ch_next = -1;
        return;
      }
      word = uniform_u32(mw[wi]);
    }
    ch_next = wi * 32 + __builtin_ctz(word);
    word &= word - 1;
    wv_next = wcol[(size_t)ch_next * n];
  };
  auto next_run = [&]() -> bool {
    while (ch_next >= 0) {
      const int ch = ch_next;
      const float wv = wv_next;
      fetch_next();
      if (ballot(wv > 0.f) == 0) continue;       // no row of this wave routes it
      bias = wv > 0.f ? p.sigma * log2f(wv) : -INFINITY;
      kb = ch * spc;
      kb_end = kb + spc;
      return true;
    }
    return false;
  };
  fetch_next();

  f32x16 oacc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) oacc[dc] = f32x16{};
  float mrun = -INFINITY, l = 0.f;
  Frag<T> kf[DS];
  Ops::load_k(kf, Kf, kb, c, h);
  bool more = true;
  while (more) {
    const int kcur = kb;
    const float bcur = bias;
    Frag<T> kc[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) kc[s] = kf[s];
    if (++kb >= kb_end) more = next_run();
    if (more) Ops::load_k(kf, Kf, kb, c, h);
    Frag<T> vf[DC][2];
    const T* vp = Vf + (size_t)kcur * (DC * 1024);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) load_frag(vf[dc][mm], vp + (dc * 2 + mm) * 512 + lane * 8);
    f32x16 s = Ops::scores(kc, qf, kcur, row0, qrow, h, true);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = fmaf(p.c2, s[r], bcur);
    float tm = max16(s);
    tm = fmaxf(tm, xor32f(tm));
    const float mnew = fmaxf(mrun, tm);
    if (mnew > mrun) {
      const float sc = exp2f(mrun - mnew);
      l *= sc;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) oacc[dc] *= sc;
      mrun = mnew;
    }
    const float msub = mrun == -INFINITY ? 0.f : mrun;
    f32x16 pw;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pw[r] = exp2f(s[r] - msub);
      l += pw[r];
    }
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      Frag<T> pf;
      acc_frag(pf, pw, mm);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) mma16(oacc[dc], vf[dc][mm], pf);
    }
  }

  const float lt = l + xor32f(l);
  const float inv = 1.0f / lt;
  float* orow = p.o + (bh * n + qrow) * D;
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * dc + 8 * g4 + 4 * h;
      store4(orow + d0, oacc[dc][4 * g4 + 0] * inv, oacc[dc][4 * g4 + 1] * inv, oacc[dc][4 * g4 + 2] * inv,
             oacc[dc][4 * g4 + 3] * inv);
    }
  if (p.lse && h == 0) p.lse[bh * n + qrow] = (mrun + log2f(lt)) * 0.69314718055994531f;
}

// ================================================================================ launch
template <typename T, int D>
static hipError_t launch_dash_t(const DashParams& p, int mode, hipStream_t s) {
  const int U = p.b * p.hkv;
  if (U == 0 || p.Tr == 0) return hipSuccess;
  if (p.Wc > DASH_NB) return hipErrorInvalidConfiguration;
  void (*route)(DashParams) = mode == 1 ? k_dash_route<T, D, 1> : mode == 2 ? k_dash_route<T, D, 2>
                                                                           : k_dash_route<T, D, 0>;
  const size_t lds = (size_t)DASH_WAVES * p.Wc * 1024 * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)route, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  prof_begin("dash_route", s);
  hipLaunchKernelGGL(route, dim3(U * p.Tr), dim3(64 * DASH_WAVES), lds, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin("dash_attn", s);
  hipLaunchKernelGGL((k_dash_attn<T, D>), dim3(U * p.G * p.Tr), dim3(64 * DASH_WAVES), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_dash(const DashParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_dash_t<__bf16, 64>(p, mode, s) : launch_dash_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_dash_t<float, 64>(p, mode, s) : launch_dash_t<float, 128>(p, mode, s);
}

}  // namespace entmax

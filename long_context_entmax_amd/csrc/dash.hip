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
      const float sc = exp2_fast(mrun - mnew);
      l *= sc;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) oacc[dc] *= sc;
      mrun = mnew;
    }
    const float msub = mrun == -INFINITY ? 0.f : mrun;
    f32x16 pw;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pw[r] = exp2_fast(s[r] - msub);
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

// ================================================================================ backward
// The backward of stages 1-2 (DashAttention (it), stage 1: gradients flow back through the
// routing to the chunk summaries). Stage 2 is softmax attention over the 64 x 64 blocks that
// the routing and the diagonal branch select, with the prior sigma ln wbar as a per-(row,
// chunk) additive term; its backward runs in the attention backward kernels (bwd.hip, mode
// 3, on 32-row query blocks: rows of a block route different chunks, and the union over 32
// rows is the forward's visiting granularity too), which also leave, per row and 32-key sub-block, the sum of dS: the gradient of the
// prior terms. Here:
//   k_dash_bwd_fine, k_dash_bwd_setup -- the stage-2 block mask of each query head at 32 x 64
//     (a key block is set when its chunk is routed by some row of the 32-row block, or it
//     lies in the block's own chunk at or before the block), the prior table sigma log2 wbar
//     and the rows' lse in base-2 units;
//   k_dash_dw -- dwbar(c, i) = sigma / wbar(c, i) * (the group's dS sums over chunk c), and
//     each head's routing weights take dwbar / G (stored as dw);
//   k_dash_route_bwd -- per (batch, KV head, 64-row tile), a wave per 32 rows as in the
//     routing forward: through the alpha-entmax Jacobian diag(g) - g g^T / sum g (g =
//     [x - tau]_+^(kappa - 1), the forward's tau) the routing logits get
//     du = g (dw - (g . dw) / sum g), stored for the summaries' gradient, and dQ = stage-2 dQ
//     + gamma scale du . ksum (on the matrix cores, the forward's logit tiles);
//   k_dash_dks -- the summaries' gradient, dksum(c) = gamma scale sum over the group's heads
//     and rows of du(c, i) q_i, as a matrix product contracted over rows (Q^T from its
//     fragment-major column copy, du^T as the B operand), one partial per (32-chunk block,
//     piece of rows); k_dash_dks_reduce adds the pieces in order.

// The chunk bits of each 32-row block: a half-wave per word, lane l of the half reads the
// block's 32 weights of chunk 32 wi + l (one 128-byte line) and the ballot packs the bits.
__global__ void k_dash_bwd_fine(DashParams p) {
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int R = p.n / 32;
  const size_t words = (size_t)p.b * p.hkv * R * p.Wc;
  const bool in = id < words * 32;
  const int l = (int)(id & 31);
  const size_t word = id >> 5;
  bool on = false;
  if (in) {
    const int wi = (int)(word % p.Wc);
    const int rb = (int)((word / p.Wc) % R);
    const size_t unit = word / ((size_t)p.Wc * R);
    const int ch = 32 * wi + l;
    if (ch < p.nc) {
      const f32x4* wr = reinterpret_cast<const f32x4*>(p.rw + (unit * p.nc + ch) * p.n + 32 * rb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = wr[j];
        on |= (v[0] > 0.f) | (v[1] > 0.f) | (v[2] > 0.f) | (v[3] > 0.f);
      }
    }
  }
  const unsigned long long bal = __ballot(on);
  if (in && l == 0) p.fine[word] = (uint32_t)(bal >> (threadIdx.x & 32));
}

// The stage-2 block mask at 32 x 64 (a key block is set when some row of the 32-row block
// routes its chunk, or it lies in the block's own chunk at or before the block), the prior
// table sigma log2 wbar and the rows' lse in base-2 units.
__global__ void k_dash_bwd_setup(DashParams p) {
  const int Tb = p.n / 64, R = p.n / 32;
  const size_t words = (size_t)p.b * p.hq * R * p.W;
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < words) {
    const int wi = (int)(id % p.W);
    const int I = (int)((id / p.W) % R);
    const size_t bh = id / ((size_t)p.W * R);
    const int bi = (int)(bh / p.hq), head = (int)(bh % p.hq);
    const int unit = bi * p.hkv + head / p.G;
    const int m = (I * 32) / p.C;                 // the block's own chunk (every row shares it)
    const uint32_t* fw = p.fine + ((size_t)unit * R + I) * p.Wc;
    uint32_t word = 0;
    for (int b = 0; b < 32; ++b) {
      const int J = wi * 32 + b;
      if (J >= Tb) break;
      const int cJ = (J * 64) / p.C;
      bool on;
      if (cJ < m) on = (fw[cJ >> 5] >> (cJ & 31)) & 1u;
      else on = cJ == m && J * 64 <= I * 32 + 31;
      word |= (on ? 1u : 0u) << b;
    }
    p.bmask[id] = word;
    return;
  }
  const size_t cells = (size_t)p.b * p.hkv * p.nc * p.n;
  const size_t e = id - words;
  if (e < cells) {
    const float wv = p.rw[e];
    p.lp[e] = wv > 0.f ? p.sigma * log2f(wv) : -INFINITY;
    return;
  }
  const size_t r = e - cells;
  if (r < (size_t)p.b * p.hq * p.n) p.lse2[r] = p.lse_in[r] * 1.44269504088896341f;
}

// dw(c, i) of a (unit, chunk, row): sigma / (G wbar) times the dS sums of the group's heads
// over the chunk's sub-blocks (heads in order, sub-blocks in order); 0 off the support
__global__ void k_dash_dw(DashParams p) {
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int n = p.n;
  if (id >= (size_t)p.b * p.hkv * p.nc * n) return;
  const int i = (int)(id % n);
  const int cc = (int)((id / n) % p.nc);
  const size_t unit = id / ((size_t)n * p.nc);
  const float wv = p.rw[id];
  float out = 0.f;
  if (wv > 0.f) {
    const int SB = p.C / 32;
    const size_t bh0 = (unit / p.hkv) * p.hq + (unit % p.hkv) * p.G;
    float s = 0.f;
    for (int g = 0; g < p.G; ++g) {
      const float* db = p.dbias + ((bh0 + g) * (size_t)(n >> 5) + (size_t)cc * SB) * n + i;
      float sm = 0.f;
      for (int u = 0; u < SB; ++u) sm += db[(size_t)u * n];
      s += sm;
    }
    out = p.sigma / (float)p.G * s / wv;
  }
  p.dw[id] = out;
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(64 * DASH_WAVES) void k_dash_route_bwd(DashParams p) {
  constexpr int DS = D / 16, DC = D / 32;
  const int U = p.b * p.hkv;
  const int bid = blockIdx.x;
  if (bid >= U * p.Tr) return;
  const int t = p.Tr - 1 - bid / U;
  const int unit = bid % U;
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int n = p.n;
  const int qrow = t * 64 + w * 32 + c;
  const int m = (t * 64) / p.C;
  const int nb = (m + 31) >> 5;
  const T* Ks = reinterpret_cast<const T*>(p.ks) + (size_t)unit * p.nc * D;
  const float* dwr = p.dw + (size_t)unit * p.nc * n + qrow;   // + chunk * n
  const float kappa = p.kappa;

  Frag<T> eye[2];
  eye_frags(eye, c, h);
  for (int g = 0; g < p.G; ++g) {
    const size_t bh = (size_t)bi * p.hq + kvh * p.G + g;
    f32x16 dqr[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) dqr[dc] = f32x16{};
    float* du = p.du + bh * p.nc * n;
    if (m > 0) {
      const T* Q = reinterpret_cast<const T*>(p.q) + bh * n * D;
      Frag<T> qf[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) load_frag(qf[s], Q + (size_t)qrow * D + 16 * s + 8 * h);
      const float tau = p.rtau[bh * n + qrow];
      // the routing logits of the forward (same products, same order), chunk block jb
      auto logits = [&](int jb, Frag<T> (&kf)[DS]) -> f32x16 {
        const int ch = 32 * jb + c;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          if (ch < m) load_frag(kf[s], Ks + (size_t)ch * D + 16 * s + 8 * h);
          else zero_frag(kf[s]);
        }
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < DS; ++s) mma16(acc, kf[s], qf[s]);
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (32 * jb + acc_row(r, h) < m) ? p.cx * acc[r] : -INFINITY;
        return x;
      };
      auto dwv = [&](int jb, f32x16& v) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = 32 * jb + acc_row(r, h);
          v[r] = cr < m ? dwr[(size_t)cr * n] : 0.f;
        }
      };
      // delta = (g . dw) / sum g over the row's chunks
      float sg = 0.f, sgd = 0.f;
      for (int jb = 0; jb < nb; ++jb) {
        Frag<T> kf[DS];
        f32x16 dv;
        dwv(jb, dv);
        const f32x16 x = logits(jb, kf);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float gg = Weight<MODE>::g(fmaxf(x[r] - tau, 0.f), kappa);
          sg += gg;
          sgd += gg * dv[r];
        }
      }
      sg += xor32f(sg);
      sgd += xor32f(sgd);
      const float delta = sgd / sg;
      for (int jb = 0; jb < nb; ++jb) {
        Frag<T> kf[DS];
        f32x16 dv;
        dwv(jb, dv);
        const f32x16 x = logits(jb, kf);
        f32x16 dz;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float gg = Weight<MODE>::g(fmaxf(x[r] - tau, 0.f), kappa);
          dz[r] = gg * (dv[r] - delta);
          const int cr = 32 * jb + acc_row(r, h);
          if (cr < p.nc) du[(size_t)cr * n + qrow] = dz[r];
        }
        // dQ^T[d][q] += ksum^T dz^T (the logit tile as the B operand)
        Frag<T> kt[2][DC];
        rows_to_cols<T, DS>(kt, kf, eye);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          Frag<T> zf;
          acc_frag(zf, dz, mm);
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) mma16(dqr[dc], kt[mm][dc], zf);
        }
      }
    }
    // chunks the row does not route (its own and later ones): no gradient
    for (int jb = nb; 32 * jb < p.nc; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int cr = 32 * jb + acc_row(r, h);
        if (cr < p.nc) du[(size_t)cr * n + qrow] = 0.f;
      }
    // dQ = stage-2 dQ + gamma scale dz . ksum
    const float* d32 = p.dq32 + (bh * n + qrow) * D;
    T* dQ = reinterpret_cast<T*>(p.dq) + (bh * n + qrow) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dc + 8 * g4 + 4 * h;
        const f32x4 a = *reinterpret_cast<const f32x4*>(d32 + d0);
        store4(dQ + d0, a[0] + p.gs * dqr[dc][4 * g4], a[1] + p.gs * dqr[dc][4 * g4 + 1],
               a[2] + p.gs * dqr[dc][4 * g4 + 2], a[3] + p.gs * dqr[dc][4 * g4 + 3]);
      }
  }
}

// Partial summary gradients: work group (unit, 32-chunk block cb, row piece pc); its four
// waves take the 32-row blocks of the piece in turn, for every head of the group, and add
// dksum^T[d][c] += sum_i Q^T[d][i] du^T[i][c]. Rows before (32 cb + 1) C route none of the
// block's chunks (du is 0 there) and are not visited.
constexpr int DKS_WAVES = 4;

template <typename T, int D>
__global__ __launch_bounds__(64 * DKS_WAVES) void k_dash_dks(DashParams p) {
  constexpr int DC = D / 32;
  __shared__ float red[(DKS_WAVES - 1) * DC * 16 * 64];
  const int U = p.b * p.hkv;
  const int bid = blockIdx.x;
  if (bid >= U * p.Wc * p.NP) return;
  const int unit = bid % U;
  const int cb = (bid / U) % p.Wc;
  const int pc = bid / (U * p.Wc);
  const int n = p.n;
  const int start = (32 * cb + 1) * p.C;        // first row that routes a chunk of the block
  const int r0 = max(pc * p.PR, start), r1 = min((pc + 1) * p.PR, n);
  if (r0 >= r1) return;                         // whole work group (the reduction skips it)
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int ch = 32 * cb + c;
  const bool live = ch < p.nc;
  f32x16 acc[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) acc[dc] = f32x16{};
  for (int g = 0; g < p.G; ++g) {
    const size_t bh = (size_t)bi * p.hq + kvh * p.G + g;
    const T* Qc = reinterpret_cast<const T*>(p.qc) + bh * n * D;
    const float* du = p.du + (bh * p.nc + (live ? ch : 0)) * n;
    for (int b = r0 / 32 + w; b < r1 / 32; b += DKS_WAVES) {
      Frag<T> a[DC][2], bf[2];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) load_frag(a[dc][mm], Qc + ((size_t)((b * DC + dc) * 2 + mm) * 64 + lane) * 8);
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        // rows 16 mm + sigma(8 h + j) of the block: two runs of four
        if (live) {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(du + 32 * b + 16 * mm + 4 * h);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(du + 32 * b + 16 * mm + 8 + 4 * h);
          set_frag(bf[mm], lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]);
        } else {
          zero_frag(bf[mm]);
        }
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16(acc[dc], a[dc][mm], bf[mm]);
    }
  }
  // the waves' sums in order (wave 0 + 1 + 2 + 3)
  if (w > 0) {
    float* dst = red + (size_t)(w - 1) * DC * 16 * 64;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(dc * 16 + r) * 64 + lane] = acc[dc][r];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int v = 0; v < DKS_WAVES - 1; ++v)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dc][r] += red[((size_t)v * DC * 16 + dc * 16 + r) * 64 + lane];
    // accumulator rows are d, columns the block's chunks
    float* out = p.dpart + (((size_t)unit * p.Wc + cb) * p.NP + pc) * D * 32;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[(32 * dc + acc_row(r, h)) * 32 + c] = acc[dc][r];
  }
}

// dksum(unit, chunk, d) = gamma scale * the pieces' partials in order
template <typename T, int D>
__global__ void k_dash_dks_reduce(DashParams p) {
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int U = p.b * p.hkv;
  if (id >= (size_t)U * p.Wc * D * 32) return;
  const int c = (int)(id & 31);
  const int d = (int)((id >> 5) % D);
  const int cb = (int)((id / (32 * D)) % p.Wc);
  const int unit = (int)(id / ((size_t)32 * D * p.Wc));
  const int ch = 32 * cb + c;
  if (ch >= p.nc) return;
  // the pieces whose work groups ran: from the one holding the block's first routing row on
  // (none when no row routes a chunk of the block)
  const int start = (32 * cb + 1) * p.C;
  const int p0 = start < p.n ? start / p.PR : p.NP;
  const float* part = p.dpart + ((size_t)unit * p.Wc + cb) * p.NP * D * 32 + d * 32 + c;
  float tot = 0.f;
  for (int pc = p0; pc < p.NP; ++pc) tot += part[(size_t)pc * D * 32];
  reinterpret_cast<T*>(p.dks)[((size_t)unit * p.nc + ch) * D + d] = (T)(p.gs * tot);
}

hipError_t launch_dash_bwd_setup(const DashParams& p, hipStream_t s) {
  const size_t lanes = (size_t)p.b * p.hkv * (p.n / 32) * p.Wc * 32;
  const size_t items = (size_t)p.b * p.hq * (p.n / 32) * p.W + (size_t)p.b * p.hkv * p.nc * p.n +
                       (size_t)p.b * p.hq * p.n;
  if (items == 0) return hipSuccess;
  prof_begin("dash_bwd_setup", s);
  hipLaunchKernelGGL(k_dash_bwd_fine, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess)
    hipLaunchKernelGGL(k_dash_bwd_setup, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, p);
  prof_end(s);
  return e != hipSuccess ? e : hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dash_route_bwd_t(const DashParams& p, int mode, hipStream_t s) {
  const int U = p.b * p.hkv;
  if (U == 0 || p.Tr == 0) return hipSuccess;
  const size_t cells = (size_t)U * p.nc * p.n;
  prof_begin("dash_dw", s);
  hipLaunchKernelGGL(k_dash_dw, dim3((unsigned)((cells + 255) / 256)), dim3(256), 0, s, p);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void (*fn)(DashParams) = mode == 1 ? k_dash_route_bwd<T, D, 1> : mode == 2 ? k_dash_route_bwd<T, D, 2>
                                                                            : k_dash_route_bwd<T, D, 0>;
  prof_begin("dash_route_bwd", s);
  hipLaunchKernelGGL(fn, dim3(U * p.Tr), dim3(64 * DASH_WAVES), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin("dash_dks", s);
  hipLaunchKernelGGL((k_dash_dks<T, D>), dim3(U * p.Wc * p.NP), dim3(64 * DKS_WAVES), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t outs = (size_t)U * p.Wc * D * 32;
  prof_begin("dash_dks_reduce", s);
  hipLaunchKernelGGL((k_dash_dks_reduce<T, D>), dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_dash_route_bwd(const DashParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (dtype == 1)
    return D == 64 ? launch_dash_route_bwd_t<__bf16, 64>(p, mode, s) : launch_dash_route_bwd_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_dash_route_bwd_t<float, 64>(p, mode, s) : launch_dash_route_bwd_t<float, 128>(p, mode, s);
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

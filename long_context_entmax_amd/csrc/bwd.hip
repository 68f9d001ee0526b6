// Backward of alpha-entmax attention: dK/dV per key block and dQ per query tile, each
// walking only the set bits of the block mask (AdaSplash-2 pages, AdaSplash-2 (zh) §2.3 and
// AdaSplash-2 (ja) §2.3: the mask lets the backward skip all-zero blocks; local accumulators
// instead of atomics).
//
// Gradient (the exact alpha-entmax Jacobian; the pages do not spell it out): with
// x = (alpha-1) s, d = [x - tau]_+, p = d^kappa, g = d^(kappa-1), dP_ij = dO_i . v_j and
// delta_i = dO_i . o~_i,
//   dS_ij = g_ij (dP_ij - delta_i),  dq_i = scale sum_j dS_ij k_j,
//   dk_j  = scale sum_i dS_ij q_i,   dv_j = sum_i p_ij dO_i.
//
// Every operand is read from a fragment-major rows copy (lanes walk rows, 8 consecutive
// head-dimension elements per lane), so a wave's operand load is one contiguous 1 KB run at
// a wave-uniform base plus lane * 16 bytes. The operands of the products contracted over
// rows (Q^T and dO^T in dK/dV, K^T in dQ: lanes walk the head dimension, 8 rows per lane in
// accumulator order) are formed from those same fragments on the matrix core
// (rows_to_cols, an exact copy), so each item's Q, dO or K rows come from memory once.
//
// k_bwd_dkv: one work group per (batch, KV head, key block J). Wave w owns the 32-key
// sub-block w % KC of J and every NS-th item of the list (query head of the GQA group,
// query tile with bit J set, 32-row chunk); K and V of the sub-block stay in registers,
// dK and dV accumulate in registers and the waves that share a sub-block add their sums
// in LDS in a fixed order (deterministic, no atomics).
// k_bwd_dq: one work group per (batch, query head, query tile I); wave w owns the 32-row
// chunk w % QCB and every NS-th (key block, 32-key sub-block) item of row I's bits.
#include "common.hpp"
#include "kernels.hpp"

namespace entmax {

namespace {

// offset (in elements) of a wave's operand fragment in a fragment-major copy
__device__ __forceinline__ size_t rows_off(int blk32, int s, int DS, int lane) {
  return ((size_t)(blk32 * DS + s) * 64 + lane) * 8;
}

}  // namespace

template <typename T, int D, int MODE, bool BIAS>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void k_bwd_dkv(BwdParams p) {
  constexpr int DS = D / 16, DC = D / 32;
  extern __shared__ float red[];
  int unit, rank;
  if (!wgmap_get(p.map, blockIdx.x, unit, rank)) return;
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int J = rank;
  const int KC = p.Bc / 32, NS = 4 / KC;
  const int ks = w % KC, slot = w / KC;
  const int key0 = J * p.Bc + 32 * ks;
  const int n = p.n;
  const int QCB = p.Br / 32;
  const float cx = p.cx, kappa = p.kappa;

  const size_t kvoff = (size_t)(bi * p.hkv + kvh) * n * D;
  const T* Kr = reinterpret_cast<const T*>(p.kr) + kvoff;
  const T* Vr = reinterpret_cast<const T*>(p.vr) + kvoff;
  Frag<T> kb[DS], vb[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    load_frag(kb[s], Kr + rows_off(key0 >> 5, s, DS, lane));
    load_frag(vb[s], Vr + rows_off(key0 >> 5, s, DS, lane));
  }
  f32x16 dk[DC], dv[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    dk[dc] = f32x16{};
    dv[dc] = f32x16{};
  }
  Frag<T> eye[2];
  eye_frags(eye, c, h);

  // This wave's items in list order: for each query head g of the group, each query tile I
  // with bit J in the head's column mask, each 32-row chunk qc of I -- every NS-th, none
  // above the diagonal. The next item's Q rows (the first operand needed) are loaded while
  // the current item is multiplied.
  // Under the causal mask the query tiles before the one holding key J*Bc have no bit: the
  // walk over each head's words starts at that tile's word.
  const int ws = p.causal ? ((J * p.Bc / p.Br) >> 5) : 0;
  int t = 0, g = 0, wi = ws, I = 0, qc = QCB;
  const uint32_t* colw = p.maskT + ((size_t)(bi * p.hq + kvh * p.G) * p.Tc + J) * p.WT;
  uint32_t word = uniform_u32(colw[ws]);
  auto next_item = [&](int& gi, int& q0i) -> bool {
    for (;;) {
      if (qc >= QCB) {
        while (word == 0) {
          if (++wi >= p.WT) {
            if (++g >= p.G) return false;
            wi = ws;
            colw = p.maskT + ((size_t)(bi * p.hq + kvh * p.G + g) * p.Tc + J) * p.WT;
          }
          word = uniform_u32(colw[wi]);
        }
        I = wi * 32 + __builtin_ctz(word);
        word &= word - 1;
        qc = 0;
      }
      const int q0c = I * p.Br + 32 * qc;
      ++qc;
      const bool mine = (t++ & (NS - 1)) == slot;   // NS is 1, 2 or 4
      if (!mine || (p.causal && key0 > q0c + 31)) continue;   // sub-tile above the diagonal
      gi = g;
      q0i = q0c;
      return true;
    }
  };
  auto row_base = [&](int gi) -> size_t { return (size_t)(bi * p.hq + kvh * p.G + gi) * n; };
  int g_next = 0, q0_next = 0;
  bool have = next_item(g_next, q0_next);
  // (head_dim 128, one wave per SIMD: the dO rows too)
  constexpr bool DEEP = D == 128;
  Frag<T> qn[DS], dn[DEEP ? DS : 1];
  // a head's Q and dO rows through buffer resources (a fixed lane offset, a scalar row
  // offset: no vector address arithmetic per fragment)
  using Ops = KvOps<T, D>;
  const uint32_t head_bytes = (uint32_t)((size_t)n * D * sizeof(T));
  auto load_rows = [&](int gi, int q0i) {
    const T* Qr = reinterpret_cast<const T*>(p.qr) + row_base(gi) * D;
    Ops::load_k_buf(qn, buffer_rsrc(Qr, head_bytes), q0i >> 5, lane);
    if constexpr (DEEP) {
      const T* DOn = reinterpret_cast<const T*>(p.dor) + row_base(gi) * D;
      Ops::load_k_buf(dn, buffer_rsrc(DOn, head_bytes), q0i >> 5, lane);
    }
  };
  if (have) load_rows(g_next, q0_next);
  while (have) {
    const int gc = g_next, q0 = q0_next;
    const int head = kvh * p.G + gc;
    const size_t qrow0 = row_base(gc);
    const T* DOr = reinterpret_cast<const T*>(p.dor) + qrow0 * D;
    const float cm = BIAS ? p.slopes[head] * p.am1 : 0.0f;   // position bias on the x-scale
    const int qb = q0 >> 5;
    Frag<T> qa[DS], da[DS];
    f32x4 tv[4], dl[4];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qa[s] = qn[s];
      if constexpr (DEEP) da[s] = dn[s];
    }
    if constexpr (!DEEP) Ops::load_k_buf(da, buffer_rsrc(DOr, head_bytes), qb, lane);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      tv[g4] = *reinterpret_cast<const f32x4*>(p.tau + qrow0 + q0 + 8 * g4 + 4 * h);
      dl[g4] = *reinterpret_cast<const f32x4*>(p.delta + qrow0 + q0 + 8 * g4 + 4 * h);
    }
    // the next item's rows are loaded on every item (the current item's again after the
    // last), so the wait before an operand counts a fixed number of newer loads and does
    // not drain the prefetch
    have = next_item(g_next, q0_next);
    load_rows(have ? g_next : gc, have ? q0_next : q0);
    f32x16 S = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(S, qa[s], kb[s]);   // S[q][key]
    // -tau of each entry's row (and the position bias): x - tau = cx S + off
    f32x16 off;
#pragma unroll
    for (int r = 0; r < 16; ++r) off[r] = -tv[r >> 2][r & 3];
    if (BIAS && cm != 0.0f) {
      const f32x16 bb = bias16<1>(0.0f, cm, (float)(q0 + 4 * h - key0 - c), p.causal);
#pragma unroll
      for (int r = 0; r < 16; ++r) off[r] += bb[r];
    }
    // P and G; rows 8(r/4) + 4h + r%4 of the chunk, key c of the sub-block
    const bool diag = p.causal && key0 + 31 > q0;
    f32x16 P, G;
    float mx = 0.f;
    if constexpr (MODE == MODE_DASH) {
      // softmax with the routing prior, in base-2 units (cx = scale log2 e, tau = lse log2 e,
      // lp = sigma log2 wbar): P = 2^(cx s - tau + lp) on a routed chunk, 2^(cx s - tau) on
      // the query's own chunk (keys after the query masked); dS = P (dP - delta) is the
      // softmax backward, so G = P
      // (the walk visits a sub-tile only when some row of its 32 routes the chunk, or on the
      // diagonal, so no sub-tile is all zero and none is skipped)
      const int cJ = key0 / p.C;
      if (q0 / p.C != cJ) {
        const float* lr = p.lp + ((size_t)(bi * p.hkv + kvh) * (n / p.C) + cJ) * n + q0;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 lv = *reinterpret_cast<const f32x4*>(lr + 8 * g4 + 4 * h);
#pragma unroll
          for (int j = 0; j < 4; ++j) P[4 * g4 + j] = exp2_fast(fmaf(cx, S[4 * g4 + j], lv[j] - tv[g4][j]));
        }
      } else if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          P[r] = exp2_fast(key0 + c > q0 + acc_row(r, h) ? -INFINITY : fmaf(cx, S[r], -tv[r >> 2][r & 3]));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) P[r] = exp2_fast(fmaf(cx, S[r], -tv[r >> 2][r & 3]));
      }
      G = P;
    } else if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float tt = fmaf(cx, S[r], off[r]);
        tt = (key0 + c <= q0 + acc_row(r, h)) ? tt : -1.0f;
        const float dm = relu_raw(tt);
        P[r] = Weight<MODE>::p(dm, kappa);
        G[r] = Weight<MODE>::g(dm, kappa);
        mx = fmaxf(mx, dm);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dm = relu_raw(fmaf(cx, S[r], off[r]));
        P[r] = Weight<MODE>::p(dm, kappa);
        G[r] = Weight<MODE>::g(dm, kappa);
        mx = fmaxf(mx, dm);
      }
    }
    if (MODE != MODE_DASH && !p.dense && ballot(mx > 0.f) == 0) continue;   // an all-zero sub-tile
    f32x16 dP = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(dP, da[s], vb[s]);  // dP[q][key]
    f32x16 dS;
#pragma unroll
    for (int r = 0; r < 16; ++r) dS[r] = G[r] * (dP[r] - dl[r >> 2][r & 3]);
    Frag<T> pf[2], sf[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      acc_frag(pf[m], P, m);
      acc_frag(sf[m], dS, m);
    }
    // Q^T and dO^T of the chunk (cols layout), one 32-wide block of the head dimension at a
    // time, each used as soon as it is formed (fewer live registers at head_dim 128)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      f32x16 tq = f32x16{}, td = f32x16{};
      mma16(tq, qa[2 * dc], eye[0]);
      mma16(td, da[2 * dc], eye[0]);
      mma16(tq, qa[2 * dc + 1], eye[1]);
      mma16(td, da[2 * dc + 1], eye[1]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        Frag<T> qt, dt;
        acc_frag(qt, tq, m);
        acc_frag(dt, td, m);
        mma16(dv[dc], dt, pf[m]);   // dV^T[d][key] += dO^T P
        mma16(dk[dc], qt, sf[m]);   // dK^T[d][key] += Q^T dS
      }
    }
  }

  // sum the NS partial accumulators of each sub-block in slot order 0, 1, ...
  float* buf = red + (size_t)ks * (2 * DC * 16 * 64);
  for (int sl = 1; sl < NS; ++sl) {
    __syncthreads();
    if (slot == sl) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          buf[((0 * DC + dc) * 16 + r) * 64 + lane] = dk[dc][r];
          buf[((1 * DC + dc) * 16 + r) * 64 + lane] = dv[dc][r];
        }
    }
    __syncthreads();
    if (slot == 0) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dk[dc][r] += buf[((0 * DC + dc) * 16 + r) * 64 + lane];
          dv[dc][r] += buf[((1 * DC + dc) * 16 + r) * 64 + lane];
        }
    }
  }
  if (slot == 0) {
    const size_t rowoff = ((size_t)(bi * p.hkv + kvh) * n + key0 + c) * D;
    T* dK = reinterpret_cast<T*>(p.dk) + rowoff;
    T* dV = reinterpret_cast<T*>(p.dv) + rowoff;
    const float sc = p.scale;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dc + 8 * g4 + 4 * h;
        store4(dK + d0, sc * dk[dc][4 * g4], sc * dk[dc][4 * g4 + 1], sc * dk[dc][4 * g4 + 2],
               sc * dk[dc][4 * g4 + 3]);
        store4(dV + d0, dv[dc][4 * g4], dv[dc][4 * g4 + 1], dv[dc][4 * g4 + 2], dv[dc][4 * g4 + 3]);
      }
  }
}

template <typename T, int D, int MODE, bool BIAS>
__global__ __launch_bounds__(256, (D == 64 ? ((sizeof(T) == 2 && !BIAS && (MODE == 1 || MODE == 2)) ? 3 : 2) : 1)) void k_bwd_dq(BwdParams p) {
  constexpr int DS = D / 16, DC = D / 32;
  extern __shared__ float red[];
  int unit, rank;
  if (!wgmap_get(p.map, blockIdx.x, unit, rank)) return;
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int bi = unit / p.hkv, kvh = unit % p.hkv;
  const int I = p.causal ? (p.Tr - 1 - rank / p.G) : (rank / p.G);
  const int head = kvh * p.G + rank % p.G;
  const int QCB = p.Br / 32, NS = 4 / QCB;
  const int qc = w % QCB, slot = w / QCB;
  const int KC = p.Bc / 32;
  const int n = p.n;
  const int q0 = I * p.Br + 32 * qc;
  const float cx = p.cx, kappa = p.kappa;

  const size_t qrow0 = (size_t)(bi * p.hq + head) * n;
  const size_t kvoff = (size_t)(bi * p.hkv + kvh) * n * D;
  const T* Kr = reinterpret_cast<const T*>(p.kr) + kvoff;
  const T* Vr = reinterpret_cast<const T*>(p.vr) + kvoff;
  Frag<T> qb[DS], db[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    load_frag(qb[s], reinterpret_cast<const T*>(p.qr) + qrow0 * D + rows_off(q0 >> 5, s, DS, lane));
    load_frag(db[s], reinterpret_cast<const T*>(p.dor) + qrow0 * D + rows_off(q0 >> 5, s, DS, lane));
  }
  const float tq = p.tau[qrow0 + q0 + c];
  const float cm = BIAS ? p.slopes[head] * p.am1 : 0.0f;   // position bias on the x-scale
  const float dq_delta = p.delta[qrow0 + q0 + c];
  f32x16 dq[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) dq[dc] = f32x16{};
  Frag<T> eye[2];
  eye_frags(eye, c, h);

  const uint32_t* roww = p.mask + ((size_t)(bi * p.hq + head) * p.Tr + I) * p.W;
  // This wave's items in list order: the 32-key sub-blocks ks of each set key block J of the
  // row's mask, every NS-th, none above the diagonal. The next item's K fragments (the first
  // operand needed) are loaded while the current item is multiplied.
  // Under the causal mask no key block after the one holding the tile's last row has a bit:
  // the walk ends at that block's word. The mask word after the current one is loaded ahead.
  const int wend = p.causal ? min(p.W, (((I * p.Br + p.Br - 1) / p.Bc) >> 5) + 1) : p.W;
  int wi = 0, t = 0, ks = KC, J = 0;
  uint32_t word = uniform_u32(roww[0]);
  uint32_t wnx = wend > 1 ? uniform_u32(roww[1]) : 0u;
  auto next_item = [&](int& kbk) -> bool {
    for (;;) {
      if (ks >= KC) {
        while (word == 0) {
          if (++wi >= wend) return false;
          word = wnx;
          wnx = wi + 1 < wend ? uniform_u32(roww[wi + 1]) : 0u;
        }
        J = wi * 32 + __builtin_ctz(word);
        word &= word - 1;
        ks = 0;
      }
      const int k0 = J * p.Bc + 32 * ks;
      ++ks;
      const bool mine = (t++ & (NS - 1)) == slot;   // NS is 1, 2 or 4
      if (!mine || (p.causal && k0 > q0 + 31)) continue;   // sub-tile above the diagonal
      kbk = k0 >> 5;
      return true;
    }
  };
  int kb_next = 0;
  bool have = next_item(kb_next);
  // K and V fragments through buffer resources over the KV head's copies: a fixed lane
  // offset and a scalar sub-block offset, so a load needs no vector address arithmetic
  using Ops = KvOps<T, D>;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kr, (uint32_t)((size_t)n * D * sizeof(T)));
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(Vr, (uint32_t)((size_t)n * D * sizeof(T)));
  Frag<T> kn[DS];
  if (have) Ops::load_k_buf(kn, krs, kb_next, lane);
  while (have) {
    const int kbk = kb_next;
    const int key0 = kbk * 32;
    Frag<T> ka[DS], va[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) ka[s] = kn[s];
    Ops::load_k_buf(va, vrs, kbk, lane);
    // loaded on every item (the current sub-block again after the last), so the waits
    // before the current item's operands do not drain the prefetch
    have = next_item(kb_next);
    Ops::load_k_buf(kn, krs, have ? kb_next : kbk, lane);
    f32x16 S = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(S, ka[s], qb[s]);   // S^T[key][q]
    // x - tau = cx S + off (the row's -tau and the position bias)
    f32x16 off;
    if (BIAS && cm != 0.0f) {
      off = bias16<-1>(-tq, cm, (float)(q0 + c - key0 - 4 * h), p.causal);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) off[r] = -tq;
    }
    const bool diag = p.causal && key0 + 31 > q0;
    f32x16 G;
    float mx = 0.f;
    if constexpr (MODE == MODE_DASH) {
      // softmax with the routing prior in base-2 units (see k_bwd_dkv); G = P
      const int cJ = key0 / p.C;
      float pr = -tq;
      if (q0 / p.C != cJ) pr += p.lp[((size_t)(bi * p.hkv + kvh) * (n / p.C) + cJ) * n + q0 + c];
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          G[r] = exp2_fast(key0 + acc_row(r, h) > q0 + c ? -INFINITY : fmaf(cx, S[r], pr));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) G[r] = exp2_fast(fmaf(cx, S[r], pr));
      }
    } else if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float tt = fmaf(cx, S[r], off[r]);
        tt = (key0 + acc_row(r, h) <= q0 + c) ? tt : -1.0f;
        const float dm = relu_raw(tt);
        G[r] = Weight<MODE>::g(dm, kappa);
        mx = fmaxf(mx, dm);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dm = relu_raw(fmaf(cx, S[r], off[r]));
        G[r] = Weight<MODE>::g(dm, kappa);
        mx = fmaxf(mx, dm);
      }
    }
    // (mode 3: the row's sum of dS over the sub-block, the gradient of its prior term)
    float* const dbr = MODE == MODE_DASH ? p.dbias + ((size_t)(bi * p.hq + head) * (n >> 5) + kbk) * n + q0 + c
                                         : nullptr;
    if (MODE != MODE_DASH && !p.dense && ballot(mx > 0.f) == 0) continue;   // an all-zero sub-tile
    f32x16 dP = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(dP, va[s], db[s]);   // dP^T[key][q]
    f32x16 dS;
#pragma unroll
    for (int r = 0; r < 16; ++r) dS[r] = G[r] * (dP[r] - dq_delta);
    if constexpr (MODE == MODE_DASH) {
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) rs += dS[r];
      rs += xor32f(rs);
      if (h == 0) *dbr = rs;
    }
    Frag<T> kt[2][DC];                   // K^T of the sub-block (cols layout)
    rows_to_cols<T, DS>(kt, ka, eye);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      Frag<T> sf;
      acc_frag(sf, dS, m);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) mma16(dq[dc], kt[m][dc], sf);   // dQ^T[d][q] += K^T dS^T
    }
  }

  float* buf = red + (size_t)qc * (DC * 16 * 64);
  for (int sl = 1; sl < NS; ++sl) {
    __syncthreads();
    if (slot == sl) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int r = 0; r < 16; ++r) buf[(dc * 16 + r) * 64 + lane] = dq[dc][r];
    }
    __syncthreads();
    if (slot == 0) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[dc][r] += buf[(dc * 16 + r) * 64 + lane];
    }
  }
  if (MODE == MODE_DASH && slot == 0) {
    // stage-2 dQ in fp32; the routing backward adds its share and writes dQ
    float* dQ = p.dq32 + (qrow0 + q0 + c) * D;
    const float sc = p.scale;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dc + 8 * g4 + 4 * h;
        *reinterpret_cast<f32x4*>(dQ + d0) = f32x4{sc * dq[dc][4 * g4], sc * dq[dc][4 * g4 + 1],
                                                  sc * dq[dc][4 * g4 + 2], sc * dq[dc][4 * g4 + 3]};
      }
  } else if (slot == 0) {
    T* dQ = reinterpret_cast<T*>(p.dq) + (qrow0 + q0 + c) * D;
    const float sc = p.scale;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dc + 8 * g4 + 4 * h;
        store4(dQ + d0, sc * dq[dc][4 * g4], sc * dq[dc][4 * g4 + 1], sc * dq[dc][4 * g4 + 2],
               sc * dq[dc][4 * g4 + 3]);
      }
  }
}

template <typename T, int D>
static hipError_t launch_dkv_t(const BwdParams& p, int mode, hipStream_t s) {
  const int KC = p.Bc / 32, DC = D / 32;
  const size_t lds = (4 / KC > 1) ? (size_t)KC * 2 * DC * 16 * 64 * sizeof(float) : 0;
  const int grid = wgmap_grid(p.map);
  if (grid == 0) return hipSuccess;
  void (*fn)(BwdParams);
  if (mode == MODE_DASH)
    fn = k_bwd_dkv<T, D, MODE_DASH, false>;
  else if (p.slopes)
    fn = mode == 1 ? k_bwd_dkv<T, D, 1, true> : mode == 2 ? k_bwd_dkv<T, D, 2, true> : k_bwd_dkv<T, D, 0, true>;
  else
    fn = mode == 1 ? k_bwd_dkv<T, D, 1, false> : mode == 2 ? k_bwd_dkv<T, D, 2, false> : k_bwd_dkv<T, D, 0, false>;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq_t(const BwdParams& p, int mode, hipStream_t s) {
  const int QCB = p.Br / 32, DC = D / 32;
  const size_t lds = (4 / QCB > 1) ? (size_t)QCB * DC * 16 * 64 * sizeof(float) : 0;
  const int grid = wgmap_grid(p.map);
  if (grid == 0) return hipSuccess;
  void (*fn)(BwdParams);
  if (mode == MODE_DASH)
    fn = k_bwd_dq<T, D, MODE_DASH, false>;
  else if (p.slopes)
    fn = mode == 1 ? k_bwd_dq<T, D, 1, true> : mode == 2 ? k_bwd_dq<T, D, 2, true> : k_bwd_dq<T, D, 0, true>;
  else
    fn = mode == 1 ? k_bwd_dq<T, D, 1, false> : mode == 2 ? k_bwd_dq<T, D, 2, false> : k_bwd_dq<T, D, 0, false>;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_dkv_t<__bf16, 64>(p, mode, s) : launch_dkv_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_dkv_t<float, 64>(p, mode, s) : launch_dkv_t<float, 128>(p, mode, s);
}

hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_dq_t<__bf16, 64>(p, mode, s) : launch_dq_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_dq_t<float, 64>(p, mode, s) : launch_dq_t<float, 128>(p, mode, s);
}

}  // namespace entmax

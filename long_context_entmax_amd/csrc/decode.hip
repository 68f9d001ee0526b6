// Decode forward of alpha-entmax attention: one new query row per (sequence, query head)
// against a KV cache. The pages leave inference to future work (AdaSplash-2 (ja) §5) and
// DashAttention decodes incrementally on the same primitives (DashAttention (it)); the threshold is
// found exactly as in the forward (AdaSplash-2 (zh) §2.1-2.2, AdaSplash-2 (ja) §2.1-2.2): a
// B-bin histogram of the row's scores gives tau_h (Proposition 1), the safeguarded hybrid
// solver refines it, and o = sum_j p_j v_j with p = [x - tau]_+^(1/(alpha-1)).
//
// MI355X decomposition. One query row is too little work for a wave to stream a long cache
// by itself, so the keys are split in slices (p.split keys), one work group per (slice, KV
// head), and the score row itself is kept: 4 bytes per key and query head against 2 d bytes
// of bf16 K per key and KV head, so the histogram and every refinement pass read the fp32
// scores instead of recomputing them from K.
//   1. k_dec_scores  (slice, KV head): x for the G query heads of the KV head on MFMA (the
//      G query rows padded to 32), stored (each row padded with -inf to whole float4
//      groups), plus the slice's max per row.
//   2. k_dec_hist    (slice, query row): the slice's counts on the row's anchored B-bin grid.
//   3. k_dec_tau     (query row): the summed histogram, tau_h, then the solver passes over
//      the stored scores (work-group reductions in a fixed order: deterministic).
//   4. k_dec_out     (p.osplit-key slice, KV head): p for the G rows, V rows read only for
//      keys where some row has p > 0, partial o per slice (smaller slices than the score
//      kernel: more waves keep V loads in flight).
//   5. k_dec_reduce  (query row): o = sum of the slice partials in a fixed order.
#include "common.hpp"
#include "kernels.hpp"
#include "solver.hpp"

namespace entmax {

namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_TAU_THREADS = 1024;

__device__ __forceinline__ int dec_len(const DecParams& p, int bi) {
  return p.lengths ? min(max(p.lengths[bi], 1), p.n) : p.n;
}

// Wave-wide reductions in a fixed order with DPP row operations (no LDS traffic): butterflies
// within each 16-lane row, then the row totals carried to lane 63; the result is uniform.
#define DEC_DPP(v, ctrl, rmask) __builtin_amdgcn_update_dpp((v), (v), ctrl, rmask, 0xF, false)
template <typename Op>
__device__ __forceinline__ int wave_red(int v, Op op) {
  v = op(v, DEC_DPP(v, 0xB1, 0xF));    // quad_perm [1,0,3,2]
  v = op(v, DEC_DPP(v, 0x4E, 0xF));    // quad_perm [2,3,0,1]
  v = op(v, DEC_DPP(v, 0x141, 0xF));   // row_half_mirror
  v = op(v, DEC_DPP(v, 0x140, 0xF));   // row_mirror
  v = op(v, DEC_DPP(v, 0x142, 0xA));   // row_bcast15 into rows 1 and 3
  v = op(v, DEC_DPP(v, 0x143, 0xC));   // row_bcast31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_fsum(float v) {
  return __int_as_float(wave_red(__float_as_int(v), [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b)); }));
}
__device__ __forceinline__ float wave_fmax(float v) {
  return __int_as_float(wave_red(__float_as_int(v), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b))); }));
}
__device__ __forceinline__ int wave_isum(int v) {
  return wave_red(v, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  return (uint32_t)wave_red((int)v, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
}

// Work-group reductions: each wave's total through LDS, then the NT/64 totals reduced by the
// same DPP steps in lanes 0..15 of every wave (fixed order, the same bits in every wave). The
// LDS slots alternate between two halves (par), so one barrier per reduction suffices: no
// wave can start the reduction after next before every wave has read this one.
constexpr int DEC_RED_SLOTS = 6;
struct DecRed {
  uint32_t v[2][DEC_RED_SLOTS][16];
};
template <int NT>
__device__ __forceinline__ uint32_t wg_gather(const DecRed* r, int par, int k, uint32_t ident) {
  const int lane = threadIdx.x & 63;
  return lane < NT / 64 ? r->v[par][k][lane] : ident;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, DecRed* r, int& par) {
  v = wave_fmax(v);
  if ((threadIdx.x & 63) == 0) r->v[par][0][threadIdx.x >> 6] = __float_as_uint(v);
  __syncthreads();
  v = wave_fmax(__uint_as_float(wg_gather<NT>(r, par, 0, __float_as_uint(-INFINITY))));
  par ^= 1;
  return v;
}

// A pass's row totals in one reduction: sums of F0, F1, Fh and of F2 (general alpha) or the
// support size, and the minimum of the smallest positive gap's bits.
template <int NT, int MODE>
__device__ __forceinline__ void block_reduce_pass(float (&f)[4], int& ci, uint32_t& mb, DecRed* r, int& par) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (MODE == 0 || k != 2) f[k] = wave_fsum(f[k]);
  if constexpr (MODE != 0) {
    ci = wave_isum(ci);
    mb = wave_umin(mb);
  }
  if ((threadIdx.x & 63) == 0) {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 4; ++k) r->v[par][k][w] = __float_as_uint(f[k]);
    r->v[par][4][w] = (uint32_t)ci;
    r->v[par][5][w] = mb;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (MODE == 0 || k != 2) f[k] = wave_fsum(__uint_as_float(wg_gather<NT>(r, par, k, 0u)));
  if constexpr (MODE != 0) {
    ci = wave_isum((int)wg_gather<NT>(r, par, 4, 0u));
    mb = wave_umin(wg_gather<NT>(r, par, 5, 0xFFFFFFFFu));
  }
  par ^= 1;
}

// the row's x_max from the per-slice maxima of the score kernel
template <int NT>
__device__ __forceinline__ float row_max(const DecParams& p, size_t row, int nsp, DecRed* r, int& par) {
  float m = -INFINITY;
  for (int s = threadIdx.x; s < nsp; s += NT) m = fmaxf(m, p.smax[row * p.nsplit + s]);
  return block_max<NT>(m, r, par);
}

}  // namespace

// ------------------------------------------------------------------------- 1. scores
// GM: a compile-time bound on the group's query heads (4 or 16). Query row g sits in
// accumulator register r with acc_row(r, h) = g, so rows below GM use registers r < RM only.
template <typename T, int D, int GM>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_scores(DecParams p) {
  constexpr int DS = D / 16;
  constexpr int RM = GM <= 4 ? 4 : 8;
  static_assert(acc_row(RM - 1, 1) >= GM - 1, "registers r < RM hold every row below GM");
  __shared__ float red[4][16];
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int w = uniform_i32(wave_id());
  const int split = blockIdx.x, bk = blockIdx.y;
  const int bi = bk / p.hkv, kvh = bk % p.hkv;
  const int G = p.G, n = p.n;
  const int L = dec_len(p, bi);
  const int k0 = split * p.split, k1 = min(k0 + p.split, L);
  const size_t row0 = (size_t)bi * p.hq + (size_t)kvh * G;   // first query row of the group

  // query fragments: lane c holds query head c of the group (zero rows beyond G)
  const T* Q = reinterpret_cast<const T*>(p.q);
  Frag<T> qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (c < G) load_frag(qf[s], Q + (row0 + c) * D + 16 * s + 8 * h);
    else zero_frag(qf[s]);
  }
  // accumulator register r holds query row acc_row(r, h) of key c: its bias slope
  float cmr[RM], mx[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const int g = acc_row(r, h);
    cmr[r] = (p.slopes && g < G) ? p.slopes[kvh * G + g] * p.am1 : 0.0f;
    mx[r] = -INFINITY;
  }
  const T* K = reinterpret_cast<const T*>(p.k) + ((size_t)bi * p.hkv + kvh) * n * D;
  // K fragments of the 32 keys from key0 (zero past the slice: nothing is read there)
  const auto load_tile = [&](int key0, Frag<T> (&f)[DS]) {
    const int j = key0 + c;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (j < k1) load_frag(f[s], K + (size_t)j * D + 16 * s + 8 * h);
      else zero_frag(f[s]);
    }
  };
  Frag<T> kf[DS];
  load_tile(k0 + 32 * w, kf);
  for (int key0 = k0 + 32 * w; key0 < k1; key0 += 128) {
    Frag<T> kn[DS];
    load_tile(key0 + 128, kn);                    // the wave's next tile, in flight meanwhile
    const int j = key0 + c;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(acc, qf[s], kf[s]);   // S[query row][key c]
    const float dist = (float)(L - 1 - j);
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const int g = acc_row(r, h);
      if (g < G && j < k1) {
        const float x = fmaf(p.cx, acc[r], -cmr[r] * dist);
        p.xs[(row0 + g) * p.ldx + j] = x;
        mx[r] = fmaxf(mx[r], x);
      }
    }
#pragma unroll
    for (int s = 0; s < DS; ++s) kf[s] = kn[s];
  }
  // max over the 32 keys of each half-wave, then over the 4 waves
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    float m = mx[r];
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int g = acc_row(r, h);
    if (c == 0 && g < G) red[w][g] = m;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < G)
    p.smax[(row0 + t) * p.nsplit + split] = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
  // the slice holding the last key pads each row to a multiple of 4 scores with -inf, so the
  // threshold kernel reads whole float4 groups without masking
  const int pad = ((L + 3) & ~3) - L;
  if (k0 <= L - 1 && L - 1 < k0 + p.split && t < G * pad)
    p.xs[(row0 + t / pad) * p.ldx + L + t % pad] = -INFINITY;
}

// ------------------------------------------------------------------------- 2. histogram
// (slice, query row): counts of the slice's scores on the row's anchored grid (bin k < B
// holds floor(x B) = T - B + 1 + k with T = floor(x_max B); lower scores are not counted),
// summed per slice so the row's histogram is their exact sum.
__global__ __launch_bounds__(DEC_THREADS) void k_dec_hist(DecParams p) {
  __shared__ uint32_t cnt_lds[16][DEC_THREADS];   // a private column of counts per thread
  __shared__ DecRed red;
  int par = 0;
  const int t = threadIdx.x;
  const int split = blockIdx.x;
  const size_t row = blockIdx.y;
  const int bi = (int)(row / p.hq);
  const int L = dec_len(p, bi);
  const int k0 = split * p.split, k1 = min(k0 + p.split, L);
  if (k0 >= L) return;                            // whole work group: slice past the cache
  const int B = p.B;
  // the slice's scores are loaded first, so their latency overlaps the row maximum's
  const float* xr = p.xs + row * p.ldx;
  constexpr int U = DEC_SPLIT_MAX / DEC_THREADS;
  float xv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = k0 + t + u * DEC_THREADS;
    xv[u] = j < k1 ? xr[j] : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) cnt_lds[k][t] = 0u;
  const float m = row_max<DEC_THREADS>(p, row, (L + p.split - 1) / p.split, &red, par);
  const float base = (float)(cvt_floor(m * (float)B) - B + 1);   // x*B is exact: B = 2^k
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float y = fmaf(xv[u], (float)B, -base);
    if (y >= 0.0f && y < (float)B) cnt_lds[(int)y][t] += 1u;
  }
  __syncthreads();
  // bin t / 16 over columns 16 (t % 16) .. + 15, then the 16 partial sums of each bin
  // (integer counts: exact in any order)
  __shared__ uint32_t part[16][16];
  {
    const int b = t >> 4, q = t & 15;
    uint32_t sum = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) sum += cnt_lds[b][16 * q + u];
    part[b][q] = sum;
  }
  __syncthreads();
  if (t < B) {
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) sum += part[t][q];
    p.hcnt[(row * p.nsplit + split) * 16 + t] = (int)sum;
  }
}

// ------------------------------------------------------------------------- 3. threshold
// candidates per thread kept in LDS for the refinement passes after the first
constexpr int DEC_CAND = 32;

// (query row): tau_h from the summed slice histograms (or the plain bracket from x_max),
// then the solver passes. The first pass scans the stored row and keeps, per thread, the
// scores that can still count: the safeguarded bracket only narrows, so every later
// evaluation point lies at or above its starting lower end (just below tau_h, or x_max - 1
// from the plain bracket), and a score at or below that end adds nothing to any sum. Each
// thread keeps its own (a fixed subset in a fixed order, so the sums stay deterministic);
// if any thread has more than DEC_CAND, every pass rescans the row.
template <int MODE>
__global__ __launch_bounds__(DEC_TAU_THREADS) void k_dec_tau(DecParams p) {
  constexpr int NT = DEC_TAU_THREADS;
  __shared__ float cand[DEC_CAND + 1][NT];        // a private column of candidate scores (+ a spill row)
  __shared__ int cnt_tot[16];
  __shared__ int part_cnt[NT / 16][16];
  __shared__ DecRed red;
  int par = 0;
  const int t = threadIdx.x;
  const size_t row = blockIdx.x;
  const int bi = (int)(row / p.hq);
  const int L = dec_len(p, bi);
  const int B = p.B;
  const int nsp = (L + p.split - 1) / p.split;
  const float* xr = p.xs + row * p.ldx;
  constexpr int U = 8;
  const float4* x4 = reinterpret_cast<const float4*>(xr);
  const int n4 = (L + 3) >> 2;                    // the score kernel pads the last group with -inf
  // every stored score of the row, four at a time with 32 in flight per thread
  const auto scan = [&](auto&& f) {
    for (int i = t; i < n4; i += U * NT) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i + u * NT;
        v[u] = ii < n4 ? x4[ii] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f(v[u].x);
        f(v[u].y);
        f(v[u].z);
        f(v[u].w);
      }
    }
  };

  // thread (part, bin) sums slices part, part + NT/16, ...; the row maximum's barrier
  // publishes the sums
  if (p.tau_init == 0) {
    const int bin = t & 15, part = t >> 4;
    int sum = 0;
    for (int s = part; s < nsp; s += NT / 16) sum += p.hcnt[(row * p.nsplit + s) * 16 + bin];
    part_cnt[part][bin] = sum;
  }
  const float m = row_max<NT>(p, row, nsp, &red, par);
  const float kappa = p.kappa, alpha = p.alpha;
  const int T = cvt_floor(m * (float)B);          // x*B is exact: B is a power of two
  int cnt[16];
  float tau_h;
  RowState st;
  if (p.tau_init == 0) {
    // then the parts in order
    if (t < B) {
      int sum = 0;
      for (int u = 0; u < NT / 16; ++u) sum += part_cnt[u][t];
      cnt_tot[t] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] = k < B ? cnt_tot[k] : 0;
    tau_h = tau_from_counts<MODE>(cnt, T, B, kappa);
    st = MODE == 0 ? RowState::from_hist_bounded(tau_h, B, m, (float)L, alpha)
                   : RowState::from_hist(tau_h, B);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] = 0;
    tau_h = m - 1.0f;
    st = RowState::from_max(m, (float)L, alpha);
  }

  const float cand_lo = st.lo;                     // a score above the bracket's lower end can still count
  const bool secant = alpha > 2.0f;
  int ncand = 0, over = 1;
  for (int npass = 0; npass < p.max_iters && !st.done;) {
    const bool first = npass == 0;
    const float thi = st.hi - st.tau;
    const float tau0 = st.tau;
    PassSums s;
    if (first) {
      scan([&](float x) {
        s.add<MODE>(x - tau0, thi, secant, kappa);
        // every score goes to the slot after the last candidate (row DEC_CAND once full) and
        // stays there only if it is one: no branch per score
        cand[min(ncand, DEC_CAND)][t] = x;
        ncand += x > cand_lo ? 1 : 0;
      });
      over = block_max<NT>(ncand > DEC_CAND ? 1.0f : 0.0f, &red, par) > 0.0f;
    } else if (over) {
      scan([&](float x) { s.add<MODE>(x - tau0, thi, false, kappa); });
    } else {
      for (int k = 0; k < ncand; ++k) s.add<MODE>(cand[k][t] - tau0, thi, false, kappa);
    }
    ++npass;
    float fr[4] = {s.F0, s.F1, s.F2, s.Fh};
    int cr = s.cnt;
    uint32_t mr = s.mrelb;
    block_reduce_pass<NT, MODE>(fr, cr, mr, &red, par);
    float tot[5];
    tot[0] = fr[0];
    tot[1] = fr[1];
    if constexpr (MODE == 0) {
      tot[2] = fr[2];
      tot[4] = INFINITY;
    } else {
      tot[2] = (float)cr;
      tot[4] = mr < 0x7F800000u ? __uint_as_float(mr) : INFINITY;
    }
    tot[3] = secant && first ? fr[3] : 0.0f;
    st.update<MODE>(tot, npass, first, thi, kappa, alpha, p.tol);
  }
  if (t == 0) {
    p.tau[row] = st.tau;
    if (p.tau_h) p.tau_h[row] = tau_h;
  }
  if (p.hist && t < B) p.hist[row * B + t] = cnt[t];
}

// ------------------------------------------------------------------------- 4. output
// GM: a compile-time bound on the group's query heads (4 or 16), so the per-head loops carry
// no branch; heads past G have tau = +inf, hence p = 0, and are not stored.
template <typename T, int D, int MODE, int GM>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_out(DecParams p) {
  constexpr int E = D / 64;                       // head-dimension elements per lane
  __shared__ float red[4][GM][D];
  __shared__ __align__(16) float pl[4][64][GM];   // a wave's weights of its 64 keys, key-major
  const int lane = lane_id();
  const int w = uniform_i32(wave_id());
  const int split = blockIdx.x, bk = blockIdx.y;
  const int bi = bk / p.hkv, kvh = bk % p.hkv;
  const int G = p.G, n = p.n;
  const int L = dec_len(p, bi);
  const int k0 = split * p.osplit, k1 = min(k0 + p.osplit, L);
  if (k0 >= L) return;                            // whole work group: slice past the cache
  const size_t row0 = (size_t)bi * p.hq + (size_t)kvh * G;
  float taug[GM], oacc[GM][E];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    taug[g] = g < G ? p.tau[row0 + g] : INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) oacc[g][e] = 0.0f;
  }
  const T* V = reinterpret_cast<const T*>(p.v) + ((size_t)bi * p.hkv + kvh) * n * D;
  // scores of the G rows at key key0 + lane (-inf past the slice and for heads past G)
  const auto load_x = [&](int key0, float (&xv)[GM]) {
    const int j = key0 + lane;
#pragma unroll
    for (int g = 0; g < GM; ++g) xv[g] = (g < G && j < k1) ? p.xs[(row0 + g) * p.ldx + j] : -INFINITY;
  };
  float xc[GM];
  load_x(k0 + 64 * w, xc);
  for (int key0 = k0 + 64 * w; key0 < k1; key0 += 256) {
    float xn[GM];                                 // the next group's scores, in flight
    load_x(key0 + 256, xn);
    float pr[GM];
    bool any = false;
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      const float d = xc[g] - taug[g];
      pr[g] = d > 0.0f ? Weight<MODE>::p(d, p.kappa) : 0.0f;
      any = any || d > 0.0f;
    }
    uint64_t bits = ballot(any);
    if (bits) {
      // the key's weights for every lane: one broadcast LDS read per key (the same address
      // in every lane)
#pragma unroll
      for (int g4 = 0; g4 < GM / 4; ++g4)
        *reinterpret_cast<f32x4*>(&pl[w][lane][4 * g4]) =
            f32x4{pr[4 * g4], pr[4 * g4 + 1], pr[4 * g4 + 2], pr[4 * g4 + 3]};
      __builtin_amdgcn_wave_barrier();            // (a wave's LDS accesses complete in order)
    }
    while (bits) {                                // keys with a non-zero weight, in order,
      int jj[8];                                  // eight V rows in flight at a time
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        jj[u] = bits ? __builtin_ctzll(bits) : -1;
        bits &= bits - 1;
      }
      // every slot loads (the group's first key stands in for an empty one, with weight 0),
      // so the loads go out back to back and no branch separates them
      float vv[8][E];
      f32x4 pw[8][GM / 4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ju = max(jj[u], 0);
        const T* vr = V + (size_t)(key0 + ju) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) vv[u][e] = (float)vr[e];
#pragma unroll
        for (int g4 = 0; g4 < GM / 4; ++g4) pw[u][g4] = *reinterpret_cast<const f32x4*>(&pl[w][ju][4 * g4]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float live = jj[u] >= 0 ? 1.0f : 0.0f;
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          const float pg = live * pw[u][g >> 2][g & 3];
#pragma unroll
          for (int e = 0; e < E; ++e) oacc[g][e] = fmaf(pg, vv[u][e], oacc[g][e]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) xc[g] = xn[g];
  }

  // sum the 4 waves' partials in wave order
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (g < G) red[w][g][lane * E + e] = oacc[g][e];
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += DEC_THREADS) {
    const int g = i / D, d = i % D;
    const float s = (red[0][g][d] + red[1][g][d]) + (red[2][g][d] + red[3][g][d]);
    p.opart[((size_t)split * p.b * p.hq + row0 + g) * D + d] = s;
  }
}

// ------------------------------------------------------------------------- 5. reduce
// thread (part, d) sums slices part, part + P, ... of element d; the P part sums are then
// added in part order (P = 1024 / D: a row's few hundred slices in a few dependent loads)
constexpr int DEC_RED_THREADS = 1024;
__global__ __launch_bounds__(DEC_RED_THREADS) void k_dec_reduce(DecParams p, int D) {
  __shared__ float part_sum[DEC_RED_THREADS];
  const size_t row = blockIdx.x;
  const int bi = (int)(row / p.hq);
  const int nsp = (dec_len(p, bi) + p.osplit - 1) / p.osplit;
  const size_t rows = (size_t)p.b * p.hq;
  const int P = DEC_RED_THREADS / D;
  const int d = threadIdx.x % D, part = threadIdx.x / D;
  float s = 0.0f;
#pragma unroll 8
  for (int k = part; k < nsp; k += P) s += p.opart[(k * rows + row) * D + d];
  part_sum[threadIdx.x] = s;
  __syncthreads();
  if (part == 0) {
    float tot = 0.0f;
    for (int u = 0; u < P; ++u) tot += part_sum[u * D + d];
    p.o[row * D + d] = tot;
  }
}

// ------------------------------------------------------------------------- launch
template <typename T, int D>
static hipError_t launch_decode_t(const DecParams& p, int mode, hipStream_t s) {
  const dim3 gs(p.nsplit, p.b * p.hkv);
  const dim3 go(p.nsplit_o, p.b * p.hkv);
  prof_begin("dec_scores", s);
  if (p.G <= 4) hipLaunchKernelGGL((k_dec_scores<T, D, 4>), gs, dim3(DEC_THREADS), 0, s, p);
  else hipLaunchKernelGGL((k_dec_scores<T, D, 16>), gs, dim3(DEC_THREADS), 0, s, p);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.tau_init == 0) {
    prof_begin("dec_hist", s);
    hipLaunchKernelGGL(k_dec_hist, dim3(p.nsplit, p.b * p.hq), dim3(DEC_THREADS), 0, s, p);
    prof_end(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  void (*tau_fn)(DecParams) = mode == 1 ? k_dec_tau<1> : mode == 2 ? k_dec_tau<2> : k_dec_tau<0>;
  prof_begin("dec_tau", s);
  hipLaunchKernelGGL(tau_fn, dim3(p.b * p.hq), dim3(DEC_TAU_THREADS), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  void (*out_fn)(DecParams);
  if (p.G <= 4)
    out_fn = mode == 1 ? k_dec_out<T, D, 1, 4> : mode == 2 ? k_dec_out<T, D, 2, 4> : k_dec_out<T, D, 0, 4>;
  else
    out_fn = mode == 1 ? k_dec_out<T, D, 1, 16> : mode == 2 ? k_dec_out<T, D, 2, 16> : k_dec_out<T, D, 0, 16>;
  prof_begin("dec_out", s);
  hipLaunchKernelGGL(out_fn, go, dim3(DEC_THREADS), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin("dec_reduce", s);
  hipLaunchKernelGGL(k_dec_reduce, dim3(p.b * p.hq), dim3(DEC_RED_THREADS), 0, s, p, D);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_decode(const DecParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (p.b * p.hq == 0) return hipSuccess;
  if (dtype == 1) return D == 64 ? launch_decode_t<__bf16, 64>(p, mode, s) : launch_decode_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_decode_t<float, 64>(p, mode, s) : launch_decode_t<float, 128>(p, mode, s);
}

}  // namespace entmax

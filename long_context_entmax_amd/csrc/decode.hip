// Decode forward of alpha-entmax attention: one new query row per (sequence, query head)
// against a KV cache. The pages leave inference to future work (page 3 section 5) and
// DashAttention decodes incrementally on the same primitives (page 4); the threshold is
// found exactly as in the forward (page 1 sections 2.1-2.2, page 3 sections 2.1-2.2): a
// B-bin histogram of the row's scores gives tau_h (Proposition 1), the safeguarded hybrid
// solver refines it, and o = sum_j p_j v_j with p = [x - tau]_+^(1/(alpha-1)).
//
// MI355X decomposition. One query row is too little work for a wave to stream a long cache
// by itself, so the keys are split in slices (p.split keys), one work group per (slice, KV
// head), and the score row itself is kept: 4 bytes per key and query head against 2 d bytes
// of bf16 K per key and KV head, so the histogram and every refinement pass read the fp32
// scores instead of recomputing them from K.
//   1. k_dec_scores  (slice, KV head): x for the G query heads of the KV head on MFMA (the
//      G query rows padded to 32), stored, plus the slice's max per row.
//   2. k_dec_hist    (slice, query row): the slice's counts on the row's anchored B-bin grid.
//   3. k_dec_tau     (query row): the summed histogram, tau_h, then the solver passes over
//      the stored scores (work-group reductions in a fixed order: deterministic).
//   4. k_dec_out     (p.osplit-key slice, KV head): p for the G rows, V rows read only for
//      keys where some row has p > 0, partial o per slice (smaller slices than the score
//      kernel: this pass waits on V loads key by key, so it wants more waves in flight).
//   5. k_dec_reduce  (query row): o = sum of the slice partials in slice order.
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

// work-group sum / min / max over NT threads in a fixed order; every thread gets the result
// (lds holds one value per wave)
template <int NT, typename V, typename Op>
__device__ __forceinline__ V block_reduce(V v, V* lds, Op op) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = op(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();   // lds may still be read from the previous reduction
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  V r = lds[0];
#pragma unroll
  for (int u = 1; u < NT / 64; ++u) r = op(r, lds[u]);
  return r;
}

// the row's x_max from the per-slice maxima of the score kernel
template <int NT>
__device__ __forceinline__ float row_max(const DecParams& p, size_t row, int nsp, float* lds) {
  float m = -INFINITY;
  for (int s = threadIdx.x; s < nsp; s += NT) m = fmaxf(m, p.smax[row * p.nsplit + s]);
  return block_reduce<NT>(m, lds, [](float a, float b) { return fmaxf(a, b); });
}

}  // namespace

// ------------------------------------------------------------------------- 1. scores
template <typename T, int D>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_scores(DecParams p) {
  constexpr int DS = D / 16;
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
  float cmr[16], mx[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int g = acc_row(r, h);
    cmr[r] = (p.slopes && g < G) ? p.slopes[kvh * G + g] * p.am1 : 0.0f;
    mx[r] = -INFINITY;
  }
  const T* K = reinterpret_cast<const T*>(p.k) + ((size_t)bi * p.hkv + kvh) * n * D;
  for (int key0 = k0 + 32 * w; key0 < k1; key0 += 128) {
    const int j = key0 + c;
    Frag<T> kf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (j < k1) load_frag(kf[s], K + (size_t)j * D + 16 * s + 8 * h);
      else zero_frag(kf[s]);
    }
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(acc, qf[s], kf[s]);   // S[query row][key c]
    const float dist = (float)(L - 1 - j);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int g = acc_row(r, h);
      if (g < G && j < k1) {
        const float x = fmaf(p.cx, acc[r], -cmr[r] * dist);
        p.xs[(row0 + g) * p.ldx + j] = x;
        mx[r] = fmaxf(mx[r], x);
      }
    }
  }
  // max over the 32 keys of each half-wave, then over the 4 waves
#pragma unroll
  for (int r = 0; r < 16; ++r) {
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
}

// ------------------------------------------------------------------------- 2. histogram
// (slice, query row): counts of the slice's scores on the row's anchored grid (bin k < B
// holds floor(x B) = T - B + 1 + k with T = floor(x_max B); lower scores are not counted),
// summed per slice so the row's histogram is their exact sum.
__global__ __launch_bounds__(DEC_THREADS) void k_dec_hist(DecParams p) {
  __shared__ uint32_t cnt_lds[16][DEC_THREADS];   // a private column of counts per thread
  __shared__ float rf[4];
  const int t = threadIdx.x;
  const int split = blockIdx.x;
  const size_t row = blockIdx.y;
  const int bi = (int)(row / p.hq);
  const int L = dec_len(p, bi);
  const int k0 = split * p.split, k1 = min(k0 + p.split, L);
  if (k0 >= L) return;                            // whole work group: slice past the cache
  const int B = p.B;
  const float m = row_max<DEC_THREADS>(p, row, (L + p.split - 1) / p.split, rf);
  const float base = (float)(cvt_floor(m * (float)B) - B + 1);   // x*B is exact: B = 2^k
#pragma unroll
  for (int k = 0; k < 16; ++k) cnt_lds[k][t] = 0u;
  const float* xr = p.xs + row * p.ldx;
  constexpr int U = DEC_SPLIT_MAX / DEC_THREADS;
  float xv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = k0 + t + u * DEC_THREADS;
    xv[u] = j < k1 ? xr[j] : -INFINITY;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float y = fmaf(xv[u], (float)B, -base);
    if (y >= 0.0f && y < (float)B) cnt_lds[(int)y][t] += 1u;
  }
  __syncthreads();
  if (t < B) {
    uint32_t sum = 0;
    for (int u = 0; u < DEC_THREADS; ++u) sum += cnt_lds[t][u];
    p.hcnt[(row * p.nsplit + split) * 16 + t] = (int)sum;
  }
}

// ------------------------------------------------------------------------- 3. threshold
// candidates per thread kept in LDS for the refinement passes after the first
constexpr int DEC_CAND = 8;

// (query row): tau_h from the summed slice histograms (or the plain bracket from x_max),
// then the solver passes. The first pass scans the stored row and keeps, per thread, the
// scores that can still count: every later evaluation point lies at or above the bracket's
// lower end, at least x_max - 1 - 1/(16B) in either start (tau_h >= T/B - 1, Proposition 1),
// so only scores with x B > T - B - 1/16 matter. Each thread keeps its own (a fixed subset in
// a fixed order, so the sums stay deterministic); if any thread has more than DEC_CAND,
// every pass rescans the row.
template <int MODE>
__global__ __launch_bounds__(DEC_TAU_THREADS) void k_dec_tau(DecParams p) {
  constexpr int NT = DEC_TAU_THREADS;
  __shared__ float cand[DEC_CAND][NT];            // a private column of candidate scores
  __shared__ int cnt_tot[16];
  __shared__ int part_cnt[NT / 16][16];
  __shared__ float rf[NT / 64];
  __shared__ int ri[NT / 64];
  __shared__ uint32_t ru[NT / 64];
  const int t = threadIdx.x;
  const size_t row = blockIdx.x;
  const int bi = (int)(row / p.hq);
  const int L = dec_len(p, bi);
  const int B = p.B;
  const int nsp = (L + p.split - 1) / p.split;
  const float* xr = p.xs + row * p.ldx;
  // every stored score of the row, four at a time with 32 in flight per thread (the row
  // stride is a multiple of 4 floats; the tail past L reads as -inf)
  const auto scan = [&](auto&& f) {
    constexpr int U = 8;
    const float4* x4 = reinterpret_cast<const float4*>(xr);
    const int n4 = (L + 3) >> 2;
    for (int i = t; i < n4; i += U * NT) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i + u * NT;
        v[u] = ii < n4 ? x4[ii] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j0 = 4 * (i + u * NT);
        f(j0 < L ? v[u].x : -INFINITY);
        f(j0 + 1 < L ? v[u].y : -INFINITY);
        f(j0 + 2 < L ? v[u].z : -INFINITY);
        f(j0 + 3 < L ? v[u].w : -INFINITY);
      }
    }
  };

  const float m = row_max<NT>(p, row, nsp, rf);
  const float kappa = p.kappa, alpha = p.alpha;
  const int T = cvt_floor(m * (float)B);          // x*B is exact: B is a power of two
  int cnt[16];
  float tau_h;
  RowState st;
  if (p.tau_init == 0) {
    // thread (part, bin) sums slices part, part + NT/16, ...; then the parts in order
    {
      const int bin = t & 15, part = t >> 4;
      int sum = 0;
      for (int s = part; s < nsp; s += NT / 16) sum += p.hcnt[(row * p.nsplit + s) * 16 + bin];
      part_cnt[part][bin] = sum;
    }
    __syncthreads();
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

  const float cand_lo = (float)(T - B) - 0.25f;   // x B above this can still count
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
        if (x * (float)B > cand_lo) {
          if (ncand < DEC_CAND) cand[ncand][t] = x;
          ++ncand;
        }
      });
      over = block_reduce<NT>(ncand > DEC_CAND ? 1 : 0, ri, [](int a, int b) { return a | b; });
    } else if (over) {
      scan([&](float x) { s.add<MODE>(x - tau0, thi, false, kappa); });
    } else {
      for (int k = 0; k < ncand; ++k) s.add<MODE>(cand[k][t] - tau0, thi, false, kappa);
    }
    ++npass;
    const auto fsum = [](float a, float b) { return a + b; };
    float tot[5];
    tot[0] = block_reduce<NT>(s.F0, rf, fsum);
    tot[1] = block_reduce<NT>(s.F1, rf, fsum);
    if constexpr (MODE == 0) {
      tot[2] = block_reduce<NT>(s.F2, rf, fsum);
      tot[4] = INFINITY;
    } else {
      tot[2] = (float)block_reduce<NT>(s.cnt, ri, [](int a, int b) { return a + b; });
      const uint32_t mb = block_reduce<NT>(s.mrelb, ru, [](uint32_t a, uint32_t b) { return min(a, b); });
      tot[4] = mb < 0x7F800000u ? __uint_as_float(mb) : INFINITY;
    }
    tot[3] = secant && first ? block_reduce<NT>(s.Fh, rf, fsum) : 0.0f;
    st.update<MODE>(tot, npass, first, thi, kappa, alpha, p.tol);
  }
  if (t == 0) {
    p.tau[row] = st.tau;
    if (p.tau_h) p.tau_h[row] = tau_h;
  }
  if (p.hist && t < B) p.hist[row * B + t] = cnt[t];
}

// ------------------------------------------------------------------------- 4. output
template <typename T, int D, int MODE>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_out(DecParams p) {
  constexpr int E = D / 64;                       // head-dimension elements per lane
  __shared__ float red[4][16][D];
  const int lane = lane_id();
  const int w = uniform_i32(wave_id());
  const int split = blockIdx.x, bk = blockIdx.y;
  const int bi = bk / p.hkv, kvh = bk % p.hkv;
  const int G = p.G, n = p.n;
  const int L = dec_len(p, bi);
  const int k0 = split * p.osplit, k1 = min(k0 + p.osplit, L);
  if (k0 >= L) return;                            // whole work group: slice past the cache
  const size_t row0 = (size_t)bi * p.hq + (size_t)kvh * G;
  float taug[16], oacc[16][E];
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    taug[g] = g < G ? p.tau[row0 + g] : INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) oacc[g][e] = 0.0f;
  }
  const T* V = reinterpret_cast<const T*>(p.v) + ((size_t)bi * p.hkv + kvh) * n * D;
  // scores of the G rows at key key0 + lane (-inf past the slice)
  const auto load_x = [&](int key0, float (&xv)[16]) {
    const int j = key0 + lane;
#pragma unroll
    for (int g = 0; g < 16; ++g) xv[g] = (g < G && j < k1) ? p.xs[(row0 + g) * p.ldx + j] : -INFINITY;
  };
  float xc[16];
  load_x(k0 + 64 * w, xc);
  for (int key0 = k0 + 64 * w; key0 < k1; key0 += 256) {
    float xn[16];                                 // the next group's scores, in flight
    load_x(key0 + 256, xn);
    float pr[16];
    bool any = false;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const float d = xc[g] - taug[g];
      pr[g] = d > 0.0f ? Weight<MODE>::p(d, p.kappa) : 0.0f;
      any = any || d > 0.0f;
    }
    uint64_t bits = ballot(any);
    while (bits) {                                // keys with a non-zero weight, in order,
      int jj[8];                                  // eight V rows in flight at a time
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        jj[u] = bits ? __builtin_ctzll(bits) : -1;
        bits &= bits - 1;
      }
      float vv[8][E];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (jj[u] >= 0) {
          const T* vr = V + (size_t)(key0 + jj[u]) * D + lane * E;
#pragma unroll
          for (int e = 0; e < E; ++e) vv[u][e] = (float)vr[e];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (jj[u] < 0) break;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          if (g < G) {
            const float pg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr[g]), jj[u]));
#pragma unroll
            for (int e = 0; e < E; ++e) oacc[g][e] = fmaf(pg, vv[u][e], oacc[g][e]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 16; ++g) xc[g] = xn[g];
  }

  // sum the 4 waves' partials in wave order
#pragma unroll
  for (int g = 0; g < 16; ++g)
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
// added in part order (P = 256 / D)
__global__ __launch_bounds__(DEC_THREADS) void k_dec_reduce(DecParams p, int D) {
  __shared__ float part_sum[DEC_THREADS];
  const size_t row = blockIdx.x;
  const int bi = (int)(row / p.hq);
  const int nsp = (dec_len(p, bi) + p.osplit - 1) / p.osplit;
  const size_t rows = (size_t)p.b * p.hq;
  const int P = DEC_THREADS / D;
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
  hipLaunchKernelGGL((k_dec_scores<T, D>), gs, dim3(DEC_THREADS), 0, s, p);
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
  void (*out_fn)(DecParams) =
      mode == 1 ? k_dec_out<T, D, 1> : mode == 2 ? k_dec_out<T, D, 2> : k_dec_out<T, D, 0>;
  prof_begin("dec_out", s);
  hipLaunchKernelGGL(out_fn, go, dim3(DEC_THREADS), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin("dec_reduce", s);
  hipLaunchKernelGGL(k_dec_reduce, dim3(p.b * p.hq), dim3(DEC_THREADS), 0, s, p, D);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_decode(const DecParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (p.b * p.hq == 0) return hipSuccess;
  if (dtype == 1) return D == 64 ? launch_decode_t<__bf16, 64>(p, mode, s) : launch_decode_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_decode_t<float, 64>(p, mode, s) : launch_decode_t<float, 128>(p, mode, s);
}

}  // namespace entmax

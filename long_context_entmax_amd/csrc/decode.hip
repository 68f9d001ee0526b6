// Decode forward of alpha-entmax attention: one new query row per (sequence, query head)
// against a KV cache. The pages leave inference to future work (page 3 section 5) and
// DashAttention decodes incrementally on the same primitives (page 4); the threshold is
// found exactly as in the forward (page 1 sections 2.1-2.2, page 3 sections 2.1-2.2): a
// B-bin histogram of the row's scores gives tau_h (Proposition 1), the safeguarded hybrid
// solver refines it, and o = sum_j p_j v_j with p = [x - tau]_+^(1/(alpha-1)).
//
// MI355X decomposition. One query row is too little work for a wave to stream a long cache
// by itself, so the keys are split in DEC_SPLIT-key slices, one work group per (slice, KV
// head), and the score row itself is kept: at 4 bytes per key and query head it is 1/32 to
// 1/64 of the K bytes it is computed from, so the histogram and every refinement pass read
// the fp32 scores instead of recomputing them from K.
//   1. k_dec_scores  (slice, KV head): x for the G query heads of the KV head on MFMA (the
//      G query rows padded to 32), stored, plus the slice's max per row.
//   2. k_dec_tau     (query row): x_max over slices, the anchored B-bin histogram, tau_h,
//      then the solver passes over the stored scores (work-group reductions in a fixed
//      order: deterministic).
//   3. k_dec_out     (slice, KV head): p for the G rows, V rows read only for keys where
//      some row has p > 0, partial o per slice.
//   4. k_dec_reduce  (query row): o = sum of the slice partials in slice order.
#include "common.hpp"
#include "kernels.hpp"
#include "solver.hpp"

namespace entmax {

namespace {

constexpr int DEC_THREADS = 256;

__device__ __forceinline__ int dec_len(const DecParams& p, int bi) {
  return p.lengths ? min(max(p.lengths[bi], 1), p.n) : p.n;
}

// work-group sum / min / max over 256 threads in a fixed order; every thread gets the result
template <typename V, typename Op>
__device__ __forceinline__ V block_reduce(V v, V* lds4, Op op) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = op(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();   // lds4 may still be read from the previous reduction
  if ((threadIdx.x & 63) == 0) lds4[w] = v;
  __syncthreads();
  return op(op(lds4[0], lds4[1]), op(lds4[2], lds4[3]));
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
  const int k0 = split * DEC_SPLIT, k1 = min(k0 + DEC_SPLIT, L);
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

// ------------------------------------------------------------------------- 2. threshold
template <int MODE>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_tau(DecParams p) {
  __shared__ uint32_t cnt_lds[16][DEC_THREADS];   // a private column of counts per thread
  __shared__ int cnt_tot[16];
  __shared__ float rf[4];
  __shared__ int ri[4];
  __shared__ uint32_t ru[4];
  const int t = threadIdx.x;
  const size_t row = blockIdx.x;
  const int bi = (int)(row / p.hq);
  const int L = dec_len(p, bi);
  const int B = p.B;
  const float* xr = p.xs + row * p.ldx;
  // every stored score of the row, four at a time with 16 in flight per thread (the row
  // stride is a multiple of 4 floats; the tail past L reads as -inf)
  const auto scan = [&](auto&& f) {
    const float4* x4 = reinterpret_cast<const float4*>(xr);
    const int n4 = (L + 3) >> 2;
    for (int i = t; i < n4; i += 4 * DEC_THREADS) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ii = i + u * DEC_THREADS;
        v[u] = ii < n4 ? x4[ii] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j0 = 4 * (i + u * DEC_THREADS);
        f(j0 < L ? v[u].x : -INFINITY);
        f(j0 + 1 < L ? v[u].y : -INFINITY);
        f(j0 + 2 < L ? v[u].z : -INFINITY);
        f(j0 + 3 < L ? v[u].w : -INFINITY);
      }
    }
  };
  const int nsp = (L + DEC_SPLIT - 1) / DEC_SPLIT;

  float m = -INFINITY;
  for (int s = t; s < nsp; s += DEC_THREADS) m = fmaxf(m, p.smax[row * p.nsplit + s]);
  m = block_reduce(m, rf, [](float a, float b) { return fmaxf(a, b); });
  const float kappa = p.kappa, alpha = p.alpha;

  int cnt[16];
  float tau_h;
  RowState st;
  const int T = cvt_floor(m * (float)B);       // x*B is exact: B is a power of two
  if (p.tau_init == 0) {
    // anchored grid: bin k < B holds floor(x B) = T - B + 1 + k (lower bins are not counted)
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt_lds[k][t] = 0u;
    const float base = (float)(T - B + 1);
    uint32_t* col = &cnt_lds[0][t];
    scan([&](float x) {
      const float y = fmaf(x, (float)B, -base);
      if (y >= 0.0f && y < (float)B) col[(int)y * DEC_THREADS] += 1u;
    });
    __syncthreads();
    if (t < B) {
      uint32_t sum = 0;
      for (int u = 0; u < DEC_THREADS; ++u) sum += cnt_lds[t][u];
      cnt_tot[t] = (int)sum;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] = k < B ? cnt_tot[k] : 0;
    tau_h = tau_from_counts<MODE>(cnt, T, B, kappa);
    st = RowState::from_hist(tau_h, B);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] = 0;
    tau_h = m - 1.0f;
    st = RowState::from_max(m, (float)L, alpha);
  }

  const bool secant = alpha > 2.0f;
  for (int npass = 0; npass < p.max_iters && !st.done;) {
    const bool first = npass == 0;
    const float thi = st.hi - st.tau;
    PassSums s;
    const float tau0 = st.tau;
    scan([&](float x) { s.add<MODE>(x - tau0, thi, secant && first, kappa); });
    ++npass;
    const auto fsum = [](float a, float b) { return a + b; };
    float tot[5];
    tot[0] = block_reduce(s.F0, rf, fsum);
    tot[1] = block_reduce(s.F1, rf, fsum);
    if constexpr (MODE == 0) {
      tot[2] = block_reduce(s.F2, rf, fsum);
      tot[4] = INFINITY;
    } else {
      tot[2] = (float)block_reduce(s.cnt, ri, [](int a, int b) { return a + b; });
      const uint32_t mb = block_reduce(s.mrelb, ru, [](uint32_t a, uint32_t b) { return min(a, b); });
      tot[4] = mb < 0x7F800000u ? __uint_as_float(mb) : INFINITY;
    }
    tot[3] = secant && first ? block_reduce(s.Fh, rf, fsum) : 0.0f;
    st.update<MODE>(tot, npass, first, thi, kappa, alpha, p.tol);
  }
  if (t == 0) {
    p.tau[row] = st.tau;
    if (p.tau_h) p.tau_h[row] = tau_h;
  }
  if (p.hist && t < B) p.hist[row * B + t] = cnt[t];
}

// ------------------------------------------------------------------------- 3. output
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
  const int k0 = split * DEC_SPLIT, k1 = min(k0 + DEC_SPLIT, L);
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
  for (int key0 = k0 + 64 * w; key0 < k1; key0 += 256) {
    const int j = key0 + lane;
    float pr[16];
    bool any = false;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      pr[g] = 0.0f;
      if (g < G && j < k1) {
        const float d = p.xs[(row0 + g) * p.ldx + j] - taug[g];
        pr[g] = d > 0.0f ? Weight<MODE>::p(d, p.kappa) : 0.0f;
        any = any || d > 0.0f;
      }
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

// ------------------------------------------------------------------------- 4. reduce
__global__ __launch_bounds__(128) void k_dec_reduce(DecParams p, int D) {
  const size_t row = blockIdx.x;
  const int bi = (int)(row / p.hq);
  const int nsp = (dec_len(p, bi) + DEC_SPLIT - 1) / DEC_SPLIT;
  const size_t rows = (size_t)p.b * p.hq;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float s = 0.0f;
    for (int k = 0; k < nsp; ++k) s += p.opart[(k * rows + row) * D + d];
    p.o[row * D + d] = s;
  }
}

// ------------------------------------------------------------------------- launch
template <typename T, int D>
static hipError_t launch_decode_t(const DecParams& p, int mode, hipStream_t s) {
  const dim3 gs(p.nsplit, p.b * p.hkv);
  prof_begin("dec_scores", s);
  hipLaunchKernelGGL((k_dec_scores<T, D>), gs, dim3(DEC_THREADS), 0, s, p);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void (*tau_fn)(DecParams) = mode == 1 ? k_dec_tau<1> : mode == 2 ? k_dec_tau<2> : k_dec_tau<0>;
  prof_begin("dec_tau", s);
  hipLaunchKernelGGL(tau_fn, dim3(p.b * p.hq), dim3(DEC_THREADS), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  void (*out_fn)(DecParams) =
      mode == 1 ? k_dec_out<T, D, 1> : mode == 2 ? k_dec_out<T, D, 2> : k_dec_out<T, D, 0>;
  prof_begin("dec_out", s);
  hipLaunchKernelGGL(out_fn, gs, dim3(DEC_THREADS), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin("dec_reduce", s);
  hipLaunchKernelGGL(k_dec_reduce, dim3(p.b * p.hq), dim3(128), 0, s, p, D);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_decode(const DecParams& p, int dtype, int D, int mode, hipStream_t s) {
  if (p.b * p.hq == 0) return hipSuccess;
  if (dtype == 1) return D == 64 ? launch_decode_t<__bf16, 64>(p, mode, s) : launch_decode_t<__bf16, 128>(p, mode, s);
  return D == 64 ? launch_decode_t<float, 64>(p, mode, s) : launch_decode_t<float, 128>(p, mode, s);
}

}  // namespace entmax

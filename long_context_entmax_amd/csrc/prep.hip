// Data-movement kernels around the attention kernels (HBM-bound, O(n d)):
//   k_frag_rows       X [H, n, D] -> fragment-major copy for operands whose rows are
//                     the 32 lanes: block b, chunk s, half h, lane c holds the 8 elements
//                     X[32b + c][16s + 8h .. +7] at ((b*DS + s)*2 + h)*32 + c (in 8-element
//                     units), so one wave's operand load is one contiguous run;
//   k_frag_cols       X [H, n, D] -> fragment-major copy for operands whose lanes walk the
//                     head dimension and whose contraction runs over rows: block b, 32-wide
//                     d chunk dc, 16-row chunk m, half h, lane c holds
//                     X[32b + 16m + sigma(8h + j)][32dc + c], j = 0..7;
//   k_transpose_perm  X [H, n, D] -> Xt [H, D, n], positions inside each 16-group in sigma
//                     order, so that a lane reads 8 consecutive elements as an MFMA operand
//                     when the contraction runs over keys or queries;
//   k_delta           delta_i = dO_i . o~_i (fp32), the row term of the entmax backward;
//   k_mask_transpose  block mask [P, Tr, W] -> column-major copy [P, Tc, WT] (bit I of the
//                     words of key block J), walked by the dK/dV kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace entmax {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_transpose_perm(const T* __restrict__ src, T* __restrict__ dst,
                                                        int n) {
  constexpr int PAD = (sizeof(T) == 2) ? 2 : 1;
  __shared__ T tile[64][D + PAD];
  const int hh = blockIdx.y;
  const int r0 = blockIdx.x * 64;
  const T* s = src + ((size_t)hh * n + r0) * D;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int r = i / D, cc = i % D;
    tile[r][cc] = (r0 + r < n) ? s[(size_t)r * D + cc] : (T)0.0f;
  }
  __syncthreads();
  T* d = dst + (size_t)hh * D * n + r0;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int dd = i / 64, pos = i % 64;
    if (r0 + pos < n) d[(size_t)dd * n + pos] = tile[(pos & ~15) | sigma16(pos & 15)][dd];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_frag_rows(const T* __restrict__ src, T* __restrict__ dst, int n) {
  constexpr int DS = D / 16;
  constexpr int V4 = 8 * sizeof(T) / 16;           // 16-byte vectors per 8-element fragment
  const size_t hh = blockIdx.y;
  const int units = (n / 32) * DS * 2 * 32;        // 8-element units per head
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int c = u & 31, h = (u >> 5) & 1, s = (u >> 6) % DS, b = (u >> 6) / DS;
  const uint4* sp = reinterpret_cast<const uint4*>(src + (hh * n + (size_t)b * 32 + c) * D + 16 * s + 8 * h);
  uint4* dp = reinterpret_cast<uint4*>(dst + hh * (size_t)n * D + (size_t)u * 8);
#pragma unroll
  for (int j = 0; j < V4; ++j) dp[j] = sp[j];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_frag_cols(const T* __restrict__ src, T* __restrict__ dst, int n) {
  constexpr int DC = D / 32;
  constexpr int PAD = (sizeof(T) == 2) ? 2 : 1;
  __shared__ T tile[32][D + PAD];
  const size_t hh = blockIdx.y;
  const int b = blockIdx.x;                         // 32-row block
  const T* sp = src + (hh * n + (size_t)b * 32) * D;
  for (int i = threadIdx.x; i < 32 * D; i += 256) tile[i / D][i % D] = sp[i];
  __syncthreads();
  // units of this block: DC * 2 (m) * 2 (h) * 32 (c)
  T* dp = dst + hh * (size_t)n * D + (size_t)b * 32 * D;
  for (int u = threadIdx.x; u < DC * 128; u += 256) {
    const int c = u & 31, h = (u >> 5) & 1, m = (u >> 6) & 1, dc = u >> 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) dp[(size_t)u * 8 + j] = tile[16 * m + sigma16(8 * h + j)][32 * dc + c];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_delta(const T* __restrict__ dout, const float* __restrict__ aux,
                                               float* __restrict__ delta, int rows) {
  constexpr int PER = D / 16;   // elements per lane, 16 lanes per row
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const T* a = dout + (size_t)row * D + j * PER;
    const float* b = aux + (size_t)row * D + j * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc += (float)a[e] * b[e];
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && j == 0) delta[row] = acc;
}

__global__ __launch_bounds__(256) void k_mask_transpose(const uint32_t* __restrict__ mask,
                                                        uint32_t* __restrict__ maskT, int planes,
                                                        int Tr, int Tc, int W, int WT) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)planes * Tc * WT;
  if (idx >= total) return;
  const int wt = (int)(idx % WT);
  const int J = (int)((idx / WT) % Tc);
  const int pl = (int)(idx / ((long long)WT * Tc));
  const uint32_t* m = mask + (size_t)pl * Tr * W;
  uint32_t word = 0;
  for (int bit = 0; bit < 32; ++bit) {
    const int I = wt * 32 + bit;
    if (I >= Tr) break;
    word |= ((m[(size_t)I * W + (J >> 5)] >> (J & 31)) & 1u) << bit;
  }
  maskT[idx] = word;
}

template <typename T>
static hipError_t relayout_one(const void* src, void* dst, int heads, int n, int D, int kind, hipStream_t s) {
  if (heads == 0 || n == 0) return hipSuccess;
  if (kind == 0) {            // permuted transpose [D][n]
    dim3 grid((n + 63) / 64, heads);
    prof_begin("transpose_perm", s);
    if (D == 64) hipLaunchKernelGGL((k_transpose_perm<T, 64>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
    else hipLaunchKernelGGL((k_transpose_perm<T, 128>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
  } else if (kind == 1) {     // fragment-major rows
    const int units = (n / 32) * (D / 16) * 64;
    dim3 grid((units + 255) / 256, heads);
    prof_begin("frag_rows", s);
    if (D == 64) hipLaunchKernelGGL((k_frag_rows<T, 64>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
    else hipLaunchKernelGGL((k_frag_rows<T, 128>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
  } else {                    // fragment-major columns
    dim3 grid(n / 32, heads);
    prof_begin("frag_cols", s);
    if (D == 64) hipLaunchKernelGGL((k_frag_cols<T, 64>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
    else hipLaunchKernelGGL((k_frag_cols<T, 128>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
  }
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_transpose(const PrepParams& p, int dtype, hipStream_t s) {
  for (int t = 0; t < p.ntrans; ++t) {
    hipError_t e = (dtype == 1) ? relayout_one<__bf16>(p.src[t], p.dst[t], p.heads[t], p.n, p.D, p.kind[t], s)
                                : relayout_one<float>(p.src[t], p.dst[t], p.heads[t], p.n, p.D, p.kind[t], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_prep(const PrepParams& p, int dtype, hipStream_t s) {
  hipError_t e = launch_transpose(p, dtype, s);
  if (e != hipSuccess) return e;
  if (p.rows > 0) {
    dim3 grid((p.rows + 15) / 16);
    prof_begin("delta", s);
    if (dtype == 1) {
      if (p.D == 64) hipLaunchKernelGGL((k_delta<__bf16, 64>), grid, dim3(256), 0, s, (const __bf16*)p.dout, p.aux, p.delta, p.rows);
      else hipLaunchKernelGGL((k_delta<__bf16, 128>), grid, dim3(256), 0, s, (const __bf16*)p.dout, p.aux, p.delta, p.rows);
    } else {
      if (p.D == 64) hipLaunchKernelGGL((k_delta<float, 64>), grid, dim3(256), 0, s, (const float*)p.dout, p.aux, p.delta, p.rows);
      else hipLaunchKernelGGL((k_delta<float, 128>), grid, dim3(256), 0, s, (const float*)p.dout, p.aux, p.delta, p.rows);
    }
    prof_end(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const long long total = (long long)p.planes * p.Tc * p.WT;
  if (total > 0) {
    prof_begin("mask_transpose", s);
    hipLaunchKernelGGL(k_mask_transpose, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p.mask,
                       p.maskT, p.planes, p.Tr, p.Tc, p.W, p.WT);
    prof_end(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace entmax

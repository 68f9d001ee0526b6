// Data-movement kernels around the attention kernels (HBM-bound, O(n d)):
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
static hipError_t transpose_one(const void* src, void* dst, int heads, int n, int D, hipStream_t s) {
  if (heads == 0 || n == 0) return hipSuccess;
  dim3 grid((n + 63) / 64, heads);
  prof_begin("transpose_perm", s);
  if (D == 64)
    hipLaunchKernelGGL((k_transpose_perm<T, 64>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
  else
    hipLaunchKernelGGL((k_transpose_perm<T, 128>), grid, dim3(256), 0, s, (const T*)src, (T*)dst, n);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_transpose(const PrepParams& p, int dtype, hipStream_t s) {
  for (int t = 0; t < p.ntrans; ++t) {
    hipError_t e = (dtype == 1) ? transpose_one<__bf16>(p.src[t], p.dst[t], p.heads[t], p.n, p.D, s)
                                : transpose_one<float>(p.src[t], p.dst[t], p.heads[t], p.n, p.D, s);
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

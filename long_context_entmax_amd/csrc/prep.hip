// Data movement around the attention kernels (HBM-bound, O(n d)), all in k_prep.
//
// A re-layout job stages one 32-row tile of X [H, n, D] in LDS and writes any of:
//   rows  fragment-major copy for MFMA operands whose 32 lanes walk rows and whose
//         contraction runs over the head dimension: 32-row block b, 16-wide chunk s,
//         half h, lane c hold X[32b + c][16s + 8h .. +7] at unit ((b*DS + s)*2 + h)*32 + c
//         (units of 8 elements), so a wave's operand is one contiguous run and its lane
//         offset is lane * 8 elements;
//   cols  fragment-major copy for operands whose lanes walk the head dimension and whose
//         contraction runs over rows: block b, 32-wide chunk dc, 16-row chunk m, half h,
//         lane c hold X[32b + 16m + sigma(8h + j)][32dc + c], j = 0..7, at unit
//         (((b*DC + dc)*2 + m)*2 + h)*32 + c (sigma: the order in which a 32x32 MFMA
//         accumulator holds the rows of a 16-row chunk);
//   delta delta_i = X_i . aux_i (fp32), the row term of the entmax backward when X = dO
//         and aux = o~ from the forward.
// The mask transpose: block mask [P, Tr, W] -> column-major copy [P, Tc, WT] (bit I of the
//   words of key block J), one 32x32 bit block per wave through 32 ballots.
// k_prep runs several re-layout jobs and the transpose in one launch (one range of work
// groups per job), so the small copies do not each pay a launch and a drain.
#include "common.hpp"
#include "kernels.hpp"

namespace entmax {

template <typename T, int D>
struct RelayoutTile {
  static constexpr int PAD = 16 / (int)sizeof(T);   // keeps 16-byte alignment of LDS rows
  static constexpr int LD = D + PAD;
  static constexpr int LDS_ELEMS = 32 * LD;
};

// one 32-row tile (block blk of head hh) of a re-layout job; tile: LDS of LDS_ELEMS elements
template <typename T, int D>
__device__ __forceinline__ void relayout_tile(const T* __restrict__ src, T* __restrict__ rows,
                                              T* __restrict__ cols, const float* __restrict__ aux,
                                              float* __restrict__ delta, int n, int blk, size_t hh,
                                              T* tile) {
  constexpr int DS = D / 16, DC = D / 32;
  constexpr int LD = RelayoutTile<T, D>::LD;
  constexpr int VEC = 16 / (int)sizeof(T);       // elements per 16-byte vector
  const T* sp = src + (hh * n + (size_t)blk * 32) * D;
  for (int i = threadIdx.x; i < 32 * D / VEC; i += 256) {
    const int r = (i * VEC) / D, cc = (i * VEC) % D;
    *reinterpret_cast<uint4*>(&tile[r * LD + cc]) = reinterpret_cast<const uint4*>(sp)[i];
  }
  __syncthreads();
  const size_t base = (hh * n + (size_t)blk * 32) * D;  // this block's 32*D elements
  if (rows) {
    for (int u = threadIdx.x; u < DS * 64; u += 256) {
      const int c = u & 31, h = (u >> 5) & 1, s = u >> 6;
      const uint4* from = reinterpret_cast<const uint4*>(&tile[c * LD + 16 * s + 8 * h]);
      uint4* to = reinterpret_cast<uint4*>(rows + base + (size_t)u * 8);
#pragma unroll
      for (int j = 0; j < 8 / VEC; ++j) to[j] = from[j];
    }
  }
  if (cols) {
    for (int u = threadIdx.x; u < DC * 128; u += 256) {
      const int c = u & 31, h = (u >> 5) & 1, m = (u >> 6) & 1, dc = u >> 7;
      T v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = tile[(16 * m + sigma16(8 * h + j)) * LD + 32 * dc + c];
      uint4* to = reinterpret_cast<uint4*>(cols + base + (size_t)u * 8);
#pragma unroll
      for (int j = 0; j < 8 / VEC; ++j) to[j] = reinterpret_cast<const uint4*>(v)[j];
    }
  }
  if (delta) {
    // 8 threads per row, D/8 elements each
    const int r = threadIdx.x >> 3, part = threadIdx.x & 7;
    const float* ap = aux + base + (size_t)r * D + part * (D / 8);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < D / 8; ++e) acc += (float)tile[r * LD + part * (D / 8) + e] * ap[e];
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (part == 0) delta[hh * n + (size_t)blk * 32 + r] = acc;
  }
}

// One wave per (plane, 32 query tiles, 32 key blocks): lane l < 32 holds the mask word of
// tile I0 + l; ballot over bit b gives the column word of key block J0 + b.
__device__ __forceinline__ void mask_transpose_wave(const uint32_t* __restrict__ mask,
                                                    uint32_t* __restrict__ maskT, int planes, int Tr,
                                                    int Tc, int W, int WT, long long wave) {
  const long long total = (long long)planes * W * WT;
  if (wave >= total) return;                        // whole wave
  const int lane = threadIdx.x & 63;
  const int wt = (int)(wave % WT);
  const int wj = (int)((wave / WT) % W);
  const int pl = (int)(wave / ((long long)WT * W));
  const int I = wt * 32 + (lane & 31);
  uint32_t word = 0;
  if (lane < 32 && I < Tr) word = mask[((size_t)pl * Tr + I) * W + wj];
  uint32_t mine = 0;
  for (int b = 0; b < 32; ++b) {
    const uint32_t col = (uint32_t)__ballot((word >> b) & 1u);   // bits of lanes 0..31
    if ((lane & 31) == b) mine = col;
  }
  const int J = wj * 32 + lane;
  if (lane < 32 && J < Tc) maskT[((size_t)pl * Tc + J) * WT + wt] = mine;
}

// Several re-layout jobs and an optional mask transpose in one launch: work groups
// [start[j], start[j + 1]) run job j (one 32-row tile each), the rest the transpose (four
// waves each).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_prep(PrepBatch b) {
  __shared__ __align__(16) T tile[RelayoutTile<T, D>::LDS_ELEMS];
  const int bid = blockIdx.x;
  for (int j = 0; j < b.njobs; ++j) {
    if (bid < b.start[j + 1]) {
      const Relayout& r = b.job[j];
      const int local = bid - b.start[j], nb = b.n / 32;
      relayout_tile<T, D>((const T*)r.src, (T*)r.rows, (T*)r.cols, r.aux, r.delta, b.n, local % nb,
                          (size_t)(local / nb), tile);
      return;
    }
  }
  mask_transpose_wave(b.mask, b.maskT, b.planes, b.Tr, b.Tc, b.W, b.WT,
                      (long long)(bid - b.start[b.njobs]) * 4 + (threadIdx.x >> 6));
}

template <typename T>
static hipError_t prep_t(PrepBatch b, int D, const char* name, hipStream_t s) {
  int grid = 0;
  for (int j = 0; j < b.njobs; ++j) {
    b.start[j] = grid;
    grid += b.job[j].heads * (b.n / 32);
  }
  b.start[b.njobs] = grid;
  if (b.mask) grid += (int)(((long long)b.planes * b.W * b.WT + 3) / 4);
  if (grid == 0) return hipSuccess;
  prof_begin(name, s);
  if (D == 64) hipLaunchKernelGGL((k_prep<T, 64>), dim3(grid), dim3(256), 0, s, b);
  else hipLaunchKernelGGL((k_prep<T, 128>), dim3(grid), dim3(256), 0, s, b);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepBatch& b, int dtype, int D, const char* name, hipStream_t s) {
  return dtype == 1 ? prep_t<__bf16>(b, D, name, s) : prep_t<float>(b, D, name, s);
}

}  // namespace entmax

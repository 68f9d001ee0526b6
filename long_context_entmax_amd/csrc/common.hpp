// Device building blocks shared by the alpha-entmax attention kernels (gfx950 / CDNA4).
//
// Tiles are 32x32 products on the matrix cores. In a 32x32 MFMA output, lane l
// (c = l % 32, h = l / 32) holds accumulator register r at
//     row R(r, h) = 8 (r / 4) + 4 h + (r % 4),   column c.
// A contraction chunk of 16 is fed as one fragment per lane: lane (c, h) holds the
// 8 consecutive contraction indices 8h .. 8h+7 of its row (A operand) or column
// (B operand). For bf16 that is one v_mfma_f32_32x32x16_bf16; for fp32 it is eight
// v_mfma_f32_32x32x2_f32 where the j-th takes elements j and 8+j.
//
// When an accumulator tile becomes the B operand of the next product (P, G or dS
// contracted over its rows), registers 8m .. 8m+7 of lane (c, h) feed chunk m and
// stand for rows 16m + sigma(8h + j), sigma(8h + j) = 8 (j / 4) + 4 h + (j % 4). The
// matching A operand is read from a transposed copy whose 16-position groups are
// stored in sigma order (the "permuted transpose" built by k_transpose_perm), so the
// same lane again reads 8 consecutive elements.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace entmax {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Row of accumulator register r for half-wave h in a 32x32 MFMA output.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Additive position bias of a lane's 16 accumulator entries, plus v0: returns
// v0 - cm * |i - j| where the entries' query-key distances are
// i - j = d0 + SGN * (8 (r / 4) + r % 4), the row offsets of a 32x32 accumulator
// (SGN = +1 when the accumulator rows are queries, -1 when they are keys). Under the
// causal mask |i - j| = i - j on every valid entry; the caller masks the others.
template <int SGN>
__device__ __forceinline__ f32x16 bias16(float v0, float cm, float d0, bool causal) {
  f32x16 b;
  if (causal) {
    const float a = fmaf(-cm, d0, v0);
#pragma unroll
    for (int r = 0; r < 16; ++r) b[r] = fmaf((float)(-SGN * (8 * (r >> 2) + (r & 3))), cm, a);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) b[r] = fmaf(-cm, fabsf(d0 + (float)(SGN * (8 * (r >> 2) + (r & 3)))), v0);
  }
  return b;
}

// acc[r] = mul * acc[r] + v0 - cm |i - j| entry by entry (distances as in bias16)
template <int SGN>
__device__ __forceinline__ void scale_add_bias16(f32x16& acc, float mul, float v0, float cm, float d0,
                                                 bool causal) {
  if (causal) {
    const float a = fmaf(-cm, d0, v0);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = fmaf(mul, acc[r], fmaf((float)(-SGN * (8 * (r >> 2) + (r & 3))), cm, a));
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[r] = fmaf(mul, acc[r], fmaf(-cm, fabsf(d0 + (float)(SGN * (8 * (r >> 2) + (r & 3)))), v0));
  }
}

// Position of row `row` (0..15 within a 16-group) in the permuted transposed layout
// (sigma is an involution: it swaps the middle two quads).
__host__ __device__ __forceinline__ constexpr int sigma16(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// ------------------------------------------------------------------------------------------
// fragments
// ------------------------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<__bf16> {
  bf16x8 v;
};
template <> struct Frag<float> {
  f32x4 a, b;
};

__device__ __forceinline__ void load_frag(Frag<__bf16>& f, const __bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  f.a = *reinterpret_cast<const f32x4*>(p);
  f.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void zero_frag(Frag<__bf16>& f) {
  f.v = bf16x8{};
}
__device__ __forceinline__ void zero_frag(Frag<float>& f) {
  f.a = f32x4{};
  f.b = f32x4{};
}

// Multiply a fragment by a power of two (exact unless it overflows or underflows).
__device__ __forceinline__ void scale_frag(Frag<__bf16>& f, float sc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (__bf16)((float)f.v[j] * sc);
}
__device__ __forceinline__ void scale_frag(Frag<float>& f, float sc) {
  f.a *= sc;
  f.b *= sc;
}

// Fragment from 8 fp32 values (bf16: round to nearest even).
__device__ __forceinline__ void set_frag(Frag<__bf16>& f, float x0, float x1, float x2, float x3,
                                         float x4, float x5, float x6, float x7) {
  f.v[0] = (__bf16)x0; f.v[1] = (__bf16)x1; f.v[2] = (__bf16)x2; f.v[3] = (__bf16)x3;
  f.v[4] = (__bf16)x4; f.v[5] = (__bf16)x5; f.v[6] = (__bf16)x6; f.v[7] = (__bf16)x7;
}
__device__ __forceinline__ void set_frag(Frag<float>& f, float x0, float x1, float x2, float x3,
                                         float x4, float x5, float x6, float x7) {
  f.a = f32x4{x0, x1, x2, x3};
  f.b = f32x4{x4, x5, x6, x7};
}
// Fragment m (0 or 1) of an accumulator tile: registers 8m .. 8m+7.
template <typename T>
__device__ __forceinline__ void acc_frag(Frag<T>& f, const f32x16& acc, int m) {
  const int o = 8 * m;
  set_frag(f, acc[o + 0], acc[o + 1], acc[o + 2], acc[o + 3], acc[o + 4], acc[o + 5], acc[o + 6],
           acc[o + 7]);
}

// acc += A_chunk * B_chunk over one contraction chunk of 16.
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[0], b.a[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[1], b.a[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[2], b.a[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[3], b.a[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[0], b.b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[1], b.b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[2], b.b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[3], b.b[3], acc, 0, 0, 0);
}

// Exact transposition of 32-column blocks through the matrix core. For a rows-layout A
// operand X (lane c = row; contraction chunk s = columns 16 s .. 16 s + 15, half h holding
// 8 h .. 8 h + 7 of them), the product X_{2 dc} E_0 + X_{2 dc + 1} E_1 with the constant B
// operands below (lane (c, h), element jj: 1 iff c == 16 sh + 8 h + jj) is the block
// X[:, 32 dc .. 32 dc + 31] in accumulator layout: lane c = column 32 dc + c, register r =
// row acc_row(r, h). Its registers 8m .. 8m + 7 are therefore the cols-layout fragment m of
// the block (rows 16 m + sigma(8 h + j)), ready as the A operand of a product contracted
// over rows. Products with 1 and sums with 0 are exact, so the copy is bit for bit.
template <typename T>
__device__ __forceinline__ void eye_frags(Frag<T> (&e)[2], int c, int h) {
#pragma unroll
  for (int sh = 0; sh < 2; ++sh) {
    const int j0 = c - 16 * sh - 8 * h;   // the element that is 1, if 0 <= j0 < 8
    set_frag(e[sh], j0 == 0 ? 1.f : 0.f, j0 == 1 ? 1.f : 0.f, j0 == 2 ? 1.f : 0.f, j0 == 3 ? 1.f : 0.f,
             j0 == 4 ? 1.f : 0.f, j0 == 5 ? 1.f : 0.f, j0 == 6 ? 1.f : 0.f, j0 == 7 ? 1.f : 0.f);
  }
}

// cols-layout fragments t[m][dc] of a 32-row block held as rows-layout fragments x[s]
template <typename T, int DS>
__device__ __forceinline__ void rows_to_cols(Frag<T> (&t)[2][DS / 2], const Frag<T> (&x)[DS],
                                             const Frag<T> (&e)[2]) {
#pragma unroll
  for (int dc = 0; dc < DS / 2; ++dc) {
    f32x16 acc = f32x16{};
    mma16(acc, x[2 * dc], e[0]);
    mma16(acc, x[2 * dc + 1], e[1]);
    acc_frag(t[0][dc], acc, 0);
    acc_frag(t[1][dc], acc, 1);
  }
}

// ------------------------------------------------------------------------------------------
// element stores
// ------------------------------------------------------------------------------------------
// Store 4 consecutive values (fp32 in registers) at p.
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// ------------------------------------------------------------------------------------------
// wave helpers
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int uniform_i32(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Value of lane l ^ 32 (the other half-wave), without going through LDS.
__device__ __forceinline__ float xor32f(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ int xor32i(int v) {
  auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)((threadIdx.x & 32) ? r[0] : r[1]);
}

// Wave-wide min with DPP row operations (no LDS traffic); the result is uniform.
#define ENTMAX_DPP(v, ctrl, rmask) \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), ctrl, rmask, 0xF, false))
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, ENTMAX_DPP(v, 0xB1, 0xF));
  v = fminf(v, ENTMAX_DPP(v, 0x4E, 0xF));
  v = fminf(v, ENTMAX_DPP(v, 0x141, 0xF));
  v = fminf(v, ENTMAX_DPP(v, 0x140, 0xF));
  v = fminf(v, ENTMAX_DPP(v, 0x142, 0xA));
  v = fminf(v, ENTMAX_DPP(v, 0x143, 0xC));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// floor(x) as int in one instruction (saturating: -inf -> INT_MIN, +inf -> INT_MAX).
__device__ __forceinline__ int cvt_floor(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// float -> unsigned with truncation; negative inputs (and NaN) give 0
__device__ __forceinline__ uint32_t cvt_u32_sat(float x) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// max(x, 0) in one instruction: without the canonicalisation (signalling-NaN quieting) that
// fmaxf adds in IEEE mode; matrix-core results and their sums are never signalling NaNs
__device__ __forceinline__ float relu_raw(float x) {
  float r;
  asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(x));
  return r;
}

// max of three without canonicalising the inputs (no IEEE-mode NaN quieting)
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max16(const f32x16& a) {
  const float m0 = max3_raw(a[0], a[1], a[2]);
  const float m1 = max3_raw(a[3], a[4], a[5]);
  const float m2 = max3_raw(a[6], a[7], a[8]);
  const float m3 = max3_raw(a[9], a[10], a[11]);
  const float m4 = max3_raw(a[12], a[13], a[14]);
  return max3_raw(max3_raw(m0, m1, m2), max3_raw(m3, m4, a[15]), m0);
}
// Wave-wide maxima of two values at once: v_permlane32_swap folds the upper half-wave of
// `a` onto the lower and the lower half of `b` onto the upper, so lanes 0-31 then reduce a
// and lanes 32-63 reduce b; DPP-fused v_max steps (s_nop 1 covers the VALU-write -> DPP-read
// hazard) finish each 32-lane half, whose result ends in lane 31 (a) and lane 63 (b).
__device__ __forceinline__ void pair_max_dpp(float a, float b, float& ma, float& mb) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  float v;
  asm volatile(
      "s_nop 1\n v_max_f32 %0, %1, %2\n"
      "s_nop 1\n v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n v_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n"
      "s_nop 4"
      : "=&v"(v)
      : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
  ma = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  mb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// v[lane] = x for a wave-uniform x and lane (lane select through M0: one SGPR operand per
// VOP3 instruction)
__device__ __forceinline__ void write_lane(float& v, float x, int lane) {
  asm volatile("s_mov_b32 m0, %2\n s_nop 1\n v_writelane_b32 %0, %1, m0" : "+v"(v) : "s"(x), "s"(lane) : "m0");
}

// 2^x with the hardware exponential alone (no rescaling around denormal results): softmax
// weights are exponentials of scores at or below the row's maximum, and one below 2^-126 of
// it is 0 to working precision. -inf gives 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------------------------
// the alpha-entmax weight: p = d^kappa, g = d^(kappa - 1) for d = x - tau > 0
// MODE 1: kappa = 1 (alpha = 2); MODE 2: kappa = 2 (alpha = 1.5); MODE 0: any kappa.
// ------------------------------------------------------------------------------------------
template <int MODE>
struct Weight {
  __device__ __forceinline__ static float p(float d, float kappa) {
    if constexpr (MODE == 1) return d;
    else if constexpr (MODE == 2) return d * d;
    else return d > 0.f ? exp2f(kappa * log2f(d)) : 0.f;
  }
  __device__ __forceinline__ static float g(float d, float kappa) {
    if constexpr (MODE == 1) return d > 0.f ? 1.f : 0.f;
    else if constexpr (MODE == 2) return d;
    else return d > 0.f ? exp2f((kappa - 1.f) * log2f(d)) : 0.f;
  }
};

// Buffer resource over `bytes` bytes at p (raw buffer: loads past the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// One 16-byte buffer load at byte offset voff (per lane) + soff (wave-uniform).
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// K operand loads and transposed score tiles of the attention kernels: fragment-major K
// (the row layout of prep.hip), tile = keys x queries, lane c of the B operand = query.
template <typename T, int D>
struct KvOps {
  static constexpr int DS = D / 16;
  static constexpr int DC = D / 32;
  // The same fragments of sub-block kb through a buffer resource over one head's K copy:
  // the per-lane offset is fixed and the sub-block offset is a scalar, so a load needs no
  // vector address arithmetic (and no address register that a wait would have to guard).
  __device__ __forceinline__ static void load_k_buf(Frag<T> (&f)[DS], __amdgpu_buffer_rsrc_t r, int kb, int lane) {
    const uint32_t soff = (uint32_t)kb * (uint32_t)(DS * 512 * sizeof(T));
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const uint32_t voff = (uint32_t)(s * 512 + lane * 8) * (uint32_t)sizeof(T);
      if constexpr (sizeof(T) == 2) {
        const u32x4 v = buffer_load16(r, voff, soff);
        f[s].v = __builtin_bit_cast(bf16x8, v);
      } else {
        const u32x4 a = buffer_load16(r, voff, soff);
        const u32x4 b = buffer_load16(r, voff + 16, soff);
        f[s].a = __builtin_bit_cast(f32x4, a);
        f[s].b = __builtin_bit_cast(f32x4, b);
      }
    }
  }
  // K fragments of sub-block kb (A operand: lane c is key 32 kb + c): one contiguous
  // 1 KB run per fragment at a wave-uniform base plus lane * 8 elements
  __device__ __forceinline__ static void load_k(Frag<T> (&f)[DS], const T* Kf, int kb, int c, int h) {
    const T* kp = Kf + (size_t)kb * (DS * 512);
    const int lo = (h * 32 + c) * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) load_frag(f[s], kp + s * 512 + lo);
  }
  // S^T tile (keys x queries) added to acc0; keys after the query (causal) become -inf
  __device__ __forceinline__ static f32x16 scores(const Frag<T> (&kc)[DS], const Frag<T> (&qf)[DS], int kb,
                                                  int row0, int qrow, int h, bool causal,
                                                  const f32x16& acc0 = f32x16{}) {
    f32x16 acc = acc0;
#pragma unroll
    for (int s = 0; s < DS; ++s) mma16(acc, kc[s], qf[s]);
    if (causal && kb * 32 + 31 > row0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + acc_row(r, h) > qrow) acc[r] = -INFINITY;
    }
    return acc;
  }
};

}  // namespace entmax

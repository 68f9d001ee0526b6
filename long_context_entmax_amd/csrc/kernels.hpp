// Kernel parameter blocks and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace entmax {

// Waves (32 query rows each) of a histogram work group at head_dim 64 in bf16, and the waves
// per SIMD its register budget is built for (both tunable at build time).
#ifndef ENTMAX_HIST_WAVES64
#define ENTMAX_HIST_WAVES64 8
#endif
#ifndef ENTMAX_HIST_OCC64
#define ENTMAX_HIST_OCC64 4
#endif

// Work-group to (unit, rank) map. A unit is one (batch, KV head); all of its work
// groups land on the same XCD (work group i runs on XCD i % 8) so K/V blocks are
// reused from that XCD's L2. rank 0 is the longest work item of the unit.
struct WgMap {
  int U;      // units
  int R;      // ranks per unit
  int xcd;    // 1: XCD-grouped order (U % 8 == 0), 0: flat order
  int fold;   // 1: the second half of the ranks in reverse (shortest first), so work groups
              // dispatched half a grid apart -- which share a CU when two fit -- pair long
              // with short items
};

__host__ __device__ inline int wgmap_grid(const WgMap& m) {
  if (m.xcd) return 8 * ((m.U + 7) / 8) * m.R;
  return m.U * m.R;
}

__device__ __forceinline__ bool wgmap_get(const WgMap& m, int bid, int& unit, int& rank) {
  if (m.xcd) {
    const int x = bid & 7, s = bid >> 3;
    const int cnt = (m.U - x + 7) >> 3;
    if (s >= cnt * m.R) return false;
    unit = x + 8 * (s % cnt);
    rank = s / cnt;
  } else {
    if (bid >= m.U * m.R) return false;
    unit = bid % m.U;
    rank = bid / m.U;
  }
  if (m.fold) {
    const int h = (m.R + 1) >> 1;
    if (rank >= h) rank = m.R - 1 - (rank - h);
  }
  return true;
}

struct FwdParams {
  const void* q;
  const void* k;
  const void* kf;        // K, fragment-major rows
  const void* vf;        // V, fragment-major columns
  float* o;              // fp32 [b, hq, n, D]
  float* tau;
  uint32_t* mask;
  float* aux;            // o~ [b, hq, n, D] fp32
  int32_t* hist;         // optional [b, hq, n, B]
  float* tau_h;          // optional [b, hq, n]
  unsigned long long* stats;  // optional [32]
  float* dmax;           // workspace: per (32-row chunk, 32-key sub-block) max of x*B (rows: dmax_row)
  float* wmax;           // workspace: per (32-row chunk, word of 32 sub-blocks) max of dmax [b*hq][n/32][NW32]
  float4* tauh_ws;       // workspace: (tau_h, x_max, refinement start, 0) per row [b*hq*n]
  int b, hq, hkv, n, G;
  int causal, Br, Bc, B, max_iters;
  float cx;              // (alpha - 1) * scale
  float alpha, kappa, tol;
  int GP;                // query heads per work group
  int RH;                // rows per head per work group
  int RG;                // row groups per head = ceil(n / RH)
  int nkb, NW32;         // 32-key sub-blocks, words of sub-block bits
  int out_lds_wave;      // refinement kernel: LDS bytes per wave (sub-block maxima as bf16, then word maxima)
  int out_lds_wmax;      // offset of the word maxima in a wave's LDS part
  int Tr, Tc, W;
  WgMap map;             // histogram kernel
  WgMap map2;            // refinement/output kernel
  int tau_init;          // 0: histogram bound; 1: plain bracket from the row max (no histogram)
  int dense;             // 1: no block skipping (every valid sub-block visited, every valid mask bit set)
  const float* slopes;   // optional [hq]: position-bias slope m of each query head (scores - m |i - j|)
};

// Offset of the sub-block maxima of (query head bh, 32-row chunk) in FwdParams::dmax: one fp32
// per 32-key sub-block the chunk can see -- under the causal mask chunk c sees sub-blocks
// 0..c, so the table is a packed lower triangle of nkb (nkb + 1) / 2 entries per head.
__host__ __device__ __forceinline__ size_t dmax_row(const FwdParams& p, size_t bh, int chunk) {
  if (p.causal) return bh * ((size_t)p.nkb * (p.nkb + 1) / 2) + (size_t)chunk * (chunk + 1) / 2;
  return (bh * p.nkb + chunk) * (size_t)p.nkb;
}

// one re-layout of X [heads, n, D] (prep.hip): any of the fragment-major row copy,
// the fragment-major column copy and delta = X . aux per row (X = dO, aux = o~)
struct Relayout {
  const void* src;
  void* rows;            // nullable
  void* cols;            // nullable
  const float* aux;      // with delta
  float* delta;          // nullable
  int heads;
  const char* name;      // timing label
};

// several re-layout jobs and an optional mask transpose in one launch (prep.hip)
struct PrepBatch {
  Relayout job[4];
  int njobs;
  int start[5];          // first work group of each job (filled by the launcher)
  int n;                 // rows per head of every job
  const uint32_t* mask;  // nullable: mask [planes, Tr, W] to transpose into maskT
  uint32_t* maskT;
  int planes, Tr, Tc, W, WT;
};

struct BwdParams {
  const void* qr;        // fragment-major rows copies (prep.hip)
  const void* dor;
  const void* kr;
  const void* vr;
  const float* tau;
  const float* delta;
  const uint32_t* mask;  // [b, hq, Tr, W]
  const uint32_t* maskT; // [b, hq, Tc, WT]
  void* dq;
  void* dk;
  void* dv;
  int b, hq, hkv, n, G;
  int causal, Br, Bc;
  float cx, scale, kappa;
  float am1;             // alpha - 1 (scales the position bias onto the x-scale)
  const float* slopes;   // optional [hq] position-bias slopes
  int Tr, Tc, W, WT;
  int dense;             // 1: every item of the mask multiplied in full (no zero-block skip)
  // mode 3, the DashAttention stage-2 backward (softmax with the routing prior), in base-2
  // units: tau holds the row's lse log2 e, cx the score scale times log2 e; key j of a routed
  // chunk c adds sigma log2 wbar(c, i)
  const float* lp;       // [b, hkv, nc, n] the prior sigma log2 wbar (-inf where wbar = 0), chunk-major
  int C;                 // keys per chunk
  float* dq32;           // [b, hq, n, D] fp32 dQ (mode 3 writes here instead of dq)
  float* dbias;          // [b, hq, n / 32, n] per (32-key sub-block, row) sums of dS (mode 3)
  WgMap map;
};

// Mode of the backward kernels for the DashAttention stage-2 softmax (modes 0-2 are the
// alpha-entmax weights)
constexpr int MODE_DASH = 3;

// decode (decode.hip): the largest key slice of a score / histogram work group
constexpr int DEC_SPLIT_MAX = 2048;

struct DecParams {
  const void* q;         // [b, hq, D]
  const void* k;         // [b, hkv, n, D] cache
  const void* v;
  const int32_t* lengths;  // optional [b]
  const float* slopes;   // optional [hq]
  float* o;              // [b, hq, D] fp32
  float* tau;            // [b, hq]
  int32_t* hist;         // optional [b, hq, B]
  float* tau_h;          // optional [b, hq]
  float* xs;             // workspace: scores [b, hq, n] fp32
  float* smax;           // workspace: per-slice max [b, hq, nsplit]
  int32_t* hcnt;         // workspace: per-slice histogram counts [b, hq, nsplit, 16]
  float* opart;          // workspace: per-output-slice partial o [nsplit_o, b, hq, D]
  int b, hq, hkv, G, n, B, max_iters, tau_init, nsplit, nsplit_o;
  int split, osplit;     // keys per slice of the score/histogram and of the output kernels
  int ldx;               // row stride of xs: n rounded up to a multiple of 4
  float cx, am1, alpha, kappa, tol;
};

// DashAttention stages 1-2 (dash.hip)
struct DashParams {
  const void* q;         // [b, hq, n, D]
  const void* ks;        // chunk summaries [b, hkv, nc, D]
  const void* kf;        // K, fragment-major rows
  const void* vf;        // V, fragment-major columns
  float* o;              // [b, hq, n, D] fp32
  float* lse;            // optional [b, hq, n]
  float* rtau;           // optional [b, hq, n]
  float* rw;             // [b, hkv, nc, n] group-averaged routing weights
  uint32_t* cmask;       // [b, hkv, Tr, Wc]
  int b, hq, hkv, n, G, C, nc, Tr, Wc, max_iters;
  float cx;              // (alpha - 1) * gamma * scale: routing logits on the x-scale
  float alpha, kappa, tol;
  float c2;              // scale * log2(e): token scores in base-2 units
  float sigma;
  // backward (entmax_dash_bwd)
  const float* dbias;    // [b, hq, n / 32, n] per (32-key sub-block, row) sums of the stage-2 dS
  const float* dq32;     // [b, hq, n, D] stage-2 dQ (fp32)
  void* dq;              // [b, hq, n, D] dQ out (dtype)
  float* lp;             // [b, hkv, nc, n] the prior sigma log2 wbar, -inf where wbar = 0
  const float* lse_in;   // [b, hq, n] stage-2 lse (natural log) of the forward
  float* lse2;           // [b, hq, n] the same times log2 e
  float* dw;             // [b, hkv, nc, n] gradient of each head's routing weights (chunk-major)
  float* du;             // [b, hq, nc, n] routing-logit gradient (chunk-major)
  const void* qc;        // Q, fragment-major columns
  float* dpart;          // [b * hkv, Wc, NP, D, 32] partial summary gradients (per row piece)
  void* dks;             // [b, hkv, nc, D] summary gradient out (dtype)
  uint32_t* fine;        // [b, hkv, n / 32, Wc] chunk bits of each 32-row block (some row routes it)
  uint32_t* bmask;       // [b, hq, n / 32, W] 32 x 64 block mask of stage 2
  int W;                 // words per block-mask row
  int NP, PR;            // row pieces of the summary-gradient product and rows per piece
  float gs;              // gamma * scale: d zbar / d (q . ksum)
};

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int mode, hipStream_t s);
hipError_t launch_dash(const DashParams& p, int dtype, int D, int mode, hipStream_t s);
hipError_t launch_dash_bwd_setup(const DashParams& p, hipStream_t s);
hipError_t launch_dash_route_bwd(const DashParams& p, int dtype, int D, int mode, hipStream_t s);
hipError_t launch_decode(const DecParams& p, int dtype, int D, int mode, hipStream_t s);
hipError_t launch_prep(const PrepBatch& b, int dtype, int D, const char* name, hipStream_t s);
hipError_t launch_bwd_dkv(const BwdParams& p, int dtype, int D, int mode, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int D, int mode, hipStream_t s);

// timing hooks (api.hip): called around every launch
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

}  // namespace entmax

// C ABI of the alpha-entmax attention library: argument checks, workspace layout,
// launch sequencing and kernel timing. See include/entmax_attn.h for the contract.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dash_attn.h"
#include "../../include/entmax_attn.h"
#include "common.hpp"
#include "kernels.hpp"

namespace entmax {

static thread_local char t_err[512];

static entmax_status fail(entmax_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_err, sizeof(t_err), fmt, ap);
  va_end(ap);
  return s;
}

static entmax_status hip_fail(hipError_t e, const char* what) {
  return fail(ENTMAX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------------------------------------
// kernel timing
// ------------------------------------------------------------------------------------------
namespace {
struct Pending {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
thread_local const char* t_name = nullptr;
thread_local hipEvent_t t_start = nullptr;

hipEvent_t take_event() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void prof_begin(const char* name, hipStream_t s) {
  t_start = nullptr;
  if (!g_on) return;
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) return;
  t_name = name;
  t_start = e;
}

void prof_end(hipStream_t s) {
  if (!g_on || !t_start) return;
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({t_name, t_start, e});
  t_start = nullptr;
}

// ------------------------------------------------------------------------------------------
// argument checks and derived sizes
// ------------------------------------------------------------------------------------------
struct Derived {
  int b, hq, hkv, n, D, G, dtype, causal, Br, Bc, B, max_iters, tau_init, dense;
  float alpha, scale, tol, kappa;
  int mode;               // 1: alpha = 2, 2: alpha = 1.5, 0: other
  int Tr, Tc, W, WT, nkb, NW32;
  size_t es;              // element size
  // forward decomposition
  int QW, GP, RH, RG;
};

static bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// decode: blocks and the causal flag are not used, seqlen is the cache capacity (any value)
static entmax_status derive(const entmax_attn_desc* d, Derived& o, bool decode = false) {
  if (!d) return fail(ENTMAX_ERR_NULL, "desc is NULL");
  o.b = d->batch; o.hq = d->heads_q; o.hkv = d->heads_kv; o.n = d->seqlen; o.D = d->head_dim;
  if (o.b < 0 || o.hq < 0 || o.hkv < 0 || o.n < 0 || o.D <= 0)
    return fail(ENTMAX_ERR_SHAPE, "negative size (batch %d, heads %d/%d, seqlen %d, head_dim %d)",
                o.b, o.hq, o.hkv, o.n, o.D);
  if (o.hkv == 0 && o.hq != 0) return fail(ENTMAX_ERR_SHAPE, "heads_kv is 0 but heads_q is %d", o.hq);
  if (o.hkv > 0 && o.hq % o.hkv != 0)
    return fail(ENTMAX_ERR_SHAPE, "heads_q (%d) is not a multiple of heads_kv (%d)", o.hq, o.hkv);
  if (!(d->alpha > 1.0f && d->alpha <= 16.0f) || !isfinite(d->alpha))
    return fail(ENTMAX_ERR_ALPHA, "alpha must be finite and in (1, 16], got %g", (double)d->alpha);
  if (d->dtype != ENTMAX_F32 && d->dtype != ENTMAX_BF16)
    return fail(ENTMAX_ERR_UNSUPPORTED, "dtype %d is not F32 (0) or BF16 (1)", d->dtype);
  if (o.D != 64 && o.D != 128) return fail(ENTMAX_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128", o.D);
  o.Br = decode ? 32 : d->block_q;
  o.Bc = decode ? 32 : d->block_k;
  if (!(o.Br == 32 || o.Br == 64 || o.Br == 128) || !(o.Bc == 32 || o.Bc == 64 || o.Bc == 128))
    return fail(ENTMAX_ERR_UNSUPPORTED, "blocks %dx%d: each must be 32, 64 or 128", o.Br, o.Bc);
  if (!decode && (o.n % o.Br != 0 || o.n % o.Bc != 0))
    return fail(ENTMAX_ERR_SHAPE, "seqlen %d is not a multiple of the blocks %dx%d", o.n, o.Br, o.Bc);
  if (decode && o.hkv > 0 && o.hq / o.hkv > 16)
    return fail(ENTMAX_ERR_UNSUPPORTED, "decode: heads_q / heads_kv = %d > 16", o.hq / o.hkv);
  if (o.n > (1 << 19)) return fail(ENTMAX_ERR_UNSUPPORTED, "seqlen %d > 524288", o.n);
  o.B = d->n_bins;
  if (!pow2(o.B) || o.B < 2 || o.B > 16)
    return fail(ENTMAX_ERR_UNSUPPORTED, "n_bins %d: must be 2, 4, 8 or 16", o.B);
  if (!decode && d->causal != 0 && d->causal != 1) return fail(ENTMAX_ERR_SHAPE, "causal must be 0 or 1");
  o.causal = decode ? 1 : d->causal;
  // default pass caps: Halley (alpha <= 1.5) converges in a few passes; Newton from
  // below shrinks a large support about by half per pass; the secant needs the most
  if (d->tau_init != 0 && d->tau_init != 1)
    return fail(ENTMAX_ERR_UNSUPPORTED, "tau_init %d: must be 0 (histogram) or 1 (plain bracket)", d->tau_init);
  o.tau_init = d->tau_init;
  if (d->dense != 0 && d->dense != 1) return fail(ENTMAX_ERR_SHAPE, "dense must be 0 or 1");
  o.dense = decode ? 0 : d->dense;
  o.max_iters = d->max_iters != 0       ? d->max_iters
                : d->alpha > 2.0f      ? 30
                : (o.tau_init == 1)    ? 15
                : d->alpha > 1.5f      ? 12
                                       : 8;
  if (o.max_iters < 1 || o.max_iters > 30)
    return fail(ENTMAX_ERR_SHAPE, "max_iters %d: must be 0 (default) or 1..30", d->max_iters);
  if (!(d->scale >= 0.0f) || !isfinite(d->scale)) return fail(ENTMAX_ERR_SHAPE, "scale must be >= 0 and finite");
  if (!(d->tol >= 0.0f) || !isfinite(d->tol)) return fail(ENTMAX_ERR_SHAPE, "tol must be >= 0 and finite");
  o.dtype = d->dtype;
  o.alpha = d->alpha;
  o.scale = d->scale == 0.0f ? (float)(1.0 / sqrt((double)o.D)) : d->scale;
  o.tol = d->tol == 0.0f ? ldexpf(1.0f, -20) : d->tol;
  o.kappa = (float)(1.0 / ((double)o.alpha - 1.0));
  o.mode = (o.alpha == 2.0f) ? 1 : (o.alpha == 1.5f ? 2 : 0);
  o.G = o.hkv > 0 ? o.hq / o.hkv : 1;
  o.Tr = o.n / o.Br;
  o.Tc = o.n / o.Bc;
  o.W = (o.Tc + 31) / 32;
  o.WT = (o.Tr + 31) / 32;
  o.nkb = o.n / 32;
  o.NW32 = (o.nkb + 31) / 32;
  o.es = o.dtype == ENTMAX_BF16 ? 2 : 4;
  // histogram work group: HW waves x 32 rows over GP query heads of one KV head (HW = 4 at
  // head_dim 128 in bf16, else 8; the kernels check that they were built for the same shape)
  o.QW = 32;
  const int HW = (o.D == 128 && d->dtype == ENTMAX_BF16) ? 4 : (o.D == 64 && d->dtype == ENTMAX_BF16) ? ENTMAX_HIST_WAVES64 : 8;
  o.GP = 1;
  for (int gp : {8, 4, 2}) {
    if (gp <= HW && o.G % gp == 0 && ((HW / gp) * o.QW) % o.Br == 0) {
      o.GP = gp;
      break;
    }
  }
  o.RH = (HW / o.GP) * o.QW;
  o.RG = (o.n + o.RH - 1) / o.RH;
  return ENTMAX_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// forward workspace: K and V fragment-major copies, then per (chunk, sub-block) maxima
static size_t fwd_kv_bytes(const Derived& o) { return align256((size_t)o.b * o.hkv * o.D * o.n * o.es); }
// per (query head, 32-row chunk) the maxima of the 32-key sub-blocks the chunk can see: a packed
// lower triangle under the causal mask
static size_t fwd_dmax_bytes(const Derived& o) {
  const size_t per_head = o.causal ? (size_t)o.nkb * (o.nkb + 1) / 2 : (size_t)o.nkb * o.nkb;
  return align256((size_t)o.b * o.hq * per_head * 4);
}
static size_t fwd_wmax_bytes(const Derived& o) { return align256((size_t)o.b * o.hq * (size_t)o.nkb * o.NW32 * 4); }
static size_t fwd_ws(const Derived& o) {
  return 2 * fwd_kv_bytes(o) + fwd_dmax_bytes(o) + fwd_wmax_bytes(o) + align256((size_t)o.b * o.hq * o.n * 16);
}

// backward workspace: delta, transposed mask, then fragment-major rows copies of Q, dO, K
// and V (the kernels form the transposed operands on the matrix core)
struct BwdLayout {
  size_t delta, maskT, qr, dor, kr, vr, total;
};
static BwdLayout bwd_ws(const Derived& o) {
  BwdLayout L;
  size_t off = 0;
  const size_t qbytes = align256((size_t)o.b * o.hq * o.D * o.n * o.es);
  const size_t kbytes = align256((size_t)o.b * o.hkv * o.D * o.n * o.es);
  L.delta = off; off += align256((size_t)o.b * o.hq * o.n * 4);
  L.maskT = off; off += align256((size_t)o.b * o.hq * o.Tc * o.WT * 4);
  L.qr = off; off += qbytes;
  L.dor = off; off += qbytes;
  L.kr = off; off += kbytes;
  L.vr = off; off += kbytes;
  L.total = off;
  return L;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static WgMap make_map(int U, int R, int fold = 0) {
  WgMap m;
  m.U = U;
  m.R = R;
  m.fold = fold;
  m.xcd = (U > 0 && U % 8 == 0) ? 1 : 0;
  return m;
}

// DashAttention forward (stages 1-2): checks and derived sizes
struct DashDerived {
  int b, hq, hkv, n, D, G, dtype, C, nc, Tr, Wc, max_iters, mode;
  float alpha, kappa, gamma, sigma, scale, tol;
  size_t es;
};

static entmax_status derive_dash(const entmax_dash_desc* d, DashDerived& o) {
  if (!d) return fail(ENTMAX_ERR_NULL, "desc is NULL");
  o.b = d->batch; o.hq = d->heads_q; o.hkv = d->heads_kv; o.n = d->seqlen; o.D = d->head_dim;
  if (o.b < 0 || o.hq < 0 || o.hkv < 0 || o.n < 0 || o.D <= 0)
    return fail(ENTMAX_ERR_SHAPE, "negative size (batch %d, heads %d/%d, seqlen %d, head_dim %d)",
                o.b, o.hq, o.hkv, o.n, o.D);
  if (o.hkv == 0 && o.hq != 0) return fail(ENTMAX_ERR_SHAPE, "heads_kv is 0 but heads_q is %d", o.hq);
  if (o.hkv > 0 && o.hq % o.hkv != 0)
    return fail(ENTMAX_ERR_SHAPE, "heads_q (%d) is not a multiple of heads_kv (%d)", o.hq, o.hkv);
  if (!(d->route_alpha > 1.0f && d->route_alpha <= 16.0f) || !isfinite(d->route_alpha))
    return fail(ENTMAX_ERR_ALPHA, "route_alpha must be finite and in (1, 16], got %g", (double)d->route_alpha);
  if (d->dtype != ENTMAX_F32 && d->dtype != ENTMAX_BF16)
    return fail(ENTMAX_ERR_UNSUPPORTED, "dtype %d is not F32 (0) or BF16 (1)", d->dtype);
  if (o.D != 64 && o.D != 128) return fail(ENTMAX_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128", o.D);
  o.C = d->chunk;
  if (o.C != 64 && o.C != 128 && o.C != 256)
    return fail(ENTMAX_ERR_UNSUPPORTED, "chunk %d: must be 64, 128 or 256", o.C);
  if (o.n % o.C != 0) return fail(ENTMAX_ERR_SHAPE, "seqlen %d is not a multiple of the chunk %d", o.n, o.C);
  o.nc = o.n / o.C;
  if (o.nc > 256) return fail(ENTMAX_ERR_UNSUPPORTED, "%d chunks: at most 256", o.nc);
  if (!(d->gamma >= 0.0f) || !isfinite(d->gamma)) return fail(ENTMAX_ERR_SHAPE, "gamma must be >= 0 and finite");
  if (!(d->sigma >= 0.0f) || !isfinite(d->sigma)) return fail(ENTMAX_ERR_SHAPE, "sigma must be >= 0 and finite");
  if (!(d->scale >= 0.0f) || !isfinite(d->scale)) return fail(ENTMAX_ERR_SHAPE, "scale must be >= 0 and finite");
  if (!(d->tol >= 0.0f) || !isfinite(d->tol)) return fail(ENTMAX_ERR_SHAPE, "tol must be >= 0 and finite");
  o.max_iters = d->max_iters != 0 ? d->max_iters : (d->route_alpha > 2.0f ? 30 : 15);
  if (o.max_iters < 1 || o.max_iters > 30)
    return fail(ENTMAX_ERR_SHAPE, "max_iters %d: must be 0 (default) or 1..30", d->max_iters);
  o.dtype = d->dtype;
  o.alpha = d->route_alpha;
  o.kappa = (float)(1.0 / ((double)o.alpha - 1.0));
  o.mode = (o.alpha == 2.0f) ? 1 : (o.alpha == 1.5f ? 2 : 0);
  o.gamma = d->gamma == 0.0f ? 1.0f : d->gamma;
  o.sigma = d->sigma;
  o.scale = d->scale == 0.0f ? (float)(1.0 / sqrt((double)o.D)) : d->scale;
  o.tol = d->tol == 0.0f ? ldexpf(1.0f, -20) : d->tol;
  o.G = o.hkv > 0 ? o.hq / o.hkv : 1;
  o.Tr = o.n / 64;
  o.Wc = (o.nc + 31) / 32;
  o.es = o.dtype == ENTMAX_BF16 ? 2 : 4;
  return ENTMAX_OK;
}

static size_t dash_kv_bytes(const DashDerived& o) { return align256((size_t)o.b * o.hkv * o.n * o.D * o.es); }

// Scratch of the allocation-free decode entry point. Every device that loads this library
// holds its own instance until the process ends. In host code `scratch` only names the
// symbol: its device address (per device) comes from hipGetSymbolAddress, and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[ENTMAX_DECODE_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};
}  // namespace

// Device address of the current device's scratch, looked up once per device (with that
// device current) and kept.
static entmax_status decode_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(ENTMAX_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                SCRATCH_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(ENTMAX_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = (char*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return ENTMAX_OK;
}

}  // namespace entmax

using namespace entmax;

extern "C" {

size_t entmax_attn_fwd_workspace_bytes(const entmax_attn_desc* desc) {
  Derived o;
  if (derive(desc, o) != ENTMAX_OK) return 0;
  return fwd_ws(o);
}

size_t entmax_attn_bwd_workspace_bytes(const entmax_attn_desc* desc) {
  Derived o;
  if (derive(desc, o) != ENTMAX_OK) return 0;
  return bwd_ws(o).total;
}

size_t entmax_attn_aux_bytes(const entmax_attn_desc* desc) {
  Derived o;
  if (derive(desc, o) != ENTMAX_OK) return 0;
  return (size_t)o.b * o.hq * o.n * o.D * sizeof(float);
}

size_t entmax_attn_mask_words(const entmax_attn_desc* desc) {
  Derived o;
  if (derive(desc, o) != ENTMAX_OK) return 0;
  return (size_t)o.b * o.hq * o.Tr * o.W;
}

entmax_status entmax_attn_fwd(const entmax_attn_desc* desc, const void* q, const void* k, const void* v,
                              const float* slopes, void* o_, float* tau, uint32_t* block_mask, void* aux,
                              int32_t* hist_counts,
                              float* tau_h, uint64_t* stats, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Derived o;
  entmax_status st = derive(desc, o);
  if (st != ENTMAX_OK) return st;
  const size_t elems = (size_t)o.b * o.hq * o.n;
  if (elems == 0) return ENTMAX_OK;
  if (!q || !k || !v || !o_ || !tau || !block_mask || !aux)
    return fail(ENTMAX_ERR_NULL, "q, k, v, o, tau, block_mask and aux are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_, 16) || !aligned(aux, 16) ||
      !aligned(tau, 4) || !aligned(block_mask, 4) || (hist_counts && !aligned(hist_counts, 4)) ||
      (tau_h && !aligned(tau_h, 4)) || (stats && !aligned(stats, 8)) || (slopes && !aligned(slopes, 4)))
    return fail(ENTMAX_ERR_ALIGN, "q, k, v, o, aux need 16-byte alignment; tau, mask, counts, slopes 4-byte");
  const size_t need = fwd_ws(o);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(ENTMAX_ERR_WORKSPACE, "forward workspace: need %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  hipStream_t s = (hipStream_t)stream;

  char* wsb = (char*)workspace;
  // fragment-major copies: K in the row layout, V in the column layout (one launch)
  PrepBatch pb{};
  pb.job[0] = Relayout{k, wsb, nullptr, nullptr, nullptr, o.b * o.hkv, "k"};
  pb.job[1] = Relayout{v, nullptr, wsb + fwd_kv_bytes(o), nullptr, nullptr, o.b * o.hkv, "v"};
  pb.njobs = 2;
  pb.n = o.n;
  hipError_t e = launch_prep(pb, o.dtype, o.D, "fwd_prep", s);
  if (e != hipSuccess) return hip_fail(e, "fragment-major copies of K and V");

  FwdParams p{};
  p.q = q; p.kf = wsb; p.vf = wsb + fwd_kv_bytes(o); p.o = (float*)o_; p.tau = tau; p.mask = block_mask; p.aux = (float*)aux;
  p.hist = hist_counts; p.tau_h = tau_h; p.stats = (unsigned long long*)stats;
  p.dmax = (float*)(wsb + 2 * fwd_kv_bytes(o));
  p.wmax = (float*)(wsb + 2 * fwd_kv_bytes(o) + fwd_dmax_bytes(o));
  p.tauh_ws = (float4*)(wsb + 2 * fwd_kv_bytes(o) + fwd_dmax_bytes(o) + fwd_wmax_bytes(o));
  p.b = o.b; p.hq = o.hq; p.hkv = o.hkv; p.n = o.n; p.G = o.G;
  p.causal = o.causal; p.Br = o.Br; p.Bc = o.Bc; p.B = o.B; p.max_iters = o.max_iters;
  p.tau_init = o.tau_init;
  p.dense = o.dense;
  p.slopes = slopes;
  p.cx = (float)(((double)o.alpha - 1.0) * (double)o.scale);
  p.alpha = o.alpha; p.kappa = o.kappa; p.tol = o.tol;
  p.GP = o.GP; p.RH = o.RH; p.RG = o.RG;
  p.nkb = o.nkb; p.NW32 = o.NW32; p.Tr = o.Tr; p.Tc = o.Tc; p.W = o.W;
  p.out_lds_wmax = (int)(((size_t)o.nkb * 2 + 15) & ~(size_t)15);
  p.out_lds_wave = p.out_lds_wmax + (int)(((size_t)o.NW32 * 4 + 15) & ~(size_t)15);
  // Causal rows differ in length. When the whole histogram grid is resident at once (two
  // 8-wave groups per CU at head_dim 64 in bf16), pair long and short groups on a CU;
  // otherwise longest first is the better order.
  p.map = make_map(o.b * o.hkv, (o.G / o.GP) * o.RG);
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      p.map.fold = o.causal && o.D == 64 && o.dtype == ENTMAX_BF16 && wgmap_grid(p.map) <= 2 * cus;
  }
  p.map2 = make_map(o.b * o.hkv, o.G * ((o.nkb + 3) / 4));
  e = launch_fwd(p, o.dtype, o.D, o.mode, s);
  if (e != hipSuccess) return hip_fail(e, "forward kernel");
  return ENTMAX_OK;
}

entmax_status entmax_attn_bwd(const entmax_attn_desc* desc, const void* q, const void* k, const void* v,
                              const void* dout, const float* slopes, const float* tau,
                              const uint32_t* block_mask, const void* aux,
                              void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Derived o;
  entmax_status st = derive(desc, o);
  if (st != ENTMAX_OK) return st;
  if ((size_t)o.b * o.hq * o.n == 0) return ENTMAX_OK;
  if (!q || !k || !v || !dout || !tau || !block_mask || !aux || !dq || !dk || !dv)
    return fail(ENTMAX_ERR_NULL, "q, k, v, dout, tau, block_mask, aux, dq, dk and dv are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(aux, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(tau, 16) ||
      !aligned(block_mask, 4) || (slopes && !aligned(slopes, 4)))
    return fail(ENTMAX_ERR_ALIGN, "tensors need 16-byte alignment (block_mask, slopes 4-byte)");
  const BwdLayout L = bwd_ws(o);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
    return fail(ENTMAX_ERR_WORKSPACE, "backward workspace: need %zu bytes, 256-byte aligned (got %zu)", L.total,
                workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  const int hq_all = o.b * o.hq, hkv_all = o.b * o.hkv;
  // one launch: fragment-major rows copies of dO (with delta = dO . o~), Q, K and V, and the
  // transposed block mask
  PrepBatch pb{};
  pb.job[0] = Relayout{dout, ws + L.dor, nullptr, (const float*)aux, (float*)(ws + L.delta), hq_all, "do"};
  pb.job[1] = Relayout{q, ws + L.qr, nullptr, nullptr, nullptr, hq_all, "q"};
  pb.job[2] = Relayout{k, ws + L.kr, nullptr, nullptr, nullptr, hkv_all, "k"};
  pb.job[3] = Relayout{v, ws + L.vr, nullptr, nullptr, nullptr, hkv_all, "v"};
  pb.njobs = 4;
  pb.n = o.n;
  pb.mask = block_mask;
  pb.maskT = (uint32_t*)(ws + L.maskT);
  pb.planes = hq_all; pb.Tr = o.Tr; pb.Tc = o.Tc; pb.W = o.W; pb.WT = o.WT;
  hipError_t e = launch_prep(pb, o.dtype, o.D, "bwd_prep", s);
  if (e != hipSuccess) return hip_fail(e, "backward preparation");

  BwdParams p{};
  p.qr = ws + L.qr; p.dor = ws + L.dor;
  p.kr = ws + L.kr; p.vr = ws + L.vr;
  p.tau = tau; p.delta = (const float*)(ws + L.delta);
  p.mask = block_mask; p.maskT = (const uint32_t*)(ws + L.maskT);
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.b = o.b; p.hq = o.hq; p.hkv = o.hkv; p.n = o.n; p.G = o.G;
  p.causal = o.causal; p.Br = o.Br; p.Bc = o.Bc;
  p.cx = (float)(((double)o.alpha - 1.0) * (double)o.scale);
  p.scale = o.scale; p.kappa = o.kappa;
  p.am1 = o.alpha - 1.0f; p.slopes = slopes;
  p.Tr = o.Tr; p.Tc = o.Tc; p.W = o.W; p.WT = o.WT;
  p.dense = o.dense;

  p.map = make_map(o.b * o.hkv, o.Tc);
  prof_begin("entmax_bwd_dkv", s);
  e = launch_bwd_dkv(p, o.dtype, o.D, o.mode, s);
  prof_end(s);
  if (e != hipSuccess) return hip_fail(e, "dK/dV kernel");

  p.map = make_map(o.b * o.hkv, o.G * o.Tr);
  prof_begin("entmax_bwd_dq", s);
  e = launch_bwd_dq(p, o.dtype, o.D, o.mode, s);
  prof_end(s);
  if (e != hipSuccess) return hip_fail(e, "dQ kernel");
  return ENTMAX_OK;
}

struct DecLayout {
  size_t xs, smax, hcnt, opart, total;
  int split, osplit, nsplit, nsplit_o, ldx;
};

// slice size: the largest power of two in [lo, hi] that still gives about 1024 work groups
// over the (slice, KV head) grid, so short caches and few heads still fill the chip
static int dec_slice(long long keys_all_heads, int lo, int hi) {
  int s = hi;
  while (s > lo && keys_all_heads / s < 1024) s >>= 1;
  return s;
}

static DecLayout dec_ws(const Derived& o) {
  DecLayout L;
  const long long keys = (long long)o.n * o.b * o.hkv;
  L.split = dec_slice(keys, 256, DEC_SPLIT_MAX);
  L.osplit = dec_slice(keys, 128, 512);
  L.nsplit = (o.n + L.split - 1) / L.split;
  L.nsplit_o = (o.n + L.osplit - 1) / L.osplit;
  const size_t rows = (size_t)o.b * o.hq;
  L.xs = 0;
  L.ldx = (o.n + 3) & ~3;
  L.smax = align256(rows * L.ldx * sizeof(float));
  L.hcnt = L.smax + align256(rows * L.nsplit * sizeof(float));
  L.opart = L.hcnt + align256(rows * L.nsplit * 16 * sizeof(int32_t));
  L.total = L.opart + align256((size_t)L.nsplit_o * rows * o.D * sizeof(float));
  return L;
}

size_t entmax_attn_decode_workspace_bytes(const entmax_attn_desc* desc) {
  Derived o;
  if (derive(desc, o, true) != ENTMAX_OK) return 0;
  return dec_ws(o).total;
}

entmax_status entmax_attn_decode(const entmax_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* lengths, const float* slopes, float* o_,
                                 float* tau, int32_t* hist_counts, float* tau_h, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Derived o;
  entmax_status st = derive(desc, o, true);
  if (st != ENTMAX_OK) return st;
  if ((size_t)o.b * o.hq == 0) return ENTMAX_OK;
  if (o.n == 0) return fail(ENTMAX_ERR_SHAPE, "decode needs a cache of at least one key (seqlen 0)");
  if (!q || !k_cache || !v_cache || !o_ || !tau)
    return fail(ENTMAX_ERR_NULL, "q, k_cache, v_cache, o and tau are required");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o_, 16) || !aligned(tau, 4) ||
      (lengths && !aligned(lengths, 4)) || (slopes && !aligned(slopes, 4)) ||
      (hist_counts && !aligned(hist_counts, 4)) || (tau_h && !aligned(tau_h, 4)))
    return fail(ENTMAX_ERR_ALIGN, "q, k_cache, v_cache, o need 16-byte alignment; the others 4-byte");
  const DecLayout L = dec_ws(o);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
    return fail(ENTMAX_ERR_WORKSPACE, "decode workspace: need %zu bytes, 256-byte aligned (got %zu)", L.total,
                workspace_bytes);
  char* ws = (char*)workspace;
  DecParams p{};
  p.q = q; p.k = k_cache; p.v = v_cache; p.lengths = lengths; p.slopes = slopes;
  p.o = o_; p.tau = tau; p.hist = hist_counts; p.tau_h = tau_h;
  p.xs = (float*)(ws + L.xs); p.smax = (float*)(ws + L.smax); p.hcnt = (int32_t*)(ws + L.hcnt); p.opart = (float*)(ws + L.opart);
  p.b = o.b; p.hq = o.hq; p.hkv = o.hkv; p.G = o.G; p.n = o.n; p.B = o.B;
  p.max_iters = o.max_iters; p.tau_init = o.tau_init; p.nsplit = L.nsplit; p.nsplit_o = L.nsplit_o;
  p.split = L.split; p.osplit = L.osplit; p.ldx = L.ldx;
  p.cx = (float)(((double)o.alpha - 1.0) * (double)o.scale);
  p.am1 = o.alpha - 1.0f; p.alpha = o.alpha; p.kappa = o.kappa; p.tol = o.tol;
  const hipError_t e = launch_decode(p, o.dtype, o.D, o.mode, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode kernels");
  return ENTMAX_OK;
}

entmax_status entmax_attn_decode_noalloc(const entmax_attn_desc* desc, const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* lengths, const float* slopes,
                                         float* o_, float* tau, int32_t* hist_counts, float* tau_h,
                                         void* stream) {
  Derived o;
  entmax_status st = derive(desc, o, true);
  if (st != ENTMAX_OK) return st;
  const size_t need = dec_ws(o).total;
  if (need > (size_t)ENTMAX_DECODE_SCRATCH_BYTES)
    return fail(ENTMAX_ERR_WORKSPACE,
                "decode without allocation: this problem needs %zu bytes of scratch, the static scratch "
                "holds %zu; call entmax_attn_decode with a workspace instead",
                need, (size_t)ENTMAX_DECODE_SCRATCH_BYTES);
  if ((size_t)o.b * o.hq == 0) return ENTMAX_OK;
  char* ws = nullptr;
  st = decode_scratch(&ws);
  if (st != ENTMAX_OK) return st;
  return entmax_attn_decode(desc, q, k_cache, v_cache, lengths, slopes, o_, tau, hist_counts, tau_h, ws, need,
                            stream);
}

size_t entmax_dash_fwd_workspace_bytes(const entmax_dash_desc* desc) {
  DashDerived o;
  if (derive_dash(desc, o) != ENTMAX_OK) return 0;
  return 2 * dash_kv_bytes(o);
}

size_t entmax_dash_mask_words(const entmax_dash_desc* desc) {
  DashDerived o;
  if (derive_dash(desc, o) != ENTMAX_OK) return 0;
  return (size_t)o.b * o.hkv * o.Tr * o.Wc;
}

entmax_status entmax_dash_fwd(const entmax_dash_desc* desc, const void* q, const void* k, const void* v,
                              const void* k_summary, float* o_, float* lse, float* route_tau, float* route_w,
                              uint32_t* chunk_mask, void* workspace, size_t workspace_bytes, void* stream) {
  DashDerived o;
  entmax_status st = derive_dash(desc, o);
  if (st != ENTMAX_OK) return st;
  if ((size_t)o.b * o.hq * o.n == 0) return ENTMAX_OK;
  if (!q || !k || !v || !k_summary || !o_ || !route_w || !chunk_mask)
    return fail(ENTMAX_ERR_NULL, "q, k, v, k_summary, o, route_w and chunk_mask are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_summary, 16) || !aligned(o_, 16) ||
      !aligned(route_w, 4) || !aligned(chunk_mask, 4) || (lse && !aligned(lse, 4)) ||
      (route_tau && !aligned(route_tau, 4)))
    return fail(ENTMAX_ERR_ALIGN, "q, k, v, k_summary, o need 16-byte alignment; the others 4-byte");
  const size_t need = 2 * dash_kv_bytes(o);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(ENTMAX_ERR_WORKSPACE, "DashAttention workspace: need %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  PrepBatch pb{};
  pb.job[0] = Relayout{k, wsb, nullptr, nullptr, nullptr, o.b * o.hkv, "k"};
  pb.job[1] = Relayout{v, nullptr, wsb + dash_kv_bytes(o), nullptr, nullptr, o.b * o.hkv, "v"};
  pb.njobs = 2;
  pb.n = o.n;
  hipError_t e = launch_prep(pb, o.dtype, o.D, "dash_prep", s);
  if (e != hipSuccess) return hip_fail(e, "fragment-major copies of K and V");
  DashParams p{};
  p.q = q; p.ks = k_summary; p.kf = wsb; p.vf = wsb + dash_kv_bytes(o);
  p.o = o_; p.lse = lse; p.rtau = route_tau; p.rw = route_w; p.cmask = chunk_mask;
  p.b = o.b; p.hq = o.hq; p.hkv = o.hkv; p.n = o.n; p.G = o.G; p.C = o.C; p.nc = o.nc; p.Tr = o.Tr; p.Wc = o.Wc;
  p.max_iters = o.max_iters;
  p.cx = (float)(((double)o.alpha - 1.0) * (double)o.gamma * (double)o.scale);
  p.alpha = o.alpha; p.kappa = o.kappa; p.tol = o.tol;
  p.c2 = (float)((double)o.scale * 1.4426950408889634);
  p.sigma = o.sigma;
  e = launch_dash(p, o.dtype, o.D, o.mode, s);
  if (e != hipSuccess) return hip_fail(e, "DashAttention kernels");
  return ENTMAX_OK;
}

// ------------------------------------------------------------------------ DashAttention backward
// Stage 2 runs through the attention backward (mode 3) as softmax attention over 32 x 64
// blocks; this is its descriptor, and the layout of the backward's workspace.
static entmax_status dash_attn_view(const DashDerived& o, Derived& a) {
  entmax_attn_desc ad{};
  ad.batch = o.b; ad.heads_q = o.hq; ad.heads_kv = o.hkv; ad.seqlen = o.n; ad.head_dim = o.D;
  ad.dtype = o.dtype; ad.alpha = 1.5f; ad.causal = 1; ad.block_q = 32; ad.block_k = 64; ad.n_bins = 16;
  ad.scale = o.scale;
  return derive(&ad, a);
}

// rows per piece of the summary-gradient product (k_dash_dks)
constexpr int DASH_DKS_ROWS = 256;

struct DashBwdLayout {
  BwdLayout att;        // the attention backward's part (at offset 0)
  size_t fine, bmask, lp, lse2, dw, qc, dq32, dbias, du, dpart, total;
  int W, NP;
};
static DashBwdLayout dash_bwd_ws(const DashDerived& o, const Derived& a) {
  DashBwdLayout L;
  L.att = bwd_ws(a);
  const size_t rows = (size_t)o.b * o.hq, units = (size_t)o.b * o.hkv;
  const int Tb = o.n / 64;
  L.W = (Tb + 31) / 32;
  L.NP = (o.n + DASH_DKS_ROWS - 1) / DASH_DKS_ROWS;
  size_t off = L.att.total;
  L.fine = off; off += align256(units * (o.n / 32) * o.Wc * 4);
  L.bmask = off; off += align256(rows * (o.n / 32) * L.W * 4);
  L.lp = off; off += align256(units * o.nc * o.n * 4);
  L.lse2 = off; off += align256(rows * o.n * 4);
  L.dw = off; off += align256(units * o.nc * o.n * 4);
  L.qc = off; off += align256(rows * o.n * o.D * o.es);
  L.dq32 = off; off += align256(rows * o.n * o.D * 4);
  L.dbias = off; off += align256(rows * (size_t)(o.n / 32) * o.n * 4);
  L.du = off; off += align256(rows * o.nc * o.n * 4);
  L.dpart = off; off += align256(units * o.Wc * L.NP * (size_t)o.D * 32 * 4);
  L.total = off;
  return L;
}

size_t entmax_dash_bwd_workspace_bytes(const entmax_dash_desc* desc) {
  DashDerived o;
  Derived a;
  if (derive_dash(desc, o) != ENTMAX_OK || dash_attn_view(o, a) != ENTMAX_OK) return 0;
  return dash_bwd_ws(o, a).total;
}

entmax_status entmax_dash_bwd(const entmax_dash_desc* desc, const void* q, const void* k, const void* v,
                              const void* k_summary, const float* o_, const float* lse, const float* route_tau,
                              const float* route_w, const uint32_t* chunk_mask, const void* dout, void* dq,
                              void* dk, void* dv, void* dk_summary, void* workspace, size_t workspace_bytes,
                              void* stream) {
  DashDerived o;
  entmax_status st = derive_dash(desc, o);
  if (st != ENTMAX_OK) return st;
  if ((size_t)o.b * o.hq * o.n == 0) return ENTMAX_OK;
  Derived a;
  if ((st = dash_attn_view(o, a)) != ENTMAX_OK) return st;
  if (!q || !k || !v || !k_summary || !o_ || !lse || !route_tau || !route_w || !chunk_mask || !dout || !dq ||
      !dk || !dv || !dk_summary)
    return fail(ENTMAX_ERR_NULL, "every argument of entmax_dash_bwd is required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_summary, 16) || !aligned(o_, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dk_summary, 16) ||
      !aligned(lse, 16) || !aligned(route_tau, 4) || !aligned(route_w, 16) || !aligned(chunk_mask, 4))
    return fail(ENTMAX_ERR_ALIGN, "tensors need 16-byte alignment (route_tau and chunk_mask 4-byte)");
  const DashBwdLayout L = dash_bwd_ws(o, a);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
    return fail(ENTMAX_ERR_WORKSPACE, "DashAttention backward workspace: need %zu bytes, 256-byte aligned (got %zu)",
                L.total, workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  DashParams dp{};
  dp.q = q; dp.ks = k_summary; dp.rtau = const_cast<float*>(route_tau); dp.rw = const_cast<float*>(route_w);
  dp.cmask = const_cast<uint32_t*>(chunk_mask);
  dp.b = o.b; dp.hq = o.hq; dp.hkv = o.hkv; dp.n = o.n; dp.G = o.G; dp.C = o.C; dp.nc = o.nc; dp.Tr = o.Tr;
  dp.Wc = o.Wc; dp.max_iters = o.max_iters;
  dp.cx = (float)(((double)o.alpha - 1.0) * (double)o.gamma * (double)o.scale);
  dp.alpha = o.alpha; dp.kappa = o.kappa; dp.tol = o.tol; dp.sigma = o.sigma;
  dp.dbias = (const float*)(ws + L.dbias); dp.dq32 = (const float*)(ws + L.dq32); dp.dq = dq;
  dp.lp = (float*)(ws + L.lp); dp.dw = (float*)(ws + L.dw); dp.du = (float*)(ws + L.du);
  dp.lse_in = lse; dp.lse2 = (float*)(ws + L.lse2);
  dp.qc = ws + L.qc; dp.dpart = (float*)(ws + L.dpart); dp.NP = L.NP; dp.PR = DASH_DKS_ROWS;
  dp.dks = dk_summary; dp.fine = (uint32_t*)(ws + L.fine); dp.bmask = (uint32_t*)(ws + L.bmask); dp.W = L.W;
  dp.gs = (float)((double)o.gamma * (double)o.scale);
  hipError_t e = launch_dash_bwd_setup(dp, s);
  if (e != hipSuccess) return hip_fail(e, "DashAttention block mask and prior");

  // stage 2: the attention backward in mode 3 (delta = dO . o)
  const int hq_all = o.b * o.hq, hkv_all = o.b * o.hkv;
  const BwdLayout& B = L.att;
  PrepBatch pb{};
  pb.job[0] = Relayout{dout, ws + B.dor, nullptr, o_, (float*)(ws + B.delta), hq_all, "do"};
  pb.job[1] = Relayout{q, ws + B.qr, ws + L.qc, nullptr, nullptr, hq_all, "q"};
  pb.job[2] = Relayout{k, ws + B.kr, nullptr, nullptr, nullptr, hkv_all, "k"};
  pb.job[3] = Relayout{v, ws + B.vr, nullptr, nullptr, nullptr, hkv_all, "v"};
  pb.njobs = 4;
  pb.n = o.n;
  pb.mask = dp.bmask;
  pb.maskT = (uint32_t*)(ws + B.maskT);
  pb.planes = hq_all; pb.Tr = a.Tr; pb.Tc = a.Tc; pb.W = a.W; pb.WT = a.WT;
  e = launch_prep(pb, o.dtype, o.D, "dash_bwd_prep", s);
  if (e != hipSuccess) return hip_fail(e, "DashAttention backward preparation");
  BwdParams p{};
  p.qr = ws + B.qr; p.dor = ws + B.dor; p.kr = ws + B.kr; p.vr = ws + B.vr;
  p.tau = dp.lse2; p.delta = (const float*)(ws + B.delta);
  p.mask = dp.bmask; p.maskT = (const uint32_t*)(ws + B.maskT);
  p.dq = nullptr; p.dk = dk; p.dv = dv;
  p.b = o.b; p.hq = o.hq; p.hkv = o.hkv; p.n = o.n; p.G = o.G;
  p.causal = 1; p.Br = a.Br; p.Bc = a.Bc;
  p.cx = (float)((double)o.scale * 1.4426950408889634); p.scale = o.scale; p.kappa = 1.0f; p.am1 = 0.0f;
  p.slopes = nullptr;
  p.Tr = a.Tr; p.Tc = a.Tc; p.W = a.W; p.WT = a.WT;
  p.dense = 0;
  p.lp = dp.lp; p.C = o.C;
  p.dq32 = (float*)(ws + L.dq32); p.dbias = (float*)(ws + L.dbias);
  p.map = make_map(o.b * o.hkv, a.Tc);
  prof_begin("dash_bwd_dkv", s);
  e = launch_bwd_dkv(p, o.dtype, o.D, MODE_DASH, s);
  prof_end(s);
  if (e != hipSuccess) return hip_fail(e, "DashAttention dK/dV kernel");
  p.map = make_map(o.b * o.hkv, o.G * a.Tr);
  prof_begin("dash_bwd_dq", s);
  e = launch_bwd_dq(p, o.dtype, o.D, MODE_DASH, s);
  prof_end(s);
  if (e != hipSuccess) return hip_fail(e, "DashAttention dQ kernel");

  // stage 1: the routing's share of dQ and the summaries' gradient
  e = launch_dash_route_bwd(dp, o.dtype, o.D, o.mode, s);
  if (e != hipSuccess) return hip_fail(e, "DashAttention routing backward");
  return ENTMAX_OK;
}

const char* entmax_status_string(entmax_status s) {
  switch (s) {
    case ENTMAX_OK: return "ok";
    case ENTMAX_ERR_NULL: return "null pointer";
    case ENTMAX_ERR_SHAPE: return "invalid shape";
    case ENTMAX_ERR_ALPHA: return "invalid alpha";
    case ENTMAX_ERR_UNSUPPORTED: return "unsupported configuration";
    case ENTMAX_ERR_ALIGN: return "misaligned pointer";
    case ENTMAX_ERR_WORKSPACE: return "workspace missing or too small";
    case ENTMAX_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* entmax_last_error(void) { return t_err; }

entmax_status entmax_attn_profile(int enable) {
  g_on = enable != 0;
  return ENTMAX_OK;
}

entmax_status entmax_attn_profile_read(entmax_kernel_time* out, int max_entries, int* n_entries) {
  std::vector<Pending> pend;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    pend.swap(g_pending);
  }
  std::map<std::string, std::pair<double, int64_t>> acc;
  std::vector<std::string> order;
  entmax_status st = ENTMAX_OK;
  for (auto& r : pend) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) st = hip_fail(e, "profile event");
    if (!acc.count(r.name)) order.push_back(r.name);
    acc[r.name].first += ms;
    acc[r.name].second += 1;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& r : pend) {
      g_pool.push_back(r.a);
      g_pool.push_back(r.b);
    }
  }
  int cnt = 0;
  for (auto& name : order) {
    if (out && cnt < max_entries) {
      memset(out[cnt].name, 0, sizeof(out[cnt].name));
      strncpy(out[cnt].name, name.c_str(), sizeof(out[cnt].name) - 1);
      out[cnt].total_ms = acc[name].first;
      out[cnt].launches = acc[name].second;
    }
    ++cnt;
  }
  if (n_entries) *n_entries = cnt;
  return st;
}

}  // extern "C"

"""alpha-entmax attention (AdaSplash-2 method) on AMD MI355X -- Python binding.

Thin ctypes layer over ``libentmax_attn.so`` (C ABI in ``include/entmax_attn.h`` and
``include/dash_attn.h``):
it checks tensor placement, allocates outputs and workspace with PyTorch and passes
raw device pointers and the current HIP stream. Every step of the computation runs
in the library's HIP kernels; there is no fallback path -- if the library is not
built, every call raises.

    o, tau, mask, aux = fwd(q, k, v, alpha=1.5, causal=True, block=(64, 64), bins=16)
    dq, dk, dv = bwd(q, k, v, do, tau, mask, aux, alpha=1.5, causal=True, block=(64, 64), bins=16)
    o = entmax_attention(q, k, v, alpha=1.5)          # autograd-aware
    o, tau, hist, tau_h = decode(q_new, k_cache, v_cache, alpha=1.5, lengths=lens)
    o, lse, route_tau, route_w, chunk_mask = dash_fwd(q, k, v, k_summary, chunk=64)
    dq, dk, dv, dk_summary = dash_bwd(q, k, v, k_summary, do, o, lse, route_tau, route_w, chunk_mask, chunk=64)

Shapes: q, do [b, hq, n, d]; k, v [b, hkv, n, d]; dtype float32 or bfloat16.
``slopes`` (optional, float32 [hq] on the device): per-head position-bias slopes; head h
adds -slopes[h] |i - j| to its scores (``nape_slopes`` gives the NAPE heads).
"""
from __future__ import annotations

import ctypes
import os
from collections import namedtuple
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libentmax_attn.so")

ENTMAX_F32, ENTMAX_BF16 = 0, 1
STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape", 3: "invalid alpha", 4: "unsupported",
          5: "misaligned pointer", 6: "workspace", 7: "HIP runtime error"}


class EntmaxError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"entmax_attn: {STATUS.get(status, status)}: {detail}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("seqlen", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("causal", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("n_bins", ctypes.c_int32), ("scale", ctypes.c_float),
        ("max_iters", ctypes.c_int32), ("tol", ctypes.c_float), ("tau_init", ctypes.c_int32),
        ("dense", ctypes.c_int32),
    ]


class DashDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("seqlen", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("route_alpha", ctypes.c_float), ("gamma", ctypes.c_float),
        ("sigma", ctypes.c_float), ("scale", ctypes.c_float), ("max_iters", ctypes.c_int32),
        ("tol", ctypes.c_float),
    ]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("total_ms", ctypes.c_double), ("launches", ctypes.c_int64)]


_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_DP = ctypes.POINTER(Desc)
_DDP = ctypes.POINTER(DashDesc)

EXPORTS = [
    "entmax_attn_fwd_workspace_bytes", "entmax_attn_bwd_workspace_bytes", "entmax_attn_aux_bytes",
    "entmax_attn_mask_words", "entmax_attn_fwd", "entmax_attn_bwd", "entmax_attn_decode_workspace_bytes",
    "entmax_attn_decode", "entmax_attn_decode_noalloc", "entmax_dash_fwd_workspace_bytes", "entmax_dash_mask_words", "entmax_dash_fwd",
    "entmax_dash_bwd_workspace_bytes", "entmax_dash_bwd", "entmax_status_string",
    "entmax_last_error", "entmax_attn_profile", "entmax_attn_profile_read",
]


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_entmax_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for f in ("entmax_attn_fwd_workspace_bytes", "entmax_attn_bwd_workspace_bytes",
                  "entmax_attn_aux_bytes", "entmax_attn_mask_words"):
            getattr(L, f).restype = _sz
            getattr(L, f).argtypes = [_DP]
        L.entmax_attn_fwd.restype = ctypes.c_int
        L.entmax_attn_fwd.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.entmax_attn_bwd.restype = ctypes.c_int
        L.entmax_attn_bwd.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.entmax_attn_decode_workspace_bytes.restype = _sz
        L.entmax_attn_decode_workspace_bytes.argtypes = [_DP]
        L.entmax_attn_decode.restype = ctypes.c_int
        L.entmax_attn_decode.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.entmax_attn_decode_noalloc.restype = ctypes.c_int
        L.entmax_attn_decode_noalloc.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        for f in ("entmax_dash_fwd_workspace_bytes", "entmax_dash_mask_words", "entmax_dash_bwd_workspace_bytes"):
            getattr(L, f).restype = _sz
            getattr(L, f).argtypes = [_DDP]
        L.entmax_dash_fwd.restype = ctypes.c_int
        L.entmax_dash_fwd.argtypes = [_DDP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.entmax_dash_bwd.restype = ctypes.c_int
        L.entmax_dash_bwd.argtypes = [_DDP] + [_vp] * 15 + [_sz, _vp]
        L.entmax_status_string.restype = ctypes.c_char_p
        L.entmax_status_string.argtypes = [ctypes.c_int]
        L.entmax_last_error.restype = ctypes.c_char_p
        L.entmax_last_error.argtypes = []
        L.entmax_attn_profile.restype = ctypes.c_int
        L.entmax_attn_profile.argtypes = [ctypes.c_int]
        L.entmax_attn_profile_read.restype = ctypes.c_int
        L.entmax_attn_profile_read.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int)]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise EntmaxError(status, lib().entmax_last_error().decode())


def make_desc(batch: int, heads_q: int, heads_kv: int, seqlen: int, head_dim: int, dtype: int,
              alpha: float, causal: bool, block: Tuple[int, int], bins: int,
              scale: Optional[float] = None, max_iters: int = 0, tol: float = 0.0,
              tau_init: int = 0, dense: bool = False) -> Desc:
    return Desc(batch, heads_q, heads_kv, seqlen, head_dim, dtype, float(alpha), int(bool(causal)),
                int(block[0]), int(block[1]), int(bins), float(scale or 0.0), int(max_iters), float(tol),
                int(tau_init), int(bool(dense)))


def _torch():
    import torch
    return torch


def _desc_for(q, k, alpha, causal, block, bins, scale, max_iters, tol, tau_init: int = 0,
              dense: bool = False) -> Desc:
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, seqlen, head_dim]")
    if q.dtype == torch.bfloat16:
        dt = ENTMAX_BF16
    elif q.dtype == torch.float32:
        dt = ENTMAX_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    b, hq, n, d = q.shape
    return make_desc(b, hq, k.shape[1], n, d, dt, alpha, causal, block, bins, scale, max_iters, tol,
                     tau_init, dense)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev) -> int:
    torch = _torch()
    return torch.cuda.current_stream(dev).cuda_stream


def _check_slopes(slopes, hq: int) -> None:
    if slopes is None:
        return
    torch = _torch()
    if slopes.dtype != torch.float32 or slopes.numel() != hq:
        raise ValueError(f"slopes must be float32 with one value per query head ({hq})")


def _require_gpu(*ts) -> None:
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("entmax_attn runs on the GPU only: tensors must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(name: str, t, shape, dtype, device) -> None:
    """Raise ValueError unless tensor ``t`` has exactly ``shape``, ``dtype`` and ``device``
    (the C ABI takes raw pointers, so a wrong size here would be read or written out of
    bounds on the device)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the device of q)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_qkv(q, k, v) -> None:
    """q [b, hq, n, d]; k and v [b, hkv, n, d] with hq % hkv == 0, one dtype and device."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k and v must be [batch, heads, seqlen, head_dim]")
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if hkv == 0 or hq % hkv != 0:
        raise ValueError(f"heads of q ({hq}) must be a multiple of the heads of k ({hkv})")
    _expect("k", k, (b, hkv, n, d), q.dtype, q.device)
    _expect("v", v, (b, hkv, n, d), q.dtype, q.device)


def _check_workspace(ws, device) -> None:
    torch = _torch()
    if ws is not None and (ws.dtype != torch.uint8 or ws.dim() != 1 or ws.device != device):
        raise ValueError("workspace must be a 1-D uint8 tensor on the device of q")


def _check_stats(stats, device) -> None:
    torch = _torch()
    if stats is not None and (stats.dtype != torch.int64 or stats.dim() != 1 or stats.numel() < 32
                              or stats.device != device):
        raise ValueError("stats must be a 1-D int64 tensor of at least 32 entries on the device of q")


def mask_shape(n: int, block: Tuple[int, int]) -> Tuple[int, int]:
    Tr, Tc = n // block[0], n // block[1]
    return Tr, (Tc + 31) // 32


FwdOut = namedtuple("FwdOut", "o tau mask aux hist tau_h")


def nape_slopes(heads: int):
    """Slopes of NAPE heads as a list: the first half of the heads without position encoding
    (slope 0), the second half ALiBi with the geometric slopes 2^(-8 k / H') of H' = heads/2
    ALiBi heads, k = 1..H'. The pages name the split (half and half, AdaSplash-2 (it) §4) but not
    which half or the slopes; this is the reading taken."""
    if heads < 2 or heads % 2:
        raise ValueError("NAPE needs an even number of heads")
    hp = heads // 2
    return [0.0] * hp + [2.0 ** (-8.0 * kk / hp) for kk in range(1, hp + 1)]


def fwd(q, k, v, alpha: float = 1.5, causal: bool = True, block=(64, 64), bins: int = 16,
        scale: Optional[float] = None, max_iters: int = 0, tol: float = 0.0,
        return_hist: bool = False, stats=None, workspace=None, out=None, tau_init: int = 0,
        slopes=None, dense: bool = False) -> FwdOut:
    """alpha-entmax attention forward. Returns (o, tau, mask, aux, hist, tau_h); o is float32.

    hist/tau_h are the histogram stage's counts [b,hq,n,B] and lower bound [b,hq,n]
    (None unless return_hist). ``stats``: optional int64 CUDA tensor [32] (accumulated).
    ``out``: optional FwdOut of preallocated tensors to write into. ``tau_init``: 0 starts
    the refinement from the histogram bound, 1 from the plain bracket below the row max.
    ``dense``: visit every causally valid key block (no block skipping; the mask comes back
    with every valid bit set) -- the ablation that times the method without sparsity.
    Every tensor is checked for shape, dtype and device before a pointer is taken.
    """
    torch = _torch()
    _check_qkv(q, k, v)
    _check_slopes(slopes, q.shape[1])
    desc = _desc_for(q, k, alpha, causal, block, bins, scale, max_iters, tol, tau_init, dense)
    b, hq, n, d = q.shape
    dev = q.device
    Tr, W = mask_shape(n, block)
    f32, i32 = torch.float32, torch.int32
    if out is not None:
        o, tau, mask, aux, hist, tau_h = out
        _expect("out.o", o, (b, hq, n, d), f32, dev)
        _expect("out.tau", tau, (b, hq, n), f32, dev)
        _expect("out.mask", mask, (b, hq, Tr, W), i32, dev)
        _expect("out.aux", aux, (b, hq, n, d), f32, dev)
        _expect("out.hist", hist, (b, hq, n, bins), i32, dev)
        _expect("out.tau_h", tau_h, (b, hq, n), f32, dev)
        if any(x is None for x in (o, tau, mask, aux)):
            raise ValueError("out needs o, tau, mask and aux")
    _check_stats(stats, dev)
    _check_workspace(workspace, dev)
    _require_gpu(q, k, v, slopes)
    L = lib()
    if out is None:
        o = torch.empty(q.shape, dtype=f32, device=dev)
        tau = torch.empty((b, hq, n), dtype=f32, device=dev)
        mask = torch.empty((b, hq, Tr, W), dtype=i32, device=dev)
        aux = torch.empty((b, hq, n, d), dtype=f32, device=dev)
        hist = torch.empty((b, hq, n, bins), dtype=i32, device=dev) if return_hist else None
        tau_h = torch.empty((b, hq, n), dtype=f32, device=dev) if return_hist else None
    nbytes = L.entmax_attn_fwd_workspace_bytes(ctypes.byref(desc))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(L.entmax_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(slopes), _ptr(o), _ptr(tau),
                             _ptr(mask), _ptr(aux), _ptr(hist), _ptr(tau_h), _ptr(stats),
                             _ptr(workspace), workspace.numel(), _stream(dev)))
    return FwdOut(o, tau, mask, aux, hist, tau_h)


def bwd(q, k, v, do, tau, mask, aux, alpha: float = 1.5, causal: bool = True, block=(64, 64),
        bins: int = 16, scale: Optional[float] = None, workspace=None, out=None, slopes=None,
        dense: bool = False):
    """alpha-entmax attention backward: (dq, dk, dv) given the forward's tau, mask, aux
    (and the forward's slopes). ``dense``: no block skipping (pass the mask of a dense
    forward). Every tensor is checked for shape, dtype and device before a pointer is taken."""
    torch = _torch()
    _check_qkv(q, k, v)
    _check_slopes(slopes, q.shape[1])
    desc = _desc_for(q, k, alpha, causal, block, bins, scale, 0, 0.0, 0, dense)
    b, hq, n, d = q.shape
    dev = q.device
    Tr, W = mask_shape(n, block)
    f32 = torch.float32
    _expect("do", do, q.shape, q.dtype, dev)
    _expect("tau", tau, (b, hq, n), f32, dev)
    _expect("mask", mask, (b, hq, Tr, W), torch.int32, dev)
    _expect("aux", aux, (b, hq, n, d), f32, dev)
    if out is not None:
        dq, dk, dv = out
        _expect("out.dq", dq, q.shape, q.dtype, dev)
        _expect("out.dk", dk, k.shape, k.dtype, dev)
        _expect("out.dv", dv, v.shape, v.dtype, dev)
        if any(x is None for x in (dq, dk, dv)):
            raise ValueError("out needs dq, dk and dv")
    _check_workspace(workspace, dev)
    _require_gpu(q, k, v, do, tau, mask, aux, slopes)
    L = lib()
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = L.entmax_attn_bwd_workspace_bytes(ctypes.byref(desc))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(L.entmax_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(slopes), _ptr(tau),
                             _ptr(mask), _ptr(aux), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                             workspace.numel(), _stream(dev)))
    return dq, dk, dv


DecodeOut = namedtuple("DecodeOut", "o tau hist tau_h")


def decode(q, k_cache, v_cache, alpha: float = 1.5, bins: int = 16, scale: Optional[float] = None,
           lengths=None, slopes=None, max_iters: int = 0, tol: float = 0.0, tau_init: int = 0,
           return_hist: bool = False, workspace=None) -> DecodeOut:
    """One decode step: q [b, hq, d] against the caches k_cache, v_cache [b, hkv, n_ctx, d].

    ``lengths``: optional int32 [b] device tensor of valid cache lengths (default n_ctx).
    Returns o [b, hq, d] (float32), tau [b, hq] and, with ``return_hist``, the histogram
    counts [b, hq, bins] and tau_h [b, hq]. Equals the last row of a causal forward.
    """
    torch = _torch()
    _require_gpu(q, k_cache, v_cache, lengths, slopes)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [b, hq, d] and the caches [b, hkv, n_ctx, d]")
    b, hq, d = q.shape
    if k_cache.shape[0] != b or k_cache.shape[3] != d or q.dtype != k_cache.dtype:
        raise ValueError("q and the caches disagree in batch, head_dim or dtype")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() != b):
        raise ValueError("lengths must be int32 with one value per sequence")
    _check_slopes(slopes, hq)
    dt = ENTMAX_BF16 if q.dtype == torch.bfloat16 else ENTMAX_F32
    desc = make_desc(b, hq, k_cache.shape[1], k_cache.shape[2], d, dt, alpha, True, (32, 32), bins,
                     scale, max_iters, tol, tau_init)
    L = lib()
    dev = q.device
    o = torch.empty((b, hq, d), dtype=torch.float32, device=dev)
    tau = torch.empty((b, hq), dtype=torch.float32, device=dev)
    hist = torch.empty((b, hq, bins), dtype=torch.int32, device=dev) if return_hist else None
    tau_h = torch.empty((b, hq), dtype=torch.float32, device=dev) if return_hist else None
    nbytes = L.entmax_attn_decode_workspace_bytes(ctypes.byref(desc))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(L.entmax_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths),
                                _ptr(slopes), _ptr(o), _ptr(tau), _ptr(hist), _ptr(tau_h), _ptr(workspace),
                                workspace.numel(), _stream(dev)))
    return DecodeOut(o, tau, hist, tau_h)


# bytes of the static scratch behind decode_noalloc (ENTMAX_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 32 << 20


def decode_noalloc(q, k_cache, v_cache, alpha: float = 1.5, bins: int = 16, scale: Optional[float] = None,
                   lengths=None, slopes=None, max_iters: int = 0, tol: float = 0.0, tau_init: int = 0,
                   out=None) -> DecodeOut:
    """``decode`` through the library's allocation-free entry point (entmax_attn_decode_noalloc):
    the library takes its scratch from a static per-device buffer of DECODE_SCRATCH_BYTES
    instead of a workspace. ``out``: optional DecodeOut of preallocated o [b, hq, d] float32,
    tau [b, hq] float32 and (both or neither) hist [b, hq, bins] int32 and tau_h [b, hq]; with
    it this call allocates nothing. Calls that overlap on one device share the scratch."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [b, hq, d] and the caches [b, hkv, n_ctx, d]")
    b, hq, d = q.shape
    if k_cache.shape[0] != b or k_cache.shape[3] != d or q.dtype != k_cache.dtype:
        raise ValueError("q and the caches disagree in batch, head_dim or dtype")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() != b):
        raise ValueError("lengths must be int32 with one value per sequence")
    _check_slopes(slopes, hq)
    dev = q.device
    if out is not None:
        o, tau, hist, tau_h = out
        _expect("out.o", o, (b, hq, d), torch.float32, dev)
        _expect("out.tau", tau, (b, hq), torch.float32, dev)
        _expect("out.hist", hist, (b, hq, bins), torch.int32, dev)
        _expect("out.tau_h", tau_h, (b, hq), torch.float32, dev)
        if o is None or tau is None:
            raise ValueError("out needs o and tau")
    _require_gpu(q, k_cache, v_cache, lengths, slopes)
    dt = ENTMAX_BF16 if q.dtype == torch.bfloat16 else ENTMAX_F32
    desc = make_desc(b, hq, k_cache.shape[1], k_cache.shape[2], d, dt, alpha, True, (32, 32), bins,
                     scale, max_iters, tol, tau_init)
    if out is None:
        o = torch.empty((b, hq, d), dtype=torch.float32, device=dev)
        tau = torch.empty((b, hq), dtype=torch.float32, device=dev)
        hist, tau_h = None, None
    _check(lib().entmax_attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(lengths), _ptr(slopes), _ptr(o), _ptr(tau), _ptr(hist),
                                            _ptr(tau_h), _stream(dev)))
    return DecodeOut(o, tau, hist, tau_h)


DashOut = namedtuple("DashOut", "o lse route_tau route_w chunk_mask")


def make_dash_desc(batch: int, heads_q: int, heads_kv: int, seqlen: int, head_dim: int, dtype: int,
                   chunk: int, route_alpha: float, gamma: float = 1.0, sigma: float = 1.0,
                   scale: Optional[float] = None, max_iters: int = 0, tol: float = 0.0) -> DashDesc:
    return DashDesc(batch, heads_q, heads_kv, seqlen, head_dim, dtype, int(chunk), float(route_alpha),
                    float(gamma), float(sigma), float(scale or 0.0), int(max_iters), float(tol))


def dash_fwd(q, k, v, k_summary, chunk: int = 64, route_alpha: float = 1.5, gamma: float = 1.0,
             sigma: float = 1.0, scale: Optional[float] = None, max_iters: int = 0, tol: float = 0.0,
             workspace=None) -> DashOut:
    """DashAttention forward, stages 1-2 (include/dash_attn.h): alpha-entmax routing of each
    query over the chunk summaries k_summary [b, hkv, n / chunk, d] (averaged over the query
    heads of a KV group), then softmax over the routed chunks plus the query's own chunk with
    sigma * ln(routing weight) added to the scores. Returns o [b, hq, n, d] (float32), lse and
    route_tau [b, hq, n], route_w [b, hkv, n / chunk, n] (chunk-major group weights) and
    chunk_mask [b, hkv, n / 64, ceil(n_chunks / 32)] (int32 view of the uint32 words)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k_summary.dim() != 4:
        raise ValueError("q [b, hq, n, d], k and v [b, hkv, n, d], k_summary [b, hkv, n_chunks, d]")
    b, hq, n, d = q.shape
    if (k.shape[0] != b or k.shape[2] != n or k.shape[3] != d or k_summary.shape[:2] != k.shape[:2]
            or k_summary.shape[3] != d or len({q.dtype, k.dtype, v.dtype, k_summary.dtype}) != 1):
        raise ValueError("q, k, v and k_summary disagree in batch, heads, length, head_dim or dtype")
    if chunk <= 0 or n % chunk or k_summary.shape[2] != n // chunk:
        raise ValueError(f"k_summary needs seqlen / chunk = {n // max(chunk, 1)} rows")
    _require_gpu(q, k, v, k_summary)
    dt = ENTMAX_BF16 if q.dtype == torch.bfloat16 else ENTMAX_F32
    desc = make_dash_desc(b, hq, k.shape[1], n, d, dt, chunk, route_alpha, gamma, sigma, scale, max_iters, tol)
    L = lib()
    dev = q.device
    nc = n // chunk
    o = torch.empty((b, hq, n, d), dtype=torch.float32, device=dev)
    lse = torch.empty((b, hq, n), dtype=torch.float32, device=dev)
    rtau = torch.empty((b, hq, n), dtype=torch.float32, device=dev)
    rw = torch.empty((b, k.shape[1], nc, n), dtype=torch.float32, device=dev)
    cmask = torch.empty((b, k.shape[1], max(n // 64, 0), (nc + 31) // 32), dtype=torch.int32, device=dev)
    nbytes = L.entmax_dash_fwd_workspace_bytes(ctypes.byref(desc))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(L.entmax_dash_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_summary), _ptr(o), _ptr(lse),
                             _ptr(rtau), _ptr(rw), _ptr(cmask), _ptr(workspace), workspace.numel(), _stream(dev)))
    return DashOut(o, lse, rtau, rw, cmask)


DashGrads = namedtuple("DashGrads", "dq dk dv dk_summary")


def dash_bwd(q, k, v, k_summary, do, o, lse, route_tau, route_w, chunk_mask, chunk: int = 64,
             route_alpha: float = 1.5, gamma: float = 1.0, sigma: float = 1.0, scale: Optional[float] = None,
             max_iters: int = 0, tol: float = 0.0, workspace=None) -> DashGrads:
    """DashAttention backward, stages 1-2 (include/dash_attn.h): given do = dL/do and the
    forward's outputs (same settings), returns dq, dk, dv and dk_summary in the inputs' dtype.
    The gradient reaches q and k_summary through the routing (the alpha-entmax Jacobian) as
    well as through the prior term sigma * ln(routing weight) of stage 2."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q [b, hq, n, d] and k [b, hkv, n, d]")
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if chunk <= 0 or n % chunk:
        raise ValueError("seqlen must be a multiple of chunk")
    nc = n // chunk
    _expect("k", k, (b, hkv, n, d), q.dtype, q.device)
    _expect("v", v, (b, hkv, n, d), q.dtype, q.device)
    _expect("k_summary", k_summary, (b, hkv, nc, d), q.dtype, q.device)
    _expect("do", do, (b, hq, n, d), q.dtype, q.device)
    _expect("o", o, (b, hq, n, d), torch.float32, q.device)
    _expect("lse", lse, (b, hq, n), torch.float32, q.device)
    _expect("route_tau", route_tau, (b, hq, n), torch.float32, q.device)
    _expect("route_w", route_w, (b, hkv, nc, n), torch.float32, q.device)
    _expect("chunk_mask", chunk_mask, (b, hkv, n // 64, (nc + 31) // 32), torch.int32, q.device)
    _require_gpu(q, k, v, k_summary, do, o, lse, route_tau, route_w, chunk_mask)
    dt = ENTMAX_BF16 if q.dtype == torch.bfloat16 else ENTMAX_F32
    desc = make_dash_desc(b, hq, hkv, n, d, dt, chunk, route_alpha, gamma, sigma, scale, max_iters, tol)
    L = lib()
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dks = torch.empty_like(k_summary)
    nbytes = L.entmax_dash_bwd_workspace_bytes(ctypes.byref(desc))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(L.entmax_dash_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_summary), _ptr(o), _ptr(lse),
                             _ptr(route_tau), _ptr(route_w), _ptr(chunk_mask), _ptr(do), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dks), _ptr(workspace), workspace.numel(), _stream(dev)))
    return DashGrads(dq, dk, dv, dks)


def workspace_bytes(desc: Desc) -> Tuple[int, int]:
    L = lib()
    return (L.entmax_attn_fwd_workspace_bytes(ctypes.byref(desc)),
            L.entmax_attn_bwd_workspace_bytes(ctypes.byref(desc)))


def profile(enable: bool) -> None:
    """Record hipEvents around every kernel launch of the library (see profile_read)."""
    _check(lib().entmax_attn_profile(int(bool(enable))))


def profile_read() -> dict:
    """Per-kernel {name: (total_ms, launches)} since the last read (waits for the events)."""
    arr = (KernelTime * 64)()
    cnt = ctypes.c_int(0)
    _check(lib().entmax_attn_profile_read(arr, 64, ctypes.byref(cnt)))
    return {arr[i].name.decode(): (arr[i].total_ms, int(arr[i].launches)) for i in range(min(cnt.value, 64))}


def _make_function():
    torch = _torch()

    class EntmaxAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, alpha, causal, block, bins, scale, slopes):
            r = fwd(q, k, v, alpha, causal, block, bins, scale, slopes=slopes)
            ctx.save_for_backward(q, k, v, r.tau, r.mask, r.aux)
            ctx.cfg = (alpha, causal, block, bins, scale, slopes)
            return r.o.to(q.dtype)

        @staticmethod
        def backward(ctx, do):
            q, k, v, tau, mask, aux = ctx.saved_tensors
            alpha, causal, block, bins, scale, slopes = ctx.cfg
            dq, dk, dv = bwd(q, k, v, do.contiguous(), tau, mask, aux, alpha, causal, block, bins, scale,
                             slopes=slopes)
            return dq, dk, dv, None, None, None, None, None, None

    return EntmaxAttentionFn


_fn = None


def entmax_attention(q, k, v, alpha: float = 1.5, causal: bool = True, block=(64, 64), bins: int = 16,
                     scale: Optional[float] = None, slopes=None):
    """Differentiable alpha-entmax attention (forward and backward in the HIP library)."""
    global _fn
    if _fn is None:
        _fn = _make_function()
    return _fn.apply(q, k, v, alpha, causal, tuple(block), bins, scale, slopes)

"""fp64 CPU oracle of alpha-entmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does. The arithmetic lives in
``entmax_oracle.c`` (plain C, double precision, one row or one key at a time);
this module only loads it, splits independent rows (or keys) over host threads
and assembles block masks from per-row bits.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms (sorted sparsemax, exact 1.5-entmax), brute-force
support enumeration, Proposition 1, the softmax limit, finite differences and
exact invariants. No function is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "entmax_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)
_up = ctypes.POINTER(ctypes.c_uint32)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_entmax_tau.restype = ctypes.c_double
        lib.oracle_entmax_tau.argtypes = [_dp, ctypes.c_long, ctypes.c_double]
        lib.oracle_histogram.restype = None
        lib.oracle_histogram.argtypes = [_dp, ctypes.c_long, ctypes.c_int, _ip, _lp]
        lib.oracle_tau_from_hist.restype = ctypes.c_double
        lib.oracle_tau_from_hist.argtypes = [_ip, ctypes.c_int64, ctypes.c_int, ctypes.c_double]
        lib.oracle_attn_fwd_rows.restype = None
        lib.oracle_attn_fwd_rows.argtypes = [
            ctypes.c_long, ctypes.c_long, _dp, _dp, _dp, ctypes.c_double, ctypes.c_double,
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_long,
            _dp, _dp, _dp, _ip, _lp, _up, _dp, _dp]
        lib.oracle_attn_bwd_rows.restype = None
        lib.oracle_attn_bwd_rows.argtypes = [
            ctypes.c_long, ctypes.c_long, _dp, _dp, _dp, _dp, _dp, ctypes.c_double,
            ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_long, ctypes.c_long, _dp, _dp]
        lib.oracle_attn_bwd_keys.restype = None
        lib.oracle_attn_bwd_keys.argtypes = [
            ctypes.c_long, ctypes.c_long, ctypes.c_long, _dp, _dp, _dp, _dp, _dp, _dp,
            ctypes.c_double, ctypes.c_double, _dp, ctypes.c_int, ctypes.c_long, ctypes.c_long,
            _dp, _dp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunks(lo: int, hi: int, parts: int):
    parts = max(1, min(parts, hi - lo))
    edges = np.linspace(lo, hi, parts + 1).astype(np.int64)
    return [(int(edges[t]), int(edges[t + 1])) for t in range(parts) if edges[t + 1] > edges[t]]


# ---------------------------------------------------------------------------------------------
# row-level primitives
# ---------------------------------------------------------------------------------------------

def entmax_tau(x, alpha: float) -> float:
    """tau* of one row of x-scale scores (x = (alpha-1) * scores), by bisection."""
    x = _f64(x).ravel()
    return float(_load().oracle_entmax_tau(_ptr(x, _dp), x.size, float(alpha)))


def entmax(z, alpha: float):
    """alpha-entmax of one score vector z: returns (p, tau) with tau on the x-scale."""
    x = (alpha - 1.0) * _f64(z).ravel()
    t = entmax_tau(x, alpha)
    d = np.maximum(x - t, 0.0)
    return np.where(d > 0, d ** (1.0 / (alpha - 1.0)), 0.0), t


def histogram(x, B: int):
    """Anchored-grid histogram of one row of x-scale scores: (counts[B], T)."""
    x = _f64(x).ravel()
    c = np.zeros(B, dtype=np.int32)
    T = np.zeros(1, dtype=np.int64)
    _load().oracle_histogram(_ptr(x, _dp), x.size, int(B), _ptr(c, _ip), _ptr(T, _lp))
    return c, int(T[0])


def tau_from_hist(counts, T: int, B: int, alpha: float) -> float:
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    return float(_load().oracle_tau_from_hist(_ptr(c, _ip), int(T), int(B), float(alpha)))


# ---------------------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------------------

def attn_fwd_head(q, k, v, alpha: float, causal: bool, B: int, Bc: int, scale: float,
                  rows=None, threads: int | None = None, slope: float = 0.0) -> dict:
    """Dense forward of one query head. q: [n, d]; k, v: [n, d] of its KV head.

    ``rows``: None for all rows, or an iterable of row indices (sampled rows).
    ``slope``: the head's position-bias slope m (scores get -m |i - j|; 0 = none).
    Returns per requested row: o [r, d], tau, tau_h, counts [r, B], T, rowbits [r, W],
    xgap, psum, and ``rows`` (the row indices).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    W = (n + 32 * Bc - 1) // (32 * Bc)
    if rows is None:
        rows_arr = np.arange(n, dtype=np.int64)
    else:
        rows_arr = np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    m = rows_arr.size
    out = {
        "rows": rows_arr,
        "o": np.zeros((m, d)), "tau": np.zeros(m), "tau_h": np.zeros(m),
        "counts": np.zeros((m, B), dtype=np.int32), "T": np.zeros(m, dtype=np.int64),
        "rowbits": np.zeros((m, W), dtype=np.uint32), "xgap": np.zeros(m), "psum": np.zeros(m),
    }
    # group consecutive rows into runs so each C call covers [r0, r1)
    runs = []
    start = 0
    for t in range(1, m + 1):
        if t == m or rows_arr[t] != rows_arr[t - 1] + 1:
            runs.append((start, t))
            start = t
    jobs = []
    nthr = threads or default_threads()
    for (a, b) in runs:
        for (u, w) in _chunks(a, b, nthr * 4 if b - a > 64 else 1):
            jobs.append((u, w))

    def run(job):
        u, w = job
        r0, r1 = int(rows_arr[u]), int(rows_arr[u]) + (w - u)
        lib.oracle_attn_fwd_rows(
            n, d, _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), float(alpha), float(scale),
            float(slope), int(bool(causal)), int(B), int(Bc), r0, r1,
            _ptr(out["o"][u:w], _dp), _ptr(out["tau"][u:w], _dp), _ptr(out["tau_h"][u:w], _dp),
            _ptr(out["counts"][u:w], _ip), _ptr(out["T"][u:w], _lp),
            _ptr(out["rowbits"][u:w], _up), _ptr(out["xgap"][u:w], _dp),
            _ptr(out["psum"][u:w], _dp))

    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(run, jobs))
    return out


def block_mask(rowbits: np.ndarray, Br: int) -> np.ndarray:
    """Tile mask [Tr, W] from per-row bits [n, W]: OR over the Br rows of each query tile."""
    n, W = rowbits.shape
    Tr = (n + Br - 1) // Br
    out = np.zeros((Tr, W), dtype=np.uint32)
    for I in range(Tr):
        out[I] = np.bitwise_or.reduce(rowbits[I * Br:(I + 1) * Br], axis=0)
    return out


def attn_bwd_rows_head(q, k, v, dout, tau, alpha: float, causal: bool, scale: float,
                       rows=None, threads: int | None = None, slope: float = 0.0) -> dict:
    """Per-row backward of one query head: dq [r, d] and delta [r] for the given rows.

    ``tau`` holds the forward tau of exactly these rows (same order as ``rows``).
    """
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    n, d = q.shape
    rows_arr = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    tau = _f64(tau).ravel()
    m = rows_arr.size
    dq = np.zeros((m, d))
    delta = np.zeros(m)
    nthr = threads or default_threads()

    def run(t0t1):
        t0, t1 = t0t1
        for t in range(t0, t1):   # one call per row: rows may be scattered
            r = int(rows_arr[t])
            lib.oracle_attn_bwd_rows(n, d, _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp),
                                     _ptr(dout, _dp), _ptr(tau[t:t + 1], _dp), float(alpha),
                                     float(scale), float(slope), int(bool(causal)), r, r + 1,
                                     _ptr(dq[t:t + 1], _dp), _ptr(delta[t:t + 1], _dp))

    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(run, _chunks(0, m, nthr * 4)))
    return {"rows": rows_arr, "dq": dq, "delta": delta}


def attn_bwd_keys_group(q_group, k, v, dout_group, tau_group, delta_group, alpha: float,
                        causal: bool, scale: float, keys=None, threads: int | None = None,
                        slopes=None) -> dict:
    """Per-key backward of one KV head: dk, dv for the given keys (default: all).

    q_group, dout_group: [G, n, d] of the KV head's query heads; tau_group,
    delta_group: [G, n] (all rows of those heads); slopes: [G] position-bias slopes of
    those heads, or None.
    """
    lib = _load()
    qg, dog = _f64(q_group), _f64(dout_group)
    tg, dg = _f64(tau_group), _f64(delta_group)
    k, v = _f64(k), _f64(v)
    G, n, d = qg.shape
    sl = None if slopes is None else _f64(slopes).ravel()
    keys_arr = np.arange(n, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    m = keys_arr.size
    dk = np.zeros((m, d))
    dv = np.zeros((m, d))
    nthr = threads or default_threads()

    def run(t0t1):
        t0, t1 = t0t1
        for t in range(t0, t1):
            j = int(keys_arr[t])
            lib.oracle_attn_bwd_keys(n, d, G, _ptr(qg, _dp), _ptr(k, _dp), _ptr(v, _dp),
                                     _ptr(dog, _dp), _ptr(tg, _dp), _ptr(dg, _dp), float(alpha),
                                     float(scale), None if sl is None else _ptr(sl, _dp),
                                     int(bool(causal)), j, j + 1,
                                     _ptr(dk[t:t + 1], _dp), _ptr(dv[t:t + 1], _dp))

    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(run, _chunks(0, m, nthr * 4)))
    return {"keys": keys_arr, "dk": dk, "dv": dv}


def attn_full(q, k, v, dout, alpha: float, causal: bool, B: int, Br: int, Bc: int,
              scale: float | None = None, threads: int | None = None, backward: bool = True,
              slopes=None) -> dict:
    """Dense forward (and backward) of a whole problem.

    q, dout: [b, hq, n, d]; k, v: [b, hkv, n, d] (any array-like; widened to fp64).
    slopes: None, or [hq] position-bias slopes (head h scores get -slopes[h] |i - j|).
    Returns o, tau, tau_h, counts, T, mask [b, hq, Tr, W], xgap, psum and, with
    ``backward``, dq, dk, dv, delta.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    Tr = (n + Br - 1) // Br
    W = (n + 32 * Bc - 1) // (32 * Bc)
    sl = np.zeros(hq) if slopes is None else _f64(slopes).ravel()
    res = {
        "o": np.zeros_like(q), "tau": np.zeros((b, hq, n)), "tau_h": np.zeros((b, hq, n)),
        "counts": np.zeros((b, hq, n, B), dtype=np.int32), "T": np.zeros((b, hq, n), dtype=np.int64),
        "mask": np.zeros((b, hq, Tr, W), dtype=np.uint32), "xgap": np.zeros((b, hq, n)),
        "psum": np.zeros((b, hq, n)),
    }
    for bi in range(b):
        for h in range(hq):
            f = attn_fwd_head(q[bi, h], k[bi, h // G], v[bi, h // G], alpha, causal, B, Bc, scale,
                              threads=threads, slope=sl[h])
            res["o"][bi, h] = f["o"]
            for key in ("tau", "tau_h", "counts", "T", "xgap", "psum"):
                res[key][bi, h] = f[key]
            res["mask"][bi, h] = block_mask(f["rowbits"], Br)
    if backward:
        do = _f64(dout)
        res["dq"] = np.zeros_like(q)
        res["delta"] = np.zeros((b, hq, n))
        res["dk"] = np.zeros_like(k)
        res["dv"] = np.zeros_like(v)
        for bi in range(b):
            for h in range(hq):
                r = attn_bwd_rows_head(q[bi, h], k[bi, h // G], v[bi, h // G], do[bi, h],
                                       res["tau"][bi, h], alpha, causal, scale, threads=threads,
                                       slope=sl[h])
                res["dq"][bi, h] = r["dq"]
                res["delta"][bi, h] = r["delta"]
            for kh in range(hkv):
                hs = slice(kh * G, (kh + 1) * G)
                kk = attn_bwd_keys_group(q[bi, hs], k[bi, kh], v[bi, kh], do[bi, hs],
                                         res["tau"][bi, hs], res["delta"][bi, hs], alpha, causal,
                                         scale, threads=threads, slopes=sl[hs])
                res["dk"][bi, kh] = kk["dk"]
                res["dv"][bi, kh] = kk["dv"]
    return res


def attn_decode(q, k_cache, v_cache, lengths, alpha: float, B: int, scale: float | None = None,
                slopes=None, heads=None, threads: int | None = None) -> dict:
    """Decode step: query row q[b, h] against keys 0..lengths[b]-1 of its KV head's cache.

    The new token follows the cache, so this is row L-1 of a causal forward over the first
    L cached keys with the query placed there (the same per-row computation as
    ``attn_fwd_head``). q: [b, hq, d]; caches [b, hkv, n_ctx, d]; lengths: [b] or None.
    ``heads``: None for all (b, h) pairs, or a list of them. Returns o [b, hq, d], tau,
    tau_h [b, hq], counts [b, hq, B] (pairs not computed stay 0).
    """
    q = _f64(q)
    kc, vc = _f64(k_cache), _f64(v_cache)
    b, hq, d = q.shape
    hkv, n = kc.shape[1], kc.shape[2]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    sl = np.zeros(hq) if slopes is None else _f64(slopes).ravel()
    lens = [n] * b if lengths is None else [min(max(int(x), 1), n) for x in lengths]
    pairs = [(bi, h) for bi in range(b) for h in range(hq)] if heads is None else list(heads)
    out = {"o": np.zeros((b, hq, d)), "tau": np.zeros((b, hq)), "tau_h": np.zeros((b, hq)),
           "counts": np.zeros((b, hq, B), dtype=np.int32)}
    for bi, h in pairs:
        L = lens[bi]
        qf = np.zeros((L, d))
        qf[L - 1] = q[bi, h]
        f = attn_fwd_head(qf, kc[bi, h // G, :L], vc[bi, h // G, :L], alpha, True, B, 32, scale,
                          rows=[L - 1], threads=threads, slope=sl[h])
        out["o"][bi, h] = f["o"][0]
        out["tau"][bi, h] = f["tau"][0]
        out["tau_h"][bi, h] = f["tau_h"][0]
        out["counts"][bi, h] = f["counts"][0]
    return out

"""GPU parity of the DashAttention forward and backward (stages 1-2, include/dash_attn.h) with the fp64
oracle ``oracle.dash`` on the same seeded inputs (DashAttention (it), stages 1 and 2).

Bars: bf16 -- max |d route_tau| <= 1e-3, max |d wbar| <= 1e-3, max |do| <= 1e-2,
max |d lse| <= 1e-3. For routing alpha > 2 the weight d^kappa (kappa < 1) is only Hoelder in
tau near the support boundary, |d(a)^kappa - d(b)^kappa| <= |a - b|^kappa, so there the
weight bar is 1e-3 + (max |d route_tau| + 1e-6)^kappa, with the tau bar unchanged; chunk-mask bits equal to the OR of the kernel's own wbar > 0, and
equal to the oracle's except on (tile, chunk) pairs whose largest weight on either side is
below 1e-3 (a routing score within rounding of tau). fp32 -- the same at 1e-5 / 1e-5 /
1e-4 / 1e-5.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import oracle.dash as odash
import synth
import long_context_entmax_amd as lce
from tests.gpu_helpers import dev, rel_fro, to64

pytestmark = pytest.mark.gpu


def _inputs(b, hq, hkv, n, d, dtype, C, seed, qk_scale=1.0):
    w = synth.Workload("dash", b, hq, hkv, n, d, dtype, 1.5, True, 64, 64, 16, "normal",
                       extra={"qk_scale": qk_scale}, seed=seed)
    inp = synth.make_inputs(w, need_grad_inputs=False)
    return inp["q"], inp["k"], inp["v"], synth.chunk_summaries(w, C)


def _run(q, k, v, ks, C, alpha, gamma, sigma):
    d0 = dev()
    r = lce.dash_fwd(q.to(d0), k.to(d0), v.to(d0), ks.to(d0), C, alpha, gamma, sigma)
    torch.cuda.synchronize()
    return {kk: getattr(r, kk).cpu() for kk in ("o", "lse", "route_tau", "route_w", "chunk_mask")}


def _mask_from_w(wbar_cm: np.ndarray, n: int) -> np.ndarray:
    """Tile words from chunk-major weights [b, hkv, nc, n]."""
    b, hkv, nc, _ = wbar_cm.shape
    act = (wbar_cm > 0).transpose(0, 1, 3, 2).reshape(b, hkv, n // 64, 64, nc).any(3)   # [b,hkv,Tr,nc]
    words = np.zeros((b, hkv, n // 64, (nc + 31) // 32), dtype=np.int64)
    for c in range(nc):
        words[..., c // 32] |= act[..., c].astype(np.int64) << (c % 32)
    return words


def _check(g, ref, n, tol, alpha):
    t_tau, t_w, t_o, t_lse = tol
    dtau = np.abs(g["route_tau"].numpy() - ref["tau"]).max()
    assert dtau < t_tau
    if alpha > 2.0:
        t_w += (dtau + 1e-6) ** (1.0 / (alpha - 1.0))
    w_gpu = g["route_w"].numpy().astype(np.float64)                    # [b, hkv, nc, n]
    w_ref = ref["wbar"].transpose(0, 1, 3, 2)                            # [b, hkv, r, nc] -> chunk-major
    assert np.abs(w_gpu - w_ref).max() < t_w
    assert np.abs(g["o"].numpy() - ref["o"]).max() < t_o
    assert np.abs(g["lse"].numpy() - ref["lse"]).max() < t_lse
    gm = g["chunk_mask"].numpy().astype(np.int64) & 0xFFFFFFFF
    np.testing.assert_array_equal(gm, _mask_from_w(w_gpu, n))
    if not np.array_equal(gm, ref["mask"]):
        # every differing bit: both sides' largest weight in that (tile, chunk) is tiny
        b, hkv, nc, _ = w_gpu.shape
        big = np.maximum(np.abs(w_gpu), np.abs(w_ref)).transpose(0, 1, 3, 2).reshape(b, hkv, n // 64, 64, nc).max(3)
        diff = gm ^ ref["mask"]
        for idx in zip(*np.nonzero(diff)):
            bits = int(diff[idx])
            for bit in range(32):
                if bits >> bit & 1:
                    c = idx[3] * 32 + bit
                    assert big[idx[0], idx[1], idx[2], c] < 1e-3, (idx, c)


DASH_CASES = [
    # (b, hq, hkv, n, d, dtype, C, alpha, gamma, sigma, qk_scale)
    (1, 4, 2, 1024, 64, "bf16", 64, 1.5, 8.0, 1.0, 1.0),
    (2, 2, 1, 2048, 128, "bf16", 128, 2.0, 16.0, 1.0, 1.0),
    (1, 8, 1, 1024, 64, "bf16", 64, 1.25, 4.0, 0.5, 1.0),
    (1, 2, 2, 1536, 128, "bf16", 256, 3.0, 8.0, 2.0, 1.0),
    (1, 4, 4, 2048, 64, "bf16", 64, 1.5, 1.0, 0.0, 1.0),        # nearly uniform routing, sigma 0
    (1, 16, 2, 4096, 128, "bf16", 64, 1.5, 24.0, 1.0, 1.0),     # GQA 8, 64 chunks
    (2, 6, 2, 768, 64, "bf16", 64, 1.5, 12.0, 1.0, 1.0),        # GQA 3 (not a power of two), batch 2
    (1, 2, 1, 64, 64, "bf16", 64, 1.5, 8.0, 1.0, 1.0),          # one chunk: no row routes anything
]


@pytest.mark.parametrize("case", DASH_CASES, ids=[str(c) for c in DASH_CASES])
def test_dash_bf16(case):
    b, hq, hkv, n, d, dt, C, alpha, gamma, sigma, qs = case
    print(f"[case] dash {case}", flush=True)
    q, k, v, ks = _inputs(b, hq, hkv, n, d, dt, C, zlib.crc32(str(case).encode()) & 0xFFFF, qs)
    ref = odash.dash_fwd(to64(q), to64(k), to64(v), to64(ks), alpha, gamma, sigma, C)
    g = _run(q, k, v, ks, C, alpha, gamma, sigma)
    _check(g, ref, n, (1e-3, 1e-3, 1e-2, 1e-3), alpha)


def test_dash_fp32():
    b, hq, hkv, n, d, C = 1, 4, 2, 1024, 64, 64
    print("[case] dash fp32", flush=True)
    q, k, v, ks = _inputs(b, hq, hkv, n, d, "f32", C, 77)
    ref = odash.dash_fwd(to64(q), to64(k), to64(v), to64(ks), 1.5, 8.0, 1.0, C)
    g = _run(q, k, v, ks, C, 1.5, 8.0, 1.0)
    _check(g, ref, n, (1e-5, 1e-5, 1e-4, 1e-5), 1.5)


def test_dash_uniform_summaries_route_every_chunk():
    """Zero summaries: every earlier chunk is routed with weight 1/m_i exactly (the oracle
    pins this case to torch's SDPA)."""
    b, hq, hkv, n, d, C = 1, 2, 1, 512, 64, 64
    print("[case] dash uniform summaries", flush=True)
    q, k, v, ks = _inputs(b, hq, hkv, n, d, "bf16", C, 5)
    ks = torch.zeros_like(ks)
    ref = odash.dash_fwd(to64(q), to64(k), to64(v), to64(ks), 1.5, 1.0, 1.0, C)
    g = _run(q, k, v, ks, C, 1.5, 1.0, 1.0)
    _check(g, ref, n, (1e-5, 1e-6, 1e-2, 1e-3), 1.5)


def test_dash_fullsize_sampled_rows():
    """The 16K benchmark shape (b1, 32 query / 2 KV heads, d 128, 256 chunks of 64, routing
    alpha 1.5, gamma 36, sigma 1), run whole in the benchmark's launch configuration; 64 rows
    (the first and last tiles' edges and evenly spaced ones) against the oracle, and the chunk
    mask against the kernel's own weights everywhere."""
    import bench
    w = bench.dash_workload()
    C, gamma, sigma = bench.DASH_CHUNK, bench.DASH_GAMMA, bench.DASH_SIGMA
    print(f"[case] dash full size {w.name}", flush=True)
    inp = synth.make_inputs(w, need_grad_inputs=False)
    ks = synth.chunk_summaries(w, C)
    g = _run(inp["q"], inp["k"], inp["v"], ks, C, w.alpha, gamma, sigma)
    n = w.seqlen
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(60, 68), np.arange(n - 8, n),
                                     np.linspace(100, n - 100, 44).astype(np.int64)]))
    ref = odash.dash_fwd(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), to64(ks), w.alpha, gamma, sigma, C,
                         rows=rows)
    assert np.abs(g["route_tau"].numpy()[:, :, rows] - ref["tau"]).max() < 1e-3
    w_gpu = g["route_w"].numpy()[:, :, :, rows].astype(np.float64)
    assert np.abs(w_gpu - ref["wbar"].transpose(0, 1, 3, 2)).max() < 1e-3
    assert np.abs(g["o"].numpy()[:, :, rows] - ref["o"]).max() < 1e-2
    assert np.abs(g["lse"].numpy()[:, :, rows] - ref["lse"]).max() < 1e-3
    gm = g["chunk_mask"].numpy().astype(np.int64) & 0xFFFFFFFF
    np.testing.assert_array_equal(gm, _mask_from_w(g["route_w"].numpy().astype(np.float64), n))


# ------------------------------------------------------------------------------ backward
# Bars (relative Frobenius error of each gradient against the oracle's, as the attention
# backward): bf16 2e-2, fp32 1e-4. Both sides see the same inputs; the kernel's backward
# takes its own forward's o, lse, route_tau and route_w, the oracle recomputes them.

def _run_bwd(q, k, v, ks, do, C, alpha, gamma, sigma):
    d0 = dev()
    q, k, v, ks, do = q.to(d0), k.to(d0), v.to(d0), ks.to(d0), do.to(d0)
    r = lce.dash_fwd(q, k, v, ks, C, alpha, gamma, sigma)
    gr = lce.dash_bwd(q, k, v, ks, do, r.o, r.lse, r.route_tau, r.route_w, r.chunk_mask, C, alpha, gamma, sigma)
    torch.cuda.synchronize()
    return {kk: getattr(gr, kk).float().cpu().numpy().astype(np.float64) for kk in ("dq", "dk", "dv", "dk_summary")}


def _inputs_bwd(b, hq, hkv, n, d, dtype, C, seed, qk_scale=1.0):
    w = synth.Workload("dash", b, hq, hkv, n, d, dtype, 1.5, True, 64, 64, 16, "normal",
                       extra={"qk_scale": qk_scale}, seed=seed)
    inp = synth.make_inputs(w, need_grad_inputs=True)
    return inp["q"], inp["k"], inp["v"], synth.chunk_summaries(w, C), inp["do"]


def _check_bwd(g, ref, bar):
    for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dk_summary", "dks")):
        if not np.any(ref[rname]):
            assert not np.any(g[name]), name
            continue
        err = rel_fro(g[name], ref[rname])
        print(f"  {name}: rel err {err:.2e}", flush=True)
        assert err < bar, (name, err)


DASH_BWD_CASES = [
    # (b, hq, hkv, n, d, dtype, C, alpha, gamma, sigma)
    (1, 4, 2, 1024, 64, "bf16", 64, 1.5, 8.0, 1.0),
    (2, 2, 1, 1024, 128, "bf16", 128, 2.0, 16.0, 1.0),
    (1, 6, 2, 768, 64, "bf16", 64, 1.25, 4.0, 0.5),      # GQA 3, routing alpha 1.25
    (1, 4, 4, 1024, 64, "bf16", 64, 1.5, 1.0, 0.0),      # sigma 0: no gradient reaches the summaries
    (1, 2, 2, 1536, 128, "bf16", 256, 1.5, 8.0, 2.0),    # chunk 256
    (1, 8, 1, 512, 64, "bf16", 64, 1.5, 12.0, 1.0),      # GQA 8
    (1, 2, 1, 64, 64, "bf16", 64, 1.5, 8.0, 1.0),        # one chunk: no routing, diagonal branch only
]


@pytest.mark.parametrize("case", DASH_BWD_CASES, ids=[str(c) for c in DASH_BWD_CASES])
def test_dash_bwd_bf16(case):
    b, hq, hkv, n, d, dt, C, alpha, gamma, sigma = case
    print(f"[case] dash bwd {case}", flush=True)
    q, k, v, ks, do = _inputs_bwd(b, hq, hkv, n, d, dt, C, zlib.crc32(str(case).encode()) & 0xFFFF)
    ref = odash.dash_bwd(to64(q), to64(k), to64(v), to64(ks), to64(do), alpha, gamma, sigma, C)
    g = _run_bwd(q, k, v, ks, do, C, alpha, gamma, sigma)
    _check_bwd(g, ref, 2e-2)


def test_dash_bwd_fp32():
    b, hq, hkv, n, d, C = 1, 4, 2, 1024, 64, 64
    print("[case] dash bwd fp32", flush=True)
    q, k, v, ks, do = _inputs_bwd(b, hq, hkv, n, d, "f32", C, 91)
    ref = odash.dash_bwd(to64(q), to64(k), to64(v), to64(ks), to64(do), 1.5, 8.0, 1.0, C)
    g = _run_bwd(q, k, v, ks, do, C, 1.5, 8.0, 1.0)
    _check_bwd(g, ref, 1e-4)


def test_dash_bwd_fullsize_sampled_rows():
    """The 16K benchmark shape in the benchmark's launch configuration, dO kept on 24 sampled
    rows (every head) and zero elsewhere, so that the oracle needs those rows only: dq of the
    sampled rows, and the whole dk, dv and dk_summary (sums over the sampled rows) against
    the oracle; dq of every other row is 0. Then, with the full dO, two sums that hold at any
    size: per KV group, sum_j dv_j = sum over the group's rows of dO_i (each row's weights
    sum to 1), and sum_j dk_j = 0 (each row's dS sums to 0)."""
    import bench
    w = bench.dash_workload()
    C, gamma, sigma = bench.DASH_CHUNK, bench.DASH_GAMMA, bench.DASH_SIGMA
    print(f"[case] dash bwd full size {w.name}", flush=True)
    inp = synth.make_inputs(w, need_grad_inputs=True)
    ks = synth.chunk_summaries(w, C)
    n = w.seqlen
    rows = np.unique(np.concatenate([np.arange(0, 2), np.arange(63, 66), np.arange(n - 3, n),
                                     np.linspace(100, n - 100, 16).astype(np.int64)]))
    keep = torch.zeros(n, dtype=inp["do"].dtype)
    keep[torch.from_numpy(rows)] = 1
    do_r = (inp["do"] * keep[None, None, :, None]).contiguous()
    g = _run_bwd(inp["q"], inp["k"], inp["v"], ks, do_r, C, w.alpha, gamma, sigma)
    ref = odash.dash_bwd(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), to64(ks), to64(do_r), w.alpha,
                         gamma, sigma, C, rows=rows)
    for name, got, want in (("dq (sampled rows)", g["dq"][:, :, rows], ref["dq"]), ("dk", g["dk"], ref["dk"]),
                            ("dv", g["dv"], ref["dv"]), ("dk_summary", g["dk_summary"], ref["dks"])):
        err = rel_fro(got, want)
        print(f"  {name}: rel err {err:.2e}", flush=True)
        assert err < 2e-2, name
    others = np.setdiff1d(np.arange(n), rows)
    assert not np.any(g["dq"][:, :, others])
    g = _run_bwd(inp["q"], inp["k"], inp["v"], ks, inp["do"], C, w.alpha, gamma, sigma)
    b, hq, hkv = w.batch, w.heads_q, w.heads_kv
    G = hq // hkv
    do64 = to64(inp["do"]).reshape(b, hkv, G, n, -1).sum(axis=(2, 3))
    assert rel_fro(g["dv"].sum(axis=2), do64) < 2e-2
    assert np.linalg.norm(g["dk"].sum(axis=2)) < 2e-2 * np.linalg.norm(g["dk"])


def test_dash_bwd_alpha3_conditioned_rows():
    """Routing alpha 3 (the general-alpha weight, kappa = 1/2). There g = (x - tau)^(kappa - 1)
    is singular at the support boundary, so du of a chunk whose logit lies just above tau
    moves by a large factor for a tau change at rounding level: such rows carry no usable
    reference. dO is zeroed on every row where some head of the group routes a chunk within
    1e-2 of its tau (by the oracle's own tau), on both sides; those rows then contribute
    nothing, and every gradient must still match to the bf16 bar."""
    case = (1, 4, 2, 1024, 64, "bf16", 64, 3.0, 8.0, 1.0)
    b, hq, hkv, n, d, dt, C, alpha, gamma, sigma = case
    print(f"[case] dash bwd alpha 3 {case}", flush=True)
    q, k, v, ks, do = _inputs_bwd(b, hq, hkv, n, d, dt, C, zlib.crc32(str(case).encode()) & 0xFFFF)
    q64, ks64 = to64(q), to64(ks)
    G = hq // hkv
    scale = 1.0 / np.sqrt(d)
    bad = np.zeros((b, hkv, n), dtype=bool)
    for bi in range(b):
        for hh in range(hq):
            g = hh // G
            for i in range(C, n):
                m = i // C
                z = gamma * scale * (ks64[bi, g, :m] @ q64[bi, hh, i])
                x = (alpha - 1.0) * z
                gap = x - oracle.entmax_tau(x, alpha)
                if np.any((gap > 0.0) & (gap < 1e-2)):
                    bad[bi, g, i] = True
    print(f"  rows zeroed: {bad.mean():.3f}", flush=True)
    assert bad.mean() < 0.5
    keep = torch.from_numpy(~np.repeat(bad, G, axis=1)).to(do.dtype)[..., None]
    do = (do * keep).contiguous()
    ref = odash.dash_bwd(q64, to64(k), to64(v), ks64, to64(do), alpha, gamma, sigma, C)
    g = _run_bwd(q, k, v, ks, do, C, alpha, gamma, sigma)
    _check_bwd(g, ref, 2e-2)

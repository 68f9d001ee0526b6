"""GPU parity of the decode path (one new query row per sequence and head against a KV
cache) with the fp64 oracle: the oracle's decode row is row L-1 of a causal forward over
the first L cached keys with the query placed there.

Bars as for the forward: bf16 max |dtau| <= 1e-3, max |do| <= 1e-2; tau_h satisfies
Proposition 1 against the oracle's tau* (AdaSplash-2 (ja) §2.1); the fp32 grid case compares
histogram counts bit for bit.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import long_context_entmax_amd as lce
from tests.gpu_helpers import dev, to64

pytestmark = pytest.mark.gpu


def _inputs(b, hq, hkv, n, d, dtype, recipe, lengths, seed, qk_scale=1.0):
    """Caches from the synthetic generator; the decode query of sequence b is row L_b - 1."""
    w = synth.Workload("dec", b, hq, hkv, n, d, dtype, 1.5, True, 32, 32, 16, recipe,
                       extra={"qk_scale": qk_scale}, seed=seed)
    inp = synth.make_inputs(w, need_grad_inputs=False)
    lens = [n] * b if lengths is None else list(lengths)
    q = torch.stack([inp["q"][bi, :, lens[bi] - 1] for bi in range(b)])   # [b, hq, d]
    return q.contiguous(), inp["k"], inp["v"], lens


def _run(q, k, v, lens, alpha, B, slopes=None, tau_init=0, pass_lengths=True):
    d0 = dev()
    ln = torch.tensor(lens, dtype=torch.int32, device=d0) if pass_lengths else None
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device=d0)
    r = lce.decode(q.to(d0), k.to(d0), v.to(d0), alpha, B, lengths=ln, slopes=sl, tau_init=tau_init,
                   return_hist=True)
    torch.cuda.synchronize()
    return {kk: getattr(r, kk).cpu() for kk in ("o", "tau", "hist", "tau_h")}


def _check(g, ref, B, tol_tau=1e-3, tol_o=1e-2, prop1=True):
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < tol_tau
    assert np.abs(g["o"].numpy() - ref["o"]).max() < tol_o
    if prop1:
        th = g["tau_h"].numpy().astype(np.float64)
        assert np.all(th <= ref["tau"] + 1e-5)
        assert np.all(ref["tau"] - th < 1.0 / B + 1e-5)


DEC_CASES = [
    # (b, hq, hkv, n_ctx, d, alpha, B, lengths, slopes?, qk_scale)
    (2, 4, 2, 1000, 64, 1.5, 16, [1000, 777], False, 1.0),
    (1, 8, 2, 4096, 128, 2.0, 16, None, True, 1.2),
    (3, 2, 2, 300, 64, 1.25, 8, [1, 2, 300], False, 1.0),
    (1, 4, 1, 5000, 64, 3.0, 8, None, False, 1.0),
    (1, 16, 1, 2500, 64, 1.5, 4, [2049], True, 1.0),
    (2, 2, 1, 2048, 128, 1.5, 16, [2048, 2047], False, 0.8),
    # nearly flat scores: most keys stay refinement candidates, more than a work group keeps
    # on chip, so the passes rescan the stored row
    (1, 2, 1, 30000, 64, 1.5, 16, None, False, 0.05),
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[str(c) for c in DEC_CASES])
def test_decode_bf16(case):
    b, hq, hkv, n, d, alpha, B, lengths, bias, qs = case
    print(f"[case] decode {case}", flush=True)
    q, k, v, lens = _inputs(b, hq, hkv, n, d, "bf16", "normal", lengths,
                          zlib.crc32(str(case).encode()) & 0xFFFF, qs)
    slopes = lce.nape_slopes(hq) if bias else None
    ref = oracle.attn_decode(to64(q), to64(k), to64(v), lens, alpha, B, slopes=slopes)
    g = _run(q, k, v, lens, alpha, B, slopes)
    _check(g, ref, B)


def test_decode_fp32_grid_bit_exact():
    """Q and K on the 2^-5 grid with (alpha - 1) scale B = 1: every score is exact in fp32,
    so the histogram counts match the oracle bit for bit."""
    b, hq, hkv, n, d = 2, 4, 2, 640, 64
    print("[case] decode fp32 grid", flush=True)
    q, k, v, lens = _inputs(b, hq, hkv, n, d, "f32", "tiny", [640, 333], 21)
    ref = oracle.attn_decode(to64(q), to64(k), to64(v), lens, 1.5, 16)
    g = _run(q, k, v, lens, 1.5, 16)
    np.testing.assert_array_equal(g["hist"].numpy(), ref["counts"])
    _check(g, ref, 16, tol_tau=1e-5, tol_o=1e-4)


def test_decode_plain_bracket_and_default_lengths():
    """The histogram-free start reaches the same tau; lengths = NULL means the whole cache."""
    b, hq, hkv, n, d = 1, 4, 2, 3000, 64
    print("[case] decode bracket start", flush=True)
    q, k, v, lens = _inputs(b, hq, hkv, n, d, "bf16", "normal", None, 8)
    ref = oracle.attn_decode(to64(q), to64(k), to64(v), lens, 1.5, 16)
    g = _run(q, k, v, lens, 1.5, 16, tau_init=1, pass_lengths=False)
    _check(g, ref, 16, prop1=False)
    assert int(np.abs(g["hist"].numpy()).sum()) == 0


def test_decode_matches_forward_last_row():
    """Decode of the query at position n - 1 equals the last row of the causal forward: tau
    to fp32 rounding; o to the bf16 rounding of P that the forward's P.V product applies
    (the decode sums p v in fp32)."""
    w = synth.Workload("t", 1, 4, 2, 512, 64, "bf16", 1.5, True, 64, 64, 16, "normal", seed=4)
    print("[case] decode vs forward", flush=True)
    inp = synth.make_inputs(w, need_grad_inputs=False)
    d0 = dev()
    qd, kd, vd = inp["q"].to(d0), inp["k"].to(d0), inp["v"].to(d0)
    f = lce.fwd(qd, kd, vd, 1.5, True, (64, 64), 16)
    r = lce.decode(qd[:, :, -1].contiguous(), kd, vd, 1.5, 16)
    torch.cuda.synchronize()
    assert (f.tau[:, :, -1] - r.tau).abs().max().item() < 1e-5
    assert (f.o[:, :, -1] - r.o).abs().max().item() < 1e-2


def test_decode_fullsize_sampled_heads():
    """The 128K GQA shape (hq 32 / hkv 8, d 64, centroid recipe): the query heads of two KV
    heads (groups of 4, as in the full problem) against their full 131072-key caches."""
    w = synth.workload("C5")
    heads = [0, 1, 2, 3, 20, 21, 22, 23]
    print(f"[case] decode full size {w.name} heads {heads}", flush=True)
    inp = synth.make_inputs(w, heads=heads, need_grad_inputs=False)
    n = w.seqlen
    q = inp["q"][:, :, n - 1].contiguous()                      # [1, 8, d]
    ref = oracle.attn_decode(to64(q), to64(inp["k"]), to64(inp["v"]), None, w.alpha, w.n_bins)
    g = _run(q, inp["k"], inp["v"], [n], w.alpha, w.n_bins)
    _check(g, ref, w.n_bins)


def test_decode_max_cache():
    """A cache of the largest supported length, 2^19 keys, and a ragged shorter one."""
    b, hq, hkv, n, d = 2, 2, 1, 1 << 19, 64
    print("[case] decode max cache", flush=True)
    q, k, v, lens = _inputs(b, hq, hkv, n, d, "bf16", "normal", [n, 300001], 31)
    ref = oracle.attn_decode(to64(q), to64(k), to64(v), lens, 1.5, 16)
    g = _run(q, k, v, lens, 1.5, 16)
    _check(g, ref, 16)

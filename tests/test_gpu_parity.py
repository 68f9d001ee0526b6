"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same inputs.

Bars: fp32 tiny configuration -- histogram counts, support and block mask bit-exact,
|dtau| <= 1e-5, |dO| <= 1e-4, gradients within 1e-4 relative Frobenius error; bf16 --
max |dO| <= 1e-2, max |dtau| <= 1e-3, gradients within 2e-2 relative Frobenius error,
block mask equal except in blocks whose nearest score lies within 1e-3 of tau*.
tau_h always satisfies Proposition 1 against the oracle's tau* (AdaSplash-2 (ja) §2.1).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import long_context_entmax_amd as lce
from tests.gpu_helpers import (mask_bits, mask_mismatch_is_ambiguous, rel_fro, run_gpu, scores_x,
                               to64, valid_block_mask)

pytestmark = pytest.mark.gpu


def _oracle(inp, w, slopes=None):
    return oracle.attn_full(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), to64(inp["do"]), w.alpha,
                            w.causal, w.n_bins, w.block_q, w.block_k, slopes=slopes)


def _check_prop1(g, ref, B):
    th = g["tau_h"].numpy().astype(np.float64)
    ts = ref["tau"]
    assert np.all(th <= ts + 1e-5), float((th - ts).max())
    assert np.all(ts - th < 1.0 / B + 1e-5), float((ts - th).max())


def test_tiny_fp32_config_bit_exact():
    """b1 h1 n256 d64 fp32 non-causal alpha 1.5 B16 32x32, Q/K on the 2^-5 grid."""
    w = synth.workload("C1")
    print(f"[case] C1 {w.as_dict()}", flush=True)
    inp = synth.make_inputs(w)
    ref = _oracle(inp, w)
    # precondition of bit-exact comparisons: no score within 1e-6 of the threshold
    assert ref["xgap"].min() > 1e-6, "test construction: a score sits on the threshold"
    g = run_gpu(inp, w)
    # histogram counts: bit-exact
    np.testing.assert_array_equal(g["hist"].numpy(), ref["counts"])
    assert np.abs(g["tau_h"].numpy() - ref["tau_h"]).max() < 1e-5
    _check_prop1(g, ref, w.n_bins)
    # tau and the support it implies (scores are exact in fp32 on this grid)
    tau = g["tau"].numpy().astype(np.float64)
    assert np.abs(tau - ref["tau"]).max() < 1e-5
    x = scores_x(to64(inp["q"]), to64(inp["k"]), w.alpha, 1.0 / math.sqrt(w.head_dim), 1)
    np.testing.assert_array_equal(x > tau[..., None], x > ref["tau"][..., None])
    np.testing.assert_array_equal(mask_bits(g["mask"].numpy()), ref["mask"].astype(np.int64))
    assert np.abs(g["o"].numpy() - ref["o"]).max() < 1e-4
    for name in ("dq", "dk", "dv"):
        err = rel_fro(g[name].numpy().astype(np.float64), ref[name])
        assert err < 1e-4, (name, err)


CASES = [
    # (b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qk_scale)
    (1, 2, 2, 256, 64, 1.5, True, 64, 64, 16, 1.0),
    (1, 2, 1, 192, 64, 2.0, True, 64, 64, 16, 1.5),
    (2, 4, 2, 128, 64, 1.5, False, 32, 64, 8, 1.0),
    (1, 4, 1, 256, 64, 1.25, True, 64, 32, 16, 1.0),
    (1, 1, 1, 96, 64, 3.0, True, 32, 32, 8, 1.0),
    (1, 2, 2, 256, 128, 1.5, True, 64, 64, 8, 1.0),
    (1, 2, 2, 384, 128, 2.0, True, 128, 64, 16, 1.2),
    (1, 1, 1, 256, 128, 1.5, False, 128, 128, 16, 0.7),
    (1, 8, 2, 128, 64, 1.5, True, 64, 64, 16, 2.0),
    # GQA 16 at both head dims, and blocks 32 x 128 (one query tile row per 32-row chunk)
    (1, 16, 1, 192, 64, 1.5, True, 64, 64, 16, 1.0),
    (2, 16, 1, 128, 128, 2.0, True, 32, 128, 8, 1.0),
    (1, 3, 1, 160, 64, 1.5, True, 32, 32, 16, 1.0),    # GQA 3: no power of two
    # no causal mask and an odd number of 32-key sub-blocks: the histogram pass's last pair
    # has a tile past the last key (masked by the score products at head_dim 64, set to -inf
    # by a branch at head_dim 128)
    (1, 2, 2, 96, 64, 2.0, False, 32, 32, 16, 1.0),
    (1, 2, 1, 96, 128, 1.5, False, 32, 32, 8, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_bf16_random_shapes(case):
    b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qs = case
    print(f"[case] bf16 {case}", flush=True)
    w = synth.Workload("t", b, hq, hkv, n, d, "bf16", alpha, causal, Br, Bc, B, "normal",
                       extra={"qk_scale": qs}, seed=hash(case) & 0xFFFF)
    inp = synth.make_inputs(w)
    ref = _oracle(inp, w)
    g = run_gpu(inp, w)
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < 1e-3
    assert np.abs(g["o"].float().numpy() - ref["o"]).max() < 1e-2
    _check_prop1(g, ref, B)
    x = scores_x(to64(inp["q"]), to64(inp["k"]), alpha, 1.0 / math.sqrt(d), hq // hkv)
    assert mask_mismatch_is_ambiguous(g["mask"].numpy(), ref["mask"], x, ref["tau"], w, 1e-3)
    for name in ("dq", "dk", "dv"):
        err = rel_fro(g[name].float().numpy().astype(np.float64), ref[name])
        assert err < 2e-2, (name, err)


# Large alpha: x = (alpha - 1) s spreads the scores so far that most rows keep one key, where
# f(tau) = sum p - 1 is flattest (slope 1/(alpha - 1) at a single key) and a test on the mass
# alone would leave tau off by up to 1e-4 (alpha - 1). tau is compared on every row. p =
# (x - tau)^(1/(alpha - 1)) and g = (x - tau)^(1/(alpha - 1) - 1) are not Lipschitz at x = tau
# (a key 1e-6 above tau already has p = 0.14 at alpha = 8), so O and the gradients are
# compared on the rows whose every valid score lies at least 1e-2 from the oracle's tau (the
# other rows get dO = 0, so they add nothing to dK and dV on either side). On these inputs
# such rows keep one key, whose weight is 1 and whose dQ and dK terms vanish: the gradient
# error is taken relative to max(|reference|, 1).
LARGE_ALPHA = [
    (1, 2, 2, 128, 64, 8.0, True, 64, 64, 16, 1.0),
    (1, 2, 1, 128, 64, 16.0, False, 64, 64, 16, 1.0),
    (1, 1, 1, 192, 128, 16.0, True, 64, 64, 8, 1.0),
]


@pytest.mark.parametrize("case", LARGE_ALPHA, ids=[str(c) for c in LARGE_ALPHA])
def test_large_alpha_single_key_rows(case):
    b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qs = case
    print(f"[case] large alpha {case}", flush=True)
    w = synth.Workload("t", b, hq, hkv, n, d, "bf16", alpha, causal, Br, Bc, B, "normal",
                       extra={"qk_scale": qs}, seed=hash(case) & 0xFFFF)
    inp = synth.make_inputs(w)
    ref = _oracle(inp, w)
    x = scores_x(to64(inp["q"]), to64(inp["k"]), alpha, 1.0 / math.sqrt(d), hq // hkv)
    if causal:
        x = np.where(np.tril(np.ones((n, n), dtype=bool))[None, None], x, np.nan)
    gap = np.nanmin(np.abs(x - ref["tau"][..., None]), axis=-1)
    support = np.nansum(x > ref["tau"][..., None], axis=-1)
    assert (support == 1).mean() > 0.5, "test construction: most rows should keep one key"
    good = gap >= 1e-2
    assert good.mean() > 0.5, "test construction: most rows should be well separated"
    inp["do"] = (inp["do"].float() * torch.from_numpy(good[..., None].astype(np.float32))).to(inp["do"].dtype)
    ref = _oracle(inp, w)
    g = run_gpu(inp, w)
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < 1e-3
    assert np.abs(g["o"].float().numpy() - ref["o"])[good].max() < 1e-2
    _check_prop1(g, ref, B)
    assert mask_mismatch_is_ambiguous(g["mask"].numpy(), ref["mask"], np.nan_to_num(x, nan=-np.inf),
                                      ref["tau"], w, 1e-3)
    for name in ("dq", "dk", "dv"):
        gg = g[name].float().numpy().astype(np.float64)
        err = float(np.linalg.norm(gg - ref[name]) / max(np.linalg.norm(ref[name]), 1.0))
        assert err < 2e-2, (name, err)


DENSE_CASES = [CASES[0], CASES[1], CASES[2], CASES[3], CASES[4], CASES[6], CASES[8], CASES[11]]


@pytest.mark.parametrize("case", DENSE_CASES, ids=[str(c) for c in DENSE_CASES])
def test_dense_ablation_matches_skipping(case):
    """The ablation without block skipping (every causally valid block multiplied in the
    refinement, output and backward kernels) returns every valid mask bit and the same
    results: tau, o and aux bit for bit (the skipped blocks add exact zeros to every sum),
    the gradients up to the fp32 order of the backward's partial sums, and both within the
    oracle's bars."""
    b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qs = case
    print(f"[case] dense ablation {case}", flush=True)
    w = synth.Workload("t", b, hq, hkv, n, d, "bf16", alpha, causal, Br, Bc, B, "normal",
                       extra={"qk_scale": qs}, seed=hash(case) & 0xFFFF)
    inp = synth.make_inputs(w)
    g = run_gpu(inp, w)
    gd = run_gpu(inp, w, dense=True)
    np.testing.assert_array_equal(mask_bits(gd["mask"].numpy()), valid_block_mask(b, hq, n, Br, Bc, causal))
    for name in ("tau", "o", "aux", "tau_h", "hist"):
        assert torch.equal(g[name], gd[name]), name
    for name in ("dq", "dk", "dv"):
        err = rel_fro(gd[name].float().numpy().astype(np.float64), g[name].float().numpy().astype(np.float64))
        assert err < 1e-3, (name, err)
    ref = _oracle(inp, w)
    assert np.abs(gd["o"].float().numpy() - ref["o"]).max() < 1e-2
    for name in ("dq", "dk", "dv"):
        assert rel_fro(gd[name].float().numpy().astype(np.float64), ref[name]) < 2e-2, name


BRACKET_CASES = [CASES[0], CASES[1], CASES[3], CASES[4], CASES[6]]


@pytest.mark.parametrize("case", BRACKET_CASES, ids=[str(c) for c in BRACKET_CASES])
def test_plain_bracket_start(case):
    """Starting the refinement from [x_max - 1, x_max - n^(1-alpha)] without the histogram
    (the ablation) reaches the same tau, output and gradients."""
    b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qs = case
    print(f"[case] bracket start {case}", flush=True)
    w = synth.Workload("t", b, hq, hkv, n, d, "bf16", alpha, causal, Br, Bc, B, "normal",
                       extra={"qk_scale": qs}, seed=hash(case) & 0xFFFF)
    inp = synth.make_inputs(w)
    ref = _oracle(inp, w)
    g = run_gpu(inp, w, tau_init=1)
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < 1e-3
    assert np.abs(g["o"].float().numpy() - ref["o"]).max() < 1e-2
    # the reported lower end is x_max - 1 <= tau*, and no counts are produced
    assert np.all(g["tau_h"].numpy() <= ref["tau"] + 1e-4)
    assert int(np.abs(g["hist"].numpy()).sum()) == 0
    for name in ("dq", "dk", "dv"):
        err = rel_fro(g[name].float().numpy().astype(np.float64), ref[name])
        assert err < 2e-2, (name, err)


BIAS_CASES = [
    # (b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qk_scale)
    (1, 4, 2, 256, 64, 1.5, True, 64, 64, 16, 1.0),
    (1, 2, 1, 192, 64, 2.0, True, 64, 64, 16, 1.5),
    (2, 4, 2, 128, 64, 1.5, False, 32, 64, 8, 1.0),
    (1, 2, 2, 256, 128, 1.5, True, 64, 64, 8, 1.0),
    (1, 4, 4, 256, 64, 1.25, True, 64, 32, 16, 0.8),
    (1, 2, 1, 96, 64, 3.0, False, 32, 32, 8, 1.0),
    (1, 4, 2, 384, 128, 2.0, True, 128, 64, 16, 1.2),
]


def _bias_slopes(hq):
    """NAPE-style split with strong slopes: heads < hq/2 unbiased, then 1/2, 1/4, ..."""
    return [0.0] * (hq // 2) + [2.0 ** -(t + 1) for t in range(hq - hq // 2)]


@pytest.mark.parametrize("case", BIAS_CASES, ids=[str(c) for c in BIAS_CASES])
def test_position_bias(case):
    """Per-head position bias (NAPE heads: half without encoding, half ALiBi)."""
    b, hq, hkv, n, d, alpha, causal, Br, Bc, B, qs = case
    slopes = _bias_slopes(hq)
    print(f"[case] bias {case} slopes {slopes}", flush=True)
    # alpha > 2: g = (x - tau)^(1/(alpha-1) - 1) is unbounded at the threshold, so a score
    # within 1e-4 of tau makes the gradient ill-conditioned; such inputs are skipped by seed
    for t in range(20):
        w = synth.Workload("t", b, hq, hkv, n, d, "bf16", alpha, causal, Br, Bc, B, "normal",
                           extra={"qk_scale": qs}, seed=(hash(case) + 7 + 1000 * t) & 0xFFFF)
        inp = synth.make_inputs(w)
        ref = _oracle(inp, w, slopes)
        if alpha <= 2.0 or ref["xgap"].min() > 1e-4:
            break
    g = run_gpu(inp, w, slopes=slopes)
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < 1e-3
    assert np.abs(g["o"].float().numpy() - ref["o"]).max() < 1e-2
    _check_prop1(g, ref, B)
    x = scores_x(to64(inp["q"]), to64(inp["k"]), alpha, 1.0 / math.sqrt(d), hq // hkv, slopes)
    assert mask_mismatch_is_ambiguous(g["mask"].numpy(), ref["mask"], x, ref["tau"], w, 1e-3)
    for name in ("dq", "dk", "dv"):
        err = rel_fro(g[name].float().numpy().astype(np.float64), ref[name])
        assert err < 2e-2, (name, err)


def test_position_bias_fp32_bit_exact():
    """The tiny fp32 configuration with slope 1/16: every biased score is exact in fp32
    (x B = score B / 2 - |i - j| / 2), so counts and the block mask match bit for bit."""
    w = synth.workload("C1")
    slopes = [0.0625]
    print(f"[case] C1 bias {slopes}", flush=True)
    inp = synth.make_inputs(w)
    ref = _oracle(inp, w, slopes)
    assert ref["xgap"].min() > 1e-6, "test construction: a score sits on the threshold"
    g = run_gpu(inp, w, slopes=slopes)
    np.testing.assert_array_equal(g["hist"].numpy(), ref["counts"])
    _check_prop1(g, ref, w.n_bins)
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < 1e-5
    np.testing.assert_array_equal(mask_bits(g["mask"].numpy()), ref["mask"].astype(np.int64))
    assert np.abs(g["o"].numpy() - ref["o"]).max() < 1e-4
    for name in ("dq", "dk", "dv"):
        err = rel_fro(g[name].numpy().astype(np.float64), ref[name])
        assert err < 1e-4, (name, err)


def test_zero_slopes_match_no_bias():
    """All-zero slopes take the bias kernels and must reproduce the unbiased run."""
    w = synth.Workload("t", 1, 4, 2, 256, 64, "bf16", 1.5, True, 64, 64, 16, "normal", seed=11)
    print("[case] zero slopes", flush=True)
    inp = synth.make_inputs(w)
    a = run_gpu(inp, w)
    z = run_gpu(inp, w, slopes=[0.0] * 4)
    for kk in ("o", "tau", "mask", "hist", "tau_h", "dq", "dk", "dv"):
        assert torch.equal(a[kk], z[kk]), kk


def test_fp32_random_causal_gqa():
    w = synth.Workload("t", 1, 4, 2, 128, 64, "f32", 1.5, True, 32, 32, 16, "tiny", seed=5)
    inp = synth.make_inputs(w)
    ref = _oracle(inp, w)
    g = run_gpu(inp, w)
    if ref["xgap"].min() > 1e-6:
        np.testing.assert_array_equal(g["hist"].numpy(), ref["counts"])
        np.testing.assert_array_equal(mask_bits(g["mask"].numpy()), ref["mask"].astype(np.int64))
    assert np.abs(g["tau"].numpy() - ref["tau"]).max() < 1e-5
    assert np.abs(g["o"].numpy() - ref["o"]).max() < 1e-4
    for name in ("dq", "dk", "dv"):
        assert rel_fro(g[name].numpy().astype(np.float64), ref[name]) < 1e-4, name


def test_determinism():
    """Two runs give bitwise identical outputs (no floating-point atomics)."""
    w = synth.Workload("t", 1, 4, 2, 256, 64, "bf16", 1.5, True, 64, 64, 16, "normal", seed=3)
    inp = synth.make_inputs(w)
    a = run_gpu(inp, w)
    b = run_gpu(inp, w)
    for kk in ("o", "tau", "mask", "aux", "hist", "tau_h", "dq", "dk", "dv"):
        assert torch.equal(a[kk], b[kk]), kk


@pytest.mark.parametrize("alpha", [1.5, 2.0, 3.0])
@pytest.mark.parametrize("causal", [True, False])
def test_all_equal_scores(alpha, causal):
    """q = 0 makes every score equal (every key in one histogram bin, every key in the
    support): p_ij = 1/n_i, so tau_i = -n_i^(1-alpha) and o_i is the mean of the valid v_j,
    with n_i = i + 1 under the causal mask and n otherwise."""
    w = synth.Workload("t", 1, 2, 1, 256, 64, "bf16", alpha, causal, 64, 64, 16, "normal", seed=13)
    print(f"[case] all-equal scores alpha {alpha} causal {causal}", flush=True)
    inp = synth.make_inputs(w)
    inp["q"] = torch.zeros_like(inp["q"])
    g = run_gpu(inp, w)
    n = w.seqlen
    ni = np.arange(1, n + 1, dtype=np.float64) if causal else np.full(n, float(n))
    tau_want = -ni ** (1.0 - alpha)
    v = to64(inp["v"])[0, 0]
    o_want = np.cumsum(v, axis=0) / ni[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
    for h in range(2):
        assert np.abs(g["tau"][0, h].numpy() - tau_want).max() < 1e-5
        assert np.abs(g["o"][0, h].numpy() - o_want).max() < 1e-2
    ref = _oracle(inp, w)
    for name in ("dq", "dk", "dv"):
        err = rel_fro(g[name].float().numpy().astype(np.float64), ref[name])
        assert err < 2e-2, (name, err)


def test_max_seqlen():
    """The longest supported sequence, 2^19 tokens (one head): the first and last query tiles
    against the oracle, and Proposition 1 on them."""
    n = 1 << 19
    w = synth.Workload("t", 1, 1, 1, n, 64, "bf16", 1.5, True, 64, 64, 16, "normal",
                       extra={"qk_scale": 1.0}, seed=19)
    print(f"[case] max seqlen {n}", flush=True)
    inp = synth.make_inputs(w, need_grad_inputs=False)
    d = torch.device("cuda:0")
    r = lce.fwd(inp["q"].to(d), inp["k"].to(d), inp["v"].to(d), w.alpha, True, (64, 64), 16,
                return_hist=True)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(inp["q"][0, 0]), to64(inp["k"][0, 0]), to64(inp["v"][0, 0])
    rows = np.concatenate([np.arange(0, 64), np.arange(n - 64, n)])
    ref = oracle.attn_fwd_head(q64, k64, v64, w.alpha, True, 16, 64, 1.0 / math.sqrt(64), rows=rows)
    tau = to64(r.tau[0, 0])[rows]
    assert np.abs(tau - ref["tau"]).max() < 1e-3
    assert np.abs(to64(r.o[0, 0])[rows] - ref["o"]).max() < 1e-2
    th = to64(r.tau_h[0, 0])[rows]
    assert np.all(th <= ref["tau"] + 1e-4) and np.all(th > ref["tau"] - 1.0 / 16 - 1e-4)


@pytest.mark.parametrize("n", [1 << 17, 65 * 1024])
def test_long_noncausal(n):
    """Long sequences without the causal mask (one head): every 32-row chunk walks all n/1024
    words of 32 sub-blocks in each refinement pass, screened 64 words at a time (2^17 keys:
    two whole groups; 65 * 1024: a whole group and a one-word group), and the backward walks
    whole mask rows and columns. Sampled query tiles against the oracle (tau, O, dQ, the
    histogram bound), and the gradient sums that hold at any size: the dK rows cancel and the
    dV rows add up to the sum of dO (each row of P sums to one)."""
    w = synth.Workload("t", 1, 1, 1, n, 64, "bf16", 1.5, False, 64, 64, 16, "normal",
                       extra={"qk_scale": 2.0}, seed=23)
    print(f"[case] long non-causal {n}", flush=True)
    inp = synth.make_inputs(w)
    d = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(d) for x in ("q", "k", "v", "do"))
    r = lce.fwd(q, k, v, w.alpha, False, (64, 64), 16, return_hist=True)
    dq, dk, dv = lce.bwd(q, k, v, do, r.tau, r.mask, r.aux, w.alpha, False, (64, 64), 16)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (to64(inp[x][0, 0]) for x in ("q", "k", "v", "do"))
    rows = np.concatenate([np.arange(0, 64), np.arange(n // 2, n // 2 + 64), np.arange(n - 64, n)])
    scale = 1.0 / math.sqrt(64)
    ref = oracle.attn_fwd_head(q64, k64, v64, w.alpha, False, 16, 64, scale, rows=rows)
    rb = oracle.attn_bwd_rows_head(q64, k64, v64, do64, ref["tau"], w.alpha, False, scale,
                                   rows=ref["rows"])
    rows = ref["rows"]
    assert np.abs(to64(r.tau[0, 0])[rows] - ref["tau"]).max() < 1e-3
    assert np.abs(to64(r.o[0, 0])[rows] - ref["o"]).max() < 1e-2
    assert rel_fro(to64(dq[0, 0])[rows], rb["dq"]) < 2e-2
    th = to64(r.tau_h[0, 0])[rows]
    assert np.all(th <= ref["tau"] + 1e-4) and np.all(th > ref["tau"] - 1.0 / 16 - 1e-4)
    dk_all, dv_all = to64(dk[0, 0]), to64(dv[0, 0])
    err_k = float((np.abs(dk_all.sum(axis=0)) / np.abs(dk_all).sum(axis=0)).max())
    sum_do = do64.sum(axis=0)
    err_v = float(np.abs(dv_all.sum(axis=0) - sum_do).max() / np.abs(sum_do).max())
    print(f"[case] long non-causal: sum dK {err_k:.2e}, sum dV vs sum dO {err_v:.2e}", flush=True)
    assert err_k <= 2.0 ** -6
    assert err_v <= 1e-2

"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks re-runs the oracle's own formula: each compares it with
an independent result -- a closed form from the literature (sorted sparsemax,
exact sort-based 1.5-entmax), brute-force support enumeration with a library
root finder, the strict bound of Proposition 1 (AdaSplash-2 pages, AdaSplash-2 (ja)
§2.1), hand-derived fixtures under tests/golden/, the softmax limit,
central finite differences and exact invariants of the gradient.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import brentq
from scipy.special import softmax

import oracle
import oracle.dash

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------------
# independent closed forms (written from the papers that define them, not from the oracle)
# ------------------------------------------------------------------------------------------------

def sparsemax_closed_form(z):
    """Sparsemax (alpha = 2) by sorting: Martins & Astudillo (2016), Algorithm 1."""
    z = np.asarray(z, dtype=np.float64)
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    k = np.arange(1, z.size + 1)
    ok = 1.0 + k * zs > cs
    kz = k[ok][-1]
    tau = (cs[kz - 1] - 1.0) / kz
    return np.maximum(z - tau, 0.0), tau


def entmax15_closed_form(z):
    """Exact 1.5-entmax by sorting: Peters, Niculae & Martins (2019), sort-based algorithm.

    On x = z/2 and a candidate support of the k largest entries, the threshold
    solves k tau^2 - 2 tau S1 + S2 - 1 = 0 (smaller root); the support is the k
    whose root lies between the k-th and (k+1)-th largest x.
    """
    x = np.asarray(z, dtype=np.float64) / 2.0
    xs = np.sort(x)[::-1]
    n = x.size
    for k in range(1, n + 1):
        top = xs[:k]
        mean = top.mean()
        ss = ((top - mean) ** 2).sum()
        disc = (1.0 - ss) / k
        if disc < 0:
            continue
        tau = mean - math.sqrt(disc)
        nxt = xs[k] if k < n else -np.inf
        if xs[k - 1] > tau >= nxt:
            return np.maximum(x - tau, 0.0) ** 2, tau
    raise AssertionError("no consistent support")


def brute_force_tau(x, alpha):
    """tau* by enumerating every support S and solving sum_S (x - tau)^kappa = 1 with brentq."""
    kappa = 1.0 / (alpha - 1.0)
    n = x.size
    found = []
    for r in range(1, n + 1):
        for S in itertools.combinations(range(n), r):
            xs = x[list(S)]
            lo_s, hi_s = xs.max() - 1.0, xs.min()
            if lo_s >= hi_s:          # tau* >= x_max - 1 would cut min_S x off
                continue
            lo_s -= 1e-9              # keep phi(lo) > 0 despite rounding of (x_max - lo)
            phi = lambda t: np.sum((xs - t) ** kappa) - 1.0
            if phi(hi_s) >= 0:        # the root would not lie below min_S x
                continue
            t = brentq(phi, lo_s, hi_s, xtol=1e-15, rtol=1e-15, maxiter=500)
            rest = np.delete(x, list(S))
            if rest.size == 0 or rest.max() <= t:
                found.append(t)
    assert len(found) == 1, found
    return found[0]


# ------------------------------------------------------------------------------------------------
# tau*, p
# ------------------------------------------------------------------------------------------------

def test_golden_entmax_values():
    with open(os.path.join(GOLDEN, "entmax_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p, tau = oracle.entmax(np.array(c["z"]), c["alpha"])
        assert abs(tau - c["tau"]) < 1e-11, c
        np.testing.assert_allclose(p, c["p"], atol=1e-11)


@pytest.mark.parametrize("n", [1, 2, 7, 256, 4096])
def test_sparsemax_closed_form(n):
    rng = np.random.default_rng(n)
    for scale in (0.1, 1.0, 5.0):
        for _ in range(5):
            z = rng.standard_normal(n) * scale
            p_ref, t_ref = sparsemax_closed_form(z)
            p, t = oracle.entmax(z, 2.0)
            assert abs(t - t_ref) < 1e-11
            np.testing.assert_array_equal(p > 0, p_ref > 0)
            np.testing.assert_allclose(p, p_ref, atol=1e-11)


@pytest.mark.parametrize("n", [1, 2, 7, 256, 4096])
def test_entmax15_closed_form(n):
    rng = np.random.default_rng(100 + n)
    for scale in (0.1, 1.0, 5.0):
        for _ in range(5):
            z = rng.standard_normal(n) * scale
            p_ref, t_ref = entmax15_closed_form(z)
            p, t = oracle.entmax(z, 1.5)
            assert abs(t - t_ref) < 1e-11
            np.testing.assert_array_equal(p > 0, p_ref > 0)
            np.testing.assert_allclose(p, p_ref, atol=1e-11)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0, 8.0, 16.0])
def test_brute_force_supports(alpha):
    rng = np.random.default_rng(int(alpha * 100))
    for n in range(1, 9):
        for _ in range(6):
            x = rng.standard_normal(n) * rng.choice([0.2, 1.0, 3.0])
            t_ref = brute_force_tau(x, alpha)
            t = oracle.entmax_tau(x, alpha)
            assert abs(t - t_ref) < 1e-10, (alpha, x)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0, 8.0, 16.0])
def test_distribution_properties(alpha):
    """Rows sum to one with exact zeros; shift and permutation behave as the definition says."""
    rng = np.random.default_rng(7)
    for n in (1, 5, 300):
        z = rng.standard_normal(n) * 2.0
        p, t = oracle.entmax(z, alpha)
        assert abs(p.sum() - 1.0) < 1e-9
        x = (alpha - 1.0) * z
        assert np.all(p[x <= t] == 0.0) and np.all(p[x > t] > 0.0)
        c = 0.7
        p2, t2 = oracle.entmax(z + c, alpha)
        assert abs(t2 - (t + (alpha - 1.0) * c)) < 1e-9
        np.testing.assert_allclose(p2, p, atol=1e-9)
        perm = rng.permutation(n)
        p3, t3 = oracle.entmax(z[perm], alpha)
        assert abs(t3 - t) < 1e-11
        np.testing.assert_allclose(p3, p[perm], atol=1e-11)
        # tau* lies in the bracket [x_max - 1, x_max - n^(1 - alpha)]
        assert x.max() - 1.0 - 1e-12 <= t <= x.max() - n ** (1.0 - alpha) + 1e-12


def test_softmax_limit():
    """As alpha -> 1, alpha-entmax approaches softmax at first order in alpha - 1."""
    rng = np.random.default_rng(3)
    errs = []
    for am1 in (1e-1, 1e-2, 1e-3):
        e = 0.0
        for _ in range(8):
            z = rng.standard_normal(256)
            p, _ = oracle.entmax(z, 1.0 + am1)
            e = max(e, np.abs(p - softmax(z)).max())
        errs.append(e)
    assert errs[0] > errs[1] > errs[2]
    assert errs[1] < 0.25 * errs[0] and errs[2] < 0.25 * errs[1]
    assert errs[2] < 5e-3


# ------------------------------------------------------------------------------------------------
# histogram and Proposition 1
# ------------------------------------------------------------------------------------------------

def test_golden_histograms():
    with open(os.path.join(GOLDEN, "histogram_anchored.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        counts, T = oracle.histogram(np.array(c["x"]), c["B"])
        assert T == c["T"], c
        expect = np.zeros(c["B"], dtype=np.int32)
        for k, v in c["nonzero"].items():
            expect[int(k)] = v
        np.testing.assert_array_equal(counts, expect)
        if "tau_h" in c:
            th = oracle.tau_from_hist(counts, T, c["B"], c["alpha"])
            assert abs(th - c["tau_h"]) < 1e-11
            ts = oracle.entmax_tau(np.array(c["x"]), c["alpha"])
            assert abs(ts - c["tau_star"]) < 1e-11


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
@pytest.mark.parametrize("B", [8, 16])
def test_proposition1_strict(alpha, B):
    """tau* - h < tau_h <= tau*, h = 1/B, on random rows of many sizes and spreads."""
    rng = np.random.default_rng(int(alpha * 1000) + B)
    h = 1.0 / B
    for n in (1, 2, 7, 256, 4096):
        for spread in (0.3, 1.0, 3.0, 10.0):
            for _ in range(6 if n < 4096 else 2):
                x = rng.standard_normal(n) * spread * (alpha - 1.0) + rng.uniform(-5, 5)
                counts, T = oracle.histogram(x, B)
                assert counts[B - 1] >= 1
                th = oracle.tau_from_hist(counts, T, B, alpha)
                ts = oracle.entmax_tau(x, alpha)
                assert th <= ts + 1e-11
                assert ts - th < h


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_proposition1_is_strict_for_a_dominant_score(alpha):
    """One dominant score half a bin above a grid line: the gap is h/2, not h.

    A window anchored at x_max itself (bins relative to the row maximum) would
    put x_max on the top bin's lower edge plus h and give tau* - tau_h = h
    exactly; the anchored grid must not.
    """
    B = 16
    h = 1.0 / B
    for base in (-3, 0, 2, 7):
        xmax = (base * B + 0.5) / B
        x = np.array([xmax, xmax - 5.0, xmax - 9.0])
        counts, T = oracle.histogram(x, B)
        th = oracle.tau_from_hist(counts, T, B, alpha)
        ts = oracle.entmax_tau(x, alpha)
        assert abs(ts - (xmax - 1.0)) < 1e-11
        assert abs((ts - th) - 0.5 * h) < 1e-10


def test_histogram_shift_by_grid_steps():
    """Shifting a row by m grid steps shifts T by m and leaves the counts unchanged."""
    rng = np.random.default_rng(11)
    for B in (8, 16):
        x = np.round(rng.standard_normal(500) * 64) / 64.0
        c0, T0 = oracle.histogram(x, B)
        for m in (-7, 3, 40):
            c1, T1 = oracle.histogram(x + m / B, B)
            assert T1 == T0 + m
            np.testing.assert_array_equal(c1, c0)


def test_support_within_histogram_window():
    """The support at tau_h contains the true support (AdaSplash-2 (es) §2A)."""
    rng = np.random.default_rng(5)
    for alpha in (1.5, 2.0):
        for _ in range(20):
            x = rng.standard_normal(1000) * 2.0 * (alpha - 1.0)
            counts, T = oracle.histogram(x, 16)
            th = oracle.tau_from_hist(counts, T, 16, alpha)
            ts = oracle.entmax_tau(x, alpha)
            assert np.all((x > ts) <= (x > th))


# ------------------------------------------------------------------------------------------------
# attention forward
# ------------------------------------------------------------------------------------------------

def _rand_problem(rng, n, d, scale=1.0):
    q = rng.standard_normal((n, d)) * scale
    k = rng.standard_normal((n, d)) * scale
    v = rng.standard_normal((n, d))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_attention_forward_closed_forms(causal):
    rng = np.random.default_rng(21)
    n, d = 96, 16
    q, k, v = _rand_problem(rng, n, d, 1.5)
    scale = 1.0 / math.sqrt(d)
    for alpha, ref in ((2.0, sparsemax_closed_form), (1.5, entmax15_closed_form)):
        f = oracle.attn_fwd_head(q, k, v, alpha, causal, 16, 32, scale)
        for i in range(n):
            nv = i + 1 if causal else n
            s = scale * (q[i] @ k[:nv].T)
            p, t = ref(s)
            assert abs(f["tau"][i] - t) < 1e-10
            np.testing.assert_allclose(f["o"][i], p @ v[:nv], atol=1e-10)
            assert abs(f["psum"][i] - 1.0) < 1e-9
            bits = np.zeros(f["rowbits"].shape[1], dtype=np.uint32)
            for j in np.nonzero(p > 0)[0]:
                J = j // 32
                bits[J // 32] |= np.uint32(1) << np.uint32(J % 32)
            np.testing.assert_array_equal(f["rowbits"][i], bits)


def test_causal_first_row_and_mask_shape():
    rng = np.random.default_rng(2)
    n, d = 128, 8
    q, k, v = _rand_problem(rng, n, d)
    scale = 1.0 / math.sqrt(d)
    for alpha in (1.5, 2.0, 3.0):
        f = oracle.attn_fwd_head(q, k, v, alpha, True, 16, 32, scale)
        np.testing.assert_allclose(f["o"][0], v[0], atol=1e-12)
        x00 = (alpha - 1.0) * scale * (q[0] @ k[0])
        assert abs(f["tau"][0] - (x00 - 1.0)) < 1e-11
        m = oracle.block_mask(f["rowbits"], 32)
        for I in range(m.shape[0]):
            assert m[I, 0] != 0                       # every row has a non-zero weight
            assert m[I, 0] >> np.uint32(I + 1) == 0   # nothing above the causal diagonal


# ------------------------------------------------------------------------------------------------
# attention backward
# ------------------------------------------------------------------------------------------------

def _loss(q, k, v, do, alpha, causal, scale):
    f = oracle.attn_fwd_head(q, k, v, alpha, causal, 16, 32, scale, threads=1)
    return float((f["o"] * do).sum()), f


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_finite_differences(alpha, causal):
    """Analytic backward vs central differences of L = sum(O * dO) in fp64."""
    n, d = 10, 4
    scale = 1.0 / math.sqrt(d)
    seed = 0
    while True:
        rng = np.random.default_rng(1000 * seed + int(alpha * 10) + causal)
        q, k, v = _rand_problem(rng, n, d, 1.2)
        do = rng.standard_normal((n, d))
        L0, f = _loss(q, k, v, do, alpha, causal, scale)
        if f["xgap"].min() > 1e-3 and seed < 50:
            break
        seed += 1
    r = oracle.attn_bwd_rows_head(q, k, v, do, f["tau"], alpha, causal, scale, threads=1)
    kk = oracle.attn_bwd_keys_group(q[None], k, v, do[None], f["tau"][None], r["delta"][None],
                                    alpha, causal, scale, threads=1)
    eps = 1e-5
    for name, arr, grad in (("q", q, r["dq"]), ("k", k, kk["dk"]), ("v", v, kk["dv"])):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            args1 = {"q": q, "k": k, "v": v}
            args2 = {"q": q, "k": k, "v": v}
            args1[name], args2[name] = a1, a2
            L1, _ = _loss(args1["q"], args1["k"], args1["v"], do, alpha, causal, scale)
            L2, _ = _loss(args2["q"], args2["k"], args2["v"], do, alpha, causal, scale)
            num[idx] = (L1 - L2) / (2 * eps)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(num), 1e-12)
        assert err < 1e-5, (name, err)


def test_gradient_invariants_gqa():
    """sum_j dK_j = 0 (rows of dS sum to zero) and sum_j dV_j = sum_i dO_i over the group."""
    rng = np.random.default_rng(9)
    b, hq, hkv, n, d = 1, 4, 2, 64, 8
    q = rng.standard_normal((b, hq, n, d)) * 1.5
    k = rng.standard_normal((b, hkv, n, d)) * 1.5
    v = rng.standard_normal((b, hkv, n, d))
    do = rng.standard_normal((b, hq, n, d))
    for alpha in (1.5, 2.0):
        res = oracle.attn_full(q, k, v, do, alpha, True, 16, 32, 32, threads=4)
        G = hq // hkv
        for kh in range(hkv):
            np.testing.assert_allclose(res["dk"][0, kh].sum(0), 0.0, atol=1e-9)
            np.testing.assert_allclose(res["dv"][0, kh].sum(0),
                                       do[0, kh * G:(kh + 1) * G].sum((0, 1)), atol=1e-9)


def test_sparsemax_backward_projection_form():
    """At alpha = 2 the Jacobian is a projection: dS = 1_S (dP - mean_S dP)."""
    rng = np.random.default_rng(4)
    n, d = 80, 8
    q, k, v = _rand_problem(rng, n, d, 2.0)
    do = rng.standard_normal((n, d))
    scale = 1.0 / math.sqrt(d)
    f = oracle.attn_fwd_head(q, k, v, 2.0, True, 16, 32, scale)
    r = oracle.attn_bwd_rows_head(q, k, v, do, f["tau"], 2.0, True, scale)
    for i in range(n):
        s = scale * (q[i] @ k[:i + 1].T)
        p, _ = sparsemax_closed_form(s)
        S = p > 0
        dp = do[i] @ v[:i + 1].T
        ds = np.where(S, dp - dp[S].mean(), 0.0)
        np.testing.assert_allclose(r["dq"][i], scale * ds @ k[:i + 1], atol=1e-10)


def test_backward_softmax_limit():
    """As alpha -> 1 the entmax backward approaches the softmax-attention backward."""
    rng = np.random.default_rng(8)
    n, d = 48, 8
    q, k, v = _rand_problem(rng, n, d)
    do = rng.standard_normal((n, d))
    scale = 1.0 / math.sqrt(d)
    S = scale * q @ k.T
    P = softmax(S, axis=1)
    dP = do @ v.T
    dS = P * (dP - (P * dP).sum(1, keepdims=True))
    dq_soft = scale * dS @ k
    errs = []
    for am1 in (1e-1, 1e-2, 1e-3):
        alpha = 1.0 + am1
        f = oracle.attn_fwd_head(q, k, v, alpha, False, 16, 32, scale)
        r = oracle.attn_bwd_rows_head(q, k, v, do, f["tau"], alpha, False, scale)
        errs.append(np.abs(r["dq"] - dq_soft).max())
    assert errs[1] < 0.25 * errs[0] and errs[2] < 0.25 * errs[1]


# ------------------------------------------------------------------------------------------------
# position bias (NAPE heads: half without position encoding, half ALiBi; AdaSplash-2 (it) §4)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_position_bias_hand_derived(causal):
    """q = 0 leaves only the bias: x_ij = -m |i - j| at alpha = 2 (sparsemax).

    Derived by hand for m = 0.05. Causal row i >= 5: the support is the k nearest keys
    with k (k - 1) < 2/m = 40, so k = 6 and tau = -(1 + m k (k - 1)/2)/k = -1.75/6,
    p_ij = 0.29167, 0.24167, ..., 0.04167 for i - j = 0..5. Full (non-causal) interior
    row: the support |i - j| <= 4 gives tau = -(1 + m r (r - 1))/(2r - 1) = -2/9 with r = 5,
    and the excluded keys at distance 5 have x = -0.25 <= tau.
    """
    n, m = 32, 0.05
    q = np.zeros((n, n))
    k = np.ones((n, n))
    v = np.eye(n)                      # o_i is the weight row p_i
    f = oracle.attn_fwd_head(q, k, v, 2.0, causal, 16, 32, 1.0, slope=m)
    if causal:
        rows, tau = range(5, n), -1.75 / 6
    else:
        rows, tau = range(4, n - 4), -2.0 / 9.0
    for i in rows:
        assert abs(f["tau"][i] - tau) < 1e-12
        dist = np.abs(i - np.arange(n))
        want = np.maximum(-m * dist - tau, 0.0)
        if causal:
            want[i + 1:] = 0.0
        np.testing.assert_allclose(f["o"][i], want, atol=1e-12)
    if causal:
        np.testing.assert_allclose(f["o"][10][5:11], [0.25 / 6 + 0.05 * t for t in range(6)], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_position_bias_closed_forms(causal):
    """Random q, k with a slope: the sort-based closed forms on the biased scores."""
    rng = np.random.default_rng(33)
    n, d = 80, 16
    q, k, v = _rand_problem(rng, n, d, 1.5)
    scale = 1.0 / math.sqrt(d)
    for alpha, ref, m in ((2.0, sparsemax_closed_form, 0.07), (1.5, entmax15_closed_form, 0.3)):
        f = oracle.attn_fwd_head(q, k, v, alpha, causal, 16, 32, scale, slope=m)
        f0 = oracle.attn_fwd_head(q, k, v, alpha, causal, 16, 32, scale)
        for i in range(n):
            nv = i + 1 if causal else n
            s = scale * (q[i] @ k[:nv].T) - m * np.abs(i - np.arange(nv))
            p, t = ref(s)
            assert abs(f["tau"][i] - t) < 1e-10
            np.testing.assert_allclose(f["o"][i], p @ v[:nv], atol=1e-10)
        # the bias moves the weight towards the diagonal
        assert np.mean(f["xgap"]) != np.mean(f0["xgap"])


def _loss_bias(q, k, v, do, alpha, causal, scale, m):
    f = oracle.attn_fwd_head(q, k, v, alpha, causal, 16, 32, scale, threads=1, slope=m)
    return float((f["o"] * do).sum()), f


@pytest.mark.parametrize("alpha", [1.5, 2.0, 3.0])
@pytest.mark.parametrize("causal", [False, True])
def test_position_bias_gradients_finite_differences(alpha, causal):
    """Analytic backward with a slope vs central differences of L = sum(O * dO)."""
    n, d, m = 10, 4, 0.35
    scale = 1.0 / math.sqrt(d)
    seed = 0
    while True:
        rng = np.random.default_rng(2000 * seed + int(alpha * 10) + causal)
        q, k, v = _rand_problem(rng, n, d, 1.2)
        do = rng.standard_normal((n, d))
        L0, f = _loss_bias(q, k, v, do, alpha, causal, scale, m)
        if f["xgap"].min() > 1e-3 and seed < 50:
            break
        seed += 1
    r = oracle.attn_bwd_rows_head(q, k, v, do, f["tau"], alpha, causal, scale, threads=1, slope=m)
    kk = oracle.attn_bwd_keys_group(q[None], k, v, do[None], f["tau"][None], r["delta"][None],
                                    alpha, causal, scale, threads=1, slopes=[m])
    eps = 1e-5
    for name, arr, grad in (("q", q, r["dq"]), ("k", k, kk["dk"]), ("v", v, kk["dv"])):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            args1 = {"q": q, "k": k, "v": v}
            args2 = {"q": q, "k": k, "v": v}
            args1[name], args2[name] = a1, a2
            L1, _ = _loss_bias(args1["q"], args1["k"], args1["v"], do, alpha, causal, scale, m)
            L2, _ = _loss_bias(args2["q"], args2["k"], args2["v"], do, alpha, causal, scale, m)
            num[idx] = (L1 - L2) / (2 * eps)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(num), 1e-12)
        assert err < 1e-5, (name, err)


def test_position_bias_gqa_heads_sum():
    """A KV head's dK/dV with per-head slopes is the sum of its heads' single-head results."""
    rng = np.random.default_rng(12)
    b, hq, hkv, n, d = 1, 4, 2, 48, 8
    q = rng.standard_normal((b, hq, n, d)) * 1.5
    k = rng.standard_normal((b, hkv, n, d)) * 1.5
    v = rng.standard_normal((b, hkv, n, d))
    do = rng.standard_normal((b, hq, n, d))
    slopes = np.array([0.0, 0.25, 0.0, 0.0625])
    res = oracle.attn_full(q, k, v, do, 1.5, True, 16, 32, 32, threads=4, slopes=slopes)
    G = hq // hkv
    scale = 1.0 / math.sqrt(d)
    for kh in range(hkv):
        dk = np.zeros((n, d))
        dv = np.zeros((n, d))
        for g in range(G):
            h = kh * G + g
            one = oracle.attn_bwd_keys_group(q[0, h][None], k[0, kh], v[0, kh], do[0, h][None],
                                             res["tau"][0, h][None], res["delta"][0, h][None],
                                             1.5, True, scale, slopes=[slopes[h]])
            dk += one["dk"]
            dv += one["dv"]
        np.testing.assert_allclose(res["dk"][0, kh], dk, atol=1e-12)
        np.testing.assert_allclose(res["dv"][0, kh], dv, atol=1e-12)
        np.testing.assert_allclose(res["dk"][0, kh].sum(0), 0.0, atol=1e-9)


# ------------------------------------------------------------------------------------------------
# decode (one new query row against a cache)
# ------------------------------------------------------------------------------------------------

def test_decode_single_key_and_hand_derived_row():
    """A one-key cache gives tau = x_0 - 1 and o = v_0; with q = 0 and slope m = 0.05 the
    decode row is the hand-derived causal sparsemax row (support: the 6 newest keys,
    tau = -1.75/6; the key at distance t gets 0.29167 - 0.05 t)."""
    rng = np.random.default_rng(5)
    d = 8
    q = rng.standard_normal((1, 2, d))
    kc = rng.standard_normal((1, 1, 40, d))
    vc = rng.standard_normal((1, 1, 40, d))
    r = oracle.attn_decode(q, kc, vc, [1], 1.5, 16, scale=0.5)
    for h in range(2):
        x0 = 0.5 * 0.5 * (q[0, h] @ kc[0, 0, 0])
        assert abs(r["tau"][0, h] - (x0 - 1.0)) < 1e-12
        np.testing.assert_allclose(r["o"][0, h], vc[0, 0, 0], atol=1e-12)
    n = 24
    q0 = np.zeros((1, 1, n))
    kc = np.ones((1, 1, n, n))
    vc = np.eye(n)[None, None]
    r = oracle.attn_decode(q0, kc, vc, [20], 2.0, 16, scale=1.0, slopes=[0.05])
    assert abs(r["tau"][0, 0] - (-1.75 / 6)) < 1e-12
    want = np.zeros(n)
    for t in range(6):
        want[19 - t] = 1.75 / 6 - 0.05 * t
    np.testing.assert_allclose(r["o"][0, 0], want, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# DashAttention stages 1-2 (DashAttention (it), stages 1 and 2)
# ------------------------------------------------------------------------------------------------

def _dash_inputs(b, hq, hkv, n, d, nc, seed, ks_zero):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, hq, n, d))
    k = rng.standard_normal((b, hkv, n, d))
    v = rng.standard_normal((b, hkv, n, d))
    ks = np.zeros((b, hkv, nc, d)) if ks_zero else rng.standard_normal((b, hkv, nc, d))
    return q, k, v, ks


@pytest.mark.parametrize("sigma", [0.0, 1.0, 2.5])
def test_dash_uniform_routing_is_biased_causal_softmax(sigma):
    """All summaries equal (zero): every routing row is uniform over its m_i earlier chunks
    (wbar = 1/m_i, so every earlier chunk is routed) and stage 2 is causal softmax attention
    with -sigma ln m_i added on the earlier chunks -- checked against torch's
    scaled_dot_product_attention in fp64 with that additive mask."""
    import torch
    b, hq, hkv, n, d, C = 1, 4, 2, 96, 16, 8
    q, k, v, ks = _dash_inputs(b, hq, hkv, n, d, n // C, 3, True)
    r = oracle.dash.dash_fwd(q, k, v, ks, 1.5, 1.0, sigma, C)
    i = np.arange(n)
    m = i // C
    for row in range(n):
        want = np.zeros(n // C)
        want[:m[row]] = 1.0 / max(m[row], 1) if m[row] else 0.0
        np.testing.assert_allclose(r["wbar"][0, :, row], np.broadcast_to(want, (hkv, n // C)), atol=1e-12)
    bias = np.full((n, n), -np.inf)
    for row in range(n):
        bias[row, :m[row] * C] = -sigma * np.log(max(m[row], 1))
        bias[row, m[row] * C:row + 1] = 0.0
    G = hq // hkv
    kk = torch.from_numpy(np.repeat(k, G, axis=1))
    vv = torch.from_numpy(np.repeat(v, G, axis=1))
    o = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kk, vv,
                                                         attn_mask=torch.from_numpy(bias))
    np.testing.assert_allclose(r["o"], o.numpy(), atol=1e-12)
    # lse: the log of the softmax denominator, from the same additive mask
    s = np.einsum("bhid,bhjd->bhij", q, np.repeat(k, G, axis=1)) / math.sqrt(d) + bias
    np.testing.assert_allclose(r["lse"], np.log(np.exp(s).sum(-1)), atol=1e-12)


def test_dash_sigma0_all_routed_is_causal_softmax():
    """sigma = 0 with every earlier chunk routed: plain causal softmax attention."""
    import torch
    b, hq, hkv, n, d, C = 2, 2, 1, 64, 8, 16
    q, k, v, ks = _dash_inputs(b, hq, hkv, n, d, n // C, 4, True)
    r = oracle.dash.dash_fwd(q, k, v, ks, 2.0, 1.0, 0.0, C)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, 2, axis=1)),
        torch.from_numpy(np.repeat(v, 2, axis=1)), is_causal=True)
    np.testing.assert_allclose(r["o"], o.numpy(), atol=1e-12)


def test_dash_hand_derived_sparsemax_routing():
    """alpha = 2 routing of row 3 with C = 1 against summaries whose logits are (1.5, 1, -5)
    for head 0 and (-5, 1, 1.5) for head 1: by hand, sparsemax gives (0.75, 0.25, 0) and
    (0, 0.25, 0.75) with tau 0.75; the group average is (0.375, 0.25, 0.375), its support
    the union of the two."""
    d = 2
    q = np.zeros((2, 4, d))
    q[0, 3] = [1.0, 0.0]
    q[1, 3] = [0.0, 1.0]
    ks = np.array([[1.5, -5.0], [1.0, 1.0], [-5.0, 1.5], [0.0, 0.0]])
    r = oracle.dash.route_group(q, ks, 2.0, 1.0, 1.0, 1, [3])
    np.testing.assert_allclose(r["what"][0, 0, :3], [0.75, 0.25, 0.0], atol=1e-12)
    np.testing.assert_allclose(r["what"][1, 0, :3], [0.0, 0.25, 0.75], atol=1e-12)
    np.testing.assert_allclose(r["tau"][:, 0], [0.75, 0.75], atol=1e-12)
    np.testing.assert_allclose(r["wbar"][0, :3], [0.375, 0.25, 0.375], atol=1e-12)
    # gamma scales the logits: gamma = 2 doubles them, sparsemax of (3, 2, -10) is (1, 0, 0)
    r2 = oracle.dash.route_group(q, ks, 2.0, 2.0, 1.0, 1, [3])
    np.testing.assert_allclose(r2["what"][0, 0, :3], [1.0, 0.0, 0.0], atol=1e-12)


def test_dash_routing_invariants_and_mask_brute_force():
    """Random summaries at alpha 1.5: each head's routing row sums to 1 over its m_i chunks,
    wbar is their mean (support = union), the first chunk's rows route nothing; the chunk
    mask equals a brute-force OR over each 64-row tile; stage 2 attends the diagonal keys
    plus C keys per routed chunk, and its weights sum to 1 (o of v = 1 is 1)."""
    b, hq, hkv, n, d, C = 1, 4, 2, 256, 16, 16
    q, k, v, ks = _dash_inputs(b, hq, hkv, n, d, n // C, 5, False)
    q *= 3.0
    r = oracle.dash.dash_fwd(q, k, v, ks, 1.5, 1.0, 1.0, C)
    G = hq // hkv
    for g in range(hkv):
        rt = oracle.dash.route_group(q[0, g * G:(g + 1) * G], ks[0, g], 1.5, 1.0, 1.0 / math.sqrt(d), C,
                                     np.arange(n))
        m = np.arange(n) // C
        sums = rt["what"].sum(-1)
        np.testing.assert_allclose(sums[:, m > 0], 1.0, atol=1e-12)
        assert np.all(sums[:, m == 0] == 0.0)
        np.testing.assert_array_equal(rt["wbar"] > 0, (rt["what"] > 0).any(0))
        assert np.all(rt["wbar"][np.arange(n)[:, None] // C <= np.arange(n // C)[None, :]] == 0.0)
        assert (rt["wbar"][m > 2] == 0).any(), "test construction: routing should be sparse"
        # brute-force tile mask
        want = np.zeros_like(r["mask"][0, g])
        for i in range(n):
            for c in range(n // C):
                if rt["wbar"][i, c] > 0:
                    want[i // 64, c // 32] |= 1 << (c % 32)
        np.testing.assert_array_equal(r["mask"][0, g], want)
        nk = (np.arange(n) % C + 1) + C * (rt["wbar"] > 0).sum(-1)
        np.testing.assert_array_equal(r["nkeys"][0, g], nk)
    ones = np.ones_like(v)
    r1 = oracle.dash.dash_fwd(q, k, ones, ks, 1.5, 1.0, 1.0, C)
    np.testing.assert_allclose(r1["o"], 1.0, atol=1e-12)


def _dash_loss(q, k, v, ks, do, alpha, gamma, sigma, C):
    return float((oracle.dash.dash_fwd(q, k, v, ks, alpha, gamma, sigma, C)["o"] * do).sum())


@pytest.mark.parametrize("alpha,G", [(1.5, 2), (2.0, 1), (1.25, 3)])
def test_dash_backward_finite_differences(alpha, G):
    """dash_bwd against central differences of sum(o * dO) in sampled coordinates of q, k, v
    and the chunk summaries (eps 1e-4 in fp64: the oracle's bisection leaves tau within
    1e-12, so a smaller step would measure that noise; a coordinate whose perturbation moved
    a routing support boundary would show as a kink, none does at these seeds)."""
    b, hkv, n, d, C = 1, 1, 80, 8, 16
    hq = G * hkv
    q, k, v, ks = _dash_inputs(b, hq, hkv, n, d, n // C, 11 + G, False)
    do = np.random.default_rng(5).standard_normal(q.shape)
    gamma, sigma = 2.0, 1.5
    gr = oracle.dash.dash_bwd(q, k, v, ks, do, alpha, gamma, sigma, C)
    rng = np.random.default_rng(7)
    eps = 1e-4
    for name, arr in (("dq", q), ("dk", k), ("dv", v), ("dks", ks)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp = _dash_loss(q, k, v, ks, do, alpha, gamma, sigma, C)
            arr[idx] = old - eps
            lm = _dash_loss(q, k, v, ks, do, alpha, gamma, sigma, C)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gr[name][idx]) < 1e-6 * max(1.0, abs(fd)) + 2e-7, (name, idx, fd, gr[name][idx])
    # the summaries get gradient through the routing alone: some must be non-zero here
    assert np.abs(gr["dks"]).max() > 1e-3


def test_dash_backward_sigma0_and_fixed_prior_against_autograd():
    """With the prior treated as a fixed additive mask, stage 2 is masked softmax attention:
    torch autograd in fp64 through scaled_dot_product_attention gives dk and dv exactly as
    dash_bwd (the routing does not reach k and v), and at sigma = 0 (no prior: the routing
    only selects chunks) also dq, with a summary gradient of exactly 0."""
    import torch
    b, hq, hkv, n, d, C = 1, 4, 2, 96, 8, 16
    q, k, v, ks = _dash_inputs(b, hq, hkv, n, d, n // C, 21, False)
    do = np.random.default_rng(9).standard_normal(q.shape)
    G = hq // hkv
    for sigma in (0.0, 1.0):
        f = oracle.dash.dash_fwd(q, k, v, ks, 1.5, 3.0, sigma, C)
        gr = oracle.dash.dash_bwd(q, k, v, ks, do, 1.5, 3.0, sigma, C)
        bias = np.full((b, hq, n, n), -np.inf)
        for g in range(hkv):
            for i in range(n):
                m = i // C
                for c in range(m):
                    w = f["wbar"][0, g, i, c]
                    if w > 0:
                        bias[0, g * G:(g + 1) * G, i, c * C:(c + 1) * C] = sigma * np.log(w)
                bias[0, g * G:(g + 1) * G, i, m * C:i + 1] = 0.0
        qt = torch.from_numpy(q).requires_grad_()
        kt = torch.from_numpy(k).requires_grad_()
        vt = torch.from_numpy(v).requires_grad_()
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1),
            attn_mask=torch.from_numpy(bias))
        (o * torch.from_numpy(do)).sum().backward()
        np.testing.assert_allclose(o.detach().numpy(), f["o"], atol=1e-12)
        np.testing.assert_allclose(gr["dk"], kt.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(gr["dv"], vt.grad.numpy(), atol=1e-10)
        if sigma == 0.0:
            np.testing.assert_allclose(gr["dq"], qt.grad.numpy(), atol=1e-10)
            assert np.abs(gr["dks"]).max() == 0.0
        else:
            assert np.abs(gr["dq"] - qt.grad.numpy()).max() > 1e-6   # the routing's share

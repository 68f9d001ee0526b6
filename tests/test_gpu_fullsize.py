"""Parity at the full workload sizes (4K to 128K tokens), in the launch configuration the
benchmark times (same entry points, default solver settings, library-sized workspaces).

The fp64 oracle cannot run whole problems of this size, so it checks what it can compute
one by one, on the same seeded inputs:

* whole query tiles (first, last and two seeded ones per sampled head): tau, the output,
  dQ, the histogram lower bound of tau and the tile's row of the block mask;
* dK and dV of sampled keys with dO kept on a sampled row set and zeroed elsewhere, so
  that only those rows contribute and the oracle needs their tau and delta only;
* properties that hold at any size: per KV head the dK rows sum to zero (each row of dS
  sums to zero) and the dV rows sum to the sum of dO over the group's query rows (each
  row of P sums to one).

Tolerances: max|d tau| <= 1e-3, max|d O| <= 1e-2, relative Frobenius <= 2e-2 for
gradients (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import long_context_entmax_amd as lce
from tests.gpu_helpers import dev, rel_fro, to64

pytestmark = pytest.mark.gpu

# every configured point of the 4K-128K study: (workload, alpha, target block sparsity)
POINTS = [("C2", 1.5, 0.0), ("C2", 1.5, 0.6), ("C2", 1.5, 0.9),
          ("C2", 2.0, 0.0), ("C2", 2.0, 0.6), ("C2", 2.0, 0.9),
          ("C3", 1.5, 0.6), ("C3", 1.5, 0.8), ("C3", 1.5, 0.95),
          ("C4", 2.0, 0.95), ("C5", 1.5, 0.97)]
TAU_TOL, O_TOL, G_TOL = 1e-3, 1e-2, 2e-2


def _pid(pt):
    return f"{pt[0]}-a{pt[1]:g}-s{pt[2]:g}"


def _sample_tiles(w, rng):
    Tr = w.seqlen // w.block_q
    picks = {0, Tr - 1}
    while len(picks) < 4:
        picks.add(int(rng.integers(1, Tr - 1)))
    return sorted(picks)


def _bits_of_tile(row_bits: np.ndarray) -> np.ndarray:
    return np.bitwise_or.reduce(row_bits, axis=0)


def _run(cfg, slopes=None, alpha=None, sparsity=None):
    w = synth.workload(cfg, alpha=alpha, sparsity=sparsity)
    d = dev()
    inp = synth.make_inputs(w, device=d)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    blk = (w.block_q, w.block_k)
    print(f"[fullsize] {cfg}: b{w.batch} hq{w.heads_q} hkv{w.heads_kv} n{w.seqlen} d{w.head_dim} "
          f"alpha {w.alpha} blocks {blk} B {w.n_bins} target sparsity {w.target_sparsity} beta {w.beta:.4g}",
          flush=True)
    desc = lce._desc_for(q, k, w.alpha, w.causal, blk, w.n_bins, None, 0, 0.0)
    fws, bws = lce.workspace_bytes(desc)
    wsf = torch.empty(max(fws, 256), dtype=torch.uint8, device=d)
    wsb = torch.empty(max(bws, 256), dtype=torch.uint8, device=d)
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device=d)
    r = lce.fwd(q, k, v, w.alpha, w.causal, blk, w.n_bins, workspace=wsf, return_hist=True, slopes=sl)
    dq, dk, dv = lce.bwd(q, k, v, do, r.tau, r.mask, r.aux, w.alpha, w.causal, blk, w.n_bins,
                         workspace=wsb, slopes=sl)
    torch.cuda.synchronize()
    return w, inp, r, (dq, dk, dv)


@pytest.fixture(scope="module", params=POINTS, ids=_pid)
def point(request):
    """One full-size run per configured point, shared by that point's tests (pytest groups
    the tests of a module-scoped parameter, so one run is held at a time)."""
    cfg, alpha, sparsity = request.param
    res = _run(cfg, alpha=alpha, sparsity=sparsity)
    yield request.param, res
    del res
    torch.cuda.empty_cache()


def test_fullsize_sampled_tiles(point):
    (cfg, _, _), (w, inp, r, (dq, dk, dv)) = point
    rng = np.random.default_rng(20260)
    G = w.heads_q // w.heads_kv
    scale = 1.0 / math.sqrt(w.head_dim)
    n, Br, Bc, B = w.seqlen, w.block_q, w.block_k, w.n_bins
    heads = sorted({0, w.heads_q - 1, int(rng.integers(0, w.heads_q))})
    bi = w.batch - 1
    worst = {"tau": 0.0, "o": 0.0, "dq": 0.0}
    for h in heads:
        kh = h // G
        q64 = to64(inp["q"][bi, h]); k64 = to64(inp["k"][bi, kh]); v64 = to64(inp["v"][bi, kh])
        do64 = to64(inp["do"][bi, h])
        tiles = _sample_tiles(w, rng)
        rows = np.concatenate([np.arange(I * Br, (I + 1) * Br) for I in tiles])
        ref = oracle.attn_fwd_head(q64, k64, v64, w.alpha, w.causal, B, Bc, scale, rows=rows)
        rb = oracle.attn_bwd_rows_head(q64, k64, v64, do64, ref["tau"], w.alpha, w.causal, scale,
                                       rows=ref["rows"])
        rows = ref["rows"]
        tau_g = to64(r.tau[bi, h])[rows]
        o_g = to64(r.o[bi, h])[rows]
        dq_g = to64(dq[bi, h])[rows]
        tau_h_g = to64(r.tau_h[bi, h])[rows]
        dtau = np.abs(tau_g - ref["tau"]).max()
        do_ = np.abs(o_g - ref["o"]).max()
        rdq = rel_fro(dq_g, rb["dq"])
        # Histogram bound: tau* - 1/B < tau_h <= tau* (up to the score rounding of bf16 x fp32)
        eps = 1e-4
        assert np.all(tau_h_g <= ref["tau"] + eps), f"{cfg} h{h}: tau_h above tau*"
        assert np.all(tau_h_g > ref["tau"] - 1.0 / B - eps), f"{cfg} h{h}: tau_h below tau* - 1/B"
        worst["tau"] = max(worst["tau"], dtau)
        worst["o"] = max(worst["o"], do_)
        worst["dq"] = max(worst["dq"], rdq)
        print(f"[fullsize] {cfg} b{bi} h{h} tiles {tiles}: max|dtau| {dtau:.2e} max|dO| {do_:.2e} "
              f"dq rel {rdq:.2e}", flush=True)
        assert dtau <= TAU_TOL, f"{cfg} h{h}: max|dtau| {dtau}"
        assert do_ <= O_TOL, f"{cfg} h{h}: max|dO| {do_}"
        assert rdq <= G_TOL, f"{cfg} h{h}: dq rel {rdq}"
        # block mask rows of the sampled tiles: a differing bit needs a score of that block
        # within the tau tolerance of the oracle's tau (a knife-edge support decision)
        mask_g = r.mask[bi, h].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        x = (w.alpha - 1.0) * scale * (q64[rows] @ k64.T)
        for t, I in enumerate(tiles):
            sl = slice(t * Br, (t + 1) * Br)
            ref_words = _bits_of_tile(ref["rowbits"][sl]).astype(np.int64)
            diff = mask_g[I] ^ ref_words
            for wi in np.nonzero(diff)[0]:
                for bit in range(32):
                    if not (int(diff[wi]) >> bit) & 1:
                        continue
                    J = int(wi) * 32 + bit
                    xs = x[sl, J * Bc:(J + 1) * Bc]
                    gap = np.abs(xs - ref["tau"][sl, None])
                    if w.causal:
                        qi = rows[sl][:, None]
                        kj = np.arange(J * Bc, (J + 1) * Bc)[None, :]
                        gap = np.where(kj <= qi, gap, np.inf)
                    assert gap.min() <= TAU_TOL, f"{cfg} h{h} tile {I} block {J}: mask differs"
    print(f"[fullsize] {cfg} worst: {worst}", flush=True)


def test_fullsize_keys_from_sampled_rows(point):
    """dK and dV at full size with dO kept on a sampled row set R and zeroed elsewhere: a row
    with dO = 0 has dP = 0 and delta = 0, so it adds nothing to dK or dV, and the oracle
    needs tau and delta of the rows in R only. Keys are sampled from the key blocks the rows
    of R attend to (non-zero gradients), plus random keys (zero or small gradients)."""
    (cfg, _, _), (w, inp, r, _) = point
    G = w.heads_q // w.heads_kv
    scale = 1.0 / math.sqrt(w.head_dim)
    n, Br, Bc, B = w.seqlen, w.block_q, w.block_k, w.n_bins
    rng = np.random.default_rng(11)
    bi = 0
    kh = int(rng.integers(0, w.heads_kv))
    hs = list(range(kh * G, (kh + 1) * G))
    Tr = n // Br
    rows_of = {}
    for h in hs:
        tiles = sorted({Tr - 1, int(rng.integers(Tr // 2, Tr - 1))})
        rows_of[h] = np.concatenate([np.arange(I * Br, (I + 1) * Br) for I in tiles])
    do_m = torch.zeros_like(inp["do"])
    for h in hs:
        idx = torch.as_tensor(rows_of[h], device=do_m.device)
        do_m[bi, h, idx] = inp["do"][bi, h, idx]
    d = dev()
    blk = (w.block_q, w.block_k)
    desc = lce._desc_for(inp["q"], inp["k"], w.alpha, w.causal, blk, w.n_bins, None, 0, 0.0)
    _, bws = lce.workspace_bytes(desc)
    wsb = torch.empty(max(bws, 256), dtype=torch.uint8, device=d)
    _, dk, dv = lce.bwd(inp["q"], inp["k"], inp["v"], do_m, r.tau, r.mask, r.aux, w.alpha,
                        w.causal, blk, w.n_bins, workspace=wsb)
    torch.cuda.synchronize()

    k64 = to64(inp["k"][bi, kh]); v64 = to64(inp["v"][bi, kh])
    qg = np.stack([to64(inp["q"][bi, h]) for h in hs])
    dog = np.stack([to64(do_m[bi, h]) for h in hs])
    taug = np.full((G, n), np.inf)      # rows outside R: no weight (their dO is zero)
    deltag = np.zeros((G, n))
    blocks = set()
    for g, h in enumerate(hs):
        rows = rows_of[h]
        ref = oracle.attn_fwd_head(qg[g], k64, v64, w.alpha, w.causal, B, Bc, scale, rows=rows)
        rb = oracle.attn_bwd_rows_head(qg[g], k64, v64, dog[g], ref["tau"], w.alpha, w.causal,
                                       scale, rows=ref["rows"])
        taug[g, ref["rows"]] = ref["tau"]
        deltag[g, ref["rows"]] = rb["delta"]
        words = np.bitwise_or.reduce(ref["rowbits"], axis=0)
        for wi, word in enumerate(words):
            for bit in range(32):
                if (int(word) >> bit) & 1:
                    blocks.add(wi * 32 + bit)
    blocks = sorted(blocks)
    pick = rng.choice(len(blocks), size=min(8, len(blocks)), replace=False)
    keys = set()
    for J in (blocks[i] for i in pick):
        keys.update(int(x) for x in rng.choice(np.arange(J * Bc, (J + 1) * Bc), 16, replace=False))
    keys.update(int(x) for x in rng.integers(0, n, 32))
    keys = np.array(sorted(keys), dtype=np.int64)
    rk = oracle.attn_bwd_keys_group(qg, k64, v64, dog, taug, deltag, w.alpha, w.causal, scale,
                                    keys=keys)
    dk_g = to64(dk[bi, kh])[keys]
    dv_g = to64(dv[bi, kh])[keys]
    assert np.linalg.norm(rk["dk"]) > 0 and np.linalg.norm(rk["dv"]) > 0
    rdk, rdv = rel_fro(dk_g, rk["dk"]), rel_fro(dv_g, rk["dv"])
    print(f"[fullsize] {cfg} b{bi} kv{kh}: {len(keys)} keys over {len(pick)} of {len(blocks)} "
          f"attended blocks: dk rel {rdk:.2e} dv rel {rdv:.2e}", flush=True)
    assert rdk <= G_TOL and rdv <= G_TOL


def test_fullsize_gradient_sums(point):
    """Per KV head the dK rows sum to zero and the dV rows sum to the group's sum of dO."""
    (cfg, _, _), (w, inp, r, (dq, dk, dv)) = point
    G = w.heads_q // w.heads_kv
    bi = 0
    for kh in sorted({0, w.heads_kv - 1}):
        hs = list(range(kh * G, (kh + 1) * G))
        dk_all = to64(dk[bi, kh])
        dv_all = to64(dv[bi, kh])
        sum_dk = dk_all.sum(axis=0)
        sum_dv = dv_all.sum(axis=0)
        sum_do = sum(to64(inp["do"][bi, h]).sum(axis=0) for h in hs)
        # the dK rows cancel: what is left must be a small fraction of their absolute mass
        # (a dropped or mis-signed term leaves a sum of the order of that mass)
        err_k = float((np.abs(sum_dk) / np.abs(dk_all).sum(axis=0)).max())
        err_v = float(np.abs(sum_dv - sum_do).max() / np.abs(sum_do).max())
        print(f"[fullsize] {cfg} kv{kh}: max |sum dK| / sum |dK| {err_k:.2e}, "
              f"sum dV vs sum dO rel {err_v:.2e}", flush=True)
        assert err_k <= 2.0 ** -6
        assert err_v <= 1e-2


@pytest.mark.parametrize("cfg", ["C3", "C4"])
def test_fullsize_nape_sampled_tiles(cfg):
    """NAPE heads at full size (half the heads ALiBi with nape_slopes): whole sampled query
    tiles of an unbiased and a biased head against the oracle with the same slopes."""
    w0 = synth.workload(cfg)
    slopes = lce.nape_slopes(w0.heads_q)
    w, inp, r, (dq, dk, dv) = _run(cfg, slopes)
    rng = np.random.default_rng(77)
    G = w.heads_q // w.heads_kv
    scale = 1.0 / math.sqrt(w.head_dim)
    Br, Bc, B = w.block_q, w.block_k, w.n_bins
    bi = 0
    for h in (0, w.heads_q - 1):
        kh = h // G
        q64 = to64(inp["q"][bi, h]); k64 = to64(inp["k"][bi, kh]); v64 = to64(inp["v"][bi, kh])
        do64 = to64(inp["do"][bi, h])
        tiles = _sample_tiles(w, rng)
        rows = np.concatenate([np.arange(I * Br, (I + 1) * Br) for I in tiles])
        ref = oracle.attn_fwd_head(q64, k64, v64, w.alpha, w.causal, B, Bc, scale, rows=rows,
                                   slope=slopes[h])
        rb = oracle.attn_bwd_rows_head(q64, k64, v64, do64, ref["tau"], w.alpha, w.causal, scale,
                                       rows=ref["rows"], slope=slopes[h])
        rows = ref["rows"]
        dtau = np.abs(to64(r.tau[bi, h])[rows] - ref["tau"]).max()
        do_ = np.abs(to64(r.o[bi, h])[rows] - ref["o"]).max()
        rdq = rel_fro(to64(dq[bi, h])[rows], rb["dq"])
        tau_h_g = to64(r.tau_h[bi, h])[rows]
        print(f"[fullsize] {cfg} NAPE h{h} slope {slopes[h]:.4g} tiles {tiles}: max|dtau| {dtau:.2e} "
              f"max|dO| {do_:.2e} dq rel {rdq:.2e}", flush=True)
        assert np.all(tau_h_g <= ref["tau"] + 1e-4)
        assert np.all(tau_h_g > ref["tau"] - 1.0 / B - 1e-4)
        assert dtau <= TAU_TOL and do_ <= O_TOL and rdq <= G_TOL

"""Calibrate the query scale beta of the centroid recipe to a target block sparsity.

Block sparsity (reading: sigma = 1 - nonzero blocks / causally valid blocks, at the
mask granularity block_q x block_k) is measured with the fp64 oracle on a seeded
sample of query tiles; beta is found by bisection on log(beta). The result table
``beta_table.json`` records beta, the achieved sample sparsity and the sample size.
It is test infrastructure: it calls only the oracle and the generator and writes
``synth/beta_table.json``, which the generator reads.

    python -m oracle.calibrate_beta            # all workloads (minutes on 8 cores)
    python -m oracle.calibrate_beta C2         # one workload
    python -m oracle.calibrate_beta --extra    # the extra sweep points not yet in the table
"""
from __future__ import annotations

import json
import math
import os
import sys
import time

import numpy as np

import oracle
from synth import Workload, make_inputs
from synth.betas import _TABLE, key, load_table

TARGETS = {
    # name: [(alpha, target sparsity), ...]; target 0 means "dense" (beta -> tiny)
    "C2": [(1.5, 0.0), (1.5, 0.6), (1.5, 0.9), (2.0, 0.0), (2.0, 0.6), (2.0, 0.9)],
    "C3": [(1.5, 0.6), (1.5, 0.8), (1.5, 0.95)],
    "C4": [(2.0, 0.95)],
    "C5": [(1.5, 0.97)],
}
# extra points of the block-sparsity sweeps (between and beyond the configured ones), so that
# the fit of step time against non-zero blocks rests on more than three points per sweep
SWEEP_EXTRA = {
    "C2": [(1.5, 0.3), (1.5, 0.8), (1.5, 0.95), (2.0, 0.3), (2.0, 0.8), (2.0, 0.95)],
    "C3": [(1.5, 0.7), (1.5, 0.9)],
}
NOMINAL_C2 = [0.5, 2.0, 6.0]


def base_workload(name: str, alpha: float, target: float) -> Workload:
    if name == "C2":
        return Workload("C2", 4, 8, 8, 4096, 64, "bf16", alpha, True, 64, 64, 16, "centroid",
                        target_sparsity=target)
    if name == "C3":
        return Workload("C3", 2, 16, 16, 16384, 128, "bf16", alpha, True, 64, 64, 8, "centroid",
                        target_sparsity=target)
    if name == "C4":
        return Workload("C4", 1, 8, 8, 65536, 128, "bf16", alpha, True, 128, 64, 16, "centroid",
                        zipf=1.1, target_sparsity=target)
    if name == "C5":
        return Workload("C5", 1, 32, 8, 131072, 64, "bf16", alpha, True, 64, 64, 16, "centroid",
                        target_sparsity=target)
    raise ValueError(name)


def sample_plan(w: Workload, tiles: int, seed: int = 1234):
    """Seeded (head, tile) sample: `tiles` tiles spread over up to 4 query heads of batch 0."""
    rng = np.random.default_rng(seed)
    Tr = w.seqlen // w.block_q
    heads = sorted(rng.choice(w.heads_q, size=min(4, w.heads_q), replace=False).tolist())
    per = max(1, tiles // len(heads))
    plan = {h: sorted(rng.choice(Tr, size=min(per, Tr), replace=False).tolist()) for h in heads}
    return plan


def block_sparsity(w: Workload, beta: float, tiles: int = 32, threads: int | None = None):
    """Oracle block sparsity of the sampled tiles at this beta: (sigma, nonzero, valid)."""
    w.beta = beta
    plan = sample_plan(w, tiles)
    heads = list(plan.keys())
    inp = make_inputs(w, heads=heads, need_grad_inputs=False)
    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    kv_index = {h: i for i, h in enumerate(inp["kv_heads"])}
    G = w.heads_q // w.heads_kv
    Br, Bc, n = w.block_q, w.block_k, w.seqlen
    scale = 1.0 / math.sqrt(w.head_dim)
    nnz = valid = 0
    for hi, h in enumerate(heads):
        rows = [I * Br + r for I in plan[h] for r in range(Br)]
        kvi = kv_index[h // G]
        f = oracle.attn_fwd_head(q[0, hi], k[0, kvi], v[0, kvi], w.alpha, w.causal, w.n_bins, Bc,
                                 scale, rows=rows, threads=threads)
        bits = f["rowbits"].reshape(len(plan[h]), Br, -1)
        for t, I in enumerate(plan[h]):
            m = np.bitwise_or.reduce(bits[t], axis=0)
            nnz += int(sum(bin(int(x)).count("1") for x in m))
            last_key = I * Br + Br - 1
            valid += (last_key // Bc + 1) if w.causal else n // Bc
    return 1.0 - nnz / valid, nnz, valid


def calibrate(name: str, alpha: float, target: float, tiles: int = 32, iters: int = 12):
    w = base_workload(name, alpha, target)
    if target <= 0.0:
        # dense end: the largest beta on a coarse grid whose sparsity is still <= 1%
        beta = 1e-5
        for lb in np.arange(-5.0, -1.0, 0.25):
            s, _, _ = block_sparsity(w, 10 ** lb, tiles)
            if s > 0.01:
                break
            beta = 10 ** lb
        s, nz, va = block_sparsity(w, beta, tiles)
        return beta, s, nz, va
    lo, hi = -5.0, 1.5          # log10 beta bracket
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        s, _, _ = block_sparsity(w, 10 ** mid, tiles)
        if s < target:
            lo = mid
        else:
            hi = mid
    beta = 10 ** (0.5 * (lo + hi))
    s, nz, va = block_sparsity(w, beta, tiles)
    return beta, s, nz, va


def main(argv):
    extra = "--extra" in argv
    args = [a for a in argv[1:] if not a.startswith("--")]
    src = SWEEP_EXTRA if extra else TARGETS
    names = args or list(src)
    table = load_table()
    for name in names:
        for alpha, target in src.get(name, []):
            if extra and key(name, alpha, target) in table:
                continue
            t0 = time.time()
            beta, s, nz, va = calibrate(name, alpha, target)
            table[key(name, alpha, target)] = {
                "beta": beta, "sample_sparsity": s, "sample_nonzero_blocks": nz,
                "sample_valid_blocks": va, "sample": "32 query tiles over up to 4 heads of batch 0, seed 1234",
            }
            print(f"{name} alpha={alpha} target={target}: beta={beta:.4g} sparsity={s:.4f} "
                  f"({nz}/{va}) [{time.time() - t0:.0f}s]", flush=True)
            with open(_TABLE, "w") as f:
                json.dump(table, f, indent=1, sort_keys=True)
        if name == "C2" and not extra:
            for beta in NOMINAL_C2:
                w = base_workload("C2", 1.5, 0.0)
                s, nz, va = block_sparsity(w, beta)
                table[f"C2/alpha=1.5/nominal_beta={beta:g}"] = {
                    "beta": beta, "sample_sparsity": s, "sample_nonzero_blocks": nz,
                    "sample_valid_blocks": va}
                print(f"C2 nominal beta={beta}: sparsity={s:.4f}", flush=True)
            with open(_TABLE, "w") as f:
                json.dump(table, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv)

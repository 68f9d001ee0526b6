"""Calibrated query scales (beta) of the centroid recipe.

The nominal "beta in {0.5, 2, 6}" does not set the block sparsity by itself
(the sparsity of the literal recipe is nearly flat in beta), so beta is found
per (workload, alpha, target sparsity) by bisection on log(beta) against the
oracle's block sparsity on a sample of query tiles. ``calibrate_beta.py`` in
this folder writes ``beta_table.json``; this module only reads it.
"""
from __future__ import annotations

import json
import os

_TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "beta_table.json")


def key(name: str, alpha: float, sparsity: float) -> str:
    return f"{name}/alpha={alpha:g}/sparsity={sparsity:g}"


def load_table() -> dict:
    if not os.path.exists(_TABLE):
        return {}
    with open(_TABLE) as f:
        return json.load(f)


def beta_for(w) -> float:
    t = load_table()
    k = key(w.name, w.alpha, w.target_sparsity)
    if k not in t:
        raise KeyError(f"no calibrated beta for {k}; run python -m oracle.calibrate_beta")
    return float(t[k]["beta"])

"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding and
the fp64 oracle on the same generated tensors, and compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth
import long_context_entmax_amd as lce


def dev():
    return torch.device("cuda:0")


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(inp: dict, w: synth.Workload, with_bwd: bool = True, stats=None, tau_init: int = 0,
            slopes=None, dense: bool = False):
    d = dev()
    q, k, v = inp["q"].to(d), inp["k"].to(d), inp["v"].to(d)
    blk = (w.block_q, w.block_k)
    sl = None if slopes is None else torch.tensor(list(slopes), dtype=torch.float32, device=d)
    r = lce.fwd(q, k, v, w.alpha, w.causal, blk, w.n_bins, return_hist=True, stats=stats,
                tau_init=tau_init, slopes=sl, dense=dense)
    out = {"o": r.o, "tau": r.tau, "mask": r.mask, "aux": r.aux, "hist": r.hist, "tau_h": r.tau_h}
    if with_bwd:
        do = inp["do"].to(d)
        dq, dk, dv = lce.bwd(q, k, v, do, r.tau, r.mask, r.aux, w.alpha, w.causal, blk, w.n_bins,
                             slopes=sl, dense=dense)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {kk: (vv.cpu() if isinstance(vv, torch.Tensor) else vv) for kk, vv in out.items()}


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def mask_bits(mask_i32: np.ndarray) -> np.ndarray:
    return mask_i32.astype(np.int64) & 0xFFFFFFFF


def scores_x(q64, k64, alpha, scale, G, slopes=None):
    """x = (alpha-1) (scale q k^T - slope |i - j|) per query head, fp64: [b, hq, n, n]."""
    kk = np.repeat(k64, G, axis=1)
    s = scale * np.einsum("bhid,bhjd->bhij", q64, kk)
    if slopes is not None:
        n = s.shape[-1]
        dist = np.abs(np.arange(n)[:, None] - np.arange(n)[None, :]).astype(np.float64)
        s = s - np.asarray(slopes, dtype=np.float64)[None, :, None, None] * dist[None, None]
    return (alpha - 1.0) * s


def mask_mismatch_is_ambiguous(gpu_mask, ref_mask, x, tau_ref, w, band):
    """Every block where the masks differ must hold a score within `band` of the oracle's tau."""
    diff = np.argwhere(mask_bits(gpu_mask) != mask_bits(ref_mask))
    for (b, h, I, wi) in diff:
        bits = int(mask_bits(gpu_mask)[b, h, I, wi] ^ mask_bits(ref_mask)[b, h, I, wi])
        for bit in range(32):
            if not (bits >> bit) & 1:
                continue
            J = wi * 32 + bit
            rows = slice(I * w.block_q, (I + 1) * w.block_q)
            cols = slice(J * w.block_k, (J + 1) * w.block_k)
            xs = x[b, h, rows, cols]
            ts = tau_ref[b, h, rows][:, None]
            valid = np.ones_like(xs, dtype=bool)
            if w.causal:
                ii = np.arange(rows.start, rows.stop)[:, None]
                jj = np.arange(cols.start, cols.stop)[None, :]
                valid = jj <= ii
            gap = np.abs(xs - ts)[valid]
            if gap.size == 0 or gap.min() > band:
                return False
    return True


def valid_block_mask(b: int, hq: int, n: int, Br: int, Bc: int, causal: bool) -> np.ndarray:
    """Mask words [b, hq, Tr, W] with every causally valid (query tile, key block) bit set."""
    Tr, Tc = n // Br, n // Bc
    W = (Tc + 31) // 32
    m = np.zeros((Tr, W), dtype=np.int64)
    for I in range(Tr):
        last = min(Tc - 1, (I * Br + Br - 1) // Bc) if causal else Tc - 1
        for J in range(last + 1):
            m[I, J // 32] |= 1 << (J % 32)
    return np.broadcast_to(m, (b, hq, Tr, W)).copy()

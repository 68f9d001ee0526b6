"""fp64 CPU oracle of DashAttention stages 1-2 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may use it.
It follows the DashAttention page (DashAttention (it), "Metodologia",
stages 1 and 2) and takes, where the page leaves a step open, the readings below.

Inputs: q [b, hq, n, d]; k, v [b, hkv, n, d]; ks [b, hkv, nc, d], the chunk summaries
of stage 0 (one vector per complete chunk of C keys, nc = n / C). Query head h belongs
to KV group g = h // G, G = hq / hkv.

Stage 1, routing (DashAttention (it), "Stadio 1"): query row i has m_i = floor(i / C) complete
chunks before its own. Its routing logits are zbar[h, i, c] = gamma * scale * q[h, i] .
ks[g, c] for c < m_i, and what[h, i, :] = alpha-entmax(zbar[h, i, :]) (tau on the x-scale
x = (alpha - 1) zbar). The query heads of a KV group average their routing weights:
wbar[g, i, c] = mean over h in g of what[h, i, c]; the shared support is {c : wbar > 0}.
A row with m_i = 0 routes nothing (tau reported as 0, wbar = 0).

Stage 2, prior-induced sparse softmax (DashAttention (it), "Stadio 2"): the softmax whose KL
reference is the prior g instead of the uniform distribution is softmax(s + log g). The
prior on key j of a routed chunk c is wbar[g, i, c] raised to sigma (sigma = 0: uniform
over the active keys; sigma = 1: the routing weights themselves); the query's own chunk
(the diagonal branch, which has no summary) keeps weight 1, over its keys j <= i. So
    s_ij = scale * q_i . k_j + sigma * ln wbar[g, i, c(j)]   (j in a routed chunk),
    s_ij = scale * q_i . k_j                                  (j in chunk m_i, j <= i),
and every other key is masked. o_i = sum_j softmax(s_i)_j v_j; lse_i = ln sum_j exp(s_ij).

Chunk mask: bit (g, query tile t of 64 rows, chunk c) is set iff some row of the tile
has wbar[g, i, c] > 0; words [b, hkv, ceil(n / 64), ceil(nc / 32)], bit c % 32 of word
c // 32.

Backward (``dash_bwd``; DashAttention (it), stage 1 "Differenziabilità": gradients flow back
through the routing to the chunk summaries). With L the loss and dO = dL/do:
  stage 2, per row and head: P = softmax(s), dP_j = dO . v_j, delta = dO . o,
    dS_j = P_j (dP_j - delta); dq += scale sum_j dS_j k_j, dk_j += scale dS_j q, dv_j += P_j dO;
    the bias sigma ln wbar_c of a routed chunk gets sum_{j in c} dS_j;
  group average: dwbar_c = sigma / wbar_c * sum over the group's heads of that chunk sum;
    each head's routing weights get dwbar / G;
  stage 1, per row and head (the alpha-entmax Jacobian diag(g) - g g^T / sum g with
    g = [x - tau]_+^(1/(alpha-1) - 1), x = (alpha - 1) zbar): dz = g (dw - (g . dw) / sum g);
    zbar = gamma scale q . ks, so dq += gamma scale sum_c dz_c ks_c, dks_c += gamma scale dz_c q.
Chunks outside the support carry no gradient (g = 0 there, and their keys are masked).

Pins (tests/test_oracle_pins.py): all-equal summaries make routing uniform, so sigma = 0
is causal softmax attention and sigma = 1 is causal softmax attention with -ln m_i added
on earlier chunks (both checked against torch's scaled_dot_product_attention in fp64); a
hand-derived sparsemax routing row; the GQA average, its union support and the chunk mask
by brute force; the backward against central finite differences of sum(o * dO) in q, k, v
and the summaries, and at sigma = 0 (no prior) a summary gradient of exactly 0 and a dq
equal to that of masked softmax attention. No function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

from . import entmax as _entmax

TILE = 64   # query rows per chunk-mask tile


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def route_group(q_group, ks, alpha: float, gamma: float, scale: float, C: int, rows) -> dict:
    """Stage 1 for the query heads of one KV group on the given rows.

    q_group [G, n, d], ks [nc, d]. Returns tau [G, r] (x-scale; 0 where m_i = 0),
    what [G, r, nc] (each head's routing weights) and wbar [r, nc] (their mean)."""
    q_group, ks = _f64(q_group), _f64(ks)
    G = q_group.shape[0]
    nc = ks.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    tau = np.zeros((G, rows.size))
    what = np.zeros((G, rows.size, nc))
    for ri, i in enumerate(rows):
        m = int(i) // C
        if m == 0:
            continue
        for h in range(G):
            z = gamma * scale * (ks[:m] @ q_group[h, i])
            p, t = _entmax(z, alpha)
            what[h, ri, :m] = p
            tau[h, ri] = t
    return {"tau": tau, "what": what, "wbar": what.mean(axis=0)}


def attend_group(q_group, k, v, wbar, sigma: float, scale: float, C: int, rows) -> dict:
    """Stage 2 for the query heads of one KV group on the given rows.

    q_group [G, n, d]; k, v [n, d]; wbar [r, nc] for the same rows. Returns o [G, r, d],
    lse [G, r] and the number of attended keys per row [r]."""
    q_group, k, v = _f64(q_group), _f64(k), _f64(v)
    G, n, d = q_group.shape
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((G, rows.size, d))
    lse = np.zeros((G, rows.size))
    nkeys = np.zeros(rows.size, dtype=np.int64)
    for ri, i in enumerate(rows):
        m = int(i) // C
        keys, bias = [], []
        for c in range(m):
            if wbar[ri, c] > 0.0:
                keys.append(np.arange(c * C, (c + 1) * C))
                bias.append(np.full(C, sigma * np.log(wbar[ri, c])))
        keys.append(np.arange(m * C, int(i) + 1))     # the diagonal branch
        bias.append(np.zeros(int(i) + 1 - m * C))
        keys = np.concatenate(keys)
        bias = np.concatenate(bias)
        nkeys[ri] = keys.size
        for h in range(G):
            s = scale * (k[keys] @ q_group[h, i]) + bias
            smax = s.max()
            e = np.exp(s - smax)
            tot = e.sum()
            o[h, ri] = (e / tot) @ v[keys]
            lse[h, ri] = smax + np.log(tot)
    return {"o": o, "lse": lse, "nkeys": nkeys}


def chunk_mask(wbar_rows, rows, n: int) -> np.ndarray:
    """Tile mask [ceil(n/64), ceil(nc/32)] from wbar of ALL rows (rows must be 0..n-1)."""
    wbar_rows = np.asarray(wbar_rows)
    nc = wbar_rows.shape[1]
    Tr, Wc = (n + TILE - 1) // TILE, (nc + 31) // 32
    words = np.zeros((Tr, Wc), dtype=np.int64)
    for ri, i in enumerate(rows):
        t = int(i) // TILE
        for c in np.nonzero(wbar_rows[ri] > 0.0)[0]:
            words[t, c // 32] |= 1 << (int(c) % 32)
    return words


def dash_fwd(q, k, v, ks, alpha: float, gamma: float, sigma: float, C: int,
             scale: float | None = None, rows=None) -> dict:
    """Stages 1-2 of a whole problem (rows=None) or of sampled rows.

    Returns o [b, hq, r, d], lse [b, hq, r], tau [b, hq, r], wbar [b, hkv, r, nc],
    nkeys [b, hkv, r], rows, and (rows=None only) mask [b, hkv, Tr, Wc]."""
    q, k, v, ks = _f64(q), _f64(k), _f64(v), _f64(ks)
    b, hq, n, d = q.shape
    hkv, nc = k.shape[1], ks.shape[2]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    full = rows is None
    rows = np.arange(n) if full else np.asarray(rows, dtype=np.int64)
    r = rows.size
    out = {"o": np.zeros((b, hq, r, d)), "lse": np.zeros((b, hq, r)), "tau": np.zeros((b, hq, r)),
           "wbar": np.zeros((b, hkv, r, nc)), "nkeys": np.zeros((b, hkv, r), dtype=np.int64), "rows": rows}
    if full:
        out["mask"] = np.zeros((b, hkv, (n + TILE - 1) // TILE, (nc + 31) // 32), dtype=np.int64)
    for bi in range(b):
        for g in range(hkv):
            qg = q[bi, g * G:(g + 1) * G]
            rt = route_group(qg, ks[bi, g], alpha, gamma, scale, C, rows)
            at = attend_group(qg, k[bi, g], v[bi, g], rt["wbar"], sigma, scale, C, rows)
            out["tau"][bi, g * G:(g + 1) * G] = rt["tau"]
            out["wbar"][bi, g] = rt["wbar"]
            out["o"][bi, g * G:(g + 1) * G] = at["o"]
            out["lse"][bi, g * G:(g + 1) * G] = at["lse"]
            out["nkeys"][bi, g] = at["nkeys"]
            if full:
                out["mask"][bi, g] = chunk_mask(rt["wbar"], rows, n)
    return out


def dash_bwd(q, k, v, ks, dout, alpha: float, gamma: float, sigma: float, C: int,
             scale: float | None = None, rows=None) -> dict:
    """Gradients of stages 1-2 of a whole problem with respect to q, k, v and the summaries ks,
    given dO (the backward written out in the module docstring). Returns dq [b, hq, n, d],
    dk, dv [b, hkv, n, d] and dks [b, hkv, nc, d].

    With ``rows`` only those query rows are taken: dq is returned for them alone
    ([b, hq, len(rows), d]; a row's dq depends on that row alone), and dk, dv and dks are the
    sums over those rows only (the whole gradients when dO is zero on every other row)."""
    q, k, v, ks, dout = _f64(q), _f64(k), _f64(v), _f64(ks), _f64(dout)
    b, hq, n, d = q.shape
    hkv, nc = k.shape[1], ks.shape[2]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kappa = 1.0 / (alpha - 1.0)
    dq, dk, dv, dks = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(ks)
    row_list = range(n) if rows is None else [int(r) for r in rows]
    for bi in range(b):
        for g in range(hkv):
            kk, vv, kg = k[bi, g], v[bi, g], ks[bi, g]
            for i in row_list:
                m = i // C
                # stage 1 forward of the row
                zs, ps, taus = [], [], []
                for h in range(G):
                    z = gamma * scale * (kg[:m] @ q[bi, g * G + h, i]) if m else np.zeros(0)
                    p, t = _entmax(z, alpha) if m else (np.zeros(0), 0.0)
                    zs.append(z); ps.append(p); taus.append(t)
                wbar = np.mean(ps, axis=0) if m else np.zeros(0)
                routed = [c for c in range(m) if wbar[c] > 0.0]
                keys = [np.arange(c * C, (c + 1) * C) for c in routed] + [np.arange(m * C, i + 1)]
                bias = [np.full(C, sigma * np.log(wbar[c])) for c in routed] + [np.zeros(i + 1 - m * C)]
                keys, bias = np.concatenate(keys), np.concatenate(bias)
                dwbar = np.zeros(m)
                for h in range(G):
                    hh = g * G + h
                    # stage 2 forward and backward of the row
                    s = scale * (kk[keys] @ q[bi, hh, i]) + bias
                    e = np.exp(s - s.max())
                    P = e / e.sum()
                    o = P @ vv[keys]
                    dP = vv[keys] @ dout[bi, hh, i]
                    dS = P * (dP - dout[bi, hh, i] @ o)
                    dq[bi, hh, i] += scale * (dS @ kk[keys])
                    dk[bi, g, keys] += scale * np.outer(dS, q[bi, hh, i])
                    dv[bi, g, keys] += np.outer(P, dout[bi, hh, i])
                    for ci, c in enumerate(routed):
                        dwbar[c] += sigma / wbar[c] * dS[ci * C:(ci + 1) * C].sum()
                if not m:
                    continue
                # stage 1 backward of the row
                for h in range(G):
                    hh = g * G + h
                    x = (alpha - 1.0) * zs[h]
                    dlt = np.maximum(x - taus[h], 0.0)
                    gg = np.zeros_like(dlt)
                    pos = dlt > 0.0
                    gg[pos] = dlt[pos] ** (kappa - 1.0)
                    dw = dwbar / G
                    dz = gg * (dw - (gg @ dw) / gg.sum())
                    dq[bi, hh, i] += gamma * scale * (dz @ kg[:m])
                    dks[bi, g, :m] += gamma * scale * np.outer(dz, q[bi, hh, i])
    if rows is not None:
        return {"dq": dq[:, :, np.asarray(row_list, dtype=np.int64)], "dk": dk, "dv": dv, "dks": dks}
    return {"dq": dq, "dk": dk, "dv": dv, "dks": dks}

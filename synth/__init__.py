"""Seeded synthetic inputs for alpha-entmax attention (shared by the tests, the
benchmark and the oracle's checks).

This module holds no part of the attention method: it only draws numbers.
Every tensor is a deterministic function of (seed, tensor id, flat element
index) through a counter-based SplitMix64 stream, so any head or row subset
can be regenerated on its own and the same call gives the same bits on the
CPU and on the GPU up to the last ulp of the Box-Muller transcendental
functions (tests copy one generated tensor to both sides, they never
regenerate it).

Workloads follow the efficiency setting of the AdaSplash-2 pages
("AdaSplash-2: Faster Differentiable Sparse Attention", gist.science summaries,
Results / efficiency benchmarks: synthetic inputs, 4K-128K tokens, swept block
sparsity):

* ``tiny``: Q, K, V, dO i.i.d. N(0,1). Q and K are rounded to multiples of
  2^-5 so that every fp32 score is exact (histogram counts, support and block
  mask can then be compared bit for bit); V and dO stay raw fp32.
* ``centroid``: keys are per-64-key-block centroids ``3 N(0,I)`` plus
  ``0.3 N(0,I)`` noise; each query tile picks 4 distinct causally valid key
  blocks (uniformly, or Zipf(1.1) on the block index) and its queries are
  ``beta * (sum of the 4 centroids + N(0,I))``. beta sets the block sparsity.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict
from typing import Optional, Sequence

import torch

# tensor ids of the counter-based streams
TID_Q, TID_K, TID_V, TID_DO, TID_CENTROID, TID_PICKS, TID_QNOISE, TID_KSUM = 1, 2, 3, 4, 5, 6, 7, 8

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _s64(u: int) -> int:
    """uint64 constant -> the int64 with the same bits."""
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 finaliser (Steele, Lea, Flood 2014) on int64 bit patterns."""
    z = (z ^ _srl(z, 30)) * _s64(_M1)
    z = (z ^ _srl(z, 27)) * _s64(_M2)
    return z ^ _srl(z, 31)


def _key(seed: int, tid: int) -> int:
    """Stream key of (seed, tensor id): one SplitMix64 output, as python int."""
    z = ((seed & 0xFFFFFFFF) << 32 | (tid & 0xFFFFFFFF)) + _GAMMA
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def bits64(seed: int, tid: int, counters: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output for state = key(seed, tid) + (counter + 1) * golden gamma."""
    k = _s64(_key(seed, tid))
    z = k + (counters.to(torch.int64) + 1) * _s64(_GAMMA)
    return _mix(z)


def uniform(seed: int, tid: int, counters: torch.Tensor) -> torch.Tensor:
    """Uniform on (0, 1) in float64 from the top 53 bits."""
    b = _srl(bits64(seed, tid, counters), 11)
    return (b.to(torch.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, tid: int, counters: torch.Tensor) -> torch.Tensor:
    """N(0,1) in float64 by Box-Muller on counters 2c and 2c+1."""
    c = counters.to(torch.int64)
    u1 = uniform(seed, tid, 2 * c)
    u2 = uniform(seed, tid, 2 * c + 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def _flat_counters(shape: Sequence[int], index: Sequence[torch.Tensor | slice | int],
                   device) -> torch.Tensor:
    """Flat row-major indices of ``torch.empty(shape)[index]`` (no storage of the full tensor)."""
    strides = []
    s = 1
    for n in reversed(shape):
        strides.append(s)
        s *= n
    strides = strides[::-1]
    out = torch.zeros((), dtype=torch.int64, device=device)
    nd = len(shape)
    for ax in range(nd):
        sel = index[ax] if ax < len(index) else slice(None)
        if isinstance(sel, slice):
            r = torch.arange(shape[ax], device=device, dtype=torch.int64)[sel]
        elif isinstance(sel, int):
            r = torch.tensor([sel], device=device, dtype=torch.int64)
        else:
            r = sel.to(device=device, dtype=torch.int64)
        view = [1] * nd
        view[ax] = r.numel()
        out = out + (r * strides[ax]).view(view)
    return out


def normal_tensor(seed: int, tid: int, shape: Sequence[int], device="cpu",
                  heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    """N(0,1) float64 tensor of ``shape`` = [b, h, ...]; ``heads`` selects a subset of axis 1."""
    idx: list = [slice(None)]
    if heads is not None:
        idx.append(torch.as_tensor(list(heads), dtype=torch.int64))
    return normal(seed, tid, _flat_counters(shape, idx, device))


# ----------------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------------

@dataclass
class Workload:
    """Shape and recipe of one synthetic alpha-entmax attention problem."""
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    dtype: str            # "f32" | "bf16"
    alpha: float
    causal: bool
    block_q: int
    block_k: int
    n_bins: int
    recipe: str           # "tiny" | "centroid" | "normal"
    beta: float = 1.0     # query scale of the centroid recipe
    zipf: Optional[float] = None   # Zipf exponent of the centroid picks (None: uniform)
    picks: int = 4
    seed: int = 0
    target_sparsity: Optional[float] = None
    extra: dict = field(default_factory=dict)

    def as_dict(self) -> dict:
        return asdict(self)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def workload(name: str, alpha: Optional[float] = None, sparsity: Optional[float] = None,
             beta: Optional[float] = None) -> Workload:
    """The five configurations of the efficiency study, by name (C1..C5).

    C1  tiny fp32 check: b1 h1 n256 d64, non-causal, alpha 1.5, B 16, 32x32 blocks.
    C2  b4 h8 n4096 d64 bf16 causal, alpha in {1.5, 2}, 64x64, B 16, sparsity ~0/0.6/0.9.
    C3  b2 h16 n16384 d128 bf16 causal, alpha 1.5, 64x64, B 8, sparsity 0.6/0.8/0.95.
    C4  b1 h8 n65536 d128 bf16 causal, alpha 2, 128x64, B 16, Zipf(1.1) picks, ~0.95.
    C5  b1 hq32/hkv8 n131072 d64 bf16 causal, alpha 1.5, 64x64, B 16, ~0.97 (LLaMA-3-1B layer).
    """
    from .betas import beta_for  # calibrated query scales (lazily: json read)
    if name == "C1":
        return Workload("C1", 1, 1, 1, 256, 64, "f32", alpha or 1.5, False, 32, 32, 16, "tiny")
    if name == "C2":
        a = alpha or 1.5
        s = 0.9 if sparsity is None else sparsity
        w = Workload("C2", 4, 8, 8, 4096, 64, "bf16", a, True, 64, 64, 16, "centroid",
                     target_sparsity=s)
    elif name == "C3":
        s = 0.95 if sparsity is None else sparsity
        w = Workload("C3", 2, 16, 16, 16384, 128, "bf16", alpha or 1.5, True, 64, 64, 8,
                     "centroid", target_sparsity=s)
    elif name == "C4":
        w = Workload("C4", 1, 8, 8, 65536, 128, "bf16", alpha or 2.0, True, 128, 64, 16,
                     "centroid", zipf=1.1, target_sparsity=0.95 if sparsity is None else sparsity)
    elif name == "C5":
        w = Workload("C5", 1, 32, 8, 131072, 64, "bf16", alpha or 1.5, True, 64, 64, 16,
                     "centroid", target_sparsity=0.97 if sparsity is None else sparsity)
    else:
        raise ValueError(f"unknown workload {name}")
    w.beta = beta if beta is not None else beta_for(w)
    return w


def _round_grid(x: torch.Tensor, bits: int) -> torch.Tensor:
    s = float(1 << bits)
    return torch.round(x * s) / s


def centroid_picks(w: Workload, device="cpu", heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Per (b, q-head, query tile) the indices of the picked 64-key blocks, -1 if unused.

    Distinct picks by Gumbel-top-k over the causally valid 64-key blocks with
    log-weights 0 (uniform) or -zipf*log(J+1) (Zipf on the block index).
    """
    n, Br = w.seqlen, w.block_q
    nb = n // 64
    Tr = n // Br
    hs = list(range(w.heads_q)) if heads is None else list(heads)
    J = torch.arange(nb, device=device, dtype=torch.int64)
    I = torch.arange(Tr, device=device, dtype=torch.int64)
    last = (I * Br + Br - 1) // 64 if w.causal else torch.full_like(I, nb - 1)
    valid = J.view(1, nb) <= last.view(Tr, 1)                          # [Tr, nb]
    u = uniform(w.seed, TID_PICKS,
                _flat_counters((w.batch, w.heads_q, Tr, nb),
                               [slice(None), torch.as_tensor(hs, dtype=torch.int64)], device))
    g = -torch.log(-torch.log(u))
    if w.zipf is not None:
        g = g - w.zipf * torch.log((J + 1).to(torch.float64)).view(1, 1, 1, nb)
    g = torch.where(valid.view(1, 1, Tr, nb), g, torch.full_like(g, -math.inf))
    k = min(w.picks, nb)
    top = torch.topk(g, k, dim=-1).indices                             # [b, h, Tr, k]
    nvalid = valid.sum(-1).view(1, 1, Tr, 1)
    slot = torch.arange(k, device=device).view(1, 1, 1, k)
    return torch.where(slot < nvalid, top, torch.full_like(top, -1))


def make_inputs(w: Workload, device="cpu", heads: Optional[Sequence[int]] = None,
                need_grad_inputs: bool = True) -> dict:
    """Q [b,hq,n,d], K/V [b,hkv,n,d], dO [b,hq,n,d] in the workload's dtype.

    ``heads`` restricts Q/dO to a subset of query heads (K/V are then the KV
    heads those query heads read, in full). The values of a head do not depend
    on which other heads are generated.
    """
    b, hq, hkv, n, d = w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim
    qh = list(range(hq)) if heads is None else list(heads)
    grp = hq // hkv
    kvh = sorted({h // grp for h in qh}) if heads is not None else list(range(hkv))
    dt = w.torch_dtype
    out = {"q_heads": qh, "kv_heads": kvh}
    if w.recipe == "tiny" or w.recipe == "normal":
        q = normal_tensor(w.seed, TID_Q, (b, hq, n, d), device, qh)
        k = normal_tensor(w.seed, TID_K, (b, hkv, n, d), device, kvh)
        scale = float(w.extra.get("qk_scale", 1.0))
        q, k = q * scale, k * scale
        if w.recipe == "tiny":
            q, k = _round_grid(q, 5), _round_grid(k, 5)
    elif w.recipe == "centroid":
        nb = n // 64
        cen = 3.0 * normal_tensor(w.seed, TID_CENTROID, (b, hkv, nb, d), device, None)
        kn = normal_tensor(w.seed, TID_K, (b, hkv, n, d), device, kvh)
        k = cen[:, kvh].repeat_interleave(64, dim=2) + 0.3 * kn
        picks = centroid_picks(w, device, qh)                         # [b, |qh|, Tr, P]
        kv_of = torch.as_tensor([h // grp for h in qh], device=device)
        csum = torch.zeros((b, len(qh), picks.shape[2], d), dtype=torch.float64, device=device)
        for p in range(picks.shape[-1]):
            idx = picks[..., p]
            ok = (idx >= 0).to(torch.float64).unsqueeze(-1)
            gi = idx.clamp(min=0)
            src = cen[:, kv_of]                                        # [b, |qh|, nb, d]
            csum = csum + ok * torch.gather(src, 2, gi.unsqueeze(-1).expand(-1, -1, -1, d))
        qn = normal_tensor(w.seed, TID_QNOISE, (b, hq, n, d), device, qh)
        q = w.beta * (csum.repeat_interleave(w.block_q, dim=2) + qn)
        del cen, kn, qn, csum
    else:
        raise ValueError(w.recipe)
    out["q"] = q.to(dt).contiguous()
    out["k"] = k.to(dt).contiguous()
    del q, k
    out["v"] = normal_tensor(w.seed, TID_V, (b, hkv, n, d), device, kvh).to(dt).contiguous()
    if need_grad_inputs:
        out["do"] = normal_tensor(w.seed, TID_DO, (b, hq, n, d), device, qh).to(dt).contiguous()
    return out


def chunk_summaries(w: Workload, chunk: int, device="cpu") -> torch.Tensor:
    """Chunk-summary keys [b, hkv, n / chunk, d] for DashAttention inputs (DashAttention (it), stage 0
    gives one vector per chunk of keys), drawn with the spread a mean of ``chunk`` keys of
    the recipe would have: N(0, qk_scale^2 / chunk) per element for ``normal`` and ``tiny``;
    for ``centroid`` (chunk 64, one centroid per chunk) the chunk's centroid plus
    0.3 N(0, 1/64). In the workload's dtype."""
    b, hkv, n, d = w.batch, w.heads_kv, w.seqlen, w.head_dim
    nc = n // chunk
    noise = normal_tensor(w.seed, TID_KSUM, (b, hkv, nc, d), device)
    if w.recipe == "centroid":
        if chunk != 64:
            raise ValueError("centroid summaries follow the 64-key centroid blocks")
        cen = 3.0 * normal_tensor(w.seed, TID_CENTROID, (b, hkv, n // 64, d), device, None)
        ks = cen + 0.3 * noise / 8.0
    else:
        ks = noise * (float(w.extra.get("qk_scale", 1.0)) / math.sqrt(chunk))
    return ks.to(w.torch_dtype).contiguous()

"""Benchmark: alpha-entmax attention fwd+bwd step on one MI355X.

A step is one forward and one backward of the whole hot path (histogram pass,
refinement, output pass, backward preparation, dK/dV and dQ kernels) over one
batch of synthetic inputs resident in HBM. The default workload is the largest
single-GPU configuration of the 4K-128K study: the LLaMA-3-1B-shaped layer at 128K
tokens (batch 1, 32 query / 8 KV heads, d 64, bf16, causal, alpha 1.5, 64x64 blocks,
B 16) with the centroid-cluster generator calibrated to ~97% block sparsity;
``--config C2|C3|C4`` and ``--alpha``/``--sparsity`` select the others.

Prints one JSON line: value = effective TFLOP/s (dense-equivalent FLOPs of a causal
attention fwd+bwd, 3.5 x 4 b h n^2 d / 2, divided by the measured step time),
plus a roofline object for the dominant kernel (algorithmic MFMA FLOPs per launch
over its HIP-event-timed average duration), the MFMA utilisation on the non-zero
blocks, and the CPU oracle timed on a bounded sample of the same workload.

``--dense`` runs the ablation without block skipping (every causally valid block is
multiplied; outputs are unchanged). ``--sweep`` times every configured point of the
block-sparsity study (and the extra sweep points), each with and without skipping,
fits step time against the non-zero block count per sweep, and prints one JSON line
per point plus a summary line (not the default line; ``--sweep-md`` writes a table).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
METRIC = "fwd+bwd ms/step & effective TFLOP/s vs block sparsity, α-entmax attn 4K–128K"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="C5")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--sparsity", type=float, default=None)
    ap.add_argument("--tau-init", choices=("hist", "bracket"), default="hist",
                    help="refinement start: the histogram bound (the method) or the plain "
                         "[x_max - 1, x_max - n^(1-alpha)] bracket (ablation)")
    ap.add_argument("--nape", action="store_true",
                    help="NAPE heads: the first half of the query heads without position "
                         "encoding, the second half ALiBi (per-head slopes of the scores)")
    ap.add_argument("--dense", action="store_true",
                    help="ablation: no block skipping (every causally valid block multiplied)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every point of the block-sparsity study, with and without skipping, "
                         "and fit step time against the non-zero block count")
    ap.add_argument("--sweep-md", default=None, help="with --sweep: write a markdown table here")
    ap.add_argument("--decode", action="store_true",
                    help="time one decode step (a new query row per head against the workload's "
                         "K/V as a cache) instead of the training step")
    ap.add_argument("--dash", action="store_true",
                    help="DashAttention training step (routing + prior-induced sparse softmax, forward and "
                         "backward) at 16K tokens instead of the entmax attention step")
    ap.add_argument("--tau-error", action="store_true",
                    help="instead of timing, print the mean |tau_p - tau*| after p = 1..15 "
                         "refinement passes for both starts (tau* = the converged tau)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--profile-only", action="store_true",
                    help="warmup + steps only (for rocprofv3 runs), still prints the JSON line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the steps, run 3 plain fp32 copies (x * 1) of this many MiB: the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


# the sources of the prefill forward/backward kernels and their launches (the decode and
# DashAttention kernels live in files of their own and do not enter the prefill counters)
PREFILL_SOURCES = ("api.hip", "bwd.hip", "common.hpp", "fwd.hip", "kernels.hpp", "prep.hip", "solver.hpp")


def src_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "long_context_entmax_amd", "csrc")
    for f in PREFILL_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def dense_eq_flops(w) -> float:
    f = 3.5 * 4.0 * w.batch * w.heads_q * float(w.seqlen) ** 2 * w.head_dim
    return f * (0.5 if w.causal else 1.0)


def valid_blocks(w) -> int:
    Tr, Tc = w.seqlen // w.block_q, w.seqlen // w.block_k
    if not w.causal:
        return Tr * Tc
    return sum(min(Tc, (I * w.block_q + w.block_q - 1) // w.block_k + 1) for I in range(Tr))


def popcount_mask(mask) -> int:
    import torch
    m = mask.to(torch.int64) & 0xFFFFFFFF
    cnt = torch.zeros_like(m)
    for b in range(32):
        cnt += (m >> b) & 1
    return int(cnt.sum().item())


def cpu_threads():
    """Threads the oracle may use: the cores this process may run on, at most 16 (the CPU
    share of one GPU on a shared host), and the host's total core count."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(16, avail)), os.cpu_count() or avail


def valid_pairs(w) -> float:
    """Causally valid (query, key) pairs over all query heads."""
    n = float(w.seqlen)
    per = n * (n + 1) / 2.0 if w.causal else n * n
    return per * w.batch * w.heads_q


def progressive_order(count: int):
    """0..count-1 in rounds of evenly spaced indices, each round halving the spacing (so any
    prefix of the sequence is spread over the whole range)."""
    step = 1
    while step * 2 <= count:
        step *= 2
    seen = set()
    while step >= 1:
        for u in range(step // 2 if step > 1 else 0, count, step):
            if u not in seen:
                seen.add(u)
                yield u
        step //= 2


def cpu_baseline(w, inp_cpu, target_s: float):
    """The fp64 oracle's fwd+bwd on a bounded sample of the workload, extrapolated.

    Row side (forward: scores, tau by bisection, o, histogram; backward per row: dq and
    delta): 64-row query tiles taken in an evenly spaced, progressively refined order over
    all (batch, head, tile) indices, one tile per host thread, until about 2/3 of the time
    budget is spent; the time per row is extrapolated to all rows (even spacing samples the
    causal row lengths). Key side (dk, dv per key, summed over the GQA group): keys of KV
    head 0 of batch 0 in the same kind of order, 32 keys per thread task, for the remaining
    third; each key scores every valid row of the group, and the rows whose tau the row side
    computed also take the support work (the others count as outside the support, about 1%
    of the key-side work at the study's sparsities); the time per key is extrapolated to
    all keys of all KV heads. Progress goes to stderr."""
    import numpy as np
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait
    import oracle
    threads, host_cores = cpu_threads()
    G = w.heads_q // w.heads_kv
    scale = 1.0 / math.sqrt(w.head_dim)
    n, b, hq = w.seqlen, w.batch, w.heads_q
    q64 = {(bi, h): (inp_cpu["q"][bi, h].double().numpy(), inp_cpu["do"][bi, h].double().numpy())
           for bi in range(b) for h in range(hq)}
    kv64 = {(bi, kh): (inp_cpu["k"][bi, kh].double().numpy(), inp_cpu["v"][bi, kh].double().numpy())
            for bi in range(b) for kh in range(w.heads_kv)}
    tile = min(64, n)
    ntiles = b * hq * n // tile
    tau_of = {}     # (bi, h) -> {row: (tau, delta)}

    def run_tile(u):
        r0 = u * tile
        bi, h, i0 = r0 // (hq * n), (r0 // n) % hq, r0 % n
        qq, do = q64[(bi, h)]
        kk, vv = kv64[(bi, h // G)]
        rows = list(range(i0, i0 + tile))
        f = oracle.attn_fwd_head(qq, kk, vv, w.alpha, w.causal, w.n_bins, w.block_k, scale, rows=rows, threads=1)
        rb = oracle.attn_bwd_rows_head(qq, kk, vv, do, f["tau"], w.alpha, w.causal, scale, rows=f["rows"],
                                       threads=1)
        return bi, h, f["rows"], f["tau"], rb["delta"]

    def run_pool(fn, order, budget):
        done, t0, tlast = [], time.time(), time.time()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            it, inflight = iter(order), set()
            while True:
                while len(inflight) < threads and time.time() - t0 < budget:
                    u = next(it, None)
                    if u is None:
                        break
                    inflight.add(ex.submit(fn, u))
                if not inflight:
                    break
                fin, inflight = wait(inflight, return_when=FIRST_COMPLETED)
                done.extend(x.result() for x in fin)
                if time.time() - tlast > 5.0:
                    tlast = time.time()
                    print(f"[cpu_baseline] {fn.__name__}: {len(done)} done, {tlast - t0:.0f} s", file=sys.stderr,
                          flush=True)
        return done, time.time() - t0

    res, t_rows = run_pool(run_tile, progressive_order(ntiles), target_s * 2.0 / 3.0)
    rows_done = len(res) * tile
    for bi, h, rows, tau, delta in res:
        d = tau_of.setdefault((bi, h), {})
        for r, t_, dl in zip(rows.tolist(), tau.tolist(), delta.tolist()):
            d[r] = (t_, dl)
    s_rows = t_rows / rows_done * (b * hq * n)

    kk, vv = kv64[(0, 0)]
    qg = np.stack([q64[(0, g)][0] for g in range(G)])
    dog = np.stack([q64[(0, g)][1] for g in range(G)])
    taug = np.full((G, n), np.inf)
    deltag = np.zeros((G, n))
    for g in range(G):
        for r, (t_, dl) in tau_of.get((0, g), {}).items():
            taug[g, r], deltag[g, r] = t_, dl

    def run_keys(js):
        oracle.attn_bwd_keys_group(qg, kk, vv, dog, taug, deltag, w.alpha, w.causal, scale, keys=js, threads=1)
        return len(js)

    korder = list(progressive_order(n))
    groups = [korder[i:i + 32] for i in range(0, n, 32)]   # 32 keys per task
    done_keys, t_keys = run_pool(run_keys, groups, target_s / 3.0)
    nkeys = sum(done_keys)
    s_keys = t_keys / nkeys * n * b * w.heads_kv
    s_per_step = s_rows + s_keys
    return {
        "value": dense_eq_flops(w) / s_per_step / 1e12,
        "unit": "TFLOP/s (effective)",
        "ms_per_step": s_per_step * 1e3,
        "cores": threads,
        "host_cores": host_cores,
        "kind": "oracle",
        "extrapolated": True,
        "sample": (f"fp64 oracle on {threads} threads ({host_cores} host cores): fwd + per-row bwd of "
                   f"{rows_done} of {b * hq * n} query rows (64-row tiles evenly spread over all heads, "
                   f"{t_rows:.1f} s; per row x all rows = {s_rows:.0f} s) and dK/dV of {nkeys} of {n} keys "
                   f"of one KV group ({t_keys:.1f} s; per key x all keys of all KV heads = {s_keys:.0f} s)"),
    }


def tau_error_study(lce, w, q, k, v, blk, wsf):
    """Mean absolute error of tau per refinement pass, histogram start vs plain bracket
    (the study of the pages' Fig. 3, AdaSplash-2 (es) §4). tau* is the histogram-started solve
    with the largest pass cap; the bracket-started solve at that cap is reported beside it."""
    import torch
    b, hq, n, d = q.shape

    def run(t_init, iters):
        r = lce.fwd(q, k, v, w.alpha, w.causal, blk, w.n_bins, max_iters=iters, workspace=wsf,
                    return_hist=True, tau_init=t_init)
        torch.cuda.synchronize()
        return r.tau.double().cpu(), r.tau_h.double().cpu()

    ref, tau_h = run(0, 15)
    out = {"study": "tau_mean_abs_error_per_pass", "workload": w.name, "alpha": w.alpha,
           "n_bins": w.n_bins, "rows": b * hq * n}
    # the refinement's first evaluation point: a quarter bin above tau_h, at alpha = 2 the
    # lowest of its four points (0.02 bin above tau_h)
    start = tau_h + (0.02 if w.alpha == 2.0 else 0.25) / w.n_bins
    out["histogram"] = {"tau_h": (tau_h - ref).abs().mean().item(),
                        "start": (start - ref).abs().mean().item(), "passes": []}
    tb15, xm1 = run(1, 15)
    out["bracket"] = {"start": (xm1 - ref).abs().mean().item(), "passes": [],
                      "cap15_vs_ref_max": (tb15 - ref).abs().max().item()}
    for it in range(1, 16):
        th, _ = run(0, it)
        tb, _ = run(1, it)
        out["histogram"]["passes"].append((th - ref).abs().mean().item())
        out["bracket"]["passes"].append((tb - ref).abs().mean().item())
    return out


def decode_bench(args, lce, w, inp, dev):
    """One decode step per iteration: q = the workload's query row n-1, the workload's K and V
    as the cache. Roofline of the score kernel: HBM bytes = the K cache read once plus the
    fp32 score row written."""
    import torch
    n = w.seqlen
    q = inp["q"][:, :, n - 1].contiguous()
    k, v = inp["k"], inp["v"]
    slopes = (torch.tensor(lce.nape_slopes(w.heads_q), dtype=torch.float32, device=dev)
              if args.nape else None)
    desc = lce.make_desc(w.batch, w.heads_q, w.heads_kv, n, w.head_dim,
                         lce.ENTMAX_BF16 if w.dtype == "bf16" else lce.ENTMAX_F32, w.alpha, True,
                         (32, 32), w.n_bins)
    ws = torch.empty(lce.lib().entmax_attn_decode_workspace_bytes(ctypes.byref(desc)),
                     dtype=torch.uint8, device=dev)
    step = lambda: lce.decode(q, k, v, w.alpha, w.n_bins, slopes=slopes, workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    lce.profile(True)
    lce.profile_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = lce.profile_read()
    lce.profile(False)
    kern = {name: t / max(c, 1) for name, (t, c) in kt.items()}
    es = 2 if w.dtype == "bf16" else 4
    kbytes = w.batch * w.heads_kv * n * w.head_dim * es + w.batch * w.heads_q * n * 4
    achieved = kbytes / (kern["dec_scores"] * 1e-3) / 1e9
    line = {
        "metric": "decode_tokens_per_s", "value": round(w.batch / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (the workload's K/V as the cache, its query row n-1)",
        "config": {"workload": f"decode against {w.name}: b{w.batch} hq{w.heads_q}/hkv{w.heads_kv} "
                               f"cache {n} d{w.head_dim} alpha {w.alpha} B {w.n_bins}",
                   "position_bias": "NAPE" if args.nape else "none"},
        "roofline": {"kernel": "dec_scores", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(achieved / 8000.0, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": kbytes},
        "kernels_ms": {kk: round(vv, 4) for kk, vv in kern.items()},
    }
    print(json.dumps(line), flush=True)


DASH_CHUNK, DASH_GAMMA, DASH_SIGMA = 64, 36.0, 1.0


def dash_workload():
    """16K-token DashAttention forward: b1, 32 query / 2 KV heads, d 128, bf16, chunks of 64
    (256 chunks), routing alpha 1.5 with gamma 36 (about 75% of the causal keys skipped on
    these inputs), sigma 1."""
    import synth
    return synth.Workload("D16K", 1, 32, 2, 16384, 128, "bf16", 1.5, True, 64, 64, 16, "normal", seed=0)


def dash_cpu_baseline(w, q, k, v, ks, do, target_s: float):
    """The fp64 DashAttention oracle, forward and backward, on evenly spaced query rows until
    ~target_s; the time per row is extrapolated to all rows (a row's cost grows with the keys
    it attends, which the even spacing samples; the backward of a row does all of that row's
    work, also what it adds to dK, dV and the summaries' gradient)."""
    import numpy as np
    import oracle.dash as odash
    n = w.seqlen
    q64, k64, v64, s64, d64 = (t.double().numpy() for t in (q, k, v, ks, do))
    done, t0, step = 0, time.time(), 1024
    while time.time() - t0 < target_s and step >= 1:
        rows = np.arange(step // 2, n, step)
        odash.dash_fwd(q64, k64, v64, s64, w.alpha, DASH_GAMMA, DASH_SIGMA, DASH_CHUNK, rows=rows)
        odash.dash_bwd(q64, k64, v64, s64, d64, w.alpha, DASH_GAMMA, DASH_SIGMA, DASH_CHUNK, rows=rows)
        done += rows.size
        step //= 2
    el = time.time() - t0
    s_per_step = el / done * n * w.batch
    return {"value": w.batch * n / s_per_step, "unit": "tokens/s", "ms_per_step": s_per_step * 1e3,
            "cores": 1, "kind": "oracle",
            "sample": f"forward and backward of {done} of {n} query rows (all heads), evenly spaced, {el:.1f} s, "
                      "extrapolated to all rows"}


def dash_bench(args, lce, dev):
    """One DashAttention training step (stages 1-2, forward then backward) per step; the
    forward alone is timed beside it. Roofline of the slowest of the three stage-2 kernels,
    on MFMA FLOPs of the tiles it must multiply: per query head and (32-row block, 32-key
    sub-block) pair where the sub-block lies in a chunk that some row of the block routes, or
    in the block's diagonal chunk, 2 d x 32 x 32 per product -- the forward's score and P.V
    products (2), the dK/dV kernel's score, dP, dV and dK products (4), the dQ kernel's score,
    dP and dQ products (3). The FLOPs per attended (row, key) pair are reported beside it."""
    import torch
    import synth
    w = dash_workload()
    inp = synth.make_inputs(w, device=dev, need_grad_inputs=True)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    ks = synth.chunk_summaries(w, DASH_CHUNK, device=dev)
    desc = lce.make_dash_desc(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim, lce.ENTMAX_BF16, DASH_CHUNK,
                              w.alpha, DASH_GAMMA, DASH_SIGMA)
    L = lce.lib()
    ws = torch.empty(L.entmax_dash_fwd_workspace_bytes(ctypes.byref(desc)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(L.entmax_dash_bwd_workspace_bytes(ctypes.byref(desc)), dtype=torch.uint8, device=dev)
    fwd = lambda: lce.dash_fwd(q, k, v, ks, DASH_CHUNK, w.alpha, DASH_GAMMA, DASH_SIGMA, workspace=ws)

    def train_step():
        r = fwd()
        g = lce.dash_bwd(q, k, v, ks, do, r.o, r.lse, r.route_tau, r.route_w, r.chunk_mask, DASH_CHUNK, w.alpha,
                         DASH_GAMMA, DASH_SIGMA, workspace=wsb)
        return r, g

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            out = fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, out

    t0 = time.time()
    ms_fwd, r = timed(fwd)
    ms, _ = timed(train_step)
    wall = time.time() - t0
    if args.copy_probe_mib > 0:
        # a plain fp32 copy of known size, the reference for scaling the traffic counters
        src = torch.ones(args.copy_probe_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    lce.profile(True)
    lce.profile_read()
    for _ in range(args.steps):
        train_step()
    torch.cuda.synchronize()
    kt = lce.profile_read()
    lce.profile(False)
    kern = {name: t / max(c, 1) for name, (t, c) in kt.items()}
    n, d, C, G = w.seqlen, w.head_dim, DASH_CHUNK, w.heads_q // w.heads_kv
    routed = (r.route_w > 0).sum(dim=2).to(torch.float64)                 # [b, hkv, n]
    rows = torch.arange(n, device=dev, dtype=torch.float64)
    keys = (routed * C + (rows % C + 1)).sum().item() * G                 # over query heads
    causal_keys = w.batch * w.heads_q * n * (n + 1) / 2.0
    # work the kernels do: every 32-key sub-block of a chunk that some row of a 32-row block
    # routes (plus the diagonal run), for each query head
    nb32 = n // 32
    blk_routed = (r.route_w > 0).view(w.batch, w.heads_kv, n // C, nb32, 32).any(dim=4)   # [b,hkv,nc,nb32]
    diag_sub = ((torch.arange(nb32, device=dev) * 32) % C) // 32 + 1                        # diagonal sub-blocks
    visited = (blk_routed.sum(dim=2).to(torch.float64) * (C // 32) + diag_sub).sum().item() * G
    tile = 2.0 * d * 32 * 32 * visited                                     # one product over the tiles
    flops = {"dash_attn": 2 * tile, "dash_bwd_dkv": 4 * tile, "dash_bwd_dq": 3 * tile}
    alg_route = 2.0 * d * w.batch * w.heads_q * float((torch.div(rows, C, rounding_mode="floor")).sum().item())
    tflops = {kk: f / (kern[kk] * 1e-3) / 1e12 for kk, f in flops.items()}
    dom = max(flops, key=lambda kk: kern[kk])
    line = {
        "metric": "dash_train_tokens_per_s", "value": round(w.batch * n / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (normal recipe; chunk summaries drawn with the spread of a 64-key mean)",
        "config": {"workload": f"DashAttention forward + backward {w.name}: b{w.batch} hq{w.heads_q}/hkv{w.heads_kv} "
                               f"n{n} d{d} bf16, chunk {C}, routing alpha {w.alpha}, gamma {DASH_GAMMA}, "
                               f"sigma {DASH_SIGMA}",
                   "key_sparsity": round(1.0 - keys / causal_keys, 4)},
        "fwd_ms_per_step": round(ms_fwd, 4),
        "fwd_tokens_per_s": round(w.batch * n / (ms_fwd * 1e-3), 1),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(tflops[dom], 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops[dom] / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": flops[dom]},
        "kernels_ms": {kk: round(vv, 4) for kk, vv in kern.items()},
        "kernel_tflops": dict({kk: round(vv, 2) for kk, vv in tflops.items()},
                              dash_route=round(alg_route / (kern["dash_route"] * 1e-3) / 1e12, 2),
                              dash_attn_per_attended_key=round(2.0 * 2.0 * d * keys / (kern["dash_attn"] * 1e-3) / 1e12,
                                                               2)),
        "dash_attn_tiles_over_attended_keys": round(tile / (2.0 * d * keys), 3),
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline and not args.profile_only:
        line["cpu_baseline"] = dash_cpu_baseline(w, q.cpu(), k.cpu(), v.cpu(), ks.cpu(), do.cpu(), args.cpu_seconds)
    print(json.dumps(line), flush=True)


def make_problem(lce, w, dev, tau_init: int = 0, nape: bool = False):
    """Inputs, outputs and workspaces of one workload, resident on the device."""
    import torch
    import synth
    inp = synth.make_inputs(w, device=dev)
    q = inp["q"]
    b, hq, n, d = q.shape
    blk = (w.block_q, w.block_k)
    Tr, W = lce.mask_shape(n, blk)
    outs = lce.FwdOut(torch.empty(q.shape, dtype=torch.float32, device=dev),
                      torch.empty((b, hq, n), dtype=torch.float32, device=dev),
                      torch.empty((b, hq, Tr, W), dtype=torch.int32, device=dev),
                      torch.empty((b, hq, n, d), dtype=torch.float32, device=dev), None, None)
    grads = (torch.empty_like(q), torch.empty_like(inp["k"]), torch.empty_like(inp["v"]))
    slopes = (torch.tensor(lce.nape_slopes(hq), dtype=torch.float32, device=dev) if nape else None)
    desc = lce._desc_for(q, inp["k"], w.alpha, w.causal, blk, w.n_bins, None, 0, 0.0, tau_init)
    fws, bws = lce.workspace_bytes(desc)
    return {"inp": inp, "outs": outs, "grads": grads, "slopes": slopes, "tau_init": tau_init, "blk": blk,
            "wsf": torch.empty(max(fws, 256), dtype=torch.uint8, device=dev),
            "wsb": torch.empty(max(bws, 256), dtype=torch.uint8, device=dev)}


def time_point(lce, w, prob, steps: int, warmup: int, dense: bool = False, copy_probe_mib: int = 0):
    """Warm up, time `steps` fwd+bwd steps between synchronisations, then the same steps with
    HIP events around every kernel, then one untimed step for the method's statistics."""
    import torch
    inp, outs, grads, blk = prob["inp"], prob["outs"], prob["grads"], prob["blk"]
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    dev = q.device

    def step(stats=None):
        r = lce.fwd(q, k, v, w.alpha, w.causal, blk, w.n_bins, workspace=prob["wsf"], out=outs, stats=stats,
                    tau_init=prob["tau_init"], slopes=prob["slopes"], dense=dense)
        lce.bwd(q, k, v, do, r.tau, r.mask, r.aux, w.alpha, w.causal, blk, w.n_bins, workspace=prob["wsb"],
                out=grads, slopes=prob["slopes"], dense=dense)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = e0.elapsed_time(e1) / steps
    if copy_probe_mib > 0:
        nel = copy_probe_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    # per-kernel HIP-event timing (same steps, separate loop, events recorded on the stream
    # each kernel is launched on)
    lce.profile(True)
    lce.profile_read()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ktimes = lce.profile_read()
    lce.profile(False)
    stats = torch.zeros(32, dtype=torch.int64, device=dev)
    step(stats)
    torch.cuda.synchronize()
    st = stats.cpu().tolist()
    b, hq, n, d = q.shape
    nnzb = popcount_mask(outs.mask)
    nvb = valid_blocks(w) * b * hq
    blockflop = 2.0 * w.block_q * w.block_k * d
    subflop = 2.0 * 32 * 32 * d
    # algorithmic MFMA FLOPs per launch: one 32x32xd score product per sub-block the
    # histogram pass scores and per refinement visit, a score and a P.V product per
    # output visit, and per non-zero Br x Bc block 4 products in dK/dV and 3 in dQ
    alg = {
        "entmax_fwd_hist": subflop * st[20],
        "entmax_fwd_refine_out": subflop * (st[21] + 2 * st[22]),
        "entmax_bwd_dkv": 4 * blockflop * nnzb,
        "entmax_bwd_dq": 3 * blockflop * nnzb,
    }
    kern = {name: tt / max(c, 1) for name, (tt, c) in ktimes.items()}
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    # MFMA utilisation on the non-zero blocks: the 10 products of a non-zero block (3
    # forward, 7 backward) over the time of the kernels that multiply blocks (refinement
    # and output, dK/dV, dQ), against the dtype's dense peak
    t_blk = sum(kern.get(nm, 0.0) for nm in ("entmax_fwd_refine_out", "entmax_bwd_dkv", "entmax_bwd_dq"))
    sbu = 10.0 * blockflop * nnzb / (t_blk * 1e-3) / 1e12 / peak if t_blk > 0 else None
    return {"ms": ms, "wall": wall, "kern": kern, "alg": alg, "stats": st, "nnzb": nnzb, "nvb": nvb,
            "sparsity": 1.0 - nnzb / nvb, "peak": peak, "sparse_block_mfma_util": sbu}


def workload_label(w):
    return (f"{w.name}: b{w.batch} hq{w.heads_q}/hkv{w.heads_kv} n{w.seqlen} d{w.head_dim} "
            f"{w.dtype} {'causal' if w.causal else 'full'} alpha {w.alpha:g} blocks "
            f"{w.block_q}x{w.block_k} B {w.n_bins}")


SWEEP_POINTS = [
    # (workload, alpha, target block sparsity, configured point of the study?)
    ("C1", None, None, True),
    ("C2", 1.5, 0.0, True), ("C2", 1.5, 0.3, False), ("C2", 1.5, 0.6, True), ("C2", 1.5, 0.8, False),
    ("C2", 1.5, 0.9, True), ("C2", 1.5, 0.95, False),
    ("C2", 2.0, 0.0, True), ("C2", 2.0, 0.3, False), ("C2", 2.0, 0.6, True), ("C2", 2.0, 0.8, False),
    ("C2", 2.0, 0.9, True), ("C2", 2.0, 0.95, False),
    ("C3", 1.5, 0.6, True), ("C3", 1.5, 0.7, False), ("C3", 1.5, 0.8, True), ("C3", 1.5, 0.9, False),
    ("C3", 1.5, 0.95, True),
    ("C4", 2.0, 0.95, True),
    ("C5", 1.5, 0.97, True),
]


def fit_line(xs, ys):
    """Least-squares t = a + b x and its R^2."""
    nn = len(xs)
    mx, my = sum(xs) / nn, sum(ys) / nn
    sxx = sum((x - mx) ** 2 for x in xs)
    sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
    bb = sxy / sxx if sxx > 0 else 0.0
    aa = my - bb * mx
    ss_tot = sum((y - my) ** 2 for y in ys)
    ss_res = sum((y - aa - bb * x) ** 2 for x, y in zip(xs, ys))
    return aa, bb, (1.0 - ss_res / ss_tot) if ss_tot > 0 else 1.0


def sweep(args, lce, dev):
    import torch
    import synth
    from synth.betas import key, load_table
    table = load_table()
    rows = []
    for name, alpha, target, configured in SWEEP_POINTS:
        if name != "C1" and key(name, alpha, target) not in table:
            print(json.dumps({"sweep_point": f"{name} alpha {alpha} sparsity {target}",
                              "skipped": "no calibrated beta"}), flush=True)
            continue
        w = synth.workload(name, alpha=alpha, sparsity=target)
        print(f"[sweep] {workload_label(w)} target sparsity {target}", file=sys.stderr, flush=True)
        prob = make_problem(lce, w, dev)
        big = w.seqlen >= 65536
        steps = 5 if big else args.steps
        r = time_point(lce, w, prob, steps, 2 if big else args.warmup)
        # the skipping run's results, to check that the ablation does not change them
        ref = prob["outs"]
        o_skip, tau_skip = ref.o.clone(), ref.tau.clone()
        g_skip = [g.clone() for g in prob["grads"]]
        print(f"[sweep] skipping: {r['ms']:.4f} ms/step", file=sys.stderr, flush=True)
        rd = time_point(lce, w, prob, 3 if big else max(3, args.steps // 4), 1, dense=True)
        print(f"[sweep] dense ablation: {rd['ms']:.4f} ms/step", file=sys.stderr, flush=True)
        eff = dense_eq_flops(w) / (r["ms"] * 1e-3) / 1e12
        alg_total = sum(r["alg"].values())
        passes = {str(p): r["stats"][p] for p in range(1, 17) if r["stats"][p]}
        row = {
            "sweep_point": workload_label(w), "configured_point": configured,
            "target_block_sparsity": target, "beta": w.beta,
            "achieved_block_sparsity": round(r["sparsity"], 4), "nonzero_blocks": r["nnzb"],
            "valid_blocks": r["nvb"], "ms_per_step": round(r["ms"], 4),
            "effective_tflops": round(eff, 2),
            "algorithmic_tflops": round(alg_total / (r["ms"] * 1e-3) / 1e12, 2),
            "algorithmic_frac_of_peak": round(alg_total / (r["ms"] * 1e-3) / 1e12 / r["peak"], 4),
            "sparse_block_mfma_util": None if r["sparse_block_mfma_util"] is None
            else round(r["sparse_block_mfma_util"], 4),
            "kernels_ms": {kk: round(vv, 4) for kk, vv in r["kern"].items()},
            "refine_passes_rows": passes,
            "dense_ablation_ms": round(rd["ms"], 4),
            "dense_ablation_kernels_ms": {kk: round(vv, 4) for kk, vv in rd["kern"].items()},
            "skip_speedup": round(rd["ms"] / r["ms"], 3),
        }
        row["dense_vs_skip_max_abs"] = {
            "o": float((ref.o - o_skip).abs().max()), "tau": float((ref.tau - tau_skip).abs().max()),
            "dq": float((prob["grads"][0].float() - g_skip[0].float()).abs().max()),
            "dk": float((prob["grads"][1].float() - g_skip[1].float()).abs().max()),
            "dv": float((prob["grads"][2].float() - g_skip[2].float()).abs().max())}
        print(json.dumps(row), flush=True)
        rows.append((name, alpha, row))
        del prob
        torch.cuda.empty_cache()
    fits = {}
    for name, alpha in (("C2", 1.5), ("C2", 2.0), ("C3", 1.5)):
        pts = [(rw["nonzero_blocks"], rw["ms_per_step"]) for nm, al, rw in rows if nm == name and al == alpha]
        if len(pts) >= 3:
            aa, bb, r2 = fit_line([p[0] for p in pts], [p[1] for p in pts])
            fits[f"{name} alpha {alpha:g}"] = {"points": len(pts), "a_ms": round(aa, 5),
                                               "b_us_per_kblock": round(bb * 1e6, 4), "r2": round(r2, 5)}
    print(json.dumps({"sweep_fits": fits}), flush=True)
    if args.sweep_md:
        with open(args.sweep_md, "w") as fh:
            fh.write("# Block-sparsity sweep: alpha-entmax attention fwd+bwd on one MI355X\n\n"
                     "Command: `python3 bench.py --sweep --sweep-md <this file>` (bench.py at the "
                     f"repository root; kernel sources digest `{src_digest()}`). Step times in ms "
                     "(forward + backward, inputs resident in HBM); the dense ablation multiplies "
                     "every causally valid block; a and b fit ms = a + b * nnzb per sweep.\n\n")
            fh.write("| point | configured | sparsity | nnzb | ms/step | eff. TFLOP/s | alg. TFLOP/s | "
                     "sparse-block MFMA util | dense ablation ms | skip speed-up | passes |\n")
            fh.write("|---|---|---|---|---|---|---|---|---|---|---|\n")
            for nm, al, rw in rows:
                fh.write(f"| {rw['sweep_point']} | {'yes' if rw['configured_point'] else 'extra'} | "
                         f"{rw['achieved_block_sparsity']} | {rw['nonzero_blocks']} | {rw['ms_per_step']} | "
                         f"{rw['effective_tflops']} | {rw['algorithmic_tflops']} | "
                         f"{rw['sparse_block_mfma_util']} | {rw['dense_ablation_ms']} | {rw['skip_speedup']} | "
                         f"{rw['refine_passes_rows']} |\n")
            fh.write("\n| sweep | points | a (ms) | b (us per 1000 non-zero blocks) | R^2 |\n|---|---|---|---|---|\n")
            for kk, vv in fits.items():
                fh.write(f"| {kk} | {vv['points']} | {vv['a_ms']} | {vv['b_us_per_kblock']} | {vv['r2']} |\n")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 (multi-GPU "
                                   "sharding is described, not implemented)"}))
        sys.exit(2)
    import torch
    import synth
    import long_context_entmax_amd as lce

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.dash:
        dash_bench(args, lce, dev)
        return
    if args.sweep:
        sweep(args, lce, dev)
        return
    w = synth.workload(args.config, alpha=args.alpha, sparsity=args.sparsity)
    if args.decode:
        inp = synth.make_inputs(w, device=dev, need_grad_inputs=False)
        decode_bench(args, lce, w, inp, dev)
        return
    tau_init = 0 if args.tau_init == "hist" else 1
    print(f"[bench] {workload_label(w)}", file=sys.stderr, flush=True)
    prob = make_problem(lce, w, dev, tau_init, args.nape)
    if args.tau_error:
        inp = prob["inp"]
        print(json.dumps(tau_error_study(lce, w, inp["q"], inp["k"], inp["v"], prob["blk"], prob["wsf"])),
              flush=True)
        return
    r = time_point(lce, w, prob, args.steps, args.warmup, dense=args.dense, copy_probe_mib=args.copy_probe_mib)
    print(f"[bench] timed: {r['ms']:.4f} ms/step", file=sys.stderr, flush=True)
    kern, alg, st = r["kern"], r["alg"], r["stats"]
    ms = r["ms"]
    dom = max(alg, key=lambda nm: kern.get(nm, 0.0))
    peak = r["peak"]
    achieved = alg[dom] / (kern[dom] * 1e-3) / 1e12
    # HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    # summary of this workload (FETCH_SIZE + WRITE_SIZE scaled by a copy of known size);
    # null when the kernel sources changed since the counters were taken
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"entmax_attn_{w.name}_traffic.json")
    if os.path.exists(tfile) and not args.dense and not args.nape and tau_init == 0:
        with open(tfile) as f:
            tj = json.load(f)
        if tj.get("src_digest") == src_digest() and tj.get("workload") == w.name:
            traffic = tj.get("kernels", {}).get(dom, {}).get("bytes_per_launch")
    passes = {str(p): st[p] for p in range(1, 17) if st[p]}
    sub_stats = {"hist_subblocks": st[20], "refine_visits": st[21], "output_visits": st[22],
                 "candidate_subblocks": st[23]}
    eff = dense_eq_flops(w) / (ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(eff, 3),
        "unit": "TFLOP/s (effective, dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded centroid-cluster generator, beta calibrated to the target block sparsity)",
        "config": {
            "workload": workload_label(w),
            "tau_start": "histogram" if tau_init == 0 else "plain bracket (ablation)",
            "position_bias": "NAPE (half the heads ALiBi)" if args.nape else "none",
            "block_skipping": "off (dense ablation)" if args.dense else "on",
            "target_block_sparsity": w.target_sparsity, "beta": w.beta,
            "achieved_block_sparsity": round(r["sparsity"], 4), "nonzero_blocks": r["nnzb"],
            "valid_blocks": r["nvb"],
        },
        "roofline": {
            "kernel": dom, "bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
            "algorithmic_flops_per_launch": alg[dom],
        },
        "sparse_block_mfma_util": None if r["sparse_block_mfma_util"] is None
        else round(r["sparse_block_mfma_util"], 4),
        "kernels_ms": {kk: round(vv, 4) for kk, vv in kern.items()},
        "kernel_tflops": {kk: round(alg[kk] / (kern[kk] * 1e-3) / 1e12, 2) for kk in alg if kk in kern},
        "refine_passes_rows": passes,
        "subblock_stats": sub_stats,
        "wall_s": round(r["wall"], 3),
    }
    if not args.no_cpu_baseline and not args.profile_only:
        inp_cpu = {kk: vv.cpu() for kk, vv in prob["inp"].items() if hasattr(vv, "cpu")}
        line["cpu_baseline"] = cpu_baseline(w, inp_cpu, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

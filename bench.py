"""Benchmark: alpha-entmax attention fwd+bwd step on one MI355X.

A step is one forward and one backward of the whole hot path (histogram pass,
refinement, output pass, backward preparation, dK/dV and dQ kernels) over one
batch of synthetic inputs resident in HBM. The default workload is the 4K-token
configuration (batch 4, 8 heads, n 4096, d 64, bf16, causal, alpha 1.5, 64x64
blocks, B 16) with the centroid-cluster generator calibrated to ~90% block
sparsity; ``--config C3|C4|C5`` and ``--alpha``/``--sparsity`` select the others.

Prints one JSON line: value = effective TFLOP/s (dense-equivalent FLOPs of a causal
attention fwd+bwd, 3.5 x 4 b h n^2 d / 2, divided by the measured step time),
plus a roofline object for the dominant kernel (algorithmic MFMA FLOPs per launch
over its HIP-event-timed average duration) and the CPU oracle timed on a bounded
sample of the same workload.
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
    ap.add_argument("--config", default="C2")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--sparsity", type=float, default=None)
    ap.add_argument("--tau-init", choices=("hist", "bracket"), default="hist",
                    help="refinement start: the histogram bound (the method) or the plain "
                         "[x_max - 1, x_max - n^(1-alpha)] bracket (ablation)")
    ap.add_argument("--nape", action="store_true",
                    help="NAPE heads: the first half of the query heads without position "
                         "encoding, the second half ALiBi (per-head slopes of the scores)")
    ap.add_argument("--decode", action="store_true",
                    help="time one decode step (a new query row per head against the workload's "
                         "K/V as a cache) instead of the training step")
    ap.add_argument("--dash", action="store_true",
                    help="DashAttention forward (routing + prior-induced sparse softmax) at 16K tokens "
                         "instead of the entmax attention step")
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


def src_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "long_context_entmax_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
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


def cpu_baseline(w, inp_cpu, target_s: float):
    """Time the fp64 oracle (fwd + bwd) on whole query heads until ~target_s, extrapolate."""
    import oracle
    threads = oracle.default_threads()
    G = w.heads_q // w.heads_kv
    scale = 1.0 / math.sqrt(w.head_dim)
    heads_done = 0
    t0 = time.time()
    for bi in range(w.batch):
        for h in range(w.heads_q):
            if heads_done > 0 and time.time() - t0 > target_s:
                break
            kh = h // G
            qh = inp_cpu["q"][bi, h].double().numpy()
            kk = inp_cpu["k"][bi, kh].double().numpy()
            vv = inp_cpu["v"][bi, kh].double().numpy()
            do = inp_cpu["do"][bi, h].double().numpy()
            f = oracle.attn_fwd_head(qh, kk, vv, w.alpha, w.causal, w.n_bins, w.block_k, scale,
                                     threads=threads)
            r = oracle.attn_bwd_rows_head(qh, kk, vv, do, f["tau"], w.alpha, w.causal, scale,
                                          threads=threads)
            # the key-side backward of this query head's share of its KV head
            oracle.attn_bwd_keys_group(qh[None], kk, vv, do[None], f["tau"][None], r["delta"][None],
                                       w.alpha, w.causal, scale, threads=threads)
            heads_done += 1
    el = time.time() - t0
    total_heads = w.batch * w.heads_q
    s_per_step = el * total_heads / heads_done
    return {
        "value": dense_eq_flops(w) / s_per_step / 1e12,
        "unit": "TFLOP/s (effective)",
        "ms_per_step": s_per_step * 1e3,
        "cores": threads,
        "kind": "oracle",
        "sample": f"{heads_done} of {total_heads} query heads, full length, fwd+bwd, {el:.1f} s, "
                  f"extrapolated linearly to all heads",
    }


def tau_error_study(lce, w, q, k, v, blk, wsf):
    """Mean absolute error of tau per refinement pass, histogram start vs plain bracket
    (the study of the pages' Fig. 3, page 5 section 4). tau* is the histogram-started solve
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


def dash_cpu_baseline(w, q, k, v, ks, target_s: float):
    """The fp64 DashAttention oracle on evenly spaced query rows until ~target_s; the time
    per row is extrapolated to all rows (its cost grows with the keys a row attends, which
    the even spacing samples)."""
    import numpy as np
    import oracle.dash as odash
    n = w.seqlen
    q64, k64, v64, s64 = (t.double().numpy() for t in (q, k, v, ks))
    done, t0, step = 0, time.time(), 1024
    while time.time() - t0 < target_s and step >= 1:
        rows = np.arange(step // 2, n, step)
        odash.dash_fwd(q64, k64, v64, s64, w.alpha, DASH_GAMMA, DASH_SIGMA, DASH_CHUNK, rows=rows)
        done += rows.size
        step //= 2
    el = time.time() - t0
    s_per_step = el / done * n * w.batch
    return {"value": w.batch * n / s_per_step, "unit": "tokens/s", "ms_per_step": s_per_step * 1e3,
            "cores": 1, "kind": "oracle",
            "sample": f"{done} of {n} query rows (all heads), evenly spaced, {el:.1f} s, extrapolated to all rows"}


def dash_bench(args, lce, dev):
    """One DashAttention forward (stages 1-2) per step. Roofline of the stage-2 kernel: MFMA
    FLOPs of the tiles it must multiply -- 4 d x 32 x 32 (score and P.V products) per query
    head and (32-row block, 32-key sub-block) pair where the sub-block lies in a chunk that
    some row of the block routes, or in the block's diagonal chunk. The FLOPs per attended
    (row, key) pair, 4 d each, are reported beside it."""
    import torch
    import synth
    w = dash_workload()
    inp = synth.make_inputs(w, device=dev, need_grad_inputs=False)
    q, k, v = inp["q"], inp["k"], inp["v"]
    ks = synth.chunk_summaries(w, DASH_CHUNK, device=dev)
    desc = lce.make_dash_desc(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim, lce.ENTMAX_BF16, DASH_CHUNK,
                              w.alpha, DASH_GAMMA, DASH_SIGMA)
    ws = torch.empty(lce.lib().entmax_dash_fwd_workspace_bytes(ctypes.byref(desc)), dtype=torch.uint8, device=dev)
    step = lambda: lce.dash_fwd(q, k, v, ks, DASH_CHUNK, w.alpha, DASH_GAMMA, DASH_SIGMA, workspace=ws)
    for _ in range(args.warmup):
        r = step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    e0.record()
    for _ in range(args.steps):
        r = step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = e0.elapsed_time(e1) / args.steps
    lce.profile(True)
    lce.profile_read()
    for _ in range(args.steps):
        r = step()
    torch.cuda.synchronize()
    kt = lce.profile_read()
    lce.profile(False)
    kern = {name: t / max(c, 1) for name, (t, c) in kt.items()}
    n, d, C, G = w.seqlen, w.head_dim, DASH_CHUNK, w.heads_q // w.heads_kv
    routed = (r.route_w > 0).sum(dim=2).to(torch.float64)                 # [b, hkv, n]
    rows = torch.arange(n, device=dev, dtype=torch.float64)
    keys = (routed * C + (rows % C + 1)).sum().item() * G                 # over query heads
    causal_keys = w.batch * w.heads_q * n * (n + 1) / 2.0
    alg_attn = 4.0 * d * keys
    # work the kernel does: every 32-key sub-block of a chunk that some row of a 32-row block
    # routes (plus the diagonal run), for each query head
    nb32 = n // 32
    blk_routed = (r.route_w > 0).view(w.batch, w.heads_kv, n // C, nb32, 32).any(dim=4)   # [b,hkv,nc,nb32]
    diag_sub = ((torch.arange(nb32, device=dev) * 32) % C) // 32 + 1                        # diagonal sub-blocks
    visited = (blk_routed.sum(dim=2).to(torch.float64) * (C // 32) + diag_sub).sum().item() * G
    visited_flops = 4.0 * d * 32 * 32 * visited
    alg_route = 2.0 * d * w.batch * w.heads_q * float((torch.div(rows, C, rounding_mode="floor")).sum().item())
    achieved = visited_flops / (kern["dash_attn"] * 1e-3) / 1e12
    line = {
        "metric": "dash_fwd_tokens_per_s", "value": round(w.batch * n / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (normal recipe; chunk summaries drawn with the spread of a 64-key mean)",
        "config": {"workload": f"DashAttention forward {w.name}: b{w.batch} hq{w.heads_q}/hkv{w.heads_kv} "
                               f"n{n} d{d} bf16, chunk {C}, routing alpha {w.alpha}, gamma {DASH_GAMMA}, "
                               f"sigma {DASH_SIGMA}",
                   "key_sparsity": round(1.0 - keys / causal_keys, 4)},
        "roofline": {"kernel": "dash_attn", "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": visited_flops},
        "kernels_ms": {kk: round(vv, 4) for kk, vv in kern.items()},
        "kernel_tflops": {"dash_route": round(alg_route / (kern["dash_route"] * 1e-3) / 1e12, 2),
                          "dash_attn": round(achieved, 2),
                          "dash_attn_per_attended_key": round(alg_attn / (kern["dash_attn"] * 1e-3) / 1e12, 2)},
        "dash_attn_tiles_over_attended_keys": round(visited_flops / alg_attn, 3),
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline and not args.profile_only:
        line["cpu_baseline"] = dash_cpu_baseline(w, q.cpu(), k.cpu(), v.cpu(), ks.cpu(), args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (multi-GPU "
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
    w = synth.workload(args.config, alpha=args.alpha, sparsity=args.sparsity)
    inp = synth.make_inputs(w, device=dev, need_grad_inputs=not args.decode)
    if args.decode:
        decode_bench(args, lce, w, inp, dev)
        return
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    blk = (w.block_q, w.block_k)
    b, hq, n, d = q.shape
    Tr, W = lce.mask_shape(n, blk)
    outs = lce.FwdOut(torch.empty(q.shape, dtype=torch.float32, device=dev),
                      torch.empty((b, hq, n), dtype=torch.float32, device=dev),
                      torch.empty((b, hq, Tr, W), dtype=torch.int32, device=dev),
                      torch.empty((b, hq, n, d), dtype=torch.float32, device=dev), None, None)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    tau_init = 0 if args.tau_init == "hist" else 1
    slopes = (torch.tensor(lce.nape_slopes(hq), dtype=torch.float32, device=dev) if args.nape else None)
    desc = lce._desc_for(q, k, w.alpha, w.causal, blk, w.n_bins, None, 0, 0.0, tau_init)
    fws, bws = lce.workspace_bytes(desc)
    wsf = torch.empty(max(fws, 256), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(bws, 256), dtype=torch.uint8, device=dev)

    if args.tau_error:
        print(json.dumps(tau_error_study(lce, w, q, k, v, blk, wsf)), flush=True)
        return

    def step(stats=None):
        r = lce.fwd(q, k, v, w.alpha, w.causal, blk, w.n_bins, workspace=wsf, out=outs, stats=stats,
                    tau_init=tau_init, slopes=slopes)
        lce.bwd(q, k, v, do, r.tau, r.mask, r.aux, w.alpha, w.causal, blk, w.n_bins, workspace=wsb,
                out=grads, slopes=slopes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.time()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = e0.elapsed_time(e1) / args.steps

    if args.copy_probe_mib > 0:
        nel = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # per-kernel HIP-event timing (same steps, separate loop, events recorded on the
    # stream each kernel is launched on)
    lce.profile(True)
    lce.profile_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = lce.profile_read()
    lce.profile(False)
    # method statistics from one extra, untimed step
    stats = torch.zeros(32, dtype=torch.int64, device=dev)
    step(stats)
    torch.cuda.synchronize()
    st = stats.cpu().tolist()
    nnzb = popcount_mask(outs.mask)
    nvb = valid_blocks(w) * b * hq
    sparsity = 1.0 - nnzb / nvb
    blockflop = 2.0 * w.block_q * w.block_k * d
    subflop = 2.0 * 32 * 32 * d
    # algorithmic MFMA FLOPs per launch: one 32x32xd score product per sub-block the
    # histogram pass scores and per refinement visit, a score and a P.V product per
    # output visit, and per non-zero 64x64 block 4 products in dK/dV and 3 in dQ
    alg = {
        "entmax_fwd_hist": subflop * st[20],
        "entmax_fwd_refine_out": subflop * (st[21] + 2 * st[22]),
        "entmax_bwd_dkv": 4 * blockflop * nnzb,
        "entmax_bwd_dq": 3 * blockflop * nnzb,
    }
    kern = {name: {"avg_ms": t / max(c, 1), "launches_per_step": c / args.steps}
            for name, (t, c) in ktimes.items()}
    dom = max(alg, key=lambda nm: kern.get(nm, {"avg_ms": 0})["avg_ms"])
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = alg[dom] / (kern[dom]["avg_ms"] * 1e-3) / 1e12
    # HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    # summary of this workload (FETCH_SIZE + WRITE_SIZE scaled by a copy of known size);
    # null when the kernel sources changed since the counters were taken
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"entmax_attn_{w.name}_traffic.json")
    if os.path.exists(tfile):
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
            "workload": f"{w.name}: b{w.batch} hq{w.heads_q}/hkv{w.heads_kv} n{w.seqlen} d{w.head_dim} "
                        f"{w.dtype} {'causal' if w.causal else 'full'} alpha {w.alpha} blocks "
                        f"{w.block_q}x{w.block_k} B {w.n_bins}",
            "tau_start": "histogram" if tau_init == 0 else "plain bracket (ablation)",
            "position_bias": "NAPE (half the heads ALiBi)" if args.nape else "none",
            "target_block_sparsity": w.target_sparsity, "beta": w.beta,
            "achieved_block_sparsity": round(sparsity, 4), "nonzero_blocks": nnzb, "valid_blocks": nvb,
        },
        "roofline": {
            "kernel": dom, "bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
            "algorithmic_flops_per_launch": alg[dom],
        },
        "kernels_ms": {kk: round(vv["avg_ms"], 4) for kk, vv in kern.items()},
        "kernel_tflops": {kk: round(alg[kk] / (kern[kk]["avg_ms"] * 1e-3) / 1e12, 2)
                          for kk in alg if kk in kern},
        "refine_passes_rows": passes,
        "subblock_stats": sub_stats,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline and not args.profile_only:
        inp_cpu = {kk: vv.cpu() for kk, vv in inp.items() if hasattr(vv, "cpu")}
        line["cpu_baseline"] = cpu_baseline(w, inp_cpu, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

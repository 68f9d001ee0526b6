"""The allocation-free decode entry point (entmax_attn_decode_noalloc, static per-device
scratch) against the workspace entry point (entmax_attn_decode) on the same inputs: two
calls in a row, the second on a smaller problem, each equal to the workspace call bit for
bit (the same kernels on the same scratch layout; a stale scratch from the first call must
not leak into the second)."""
import pytest
import torch

import synth
import long_context_entmax_amd as lce

pytestmark = pytest.mark.gpu


def _inputs(b, hq, hkv, n, d, dtype, seed):
    w = synth.Workload("dec", b, hq, hkv, n, d, dtype, 1.5, True, 32, 32, 16, "normal", seed=seed)
    inp = synth.make_inputs(w, device=torch.device("cuda:0"), need_grad_inputs=False)
    return inp["q"][:, :, n - 1].contiguous(), inp["k"], inp["v"]


def _same(a, b):
    assert a.shape == b.shape and torch.equal(a, b), (a - b).abs().max().item()


@pytest.mark.parametrize("first,second", [
    ((2, 8, 2, 4096, 64, "bf16", 1.5, [4096, 3001]), (1, 4, 1, 1000, 128, "bf16", 2.0, None)),
    ((1, 32, 8, 131072, 64, "bf16", 1.5, None), (2, 2, 2, 257, 64, "f32", 1.25, [257, 1])),
])
def test_noalloc_decode_matches_workspace_decode(first, second):
    dev = torch.device("cuda:0")
    for case in (first, second):
        b, hq, hkv, n, d, dtype, alpha, lens = case
        print(f"[case] decode_noalloc {case}", flush=True)
        q, k, v = _inputs(b, hq, hkv, n, d, dtype, seed=n + hq)
        lengths = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
        slopes = torch.tensor(lce.nape_slopes(hq), dtype=torch.float32, device=dev) if hq % 2 == 0 else None
        ref = lce.decode(q, k, v, alpha, 16, lengths=lengths, slopes=slopes, return_hist=True)
        out = lce.DecodeOut(torch.empty((b, hq, d), dtype=torch.float32, device=dev),
                            torch.empty((b, hq), dtype=torch.float32, device=dev),
                            torch.empty((b, hq, 16), dtype=torch.int32, device=dev),
                            torch.empty((b, hq), dtype=torch.float32, device=dev))
        got = lce.decode_noalloc(q, k, v, alpha, 16, lengths=lengths, slopes=slopes, out=out)
        torch.cuda.synchronize()
        for name in ("o", "tau", "hist", "tau_h"):
            _same(getattr(got, name), getattr(ref, name))
        # without out=: outputs allocated by the binding, counts not requested
        got2 = lce.decode_noalloc(q, k, v, alpha, 16, lengths=lengths, slopes=slopes)
        torch.cuda.synchronize()
        _same(got2.o, ref.o)
        _same(got2.tau, ref.tau)

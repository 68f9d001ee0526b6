"""bench.py on the host: the multi-GPU refusal and the source digest that guards the
committed counter summaries (no GPU needed)."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_digest_covers_the_prefill_sources_only():
    b = _bench()
    csrc = os.path.join(ROOT, "long_context_entmax_amd", "csrc")
    for f in b.PREFILL_SOURCES:
        assert os.path.exists(os.path.join(csrc, f)), f
    assert "decode.hip" not in b.PREFILL_SOURCES and "dash.hip" not in b.PREFILL_SOURCES
    d = b.src_digest()
    assert len(d) == 16 and d == b.src_digest()


def test_committed_traffic_summaries_name_their_workload():
    for w in ("C2", "C3", "C5"):
        with open(os.path.join(ROOT, "profiles", f"entmax_attn_{w}_traffic.json")) as fh:
            tj = json.load(fh)
        assert tj["workload"] == w
        k = tj["kernels"]["entmax_fwd_hist"]
        assert abs(k["bytes_per_launch"] - (k["fetch_bytes"] + k["write_bytes"])) <= 1
        assert tj["copy_probe"]["fetch_scale"] > 0 and tj["copy_probe"]["write_scale"] > 0

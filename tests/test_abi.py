"""Host-side checks of the C ABI: the library loads, exports every declared entry point,
and rejects bad arguments before touching the GPU (these calls make no HIP call, so
they run without a GPU)."""
import ctypes
import os
import re

import pytest

import long_context_entmax_amd as lce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "entmax_attn.h")
DASH_HEADER = os.path.join(ROOT, "include", "dash_attn.h")


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(entmax_[a-z_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lce.LIB_PATH):
        pytest.fail("libentmax_attn.so is not built (python -m long_context_entmax_amd.build)")
    return lce.lib()


@pytest.mark.parametrize("header,struct,cls", [(HEADER, "entmax_attn_desc", lce.Desc),
                                               (DASH_HEADER, "entmax_dash_desc", lce.DashDesc)])
def test_desc_fields_match_header(header, struct, cls):
    """The binding's descriptors have the header structs' fields, in order, 4-byte types."""
    src = open(header).read()
    body = re.search(r"typedef struct \{(.*?)\} " + struct + ";", src, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        typ, _, rest = decl.partition(" ")
        assert typ in ("int32_t", "float"), decl
        names += [x.strip() for x in rest.split(",")]
    assert names == [f[0] for f in cls._fields_]
    assert ctypes.sizeof(cls) == 4 * len(names)


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lce.EXPORTS)


def _desc(**kw):
    base = dict(batch=1, heads_q=2, heads_kv=1, seqlen=256, head_dim=64, dtype=lce.ENTMAX_BF16,
                alpha=1.5, causal=True, block=(64, 64), bins=16)
    base.update(kw)
    blk = base.pop("block")
    return lce.make_desc(base["batch"], base["heads_q"], base["heads_kv"], base["seqlen"],
                         base["head_dim"], base["dtype"], base["alpha"], base["causal"], blk,
                         base["bins"], base.get("scale"), base.get("max_iters", 0), base.get("tol", 0.0),
                         base.get("tau_init", 0))


BAD = [
    (dict(alpha=1.0), 3), (dict(alpha=float("nan")), 3), (dict(alpha=0.5), 3), (dict(alpha=17.0), 3),
    (dict(heads_q=3, heads_kv=2), 2), (dict(seqlen=100), 2), (dict(seqlen=-64), 2),
    (dict(head_dim=96), 4), (dict(block=(48, 64)), 4), (dict(block=(64, 256)), 4),
    (dict(bins=12), 4), (dict(bins=32), 4), (dict(dtype=7), 4), (dict(seqlen=1 << 20), 4),
    (dict(max_iters=31), 2), (dict(heads_kv=0), 2), (dict(tau_init=2), 4), (dict(tau_init=-1), 4),
]


@pytest.mark.parametrize("kw,status", BAD, ids=[str(b[0]) for b in BAD])
def test_argument_errors(L, kw, status):
    d = _desc(**kw)
    assert L.entmax_attn_fwd_workspace_bytes(ctypes.byref(d)) == 0
    fake = ctypes.c_void_p(256)
    st = L.entmax_attn_fwd(ctypes.byref(d), fake, fake, fake, None, fake, fake, fake, fake, None, None,
                           None, fake, 1 << 30, None)
    assert st == status, L.entmax_last_error()
    assert len(L.entmax_last_error()) > 0
    st = L.entmax_attn_bwd(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, fake, fake, fake,
                           fake, fake, 1 << 30, None)
    assert st == status


def test_null_pointers_alignment_workspace(L):
    d = _desc()
    f = ctypes.c_void_p(4096)
    assert L.entmax_attn_fwd(None, f, f, f, None, f, f, f, f, None, None, None, f, 1 << 30, None) == 1
    assert L.entmax_attn_fwd(ctypes.byref(d), None, f, f, None, f, f, f, f, None, None, None, f, 1 << 30,
                             None) == 1
    mis = ctypes.c_void_p(4098)
    assert L.entmax_attn_fwd(ctypes.byref(d), mis, f, f, None, f, f, f, f, None, None, None, f, 1 << 30,
                             None) == 5
    # slopes need 4-byte alignment
    assert L.entmax_attn_fwd(ctypes.byref(d), f, f, f, mis, f, f, f, f, None, None, None, f, 1 << 30,
                             None) == 5
    need = L.entmax_attn_fwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert L.entmax_attn_fwd(ctypes.byref(d), f, f, f, None, f, f, f, f, None, None, None, f, need - 1,
                             None) == 6
    assert L.entmax_attn_fwd(ctypes.byref(d), f, f, f, None, f, f, f, f, None, None, None, None, need,
                             None) == 6
    nb = L.entmax_attn_bwd_workspace_bytes(ctypes.byref(d))
    assert L.entmax_attn_bwd(ctypes.byref(d), f, f, f, f, None, f, f, f, f, f, f, f, nb - 1, None) == 6
    assert L.entmax_attn_bwd(ctypes.byref(d), f, f, f, None, None, f, f, f, f, f, f, f, nb, None) == 1
    assert L.entmax_attn_bwd(ctypes.byref(d), f, f, f, f, mis, f, f, f, f, f, f, f, nb, None) == 5


def test_empty_problem_is_a_no_op(L):
    for kw in (dict(batch=0), dict(heads_q=0, heads_kv=1), dict(seqlen=0)):
        d = _desc(**kw)
        assert L.entmax_attn_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None, None,
                                 None, None, None, 0, None) == 0
        assert L.entmax_attn_bwd(ctypes.byref(d), None, None, None, None, None, None, None, None, None,
                                 None, None, None, 0, None) == 0


def test_sizes(L):
    d = _desc(batch=2, heads_q=8, heads_kv=2, seqlen=4096, head_dim=64, block=(128, 64))
    Tr, W = 4096 // 128, (4096 // 64 + 31) // 32
    assert L.entmax_attn_mask_words(ctypes.byref(d)) == 2 * 8 * Tr * W
    assert L.entmax_attn_aux_bytes(ctypes.byref(d)) == 2 * 8 * 4096 * 64 * 4
    assert L.entmax_attn_fwd_workspace_bytes(ctypes.byref(d)) >= 2 * 2 * 4096 * 64 * 2
    assert L.entmax_status_string(0) == b"ok"
    assert L.entmax_status_string(7) == b"HIP runtime error"


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        lce.fwd(q, q, q)


def test_decode_arguments(L):
    """Decode: seqlen is a cache capacity (no block multiple), group size at most 16,
    required pointers, alignment and workspace size."""
    d = _desc(seqlen=1000, heads_q=4, heads_kv=2)
    nb = L.entmax_attn_decode_workspace_bytes(ctypes.byref(d))
    assert nb > 0
    assert L.entmax_attn_fwd_workspace_bytes(ctypes.byref(d)) == 0     # not a forward shape
    f = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4098)
    dec = L.entmax_attn_decode
    assert dec(ctypes.byref(d), None, f, f, None, None, f, f, None, None, f, nb, None) == 1
    assert dec(ctypes.byref(d), f, f, f, None, None, None, f, None, None, f, nb, None) == 1
    assert dec(ctypes.byref(d), f, mis, f, None, None, f, f, None, None, f, nb, None) == 5
    assert dec(ctypes.byref(d), f, f, f, mis, None, f, f, None, None, f, nb, None) == 5
    assert dec(ctypes.byref(d), f, f, f, None, None, f, f, None, None, f, nb - 1, None) == 6
    big = _desc(seqlen=1000, heads_q=32, heads_kv=1)
    assert L.entmax_attn_decode_workspace_bytes(ctypes.byref(big)) == 0
    assert dec(ctypes.byref(big), f, f, f, None, None, f, f, None, None, f, 1 << 30, None) == 4
    empty = _desc(seqlen=0)
    assert dec(ctypes.byref(empty), f, f, f, None, None, f, f, None, None, f, 1 << 30, None) == 2
    assert dec(ctypes.byref(_desc(batch=0)), None, None, None, None, None, None, None, None, None,
               None, 0, None) == 0


def _dash_desc(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, seqlen=1024, head_dim=64, dtype=lce.ENTMAX_BF16,
                chunk=64, route_alpha=1.5, gamma=1.0, sigma=1.0)
    base.update(kw)
    return lce.make_dash_desc(base["batch"], base["heads_q"], base["heads_kv"], base["seqlen"], base["head_dim"],
                              base["dtype"], base["chunk"], base["route_alpha"], base["gamma"], base["sigma"],
                              base.get("scale"), base.get("max_iters", 0), base.get("tol", 0.0))


DASH_BAD = [
    (dict(route_alpha=1.0), 3), (dict(route_alpha=float("inf")), 3), (dict(heads_q=3), 2),
    (dict(chunk=32), 4), (dict(chunk=96), 4), (dict(seqlen=1000), 2), (dict(seqlen=64 * 257), 4),
    (dict(head_dim=80), 4), (dict(dtype=3), 4), (dict(sigma=-1.0), 2), (dict(gamma=float("nan")), 2),
    (dict(max_iters=31), 2), (dict(seqlen=-64), 2),
]


@pytest.mark.parametrize("kw,status", DASH_BAD, ids=[str(b[0]) for b in DASH_BAD])
def test_dash_argument_errors(L, kw, status):
    d = _dash_desc(**kw)
    assert L.entmax_dash_fwd_workspace_bytes(ctypes.byref(d)) == 0
    assert L.entmax_dash_mask_words(ctypes.byref(d)) == 0
    f = ctypes.c_void_p(256)
    st = L.entmax_dash_fwd(ctypes.byref(d), f, f, f, f, f, None, None, f, f, f, 1 << 30, None)
    assert st == status, L.entmax_last_error()
    assert L.entmax_dash_bwd_workspace_bytes(ctypes.byref(d)) == 0
    st = L.entmax_dash_bwd(ctypes.byref(d), *([f] * 14), f, 1 << 30, None)
    assert st == status, L.entmax_last_error()


def test_dash_pointers_workspace_and_sizes(L):
    d = _dash_desc()
    f = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4098)
    need = L.entmax_dash_fwd_workspace_bytes(ctypes.byref(d))
    assert need == 2 * 1 * 2 * 1024 * 64 * 2           # K and V fragment-major copies
    assert L.entmax_dash_mask_words(ctypes.byref(d)) == 1 * 2 * (1024 // 64) * 1
    assert L.entmax_dash_fwd(None, f, f, f, f, f, None, None, f, f, f, need, None) == 1
    assert L.entmax_dash_fwd(ctypes.byref(d), f, f, f, None, f, None, None, f, f, f, need, None) == 1
    assert L.entmax_dash_fwd(ctypes.byref(d), f, f, f, f, f, None, None, None, f, f, need, None) == 1
    assert L.entmax_dash_fwd(ctypes.byref(d), f, f, f, mis, f, None, None, f, f, f, need, None) == 5
    assert L.entmax_dash_fwd(ctypes.byref(d), f, f, f, f, f, mis, None, f, f, f, need, None) == 5
    assert L.entmax_dash_fwd(ctypes.byref(d), f, f, f, f, f, None, None, f, f, f, need - 1, None) == 6
    assert L.entmax_dash_fwd(ctypes.byref(d), f, f, f, f, f, None, None, f, f, None, need, None) == 6
    for kw in (dict(batch=0), dict(seqlen=0)):
        e = _dash_desc(**kw)
        assert L.entmax_dash_fwd(ctypes.byref(e), None, None, None, None, None, None, None, None, None, None, 0,
                                 None) == 0


def test_dash_bwd_pointers_workspace_and_sizes(L):
    d = _dash_desc()
    f = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4098)
    need = L.entmax_dash_bwd_workspace_bytes(ctypes.byref(d))
    b, hq, hkv, n, D, nc = 1, 4, 2, 1024, 64, 16
    # at least: delta, the fragment-major copies of Q (rows and columns), dO, K and V, the
    # block mask, the prior table and the weight gradient, fp32 dQ, the per-(sub-block, row)
    # dS sums, the routing-logit gradient and the per-piece summary-gradient partials
    low = (b * hq * n * 4 + 3 * b * hq * n * D * 2 + 2 * b * hkv * n * D * 2 + b * hq * (n // 32) * 4
           + 2 * b * hkv * nc * n * 4 + b * hq * n * 4 + b * hq * n * D * 4 + b * hq * (n // 32) * n * 4 + b * hq * nc * n * 4
           + b * hkv * 1 * (n // 256) * D * 32 * 4)
    assert low <= need <= low + 64 * 1024
    args = [f] * 14

    def call(i=None, val=None, ws=f, nbytes=need, desc=ctypes.byref(d)):
        a = list(args)
        if i is not None:
            a[i] = val
        return L.entmax_dash_bwd(desc, *a, ws, nbytes, None)

    assert call(desc=None) == 1
    for i in range(14):                       # every tensor is required
        assert call(i, None) == 1, i
    assert call(3, mis) == 5                  # k_summary
    assert call(4, mis) == 5                  # o
    assert call(9, mis) == 5                  # dout
    assert call(13, mis) == 5                 # dk_summary
    assert call(nbytes=need - 1) == 6
    assert call(ws=None) == 6
    assert call(ws=ctypes.c_void_p(4096 + 16)) == 6
    for kw in (dict(batch=0), dict(seqlen=0)):
        e = _dash_desc(**kw)
        assert L.entmax_dash_bwd(ctypes.byref(e), *([None] * 14), None, 0, None) == 0


def test_plain_c_program_uses_the_abi(L, tmp_path):
    """tests/c_abi/abi_check.c, compiled with gcc against include/ and linked to the library,
    exercises the size queries and argument checks from plain C (no Python, no GPU)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(lce.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-o", str(exe),
                           "-L", libdir, "-lentmax_attn", "-Wl,-rpath," + libdir])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout


def _cpu_problem(b=1, hq=4, hkv=2, n=128, d=64):
    import torch
    q = torch.zeros(b, hq, n, d, dtype=torch.bfloat16)
    k = torch.zeros(b, hkv, n, d, dtype=torch.bfloat16)
    return q, k, k.clone()


def _fwd_out(b=1, hq=4, n=128, d=64, Tr=2, W=1, bins=16):
    import torch
    return lce.FwdOut(torch.zeros(b, hq, n, d), torch.zeros(b, hq, n), torch.zeros(b, hq, Tr, W, dtype=torch.int32),
                      torch.zeros(b, hq, n, d), torch.zeros(b, hq, n, bins, dtype=torch.int32), torch.zeros(b, hq, n))


@pytest.mark.parametrize("case,match", [
    ("k_batch", "k must have shape"), ("k_seqlen", "k must have shape"), ("k_dim", "k must have shape"),
    ("k_dtype", "k must be"), ("v_shape", "v must have shape"), ("heads", "multiple of the heads"),
    ("o_dtype", "out.o must be"), ("tau_shape", "out.tau must have shape"),
    ("mask_block", "out.mask must have shape"), ("aux_shape", "out.aux must have shape"),
    ("hist_bins", "out.hist must have shape"), ("stats_short", "stats must be"),
    ("stats_dtype", "stats must be"), ("ws_dtype", "workspace must be"),
])
def test_binding_checks_forward_tensors(case, match):
    """Every tensor of the forward binding is checked (shape, dtype, device) before any
    pointer is taken: a mismatch raises ValueError naming the tensor, not a device fault."""
    import torch
    q, k, v = _cpu_problem()
    kw = {}
    if case == "k_batch":
        k = torch.zeros(2, 2, 128, 64, dtype=torch.bfloat16)
    elif case == "k_seqlen":
        k = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    elif case == "k_dim":
        k = torch.zeros(1, 2, 128, 128, dtype=torch.bfloat16)
    elif case == "k_dtype":
        k = k.float()
    elif case == "v_shape":
        v = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    elif case == "heads":
        k = torch.zeros(1, 3, 128, 64, dtype=torch.bfloat16)
        v = k.clone()
    else:
        out = _fwd_out()
        if case == "o_dtype":
            out = out._replace(o=out.o.bfloat16())
        elif case == "tau_shape":
            out = out._replace(tau=torch.zeros(1, 4, 64))
        elif case == "mask_block":   # the mask of a 32x32-block run is 4 x 1 words per head
            out = out._replace(mask=torch.zeros(1, 4, 4, 1, dtype=torch.int32))
        elif case == "aux_shape":
            out = out._replace(aux=torch.zeros(1, 4, 128, 32))
        elif case == "hist_bins":
            out = out._replace(hist=torch.zeros(1, 4, 128, 8, dtype=torch.int32))
        elif case == "stats_short":
            kw["stats"] = torch.zeros(16, dtype=torch.int64)
        elif case == "stats_dtype":
            kw["stats"] = torch.zeros(32, dtype=torch.float32)
        elif case == "ws_dtype":
            kw["workspace"] = torch.zeros(1024, dtype=torch.float32)
        kw["out"] = out
    with pytest.raises(ValueError, match=match):
        lce.fwd(q, k, v, 1.5, True, (64, 64), 16, **kw)


@pytest.mark.parametrize("case,match", [
    ("do_shape", "do must have shape"), ("tau_dtype", "tau must be"), ("tau_shape", "tau must have shape"),
    ("mask_block", "mask must have shape"), ("mask_dtype", "mask must be"), ("aux_shape", "aux must have shape"),
    ("dq_shape", "out.dq must have shape"), ("dk_dtype", "out.dk must be"), ("dv_shape", "out.dv must have shape"),
])
def test_binding_checks_backward_tensors(case, match):
    import torch
    q, k, v = _cpu_problem()
    do = torch.zeros_like(q)
    tau = torch.zeros(1, 4, 128)
    mask = torch.zeros(1, 4, 2, 1, dtype=torch.int32)
    aux = torch.zeros(1, 4, 128, 64)
    kw = {}
    if case == "do_shape":
        do = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16)
    elif case == "tau_dtype":
        tau = tau.bfloat16()
    elif case == "tau_shape":
        tau = torch.zeros(1, 2, 128)
    elif case == "mask_block":
        mask = torch.zeros(1, 4, 4, 1, dtype=torch.int32)
    elif case == "mask_dtype":
        mask = mask.long()
    elif case == "aux_shape":
        aux = torch.zeros(1, 4, 128, 32)
    elif case == "dq_shape":
        kw["out"] = (torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16), torch.zeros_like(k), torch.zeros_like(v))
    elif case == "dk_dtype":
        kw["out"] = (torch.zeros_like(q), torch.zeros(k.shape), torch.zeros_like(v))
    elif case == "dv_shape":
        kw["out"] = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=match):
        lce.bwd(q, k, v, do, tau, mask, aux, 1.5, True, (64, 64), 16, **kw)


def test_binding_accepts_consistent_cpu_tensors_up_to_the_device_check():
    """A consistent set of tensors passes every shape check and stops only at the device
    check (the library runs on the GPU only)."""
    import torch
    q, k, v = _cpu_problem()
    with pytest.raises(ValueError, match="GPU only"):
        lce.fwd(q, k, v, 1.5, True, (64, 64), 16, out=_fwd_out(), stats=torch.zeros(32, dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU only"):
        lce.bwd(q, k, v, torch.zeros_like(q), torch.zeros(1, 4, 128), torch.zeros(1, 4, 2, 1, dtype=torch.int32),
                torch.zeros(1, 4, 128, 64), 1.5, True, (64, 64), 16)


def test_noalloc_decode_rejects_problems_beyond_the_scratch(L):
    """The allocation-free decode refuses, before any HIP call, a problem whose workspace
    exceeds the static scratch, and accepts the 128K-key, 32-query-head cache."""
    big = lce.make_desc(4, 32, 8, 131072, 64, lce.ENTMAX_BF16, 1.5, True, (32, 32), 16)
    assert L.entmax_attn_decode_workspace_bytes(ctypes.byref(big)) > lce.DECODE_SCRATCH_BYTES
    st = L.entmax_attn_decode_noalloc(ctypes.byref(big), 16, 16, 16, None, None, 16, 16, None, None, None)
    assert st == 6 and b"static scratch" in L.entmax_last_error()
    c5 = lce.make_desc(1, 32, 8, 131072, 64, lce.ENTMAX_BF16, 1.5, True, (32, 32), 16)
    assert L.entmax_attn_decode_workspace_bytes(ctypes.byref(c5)) <= lce.DECODE_SCRATCH_BYTES
    bad = lce.make_desc(1, 32, 8, 131072, 64, lce.ENTMAX_BF16, 0.5, True, (32, 32), 16)
    assert L.entmax_attn_decode_noalloc(ctypes.byref(bad), 16, 16, 16, None, None, 16, 16, None, None, None) == 3


def _dash_cpu_args():
    import torch
    b, hq, hkv, n, d, C = 1, 4, 2, 256, 64, 64
    bf = torch.bfloat16
    return dict(q=torch.zeros(b, hq, n, d, dtype=bf), k=torch.zeros(b, hkv, n, d, dtype=bf),
                v=torch.zeros(b, hkv, n, d, dtype=bf), k_summary=torch.zeros(b, hkv, n // C, d, dtype=bf),
                do=torch.zeros(b, hq, n, d, dtype=bf), o=torch.zeros(b, hq, n, d), lse=torch.zeros(b, hq, n),
                route_tau=torch.zeros(b, hq, n), route_w=torch.zeros(b, hkv, n // C, n),
                chunk_mask=torch.zeros(b, hkv, n // 64, 1, dtype=torch.int32))


@pytest.mark.parametrize("name,bad,match", [
    ("k", lambda a: a["k"][:, :, :128].contiguous(), "k must have shape"),
    ("k_summary", lambda a: a["k_summary"][:, :, :2].contiguous(), "k_summary must have shape"),
    ("do", lambda a: a["do"].float(), "do must be"),
    ("o", lambda a: a["o"].bfloat16(), "o must be"),
    ("lse", lambda a: a["lse"][:, :2].contiguous(), "lse must have shape"),
    ("route_tau", lambda a: a["route_tau"].double(), "route_tau must be"),
    ("route_w", lambda a: a["route_w"].transpose(2, 3).contiguous(), "route_w must have shape"),
    ("chunk_mask", lambda a: a["chunk_mask"].long(), "chunk_mask must be"),
])
def test_dash_binding_checks_backward_tensors(name, bad, match):
    """The DashAttention backward binding checks every tensor's shape and dtype before the
    device check and before any pointer is taken."""
    a = _dash_cpu_args()
    a[name] = bad(a)
    with pytest.raises(ValueError, match=match):
        lce.dash_bwd(a["q"], a["k"], a["v"], a["k_summary"], a["do"], a["o"], a["lse"], a["route_tau"],
                     a["route_w"], a["chunk_mask"], chunk=64)


def test_dash_binding_consistent_cpu_tensors_stop_at_the_device_check():
    a = _dash_cpu_args()
    with pytest.raises(ValueError, match="GPU only"):
        lce.dash_bwd(a["q"], a["k"], a["v"], a["k_summary"], a["do"], a["o"], a["lse"], a["route_tau"],
                     a["route_w"], a["chunk_mask"], chunk=64)
    with pytest.raises(ValueError, match="GPU only"):
        lce.dash_fwd(a["q"], a["k"], a["v"], a["k_summary"], chunk=64)
    with pytest.raises(ValueError, match="seqlen / chunk"):
        lce.dash_fwd(a["q"], a["k"], a["v"], a["k_summary"][:, :, :2].contiguous(), chunk=64)

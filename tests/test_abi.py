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
    (dict(max_iters=16), 2), (dict(heads_kv=0), 2), (dict(tau_init=2), 4), (dict(tau_init=-1), 4),
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
    (dict(max_iters=16), 2), (dict(seqlen=-64), 2),
]


@pytest.mark.parametrize("kw,status", DASH_BAD, ids=[str(b[0]) for b in DASH_BAD])
def test_dash_argument_errors(L, kw, status):
    d = _dash_desc(**kw)
    assert L.entmax_dash_fwd_workspace_bytes(ctypes.byref(d)) == 0
    assert L.entmax_dash_mask_words(ctypes.byref(d)) == 0
    f = ctypes.c_void_p(256)
    st = L.entmax_dash_fwd(ctypes.byref(d), f, f, f, f, f, None, None, f, f, f, 1 << 30, None)
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

"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects invalid arguments on the host before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

from moe_layer_03_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(B.EXPORTED)


def test_product_never_imports_the_oracle():
    """No CPU fallback: nothing in the package imports, loads or builds the oracle."""
    pkg = os.path.join(ROOT, "moe_layer_03_amd")
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|from\s+\.\.\s*import\s+oracle)|liboracle", re.M)
    for f in glob.glob(os.path.join(pkg, "**", "*.*"), recursive=True):
        if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
            assert not pat.search(open(f).read()), f


def _shape(**kw):
    base = dict(T=64, H=256, E=8, K=2, I=128, e_begin=0, e_end=8)
    base.update(kw)
    return B.Shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(K=0), B.MOE_ERR_INVALID_ARG),
    (dict(K=9), B.MOE_ERR_INVALID_ARG),           # K > E
    (dict(E=2000, e_end=8), B.MOE_ERR_INVALID_ARG),
    (dict(e_begin=4, e_end=4), B.MOE_ERR_INVALID_ARG),
    (dict(e_end=9), B.MOE_ERR_INVALID_ARG),
    (dict(e_begin=-1), B.MOE_ERR_INVALID_ARG),
    (dict(H=100), B.MOE_ERR_UNSUPPORTED),
    (dict(I=96), B.MOE_ERR_UNSUPPORTED),
    (dict(E=128, K=65, e_end=128), B.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 28, K=8), B.MOE_ERR_INVALID_ARG),   # T*K >= 2^31
])
def test_invalid_shapes(kw, status):
    lib = B.load()
    s = _shape(**kw).c()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    assert lib.moe_route(ctypes.byref(s), fake, B.MOE_BF16, fake, B.MOE_BF16, None, fake, fake, None, None, 0,
                         None) == status
    assert lib.moe_combine(ctypes.byref(s), fake, B.MOE_BF16, fake, fake, fake, None) == status
    assert lib.moe_layer_workspace_bytes(ctypes.byref(s)) == 0
    assert lib.moe_packed_weight_bytes(ctypes.byref(s)) == 0


def test_invalid_pointers_and_enums():
    lib = B.load()
    s = _shape().c()
    p16 = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    S = ctypes.byref(s)
    R = lib.moe_route
    assert R(S, None, B.MOE_BF16, p16, B.MOE_BF16, None, p16, p16, None, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert R(S, odd, B.MOE_BF16, p16, B.MOE_BF16, None, p16, p16, None, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert R(S, p16, B.MOE_BF16, p16, B.MOE_F32, None, p16, p16, None, None, 0, None) == B.MOE_ERR_UNSUPPORTED
    assert R(S, p16, 7, p16, 7, None, p16, p16, None, None, 0, None) == B.MOE_ERR_UNSUPPORTED
    # the screened router's workspace: 128 experts, bf16
    s128 = _shape(T=1000, E=128, K=8, e_end=32).c()
    S128 = ctypes.byref(s128)
    rneed = lib.moe_route_workspace_bytes(S128)
    assert rneed > 0
    assert R(S128, p16, B.MOE_BF16, p16, B.MOE_BF16, None, p16, p16, None, p16, rneed - 1,
             None) == B.MOE_ERR_WORKSPACE
    assert R(S128, p16, B.MOE_BF16, p16, B.MOE_BF16, None, p16, p16, None, odd, rneed,
             None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_workspace_bytes(S) == 64 * 8 * 4   # 8 experts: no screened path; the tiled path's logits
    s192 = _shape(T=1000, E=128, K=8, e_end=32, H=192).c()
    assert lib.moe_route_workspace_bytes(ctypes.byref(s192)) == 0   # H not a multiple of 128
    assert lib.moe_layer_workspace_bytes(S128) >= rneed
    G = lib.moe_grouped_gemm
    assert G(S, p16, B.MOE_BF16, None, p16, p16, 5, 0, p16, B.MOE_BF16, None) == B.MOE_ERR_INVALID_ARG
    assert G(S, p16, B.MOE_F16, None, p16, p16, B.MOE_GEMM_DOWN, B.MOE_EPI_SWIGLU, p16, B.MOE_BF16,
             None) == B.MOE_ERR_INVALID_ARG
    assert G(S, p16, B.MOE_BF16, None, p16, p16, 0, 0, p16, 9, None) == B.MOE_ERR_UNSUPPORTED
    assert G(S, p16, B.MOE_BF16, None, p16, p16, B.MOE_GEMM_DOWN, 0, p16, B.MOE_F16, None) == B.MOE_ERR_UNSUPPORTED
    assert G(S, p16, B.MOE_F32, None, p16, p16, B.MOE_GEMM_GATE_UP, 0, p16, B.MOE_F16, None) == B.MOE_ERR_UNSUPPORTED
    assert G(S, p16, B.MOE_BF16, odd, p16, p16, 0, 0, p16, B.MOE_F16, None) == B.MOE_ERR_INVALID_ARG
    need = lib.moe_dispatch_workspace_bytes(S)
    assert need > 0
    assert lib.moe_dispatch(S, p16, None, 0, p16, p16, p16, p16, p16, None, p16, need - 1,
                            None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(S, p16, p16, B.MOE_BF16, p16, p16, p16, p16, p16, None, p16, need,
                            None) == B.MOE_ERR_INVALID_ARG   # x without x_packed
    lneed = lib.moe_layer_workspace_bytes(S)
    assert lib.moe_layer(S, p16, 1, p16, 1, None, p16, p16, None, None, None, None, None, None, None, p16,
                         lneed - 1, None) == B.MOE_ERR_WORKSPACE


def test_workspace_sizes_grow_with_tokens():
    lib = B.load()
    prev = 0
    for T in (1, 64, 65, 1000, 6000):
        s = B.Shape(T, 4096, 128, 8, 1536, 0, 32).c()
        n = lib.moe_layer_workspace_bytes(ctypes.byref(s))
        assert n > prev
        prev = n
    s = B.Shape(6000, 4096, 128, 8, 1536, 0, 32)
    cap = s.cap
    # the packed-activation, SwiGLU and down buffers alone
    assert B.moe_layer_workspace_bytes(s) >= cap * (4096 * 2 + 1536 * 2 + 4096 * 2)
    assert B.moe_packed_weight_bytes(s) == 32 * 3 * 4096 * 1536 * 2


def test_status_strings():
    for st in (B.MOE_OK, B.MOE_ERR_INVALID_ARG, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE, B.MOE_ERR_HIP):
        assert B.status_string(st).startswith("MOE_")
    assert B.status_string(12345) == "unknown status"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for several it exits with status 2 and says why."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_route_screen_layout_host_only():
    """The screened router's workspace layout: regions in order, inside the workspace, and no layout for
    shapes that do not take the screened path."""
    s = B.Shape(T=6000, H=4096, E=128, K=8, I=1536, e_begin=0, e_end=32)
    info = B.moe_route_screen_layout(s)
    S, T, E = info["slices"], s.T, s.E
    assert S >= 1 and s.H % S == 0
    assert info["bytes"] == B.moe_route_workspace_bytes(s)
    assert info["part_offset"] + S * T * E * 4 <= info["nx_offset"]
    assert info["nx_offset"] + S * T * 4 <= info["nw_offset"]
    assert info["nw_offset"] + S * E * 4 <= info["bytes"]
    for bad in (B.Shape(T=511, H=4096, E=128, K=8, I=64, e_begin=0, e_end=128),
                B.Shape(T=600, H=192, E=128, K=8, I=64, e_begin=0, e_end=128),
                B.Shape(T=600, H=256, E=64, K=8, I=64, e_begin=0, e_end=64)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_route_screen_layout(bad)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as ei:
        B.moe_route_screen_layout(s, B.MOE_F32, B.MOE_F32)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED

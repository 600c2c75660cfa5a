"""Host-side checks of the C-ABI library (CPU only, no GPU call):
the library loads, exports every function include/*.h declares, and its
host-only queries (config validation, parameter count and layout, workspace
size) behave as documented."""

import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gpt_transformer_lm_amd", "libgpt2_hip.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def declared_functions():
    names = set()
    for h in ("gpt2.h", "gpt2_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(gpt2_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    declared = declared_functions()
    assert len(declared) >= 30
    missing = declared - exported
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    from gpt_transformer_lm_amd import lib
    assert declared_functions() == set(lib.exported_symbols())
    L = lib.load()
    for name in declared_functions():
        assert hasattr(L, name)


def cfg(**kw):
    from gpt_transformer_lm_amd import lib
    base = dict(V=50257, Vp=50304, maxT=1024, L=12, H=12, C_=768, B=24, T=1024, dtype=1)
    base.update(kw)
    return lib.make_config(**base)


def test_gpt2_124m_parameter_count():
    from gpt_transformer_lm_amd import lib
    L = lib.load()
    c = cfg()
    assert L.gpt2_validate_config(C.byref(c)) == 0
    # 124M with the token table padded to 50304 rows, and with 50257 rows
    assert L.gpt2_num_parameters(C.byref(c), 1) == 124475904
    assert L.gpt2_num_parameters(C.byref(c), 0) == 124439808


@pytest.mark.parametrize("L_,H,C_,expect", [(24, 16, 1024, 354871296), (48, 25, 1600, 1557686400)])
def test_miniseries_parameter_counts(L_, H, C_, expect):
    from gpt_transformer_lm_amd import lib
    c = cfg(L=L_, H=H, C_=C_, B=8)
    assert lib.load().gpt2_num_parameters(C.byref(c), 1) == expect


def test_param_layout_is_contiguous_and_ordered():
    from gpt_transformer_lm_amd import lib, synthetic
    c = cfg(V=512, Vp=512, maxT=64, L=2, H=4, C_=64, B=4, T=64, dtype=0)
    lay = lib.param_layout(c)
    names = [n for n, _, _ in lay]
    assert names == [n for n, _ in synthetic.param_table(512, 512, 64, 2, 64)]
    off = 0
    for (name, o, shape), (_, shp) in zip(lay, synthetic.param_table(512, 512, 64, 2, 64)):
        assert o == off and tuple(shape) == tuple(shp), name
        off += int(np.prod(shape))
    assert off == lib.load().gpt2_num_parameters(C.byref(c), 1)


@pytest.mark.parametrize("bad", [
    dict(C_=100),                 # not a multiple of 64
    dict(H=5),                    # does not divide C
    dict(H=24),                   # head dim 32 is valid; replaced below by an invalid head dim
    dict(Vp=50300),               # not a multiple of 64
    dict(Vp=50240),               # smaller than V
    dict(T=2048),                 # beyond maxT
    dict(B=0),
    dict(B=64),                   # bf16 logits of B*T rows reach 4 GiB
    dict(B=4160, T=1024, maxT=1024, dtype=0),   # B*T beyond the key sort's 4194304
    dict(dtype=7),
    dict(L=-1),
    dict(B=1, T=1000),            # B*T not a multiple of 64
    dict(H=2, C_=192),            # head dim 96 unsupported
])
def test_invalid_configs_are_rejected(bad):
    from gpt_transformer_lm_amd import lib
    L = lib.load()
    c = cfg(**bad)
    if bad == dict(H=24):
        assert L.gpt2_validate_config(C.byref(c)) == 0
        c = cfg(H=6, C_=1408)            # 1408 / 6 is not an integer
    rc = L.gpt2_validate_config(C.byref(c))
    assert rc == 1
    assert L.gpt2_last_error()
    assert L.gpt2_num_parameters(C.byref(c), 1) == -1
    assert L.gpt2_workspace_bytes(C.byref(c)) == 0


def test_workspace_is_sized_for_the_124m_step():
    from gpt_transformer_lm_amd import lib
    c = cfg()
    ws = lib.load().gpt2_workspace_bytes(C.byref(c))
    P = 124475904
    BT, Cc, Lr, Vp = 24 * 1024, 768, 12, 50304
    lower = P * (16 + 2) + BT * Vp * 2 + Lr * BT * Cc * 2 * 16
    assert lower < ws < lower * 1.5 + (2 << 30)
    # fits one MI355X (288 GB HBM3E) with plenty of room
    assert ws < 40 * (1 << 30)


def test_status_strings_and_null_create():
    from gpt_transformer_lm_amd import lib
    L = lib.load()
    for st in range(6):
        assert L.gpt2_status_string(st) != b"unknown status"
    assert L.gpt2_create(None, 0, None, None, 0, None) == 1


def test_failed_host_allocation_is_a_status_not_a_crash():
    """A host allocation that fails inside the library (forced by the test
    hook) comes back through the C ABI as GPT2_E_OOM / a zero size with the
    reason in gpt2_last_error(), and the next call works again."""
    from gpt_transformer_lm_amd import lib
    L = lib.load()
    c = cfg()
    good = L.gpt2_workspace_bytes(C.byref(c))
    assert good > 0
    assert L.gpt2_test_fail_host_allocations(1) == 0
    assert L.gpt2_workspace_bytes(C.byref(c)) == 0
    assert b"host allocation" in L.gpt2_last_error()
    assert L.gpt2_workspace_bytes(C.byref(c)) == good          # the hook fired once
    n = C.c_int(-1)
    assert L.gpt2_test_fail_host_allocations(2) == 0
    assert L.gpt2_step_gemm_plans(C.byref(c), None, 0, C.byref(n)) == 3
    assert b"host allocation" in L.gpt2_last_error()
    L.gpt2_test_fail_host_allocations(0)
    assert L.gpt2_step_gemm_plans(C.byref(c), None, 0, C.byref(n)) == 0 and n.value > 0


def test_arch_flags():
    from gpt_transformer_lm_amd import lib
    L = lib.load()
    c = cfg()
    for f in range(8):          # every combination of ReLU^2, QK-Norm and rotary embeddings
        c.arch_flags = f
        assert L.gpt2_validate_config(C.byref(c)) == 0
    c.arch_flags = 8
    assert L.gpt2_validate_config(C.byref(c)) == 1
    assert b"arch_flags" in L.gpt2_last_error()
    # the ReLU^2 variant changes the fc epilogue only
    c.arch_flags = lib.GPT2_ARCH_RELU2
    plans = {p["site"]: lib.EPILOGUES[p["epilogue"]] for p in lib.step_gemm_plans(c)}
    assert plans["fc"] == "bias+relu2" and plans["fcproj_dx"] == "mul"
    c.arch_flags = 0
    assert {p["site"]: lib.EPILOGUES[p["epilogue"]] for p in lib.step_gemm_plans(c)}["fc"] == "bias+gelu"


# The three GPT-2 sizes at their benchmark batch (T = 1024).
SIZES = {"124m": dict(L=12, H=12, C_=768, B=24), "350m": dict(L=24, H=16, C_=1024, B=16),
         "1.6b": dict(L=48, H=25, C_=1600, B=8)}
PLAN_KEYS = ("M", "N", "K", "epilogue", "a_kmajor", "b_kmajor", "tile_m", "tile_n", "waves", "k_groups",
             "k_splits", "bias_grad")


def op_plan_for_site(site, BT, Cc, Vp):
    """The op-level linear call (and which of its three GEMMs) that performs
    the step's GEMM at `site`, with the options the step uses there."""
    from gpt_transformer_lm_amd import lib
    layer = {"qkv": (3 * Cc, Cc, dict(bias=True)), "attproj": (Cc, Cc, dict(bias=True, residual=True)),
             "fc": (4 * Cc, Cc, dict(bias=True, gelu=True)), "fcproj": (Cc, 4 * Cc, dict(bias=True, residual=True)),
             "logits": (Vp, Cc, dict())}
    if site in layer:
        N, K, kw = layer[site]
        return lib.op_linear_plans(1, BT, N, K, **kw)[0]
    base, kind = site.rsplit("_", 1)
    name = {"cls": "logits"}.get(base, base)
    N, K, _ = layer[name]
    if kind == "dw":
        return lib.op_linear_plans(1, BT, N, K, db=name != "logits")[1]
    # dX of the fc-proj layer multiplies by the fc layer's saved GELU'
    return lib.op_linear_plans(1, BT, N, K, gelu=name == "fcproj")[2]


@pytest.mark.parametrize("size", sorted(SIZES))
def test_step_gemm_plans_reached_by_the_full_width_tests(size):
    """Every GEMM instantiation the full-depth step launches is launched by
    the two-layer step at the same width and batch (the GEMM shapes do not
    depend on L) and by the op-level linear calls at the same shapes: the
    full-width step-parity tests and the full-size op tests reach the same
    kernels as the benchmarked step."""
    from gpt_transformer_lm_amd import lib
    k = SIZES[size]
    full = lib.step_gemm_plans(cfg(**k))
    two = lib.step_gemm_plans(cfg(**dict(k, L=2)))
    assert len(full) == 12 * k["L"] + 3
    key = lambda p: (p["site"],) + tuple(p[x] for x in PLAN_KEYS)
    assert {key(p) for p in full} == {key(p) for p in two}
    seen = {}
    for p in full:
        seen.setdefault(p["site"], p)
    assert len(seen) == 15
    for site, p in seen.items():
        o = op_plan_for_site(site, k["B"] * 1024, k["C_"], 50304)
        assert tuple(o[x] for x in PLAN_KEYS) == tuple(p[x] for x in PLAN_KEYS), (site, o, p)


def test_ragged_384x192_test_shapes_reach_that_tile():
    """test_linear_384x192_ragged_rows (GPU) runs the 8-wave 384x192 tile:
    its forward with and without the residual, and its backward's dX."""
    from gpt_transformer_lm_amd import lib
    M, N, K = 8392, 768, 1096
    for kw in (dict(), dict(bias=True, residual=True)):
        p = lib.op_linear_plans(1, M, N, K, **kw)[0]
        assert (p["tile_m"], p["tile_n"], p["waves"], p["k_splits"]) == (384, 192, 8, 1), (kw, p)
    p = lib.op_linear_plans(1, M, K, N, db=True)[2]     # dX: M x 768, reduced over 1096
    assert (p["N"], p["tile_m"], p["tile_n"], p["waves"]) == (N, 384, 192, 8), p

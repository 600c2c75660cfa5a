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
    dict(B=64),                   # B*T > 32768
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
    for st in range(5):
        assert L.gpt2_status_string(st)
    assert L.gpt2_create(None, 0, None, None, 0, None) == 1

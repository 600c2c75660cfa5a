"""The allocation-free attention backward (gpt2_op_attention_backward_noalloc):
the same results as gpt2_op_attention_backward with a caller workspace, on
two calls in a row that share the library's scratch array (the second one
smaller), and its size limit checked on the host before anything runs."""

import ctypes as C
import math
import os

import numpy as np
import pytest

import oracle as O
from gpt_transformer_lm_amd import lib
from gpu_util import BF16, FP32, as_input, dev, empty, empty32, host, rel, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gpt_transformer_lm_amd", "libgpt2_hip.so")
SCRATCH = 8 << 20


def rows_that_fit(H, T):
    """Largest batch whose 2 x B*H*T scratch floats (rows rounded up to 64,
    plus 256 bytes) fit the scratch array."""
    B = 1
    while 2 * ((((B + 1) * H * T) + 63) // 64 * 64) * 4 + 256 <= SCRATCH:
        B += 1
    return B


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_noalloc_rejects_oversized_shapes_on_the_host():
    L = lib.load()
    fn = L.gpt2_op_attention_backward_noalloc
    B = rows_that_fit(12, 1024)
    # one batch row more than fits: rejected before any buffer is touched
    rc = fn(BF16, B + 1, 1024, 12, 64, None, None, None, None, None, None)
    assert rc == 1 and b"scratch" in L.gpt2_last_error()
    # a shape that fits gets as far as the buffer check
    rc = fn(BF16, B, 1024, 12, 64, None, None, None, None, None, None)
    assert rc == 1 and b"NULL buffer" in L.gpt2_last_error()


def _inputs(B, T, H, hd, dtype, seed):
    torch = __import__("torch")
    gen = torch.Generator(device="cuda").manual_seed(seed)
    Cc = H * hd
    st = torch.bfloat16 if dtype == BF16 else torch.float32
    qkv = torch.randn((B, T, 3 * Cc), generator=gen, device="cuda").to(st)
    dout = torch.randn((B, T, Cc), generator=gen, device="cuda").to(st)
    out = torch.empty((B, T, Cc), dtype=st, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    lib.attention_forward(dtype, B, T, H, hd, qkv, out, lse)
    return qkv, out, dout, lse


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [BF16, FP32], ids=["bf16", "fp32"])
def test_noalloc_matches_workspace_version_two_calls(dtype):
    torch = __import__("torch")
    if dtype == BF16:
        # the largest batch of 12 x 1024 rows the scratch holds, then a small ragged one
        shapes = [(rows_that_fit(12, 1024), 1024, 12, 64), (2, 200, 3, 64)]
    else:
        shapes = [(6, 1024, 4, 32), (1, 130, 2, 16)]
    for i, (B, T, H, hd) in enumerate(shapes):
        say("noalloc attention backward", "bf16" if dtype == BF16 else "fp32", B, T, H, hd)
        qkv, out, dout, lse = _inputs(B, T, H, hd, dtype, seed=31 + i)
        ref = torch.full((B, T, 3 * H * hd), float("nan"), dtype=qkv.dtype, device="cuda")
        lib.attention_backward(dtype, B, T, H, hd, qkv, out, dout, lse, ref)
        got = torch.full_like(ref, float("nan"))
        lib.attention_backward_noalloc(dtype, B, T, H, hd, qkv, out, dout, lse, got)
        torch.cuda.synchronize()
        # same kernels, same inputs: identical bits
        assert torch.equal(got, ref), (B, T, H, hd)
    # the small (second) call also against the oracle, to the attention tolerances
    B, T, H, hd = shapes[-1]
    Cc = H * hd
    qn = qkv.float().cpu().numpy().astype(np.float64)
    dn = dout.float().cpu().numpy().astype(np.float64)
    gn = got.float().cpu().numpy()
    tol = 1e-2 if dtype == BF16 else 1e-5
    for b in range(B):
        for h in range(H):
            sl = slice(h * hd, (h + 1) * hd)
            q, k, v = qn[b, :, sl], qn[b, :, Cc + h * hd:Cc + (h + 1) * hd], qn[b, :, 2 * Cc + h * hd:2 * Cc + (h + 1) * hd]
            _, p = O.causal_attention_forward(q[None], k[None], v[None])
            gq, gk, gv = O.causal_attention_backward(dn[b, :, sl][None], q[None], k[None], v[None], p)
            assert rel(gn[b, :, sl], gq[0]) < tol
            assert rel(gn[b, :, Cc + h * hd:Cc + (h + 1) * hd], gk[0]) < tol
            assert rel(gn[b, :, 2 * Cc + h * hd:2 * Cc + (h + 1) * hd], gv[0]) < tol

"""Pins of the oracle's single layers against what mathematics and independent
library routines fix (CPU only, float64).

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand) fails it: torch's own CPU
implementations (F.layer_norm, F.gelu(approximate='tanh'),
F.scaled_dot_product_attention(is_causal=True), F.cross_entropy,
torch.optim.AdamW) with autograd for the gradients, closed forms, invariants
and brute-force loops.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

torch.set_default_dtype(torch.float64)
RNG = np.random.Generator(np.random.PCG64(1234))


def t(a, grad=False):
    x = torch.tensor(np.asarray(a), dtype=torch.float64)
    return x.requires_grad_(grad)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- linear

def test_linear_matches_torch():
    x = RNG.standard_normal((9, 12))
    w = RNG.standard_normal((7, 12))
    b = RNG.standard_normal(7)
    dy = RNG.standard_normal((9, 7))
    y = O.linear_forward(x, w, b)
    dx, dw, db = O.linear_backward(dy, x, w)
    tx, tw, tb = t(x, True), t(w, True), t(b, True)
    ty = F.linear(tx, tw, tb)
    ty.backward(t(dy))
    assert rel(y, ty.detach().numpy()) < 1e-14
    assert rel(dx, tx.grad.numpy()) < 1e-14
    assert rel(dw, tw.grad.numpy()) < 1e-14
    assert rel(db, tb.grad.numpy()) < 1e-14


# ---------------------------------------------------------------- LayerNorm

def test_layernorm_matches_torch_forward_and_backward():
    x = RNG.standard_normal((3, 5, 48)) * 2.0 + 0.7
    w = 1.0 + RNG.standard_normal(48) * 0.3
    b = RNG.standard_normal(48) * 0.3
    dy = RNG.standard_normal((3, 5, 48))
    y, cache = O.layernorm_forward(x, w, b)
    dx, dw, db = O.layernorm_backward(dy, cache)
    tx, tw, tb = t(x, True), t(w, True), t(b, True)
    ty = F.layer_norm(tx, (48,), tw, tb, eps=1e-5)
    ty.backward(t(dy))
    assert rel(y, ty.detach().numpy()) < 1e-13
    assert rel(dx, tx.grad.numpy()) < 1e-12
    assert rel(dw, tw.grad.numpy()) < 1e-12
    assert rel(db, tb.grad.numpy()) < 1e-12


def test_layernorm_backward_invariants():
    # sum_c dx = 0 for every row (any eps); with eps = 0 also
    # sum_c dx * xhat = 0, and with eps > 0 it equals
    # rstd * sum_c(g xhat) * eps / (var + eps)  (since sum_c xhat^2 = C var/(var+eps)).
    x = RNG.standard_normal((7, 64)) * 3.0
    dy = RNG.standard_normal((7, 64))
    w = 1.0 + RNG.standard_normal(64) * 0.2
    _, cache0 = O.layernorm_forward(x, w, np.zeros(64), eps=0.0)
    dx0, _, _ = O.layernorm_backward(dy, cache0)
    assert np.abs(dx0.sum(-1)).max() < 1e-12
    assert np.abs((dx0 * cache0[0]).sum(-1)).max() < 1e-12
    x = x * 1e-3       # var comparable to eps so the eps term is visible
    _, cache = O.layernorm_forward(x, w, np.zeros(64))
    dx, _, _ = O.layernorm_backward(dy, cache)
    xhat, rstd, _ = cache
    var = x.var(-1, keepdims=True)
    expect = rstd * ((dy * w) * xhat).sum(-1, keepdims=True) * 1e-5 / (var + 1e-5)
    assert np.abs(dx.sum(-1)).max() < 1e-9
    assert np.allclose((dx * xhat).sum(-1, keepdims=True), expect, rtol=1e-9, atol=1e-12)


def test_layernorm_output_statistics():
    x = RNG.standard_normal((4, 256)) * 5 + 3
    y, _ = O.layernorm_forward(x, np.ones(256), np.zeros(256))
    assert np.abs(y.mean(-1)).max() < 1e-12
    # biased variance with eps: var(y) = var / (var + eps)
    v = x.var(-1)
    assert np.allclose(y.var(-1), v / (v + 1e-5), rtol=1e-12)


# ---------------------------------------------------------------- GELU

def test_gelu_matches_torch_tanh_form():
    u = np.linspace(-8, 8, 2001)
    dg = RNG.standard_normal(u.shape)
    tu = t(u, True)
    tg = F.gelu(tu, approximate="tanh")
    tg.backward(t(dg))
    assert rel(O.gelu_tanh(u), tg.detach().numpy()) < 1e-14
    assert rel(O.gelu_tanh_backward(u, dg), tu.grad.numpy()) < 1e-13


def test_gelu_special_values():
    assert O.gelu_tanh(np.array(0.0)) == 0.0
    assert O.gelu_tanh_backward(np.array(0.0), np.array(1.0)) == 0.5
    # tends to identity for large u, to 0 for very negative u
    assert abs(O.gelu_tanh(np.array(20.0)) - 20.0) < 1e-12
    assert abs(O.gelu_tanh(np.array(-20.0))) < 1e-12


def test_gelu_backward_central_difference():
    u = np.linspace(-5, 5, 101)
    h = 1e-6
    fd = (O.gelu_tanh(u + h) - O.gelu_tanh(u - h)) / (2 * h)
    assert np.abs(fd - O.gelu_tanh_backward(u, np.ones_like(u))).max() < 1e-8


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("H,T,hd", [(2, 7, 4), (3, 33, 16), (1, 64, 64)])
def test_attention_matches_torch_sdpa(H, T, hd):
    q = RNG.standard_normal((H, T, hd))
    k = RNG.standard_normal((H, T, hd))
    v = RNG.standard_normal((H, T, hd))
    do = RNG.standard_normal((H, T, hd))
    o, p = O.causal_attention_forward(q, k, v)
    dq, dk, dv = O.causal_attention_backward(do, q, k, v, p)
    tq, tk, tv = t(q, True), t(k, True), t(v, True)
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    to.backward(t(do))
    assert rel(o, to.detach().numpy()) < 1e-12
    assert rel(dq, tq.grad.numpy()) < 1e-11
    assert rel(dk, tk.grad.numpy()) < 1e-11
    assert rel(dv, tv.grad.numpy()) < 1e-11


def test_attention_probabilities_are_causal_and_normalised():
    q, k, v = (RNG.standard_normal((2, 20, 8)) for _ in range(3))
    _, p = O.causal_attention_forward(q, k, v)
    assert np.abs(p.sum(-1) - 1.0).max() < 1e-14
    upper = np.triu(np.ones((20, 20), dtype=bool), k=1)
    assert np.all(p[:, upper] == 0.0)


def test_attention_single_position_returns_value():
    q, k, v = (RNG.standard_normal((3, 1, 16)) for _ in range(3))
    o, _ = O.causal_attention_forward(q, k, v)
    assert np.array_equal(o, v)


def test_attention_first_row_attends_only_to_itself():
    q, k, v = (RNG.standard_normal((2, 9, 8)) for _ in range(3))
    o, _ = O.causal_attention_forward(q, k, v)
    assert np.allclose(o[:, 0], v[:, 0], rtol=0, atol=1e-15)


# ---------------------------------------------------------------- softmax CE

def test_cross_entropy_matches_torch():
    z = RNG.standard_normal((13, 50)) * 3
    y = RNG.integers(0, 50, 13)
    losses, dz = O.softmax_cross_entropy(z, y)
    tz = t(z, True)
    tl = F.cross_entropy(tz, torch.tensor(y), reduction="mean")
    tl.backward()
    assert abs(losses.mean() - tl.item()) < 1e-13
    assert rel(dz, tz.grad.numpy()) < 1e-13


def test_cross_entropy_uniform_logits_give_log_v():
    V = 512
    z = np.zeros((5, V))
    y = np.array([0, 3, 511, 7, 100])
    losses, dz = O.softmax_cross_entropy(z, y)
    assert np.all(losses == np.float64(math.log(V))) or np.abs(losses - math.log(V)).max() < 1e-15
    assert np.abs(dz.sum(-1)).max() < 1e-15
    expect = np.full((5, V), 1.0 / V)
    expect[np.arange(5), y] -= 1.0
    assert np.abs(dz - expect / 5).max() < 1e-17


def test_cross_entropy_shift_invariance_and_large_logits():
    z = RNG.standard_normal((4, 30))
    y = np.array([1, 2, 3, 4])
    l0, d0 = O.softmax_cross_entropy(z, y)
    l1, d1 = O.softmax_cross_entropy(z + 1000.0, y)
    assert np.allclose(l0, l1, atol=1e-10) and np.allclose(d0, d1, atol=1e-15)


# ---------------------------------------------------------------- encoder

def test_encoder_forward_and_backward_brute_force():
    V, maxT, C, B, T = 11, 9, 5, 3, 6
    wte = RNG.standard_normal((V, C))
    wpe = RNG.standard_normal((maxT, C))
    tok = RNG.integers(0, V, (B, T))
    tok[0, :3] = 4          # repeated ids must accumulate
    x0 = O.encoder_forward(wte, wpe, tok)
    for b in range(B):
        for s in range(T):
            assert np.array_equal(x0[b, s], wte[tok[b, s]] + wpe[s])
    dx = RNG.standard_normal((B, T, C))
    dwte, dwpe = O.encoder_backward(dx, tok, V, maxT)
    ew = np.zeros((V, C))
    ep = np.zeros((maxT, C))
    for b in range(B):
        for s in range(T):
            ew[tok[b, s]] += dx[b, s]
            ep[s] += dx[b, s]
    assert np.allclose(dwte, ew, rtol=0, atol=1e-14)
    assert np.allclose(dwpe, ep, rtol=0, atol=1e-14)
    assert np.all(dwpe[T:] == 0)


# ---------------------------------------------------------------- AdamW

def test_adamw_first_step_closed_form():
    # At t = 1: mhat = g and vhat = g^2, so
    # theta_1 = theta_0 (1 - lr wd) - lr g / (|g| + eps).
    th = RNG.standard_normal(1000)
    g = RNG.standard_normal(1000)
    lr, wd, eps = 1e-3, 0.1, 1e-8
    new, m, v = O.adamw_update(th, g, np.zeros(1000), np.zeros(1000), lr, 0.9, 0.999, eps, wd, 1)
    expect = th * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.abs(new - expect).max() < 1e-15
    assert np.allclose(m, 0.1 * g) and np.allclose(v, 0.001 * g * g)


def test_adamw_multi_step_matches_torch():
    th = RNG.standard_normal(257)
    tp = torch.nn.Parameter(t(th))
    opt = torch.optim.AdamW([tp], lr=6e-4, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    m = np.zeros_like(th)
    v = np.zeros_like(th)
    for step in range(1, 6):
        g = RNG.standard_normal(257)
        th, m, v = O.adamw_update(th, g, m, v, 6e-4, 0.9, 0.95, 1e-8, 0.1, step)
        tp.grad = t(g)
        opt.step()
    assert rel(th, tp.detach().numpy()) < 1e-14


def test_adamw_zero_gradient_zero_param_is_fixed_point():
    # Padded token-table rows: zero init and zero gradient stay exactly zero.
    z = np.zeros(64)
    new, m, v = O.adamw_update(z, z, z, z, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    assert np.all(new == 0) and np.all(m == 0) and np.all(v == 0)

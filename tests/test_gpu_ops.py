"""Op-level parity of the HIP kernels against the CPU oracle, through the
C ABI (include/gpt2_ops.h).  Same seeded inputs on both sides; bf16 inputs
are the bf16-rounded values on both sides.

Tolerances (relative L2, oracle as reference), from the arithmetic:
  * fp32 storage, fp32 arithmetic: 1e-5 (reassociation only);
  * bf16 outputs: each element is rounded to nearest bf16 (relative error
    <= 2^-9 = 1.95e-3), so 3e-3, and 6e-3 where a bf16-rounded intermediate
    feeds a second product (attention);
  * fp32 outputs of bf16 inputs (weight / bias gradients): products are exact
    in fp32, only the fp32 summation order differs: 1e-5.
Integer and layout results (encoder gather, padded columns) are bit-exact.
"""

import math

import numpy as np
import pytest

import oracle as O
from gpt_transformer_lm_amd import lib
from gpt_transformer_lm_amd import synthetic as S
from gpu_util import BF16, FP32, as_input, dev, dev_i32, empty, empty32, host, rel, say

pytestmark = pytest.mark.gpu

TOL_OUT = {FP32: 1e-5, BF16: 3e-3}
TOL_F32 = 1e-5
DT = [FP32, BF16]
DTN = {FP32: "fp32", BF16: "bf16"}


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- GEMM / linear

# (M, N, K): several tiles with ragged tails in every dimension; M >= 2048 and
# N >= 2048 select the 256-row / 256-column block tiles.
SHAPES = [(256, 192, 64), (200, 136, 128), (64, 64, 64), (320, 200, 192), (2104, 2056, 136), (2104, 1000, 264),
          (136, 8200, 72)]  # the last one has a long dX reduction (split over N)


@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("epi", ["store", "bias", "bias_res", "bias_gelu"])
def test_linear_forward(dtype, M, N, K, epi):
    """The four forward epilogues of the step: plain (logits), bias (QKV),
    bias + residual (attention and MLP projections) and bias + GELU with
    GELU' saved (fc)."""
    say("linear_forward", DTN[dtype], M, N, K, epi)
    r = rng(M * 7 + N + K)
    x, W = r.standard_normal((M, K)), r.standard_normal((N, K)) * 0.1
    b, res = r.standard_normal(N) * 0.5, r.standard_normal((M, N))
    xi, Wi, bi, ri = (as_input(a, dtype).astype(np.float64) for a in (x, W, b, res))
    y = empty((M, N), dtype)
    g = empty((M, N), dtype) if epi == "bias_gelu" else None
    lib.linear_forward(dtype, dev(x, dtype), dev(W, dtype), b=None if epi == "store" else dev(b, dtype),
                       residual=dev(res, dtype) if epi == "bias_res" else None, gelu_grad=g, y=y)
    ref = O.linear_forward(xi, Wi, None if epi == "store" else bi)
    if epi == "bias_res":
        ref = ref + ri
    if g is None:
        assert rel(host(y), ref) < TOL_OUT[dtype]
    else:
        assert rel(host(y), O.gelu_tanh(ref)) < TOL_OUT[dtype]
        assert rel(host(g), O.gelu_tanh_backward(ref, np.ones_like(ref))) < TOL_OUT[dtype]


@pytest.mark.parametrize("epi", ["store", "bias_res"])
def test_linear_384x192_ragged_rows(epi):
    """The 8-wave 384x192 tile (plain stores and residual adds with N a
    multiple of 192 and M >= 8192) with a partial last row tile and a partial
    last K step; the residual comes straight to registers after the main
    loop.  Its backward: dX of an N = 768 input layer on the same tile."""
    M, N, K = 8392, 768, 1096   # (test_abi_host checks these reach the 384x192 plans)
    say("linear 384x192", epi, M, N, K)
    r = rng(M + N + K + len(epi))
    x, W = r.standard_normal((M, K)), r.standard_normal((N, K)) * 0.1
    b, res = r.standard_normal(N) * 0.5, r.standard_normal((M, N))
    xi, Wi, bi, ri = (as_input(a, BF16).astype(np.float64) for a in (x, W, b, res))
    y = empty((M, N), BF16)
    lib.linear_forward(BF16, dev(x, BF16), dev(W, BF16), b=None if epi == "store" else dev(b, BF16),
                       residual=dev(res, BF16) if epi == "bias_res" else None, y=y)
    ref = O.linear_forward(xi, Wi, None if epi == "store" else bi)
    if epi == "bias_res":
        ref = ref + ri
    assert rel(host(y), ref) < TOL_OUT[BF16]
    # backward of a layer with 768 inputs and 200 outputs: dX = dY W is M x 768
    dy, x2, W2 = r.standard_normal((M, K)), r.standard_normal((M, N)), r.standard_normal((K, N)) * 0.1
    dx, dW, db = empty((M, N), BF16), empty32((K, N)), empty32((K,))
    lib.linear_backward(BF16, dev(dy, BF16), dev(x2, BF16), dev(W2, BF16), dx=dx, dW=dW, db=db)
    rdx, rdW, rdb = O.linear_backward(*(as_input(a, BF16).astype(np.float64) for a in (dy, x2, W2)))
    assert rel(host(dx), rdx) < TOL_OUT[BF16]
    assert rel(host(dW), rdW) < TOL_F32
    assert rel(host(db), rdb) < TOL_F32


@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
@pytest.mark.parametrize("M,N,K", [(96, 100, 64), (2056, 2052, 72)])
def test_linear_forward_unaligned_columns(dtype, M, N, K):
    """N not a multiple of 8: the epilogue falls back to element stores."""
    say("linear_forward unaligned", DTN[dtype], M, N, K)
    r = rng(M + N + K)
    x, W, b, res = r.standard_normal((M, K)), r.standard_normal((N, K)) * 0.1, r.standard_normal(N), \
        r.standard_normal((M, N))
    y = empty((M, N), dtype)
    lib.linear_forward(dtype, dev(x, dtype), dev(W, dtype), b=dev(b, dtype), residual=dev(res, dtype), y=y)
    xi, Wi, bi, ri = (as_input(a, dtype).astype(np.float64) for a in (x, W, b, res))
    assert rel(host(y), O.linear_forward(xi, Wi, bi) + ri) < TOL_OUT[dtype]


@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("gelu", [False, True])
def test_linear_backward(dtype, M, N, K, gelu):
    """dX (plain, or multiplied by a saved GELU'(u) as in the fc-projection
    layer's backward), dW and the fused bias gradient."""
    say("linear_backward", DTN[dtype], M, N, K, "gelu" if gelu else "")
    r = rng(M + 3 * N + 5 * K + gelu)
    dy, x, W, u = r.standard_normal((M, N)), r.standard_normal((M, K)), r.standard_normal((N, K)) * 0.1, \
        r.standard_normal((M, K))
    dgelu = O.gelu_tanh_backward(u, np.ones_like(u))       # the derivative the forward saves
    dyi, xi, Wi, di = (as_input(a, dtype).astype(np.float64) for a in (dy, x, W, dgelu))
    dx = empty((M, K), dtype)
    dW = empty32((N, K))
    db = empty32((N,))
    lib.linear_backward(dtype, dev(dy, dtype), dev(x, dtype), dev(W, dtype), dx=dx, dW=dW, db=db,
                        gelu_grad=dev(dgelu, dtype) if gelu else None)
    rdx, rdW, rdb = O.linear_backward(dyi, xi, Wi)
    if gelu:
        rdx = rdx * di
    assert rel(host(dx), rdx) < TOL_OUT[dtype]
    assert rel(host(dW), rdW) < TOL_F32
    assert rel(host(db), rdb) < TOL_F32


@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
def test_linear_backward_accumulates(dtype):
    say("linear_backward accumulate", DTN[dtype])
    r = rng(5)
    M, N, K = 128, 64, 192
    dy, x, W = r.standard_normal((M, N)), r.standard_normal((M, K)), r.standard_normal((N, K))
    base_w, base_b = r.standard_normal((N, K)), r.standard_normal(N)
    dW, db = dev(base_w, FP32), dev(base_b, FP32)
    lib.linear_backward(dtype, dev(dy, dtype), dev(x, dtype), dev(W, dtype), dW=dW, db=db, accumulate=True)
    _, rdW, rdb = O.linear_backward(as_input(dy, dtype).astype(np.float64), as_input(x, dtype).astype(np.float64),
                                    W)
    assert rel(host(dW), base_w.astype(np.float32) + rdW) < TOL_F32
    assert rel(host(db), base_b.astype(np.float32) + rdb) < TOL_F32


# The GEMMs of the GPT-2 124M, 350M and 1.6B steps at their benchmark batch
# (B*T = 24576, 16384, 8192; Vp = 50304) at full size, with the epilogues the
# step uses at each site, so every (tile, waves, K-groups, K-splits,
# epilogue, layout) the steps launch runs here (the host test
# test_step_gemm_plans_reached_by_the_full_width_tests checks that the plans
# agree).  512 sampled outputs of each product are recomputed as float64 dot
# products from the same bf16 operands.
FULL_SIZES = {"124m": (24576, 768), "350m": (16384, 1024), "1.6b": (8192, 1600)}
FULL_SITES = ["qkv", "attproj", "fc", "fcproj", "logits"]


def _site_shape(site, Cc):
    return {"qkv": (3 * Cc, Cc), "attproj": (Cc, Cc), "fc": (4 * Cc, Cc), "fcproj": (Cc, 4 * Cc),
            "logits": (50304, Cc)}[site]


@pytest.mark.parametrize("site", FULL_SITES)
@pytest.mark.parametrize("size", sorted(FULL_SIZES))
def test_linear_full_size_sampled(size, site):
    M, Cc = FULL_SIZES[size]
    N, K = _site_shape(site, Cc)
    say("full-size linear", size, site, M, N, K)
    torch = __import__("torch")
    bias, residual, gelu = site != "logits", site in ("attproj", "fcproj"), site == "fc"
    gelu_dx = site == "fcproj"        # the fc-projection dX multiplies by the fc layer's saved GELU'
    gen = torch.Generator(device="cuda").manual_seed(11 + M + N)
    bf = torch.bfloat16
    x = torch.randn((M, K), generator=gen, device="cuda").to(bf)
    W = (torch.randn((N, K), generator=gen, device="cuda") * 0.05).to(bf)
    b = (torch.randn((N,), generator=gen, device="cuda") * 0.1).to(bf) if bias else None
    res = torch.randn((M, N), generator=gen, device="cuda").to(bf) if residual else None
    dy = (torch.randn((M, N), generator=gen, device="cuda") * 0.1).to(bf)
    dg = (torch.rand((M, K), generator=gen, device="cuda") * 1.4 - 0.2).to(bf) if gelu_dx else None
    y = torch.empty((M, N), dtype=bf, device="cuda")
    g = torch.empty((M, N), dtype=bf, device="cuda") if gelu else None
    lib.linear_forward(BF16, x, W, b=b, residual=res, gelu_grad=g, y=y)
    dx = torch.empty((M, K), dtype=bf, device="cuda")
    dW = torch.empty((N, K), dtype=torch.float32, device="cuda")
    db = torch.empty((N,), dtype=torch.float32, device="cuda") if bias else None
    lib.linear_backward(BF16, dy, x, W, dx=dx, dW=dW, db=db, gelu_grad=dg)
    torch.cuda.synchronize()
    r = rng(M + N + K)
    im, in_, ik = r.integers(0, M, 512), r.integers(0, N, 512), r.integers(0, K, 512)
    tim, tin, tik = (torch.from_numpy(a).cuda() for a in (im, in_, ik))
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    # forward at the sampled (m, n) pairs
    u = np.einsum("ik,ik->i", f64(x[tim]), f64(W[tin]))
    if bias:
        u = u + f64(b)[in_]
    if residual:
        u = u + f64(res[tim, tin])
    if gelu:
        assert rel(f64(y[tim, tin]), O.gelu_tanh(u)) < 3e-3
        assert rel(f64(g[tim, tin]), O.gelu_tanh_backward(u, np.ones_like(u))) < 3e-3
    else:
        assert rel(f64(y[tim, tin]), u) < 3e-3
    # dX at the sampled (m, k) pairs
    rdx = np.einsum("in,in->i", f64(dy[tim]), f64(W[:, tik].T.contiguous()))
    if gelu_dx:
        rdx = rdx * f64(dg[tim, tik])
    assert rel(f64(dx[tim, tik]), rdx) < 3e-3
    # dW at the sampled (n, k) pairs, reduced over every row
    rdw = np.einsum("mi,mi->i", f64(dy[:, tin]), f64(x[:, tik]))
    assert rel(dW[tin, tik].cpu().numpy(), rdw) < 1e-4
    if bias:
        assert rel(db.cpu().numpy(), f64(dy).sum(0)) < 1e-4


# ---------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
@pytest.mark.parametrize("N,C", [(200, 64), (77, 768), (130, 1600), (24576, 768)])
def test_layernorm_forward_backward(dtype, N, C):
    say("layernorm", DTN[dtype], N, C)
    r = rng(N + C)
    x = r.standard_normal((N, C)) * 2 + 0.5
    w, b = 1 + r.standard_normal(C) * 0.2, r.standard_normal(C) * 0.2
    dy, dres0 = r.standard_normal((N, C)), r.standard_normal((N, C))
    xi, wi, bi, dyi = (as_input(a, dtype).astype(np.float64) for a in (x, w, b, dy))
    y, mean, rstd = empty((N, C), dtype), empty32((N,)), empty32((N,))
    lib.layernorm_forward(dtype, dev(x, dtype), dev(w, dtype), dev(b, dtype), y, mean, rstd)
    ry, cache = O.layernorm_forward(xi, wi, bi)
    assert rel(host(y), ry) < TOL_OUT[dtype]
    assert rel(host(rstd), cache[1][:, 0]) < 1e-5
    assert rel(host(mean), xi.mean(-1)) < 1e-5
    dres = dev(dres0, FP32)
    copy = empty((N, C), dtype) if dtype == BF16 else None
    dw, db = empty32((C,)), empty32((C,))
    lib.layernorm_backward(dtype, dev(dy, dtype), dev(x, dtype), dev(w, dtype), mean, rstd, dres, False, copy,
                           dw, db)
    rdx, rdw, rdb = O.layernorm_backward(dyi, cache)
    expect = dres0.astype(np.float32).astype(np.float64) + rdx
    assert rel(host(dres), expect) < 1e-5
    if copy is not None:
        assert rel(host(copy), expect) < 3e-3
    assert rel(host(dw), rdw) < 1e-5
    assert rel(host(db), rdb) < 1e-5
    # overwrite mode
    lib.layernorm_backward(dtype, dev(dy, dtype), dev(x, dtype), dev(w, dtype), mean, rstd, dres, True, None, dw, db)
    assert rel(host(dres), rdx) < 1e-5


# ---------------------------------------------------------------- attention

def qkv_heads(qkv, B, T, H, hd):
    C = H * hd
    q = qkv[:, :, :C].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    k = qkv[:, :, C:2 * C].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    v = qkv[:, :, 2 * C:].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    return q, k, v


ATT = [(2, 64, 4, 16), (2, 200, 3, 64), (1, 1, 2, 64), (3, 130, 2, 32), (1, 96, 1, 128), (2, 256, 2, 64)]


@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
@pytest.mark.parametrize("B,T,H,hd", ATT)
def test_attention_forward_backward(dtype, B, T, H, hd):
    say("attention", DTN[dtype], B, T, H, hd)
    r = rng(B * 1000 + T + H + hd)
    C = H * hd
    qkv = r.standard_normal((B, T, 3 * C))
    dout = r.standard_normal((B, T, C))
    qi, doi = as_input(qkv, dtype).astype(np.float64), as_input(dout, dtype).astype(np.float64)
    out, lse = empty((B, T, C), dtype), empty32((B, H, T))
    dq = dev(qkv, dtype)
    lib.attention_forward(dtype, B, T, H, hd, dq, out, lse)
    dqkv = empty((B, T, 3 * C), dtype)
    lib.attention_backward(dtype, B, T, H, hd, dq, out, dev(dout, dtype), lse, dqkv)
    q, k, v = qkv_heads(qi, B, T, H, hd)
    ro = np.empty((B, H, T, hd))
    rg = np.empty((B, T, 3 * C))
    rlse = np.empty((B, H, T))
    for b in range(B):
        o, p = O.causal_attention_forward(q[b], k[b], v[b])
        ro[b] = o
        s = np.matmul(q[b], np.swapaxes(k[b], -1, -2)) / math.sqrt(hd)
        s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
        mx = s.max(-1)
        rlse[b] = mx + np.log(np.exp(s - mx[..., None]).sum(-1))
        do = doi[b].reshape(T, H, hd).transpose(1, 0, 2)
        gq, gk, gv = O.causal_attention_backward(do, q[b], k[b], v[b], p)
        rg[b, :, :C] = gq.transpose(1, 0, 2).reshape(T, C)
        rg[b, :, C:2 * C] = gk.transpose(1, 0, 2).reshape(T, C)
        rg[b, :, 2 * C:] = gv.transpose(1, 0, 2).reshape(T, C)
    tol = {FP32: 1e-5, BF16: 6e-3}[dtype]
    assert rel(host(out), ro.transpose(0, 2, 1, 3).reshape(B, T, C)) < tol
    assert rel(host(lse), rlse) < 1e-5 if dtype == FP32 else rel(host(lse), rlse) < 1e-3
    assert rel(host(dqkv), rg) < (1e-5 if dtype == FP32 else 1e-2)


def test_attention_full_size_sampled_heads():
    """GPT-2 124M attention (B=24, T=1024, H=12, hd=64) in bf16: three sampled
    (batch, head) pairs recomputed by the oracle."""
    B, T, H, hd = 24, 1024, 12, 64
    say("attention full size", B, T, H, hd)
    torch = __import__("torch")
    C = H * hd
    gen = torch.Generator(device="cuda").manual_seed(3)
    qkv = torch.randn((B, T, 3 * C), generator=gen, device="cuda").to(torch.bfloat16)
    dout = torch.randn((B, T, C), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    lib.attention_forward(BF16, B, T, H, hd, qkv, out, lse)
    dqkv = torch.empty((B, T, 3 * C), dtype=torch.bfloat16, device="cuda")
    lib.attention_backward(BF16, B, T, H, hd, qkv, out, dout, lse, dqkv)
    torch.cuda.synchronize()
    qn = qkv.float().cpu().numpy().astype(np.float64)
    dn = dout.float().cpu().numpy().astype(np.float64)
    on, gn = out.float().cpu().numpy(), dqkv.float().cpu().numpy()
    for b, h in [(0, 0), (11, 7), (23, 11)]:
        sl = slice(h * hd, (h + 1) * hd)
        q, k, v = qn[b, :, sl], qn[b, :, C + h * hd:C + (h + 1) * hd], qn[b, :, 2 * C + h * hd:2 * C + (h + 1) * hd]
        o, p = O.causal_attention_forward(q[None], k[None], v[None])
        gq, gk, gv = O.causal_attention_backward(dn[b, :, sl][None], q[None], k[None], v[None], p)
        assert rel(on[b, :, sl], o[0]) < 6e-3
        assert rel(gn[b, :, sl], gq[0]) < 1e-2
        assert rel(gn[b, :, C + h * hd:C + (h + 1) * hd], gk[0]) < 1e-2
        assert rel(gn[b, :, 2 * C + h * hd:2 * C + (h + 1) * hd], gv[0]) < 1e-2


# ---------------------------------------------------------------- softmax CE

@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
@pytest.mark.parametrize("N,V,Vp", [(300, 1000, 1024), (64, 512, 512), (33, 50257, 50304), (5, 8, 64)])
def test_softmax_xent(dtype, N, V, Vp):
    say("softmax_xent", DTN[dtype], N, V, Vp)
    r = rng(N + V)
    z = r.standard_normal((N, Vp)) * 2
    z[:, V:] = 30.0          # padded columns must not matter
    y = r.integers(0, V, N)
    zi = as_input(z, dtype).astype(np.float64)
    logits = dev(z, dtype)
    losses = empty32((N,))
    lib.softmax_xent(dtype, logits, dev_i32(y), losses, V, 1.0 / N)
    rl, rdz = O.softmax_cross_entropy(zi[:, :V], y)
    assert rel(host(losses), rl) < 1e-5
    g = host(logits)
    assert np.all(g[:, V:] == 0.0)
    assert rel(g[:, :V], rdz) < TOL_OUT[dtype]
    # each row of dlogits sums to zero (up to the output rounding)
    assert np.abs(g.sum(-1)).max() < 1e-2 / N


@pytest.mark.parametrize("N", [24 * 1024, 24 * 1024 - 104])
def test_classifier_full_size(N):
    """The stand-alone classifier at GPT-2 124M shape (hidden 24x1024x768 ~
    N(0,1), tied table 50304x768 ~ N(0,0.02) including its padded rows,
    labels uniform in [0, 50257)), through the step's own kernels (d_hidden
    reads the table through the transposed copy with the K-grouped 192x192
    tile over the whole vocabulary).  The oracle runs on every row, in row
    chunks: the losses of all rows, dlogits and d_hidden of sampled rows,
    and 64 sampled rows of d_wte element by element (the mean-loss gradient
    over all rows is the sum of the chunks' gradients, each scaled by its
    share of the rows); padded rows of dlogits and d_wte are exactly zero.
    The second row count (a multiple of 8, as the bf16 GEMMs require of every
    reduction length) leaves a ragged last row tile in every product and a
    partial last K step in d_wte."""
    C, V, Vp = 768, 50257, 50304
    say("classifier full size", N, C, V, Vp)
    torch = __import__("torch")
    hidden, wte, labels = S.classifier_inputs(N, C, V, Vp, seed=17)
    h_d, w_d = dev(hidden, BF16), dev(wte, BF16)
    losses = empty32((N,))
    logits = torch.empty((N, Vp), dtype=torch.bfloat16, device="cuda")
    d_hidden = torch.empty((N, C), dtype=torch.bfloat16, device="cuda")
    d_wte = torch.empty((Vp, C), dtype=torch.float32, device="cuda")
    lib.classifier_fwd_bwd(BF16, h_d, w_d, dev_i32(labels), V, losses, logits, d_hidden, d_wte)
    torch.cuda.synchronize()
    hi = S.bf16_round(hidden).astype(np.float32)
    wi = S.bf16_round(wte)[:V].astype(np.float32)
    rows = np.unique(np.concatenate([rng(1).integers(0, N, 48), [0, N - 1, N - 37]]))
    vrows = np.unique(np.concatenate([rng(2).integers(0, V, 60), [0, V - 1], labels[rows[:2]]]))
    rl = np.empty(N)
    rdwte = np.zeros((len(vrows), C))
    rdz, rdh = {}, {}
    chunk = 2048
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        l, dz = O.softmax_cross_entropy(hi[r0:r1] @ wi.T, labels[r0:r1])
        dz = dz.astype(np.float64) * ((r1 - r0) / N)        # chunk mean -> share of the mean over N rows
        rl[r0:r1] = l
        rdwte += dz[:, vrows].T @ hi[r0:r1].astype(np.float64)
        for i in rows[(rows >= r0) & (rows < r1)]:
            rdz[i] = dz[i - r0]
            rdh[i] = dz[i - r0] @ wi.astype(np.float64)
    assert rel(losses.cpu().numpy(), rl) < 1e-3
    trows = torch.from_numpy(rows).cuda()
    gdz = logits[trows].float().cpu().numpy()
    assert np.all(gdz[:, V:] == 0)
    assert rel(gdz[:, :V], np.stack([rdz[i] for i in rows])) < 1e-2
    assert rel(d_hidden[trows].float().cpu().numpy(), np.stack([rdh[i] for i in rows])) < 1e-2
    dw = d_wte.cpu().numpy().astype(np.float64)
    assert np.all(dw[V:] == 0)
    assert rel(dw[vrows], rdwte) < 1e-2
    for j, v in enumerate(vrows[:8]):            # and row by row
        assert rel(dw[v], rdwte[j]) < 3e-2, v
    assert np.isfinite(dw).all()


# ---------------------------------------------------------------- encoder

@pytest.mark.parametrize("dtype", DT, ids=DTN.get)
# (40, 1024): more positions than one workgroup's key sort held (32768);
# (1, 5000): a non-power-of-two count above the 4096-key LDS chunk
@pytest.mark.parametrize("B,T,C,V", [(4, 64, 64, 512), (24, 1024, 768, 50257), (3, 40, 128, 300),
                                     (40, 1024, 64, 50257), (1, 5000, 64, 300)])
def test_encoder(dtype, B, T, C, V):
    say("encoder", DTN[dtype], B, T, C, V)
    r = rng(B + T + C)
    maxT = T + 8
    if V >= 50000:
        tok, _ = S.zipf_batch(B, T, seed=5)
    else:
        tok = r.integers(0, V, (B, T)).astype(np.int32)
        tok[0, : T // 2] = 3          # a hot row
    wte, wpe = r.standard_normal((V, C)), r.standard_normal((maxT, C))
    out = empty((B, T, C), dtype)
    lib.encoder_forward(dtype, dev_i32(tok), dev(wte, dtype), dev(wpe, dtype), out, V)
    ref = O.encoder_forward(as_input(wte, dtype).astype(np.float64), as_input(wpe, dtype).astype(np.float64), tok)
    expect = as_input(ref, dtype)
    assert np.array_equal(host(out).astype(np.float32), expect)
    dx0 = r.standard_normal((B, T, C)).astype(np.float32)
    base = r.standard_normal((V, C)).astype(np.float32)
    dwte, dwpe = dev(base, FP32), empty32((T, C))
    lib.encoder_backward(dev_i32(tok), dev(dx0, FP32), dwte, dwpe, V)
    rw, rp = O.encoder_backward(dx0.astype(np.float64), tok, V, T)
    got = host(dwte)
    assert rel(got, base + rw) < 1e-6
    assert rel(host(dwpe), rp) < 1e-6
    # deterministic: a second run gives identical bits
    dwte2 = dev(base, FP32)
    lib.encoder_backward(dev_i32(tok), dev(dx0, FP32), dwte2, dwpe, V)
    assert np.array_equal(host(dwte2), got)


@pytest.mark.parametrize("B,T,C,V", [(2, 300, 6, 40), (3, 200, 20, 5)])
def test_encoder_backward_narrow(B, T, C, V):
    # widths that are not a multiple of 4 (the scalar channel path), and a
    # vocabulary so small that runs of one token cross many 64-position pieces
    say("encoder_backward", B, T, C, V)
    r = rng(B * T + C)
    tok = r.integers(0, V, (B, T)).astype(np.int32)
    dx0 = r.standard_normal((B, T, C)).astype(np.float32)
    base = r.standard_normal((V, C)).astype(np.float32)
    dwte, dwpe = dev(base, FP32), empty32((T, C))
    lib.encoder_backward(dev_i32(tok), dev(dx0, FP32), dwte, dwpe, V)
    rw, rp = O.encoder_backward(dx0.astype(np.float64), tok, V, T)
    assert rel(host(dwte), base + rw) < 1e-6
    assert rel(host(dwpe), rp) < 1e-6


# ---------------------------------------------------------------- AdamW

@pytest.mark.parametrize("n", [1000003, 64, 5])
def test_adamw(n):
    say("adamw", n)
    torch = __import__("torch")
    r = rng(n)
    th, g = r.standard_normal(n).astype(np.float32), r.standard_normal(n).astype(np.float32)
    m0 = (r.standard_normal(n) * 0.1).astype(np.float32)
    v0 = np.abs(r.standard_normal(n) * 0.1).astype(np.float32)
    M, G, Mm, Vv = (dev(a, FP32) for a in (th, g, m0, v0))
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    lib.adamw(M, G, Mm, Vv, pb, 6e-4, 0.9, 0.95, 1e-8, 0.1, 3)
    rt, rm, rv = O.adamw_update(th.astype(np.float64), g.astype(np.float64), m0.astype(np.float64),
                                v0.astype(np.float64), 6e-4, 0.9, 0.95, 1e-8, 0.1, 3)
    assert rel(host(M), rt) < 1e-6
    # the update itself (~lr): fp32 rounding of theta (~6e-8) bounds its relative error by ~1e-4
    assert rel(host(M) - th, rt - th) < 1e-3
    assert rel(host(Mm), rm) < 1e-6 and rel(host(Vv), rv) < 1e-6
    assert np.array_equal(host(pb).astype(np.float32), S.bf16_round(host(M).astype(np.float32)))

"""Plain CPU oracle of one GPT-2 training step: forward, hand-written backward
and AdamW, in numpy, generic over float32 / float64.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP library and imports nothing from it.

What is computed, and where it comes from
-----------------------------------------
The page "State of the Union [May 3, 2024]" (karpathy/llm.c discussion #344)
is the primary source.  Its opening bullet list names bf16 mixed precision
with an fp32 master copy, a fused classifier that evaluates the loss only at
the label's index, and flash attention; its kernel table (section "Runtime,
DRAM traffic, instructions") lists the kernels of one step: encoder
forward/backward, layernorm forward/backward, GEMMs, attention, gelu
forward/backward, residual add, fused classifier and adamw; its "Fine print"
section fixes the vocabulary padding 50257 -> 50304 with the padded logits
masked to -inf.

Every fused or faster piece of that design reaches the plain mathematical
result up to rounding (flash attention is exact attention, the fused
classifier is softmax cross-entropy read at the label), so this oracle is the
plain definition written out, with no blocking, fusion or reordering:

* LayerNorm: biased variance over the channel axis, eps = 1e-5 inside the
  square root (the pages are silent; standard GPT-2 reading).
* GELU: tanh approximation 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))
  (the pages only name the kernels; Hendrycks & Gimpel 2016).
* Attention: scale 1/sqrt(hd), keys j > i masked to -inf, softmax over keys.
* Classifier: tied to the token table, no bias; only the V real rows exist
  here (padding is a property of the GPU layout, checked separately).
* Loss: mean over all B*T positions, no ignore index.
* AdamW: Loshchilov & Hutter decoupled decay with bias correction, eps added
  to sqrt(v_hat), decay applied to every parameter.

The oracle's parameters are a dict ``name -> ndarray`` with weights stored
[out, in] (y = x W^T + b) and the QKV output columns ordered [q | k | v],
head h owning columns h*hd .. h*hd+hd-1 inside each.

Pins (see tests/test_oracle_*.py): finite differences in float64, torch CPU
float64 library routines for single layers and a whole-model autograd check,
the closed form of the initial loss, the exact ln V loss with a zero token
table, causality, softmax row sums, AdamW's closed form at t = 1 and brute
force loops for the encoder scatter; for accumulation and clipping, the
identity with the concatenated batch, the clipping closed forms and torch's
clip_grad_norm_ + AdamW on the whole tiny model.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .fp8 import fp8_linear_backward, fp8_linear_forward

LN_EPS = 1e-5
GELU_K0 = math.sqrt(2.0 / math.pi)
GELU_K1 = 0.044715


@dataclass(frozen=True)
class OracleConfig:
    vocab_size: int      # V, real token ids 0..V-1
    max_seq_len: int     # rows of the position table
    num_layers: int      # L
    num_heads: int       # H
    channels: int        # C
    # architecture variants (see "Architecture variants" below); all off is GPT-2
    relu2: bool = False
    qk_norm: bool = False
    rope: bool = False
    # FP8 products (oracle/fp8.py) for the QKV projection, the MLP and the head
    fp8: bool = False

    @property
    def head_dim(self) -> int:
        return self.channels // self.num_heads


def param_shapes(cfg: OracleConfig):
    """Shapes of every parameter tensor, [out, in] for weights, in the order
    the step visits them (token table first, final LayerNorm last)."""
    V, T, L, C = cfg.vocab_size, cfg.max_seq_len, cfg.num_layers, cfg.channels
    return [
        ("wte", (V, C)),
        ("wpe", (T, C)),
        ("ln1w", (L, C)),
        ("ln1b", (L, C)),
        ("qkvw", (L, 3 * C, C)),
        ("qkvb", (L, 3 * C)),
        ("attprojw", (L, C, C)),
        ("attprojb", (L, C)),
        ("ln2w", (L, C)),
        ("ln2b", (L, C)),
        ("fcw", (L, 4 * C, C)),
        ("fcb", (L, 4 * C)),
        ("fcprojw", (L, C, 4 * C)),
        ("fcprojb", (L, C)),
        ("lnfw", (C,)),
        ("lnfb", (C,)),
    ]


# --------------------------------------------------------------------------
# Layer definitions
# --------------------------------------------------------------------------

def layernorm_forward(x, w, b, eps=LN_EPS):
    """y = (x - mean) / sqrt(var + eps) * w + b over the last axis (biased var).

    Returns y and the cache (xhat, rstd, w) the backward needs."""
    mean = x.mean(axis=-1, keepdims=True)
    xc = x - mean
    var = (xc * xc).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = xc * rstd
    return xhat * w + b, (xhat, rstd, w)


def layernorm_backward(dy, cache):
    """Gradient of LayerNorm: dx, dw, db (dw/db summed over all leading axes).

    With g = dy * w:  dx = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat))."""
    xhat, rstd, w = cache
    lead = tuple(range(dy.ndim - 1))
    dw = (dy * xhat).sum(axis=lead)
    db = dy.sum(axis=lead)
    g = dy * w
    dx = rstd * (g - g.mean(axis=-1, keepdims=True)
                 - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dx, dw, db


def gelu_tanh(u):
    """0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(GELU_K0 * (u + GELU_K1 * u ** 3)))


def gelu_tanh_backward(u, dg):
    """dg * d/du GELU_tanh(u), differentiated by hand from the formula above."""
    kappa = GELU_K0 * (u + GELU_K1 * u ** 3)
    th = np.tanh(kappa)
    dkappa = GELU_K0 * (1.0 + 3.0 * GELU_K1 * u * u)
    return dg * (0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * dkappa)


def linear_forward(x, w, b=None):
    """y = x W^T (+ b) for W stored [out, in]."""
    y = x @ w.T
    return y if b is None else y + b


def linear_backward(dy, x, w):
    """Gradients of y = x W^T + b:  dx = dy W,  dW = dy^T x,  db = sum over rows of dy."""
    dy2 = dy.reshape(-1, dy.shape[-1])
    x2 = x.reshape(-1, x.shape[-1])
    return (dy @ w), dy2.T @ x2, dy2.sum(axis=0)


def _softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def causal_attention_forward(q, k, v):
    """Exact causal attention for one batch row.

    q, k, v: [H, T, hd].  S = q k^T / sqrt(hd), keys j > i set to -inf,
    P = softmax over keys, O = P v.  Returns O [H, T, hd] and P [H, T, T]."""
    H, T, hd = q.shape
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * (1.0 / math.sqrt(hd))
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    p = _softmax_rows(s)
    return np.matmul(p, v), p


def causal_attention_backward(do, q, k, v, p):
    """Gradients of causal attention for one batch row (textbook softmax
    Jacobian):  dV = P^T dO;  dP = dO V^T;  dS = P * (dP - sum_j P dP);
    dQ = dS K / sqrt(hd);  dK = dS^T Q / sqrt(hd)."""
    hd = q.shape[-1]
    scale = 1.0 / math.sqrt(hd)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) * scale
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) * scale
    return dq, dk, dv


def softmax_cross_entropy(z, y):
    """Per-row loss logsumexp(z_i) - z_i[y_i] and the gradient of the MEAN loss,
    dz = (softmax(z) - onehot(y)) / N, for z [N, V], y [N]."""
    n = z.shape[0]
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    rows = np.arange(n)
    losses = lse - z[rows, y]
    dz = e / s
    dz[rows, y] -= 1.0
    dz /= n
    return losses, dz


def encoder_forward(wte, wpe, tokens):
    """x0[b, t] = wte[tokens[b, t]] + wpe[t]."""
    T = tokens.shape[1]
    return wte[tokens] + wpe[:T][None, :, :]


def encoder_backward(dx0, tokens, vocab_size, max_seq_len):
    """Scatter-add of dx0 rows into the token table by token id, and the sum
    over the batch for the position table.  Written as plain loops over the
    positions (np.add.at), the definition of the scatter."""
    B, T, C = dx0.shape
    dwte = np.zeros((vocab_size, C), dtype=dx0.dtype)
    np.add.at(dwte, tokens.reshape(-1), dx0.reshape(-1, C))
    dwpe = np.zeros((max_seq_len, C), dtype=dx0.dtype)
    dwpe[:T] = dx0.sum(axis=0)
    return dwte, dwpe


def adamw_update(theta, g, m, v, lr, beta1, beta2, eps, wd, t):
    """One AdamW update (Loshchilov & Hutter 2019, decoupled decay, bias
    corrected, eps added to sqrt(v_hat)).  Returns new (theta, m, v)."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    theta = theta - lr * (mhat / (np.sqrt(vhat) + eps) + wd * theta)
    return theta, m, v


# --------------------------------------------------------------------------
# Architecture variants
# --------------------------------------------------------------------------
# The page "NanoGPT (124M) in 90 seconds" (section "How it works", item
# "Architecture Changes") names rotary embeddings, QK-Norm and ReLU^2 and
# gives no formula.  The readings here are the plainest ones:
# * ReLU^2: the MLP activation relu(u)^2 in place of GELU-tanh.
# * QK-Norm: q and k of every head divided by their root mean square over the
#   head dimension, sqrt(mean(x^2) + eps) with eps = 1e-6, no learned gain;
#   the attention scale stays 1/sqrt(hd).
# * Rotary embedding (Su et al., RoFormer, 2021): at position t the pair of
#   head coordinates (i, i + hd/2), i < hd/2, is rotated by the angle
#   t * 10000^(-2i/hd): (a, b) -> (a cos - b sin, a sin + b cos).  It acts on
#   q and k after QK-Norm; the learned position table is then not added to
#   the token embedding (it stays a parameter, with zero gradient).

RMS_EPS = 1e-6
ROPE_BASE = 10000.0


def relu2(u):
    """relu(u)^2."""
    r = np.maximum(u, 0.0)
    return r * r


def relu2_backward(u, dg):
    """dg * d/du relu(u)^2 = dg * 2 relu(u)."""
    return dg * (2.0 * np.maximum(u, 0.0))


def rms_norm_forward(x, eps=RMS_EPS):
    """y = x / sqrt(mean(x^2) + eps) over the last axis; returns y and the
    cache (y, r) with r = 1 / sqrt(mean(x^2) + eps)."""
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    y = x * r
    return y, (y, r)


def rms_norm_backward(dy, cache):
    """Gradient of rms_norm_forward: with y = x r and dr/dx = -r^3 x / n,
    dx = r (dy - y mean(dy * y))."""
    y, r = cache
    return r * (dy - y * (dy * y).mean(axis=-1, keepdims=True))


def rope_angles(T, hd, base=ROPE_BASE):
    """[T, hd/2] angles t * base^(-2i/hd)."""
    i = np.arange(hd // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / hd)
    return np.arange(T, dtype=np.float64)[:, None] * theta[None, :]


def rope_forward(x, ang):
    """Rotate the (i, i + hd/2) coordinate pairs of x [..., T, hd] by ang [T, hd/2]."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_backward(dy, ang):
    """Gradient of rope_forward: the transposed (inverse) rotation of dy."""
    h = dy.shape[-1] // 2
    da, db = dy[..., :h], dy[..., h:]
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([da * c + db * s, -da * s + db * c], axis=-1)


# --------------------------------------------------------------------------
# Whole model
# --------------------------------------------------------------------------

def _split_heads(x, H):
    T, C = x.shape
    return x.reshape(T, H, C // H).transpose(1, 0, 2)


def _wgrad(dy, x):
    """Weight gradient of y = x W^T: dW[n, k] = sum over positions dy[., n] x[., k]."""
    return dy.reshape(-1, dy.shape[-1]).T @ x.reshape(-1, x.shape[-1])


def _merge_heads(x):
    H, T, hd = x.shape
    return x.transpose(1, 0, 2).reshape(T, H * hd)


def _lin(cfg, x, w, b=None):
    """A linear layer of the FP8 set (QKV, fc, fc-proj, head): the fp8
    product when cfg.fp8 (its cache kept for the backward), else x W^T + b."""
    if cfg.fp8:
        y, c = fp8_linear_forward(x, w, b)
        return y.astype(x.dtype), c
    return linear_forward(x, w, b), None


def _lin_grads(cfg, dy, x, w, cache):
    """(dx, dW, db) of a layer of the FP8 set."""
    if cfg.fp8:
        dx, dw, db = fp8_linear_backward(dy, cache)
        return dx.astype(dy.dtype), dw.astype(dy.dtype), db
    return dy @ w, _wgrad(dy, x), dy.reshape(-1, dy.shape[-1]).sum(axis=0)


def gpt2_forward(params, tokens, targets, cfg: OracleConfig):
    """Forward pass.  tokens, targets: int arrays [B, T] (targets may be None).

    Returns (mean_loss or None, per-position losses or None, logits, cache)."""
    B, T = tokens.shape
    C, H, L = cfg.channels, cfg.num_heads, cfg.num_layers
    if cfg.rope:     # positions enter through the rotation only
        x = params["wte"][tokens]
    else:
        x = encoder_forward(params["wte"], params["wpe"], tokens)
    ang = rope_angles(T, C // H) if cfg.rope else None
    layers = []
    for l in range(L):
        ln1, ln1_c = layernorm_forward(x, params["ln1w"][l], params["ln1b"][l])
        qkv, qkv_q = _lin(cfg, ln1, params["qkvw"][l], params["qkvb"][l])
        att = np.empty_like(x)
        probs, qk = [], []
        for b in range(B):
            q = _split_heads(qkv[b, :, 0:C], H)
            k = _split_heads(qkv[b, :, C:2 * C], H)
            v = _split_heads(qkv[b, :, 2 * C:3 * C], H)
            qc = kc = None
            if cfg.qk_norm:
                q, qc = rms_norm_forward(q)
                k, kc = rms_norm_forward(k)
            if cfg.rope:
                q, k = rope_forward(q, ang), rope_forward(k, ang)
            o, p = causal_attention_forward(q, k, v)
            att[b] = _merge_heads(o)
            probs.append(p)
            qk.append((q, k, qc, kc))
        h = x + att @ params["attprojw"][l].T + params["attprojb"][l]
        ln2, ln2_c = layernorm_forward(h, params["ln2w"][l], params["ln2b"][l])
        u, fc_q = _lin(cfg, ln2, params["fcw"][l], params["fcb"][l])
        g = relu2(u) if cfg.relu2 else gelu_tanh(u)
        proj, fcproj_q = _lin(cfg, g, params["fcprojw"][l], params["fcprojb"][l])
        x_next = h + proj
        layers.append(dict(x=x, ln1=ln1, ln1_c=ln1_c, qkv=qkv, att=att, qk=qk,
                           probs=probs, h=h, ln2=ln2, ln2_c=ln2_c, u=u, g=g,
                           qkv_q=qkv_q, fc_q=fc_q, fcproj_q=fcproj_q))
        x = x_next
    lnf, lnf_c = layernorm_forward(x, params["lnfw"], params["lnfb"])
    logits, head_q = _lin(cfg, lnf.reshape(B * T, C), params["wte"])
    cache = dict(tokens=tokens, layers=layers, xL=x, lnf=lnf, lnf_c=lnf_c,
                 logits=logits, B=B, T=T, ang=ang, head_q=head_q)
    if targets is None:
        return None, None, logits.reshape(B, T, -1), cache
    losses, dz = softmax_cross_entropy(logits, targets.reshape(-1))
    cache["dlogits"] = dz
    return losses.mean(), losses.reshape(B, T), logits.reshape(B, T, -1), cache


def gpt2_backward(params, cache, cfg: OracleConfig):
    """Backward pass of the mean loss; returns a dict of parameter gradients
    with the same keys and shapes as ``params``."""
    B, T = cache["B"], cache["T"]
    C, H, L = cfg.channels, cfg.num_heads, cfg.num_layers
    grads = {k: np.zeros_like(v) for k, v in params.items()}
    dz = cache["dlogits"]                                    # [BT, V]
    lnf = cache["lnf"].reshape(B * T, C)
    dlnf, dwte_head, _ = _lin_grads(cfg, dz, lnf, params["wte"], cache["head_q"])
    grads["wte"] += dwte_head
    dlnf = dlnf.reshape(B, T, C)
    dx, grads["lnfw"], grads["lnfb"] = layernorm_backward(dlnf, cache["lnf_c"])
    for l in reversed(range(L)):
        c = cache["layers"][l]
        # x_next = h + g Wp^T + bp
        dg, grads["fcprojw"][l], grads["fcprojb"][l] = _lin_grads(cfg, dx, c["g"], params["fcprojw"][l],
                                                                  c["fcproj_q"])
        du = relu2_backward(c["u"], dg) if cfg.relu2 else gelu_tanh_backward(c["u"], dg)
        dln2, grads["fcw"][l], grads["fcb"][l] = _lin_grads(cfg, du, c["ln2"], params["fcw"][l], c["fc_q"])
        dh_ln, grads["ln2w"][l], grads["ln2b"][l] = layernorm_backward(dln2, c["ln2_c"])
        dh = dx + dh_ln
        # h = x + att Wo^T + bo
        datt = dh @ params["attprojw"][l]
        grads["attprojw"][l] = _wgrad(dh, c["att"])
        grads["attprojb"][l] = dh.sum(axis=(0, 1))
        dqkv = np.empty_like(c["qkv"])
        for b in range(B):
            q, k, qc, kc = c["qk"][b]          # as the attention saw them
            v = _split_heads(c["qkv"][b, :, 2 * C:3 * C], H)
            do = _split_heads(datt[b], H)
            dq, dk, dv = causal_attention_backward(do, q, k, v, c["probs"][b])
            if cfg.rope:
                dq, dk = rope_backward(dq, cache["ang"]), rope_backward(dk, cache["ang"])
            if cfg.qk_norm:
                dq, dk = rms_norm_backward(dq, qc), rms_norm_backward(dk, kc)
            dqkv[b, :, 0:C] = _merge_heads(dq)
            dqkv[b, :, C:2 * C] = _merge_heads(dk)
            dqkv[b, :, 2 * C:3 * C] = _merge_heads(dv)
        dln1, grads["qkvw"][l], grads["qkvb"][l] = _lin_grads(cfg, dqkv, c["ln1"], params["qkvw"][l], c["qkv_q"])
        dx_ln, grads["ln1w"][l], grads["ln1b"][l] = layernorm_backward(dln1, c["ln1_c"])
        dx = dh + dx_ln
    dwte, dwpe = encoder_backward(dx, cache["tokens"], cfg.vocab_size, cfg.max_seq_len)
    grads["wte"] += dwte
    if not cfg.rope:         # with rotary embeddings the position table is not used
        grads["wpe"] += dwpe
    return grads


def gpt2_step(params, tokens, targets, cfg: OracleConfig, adam_state, lr, beta1,
              beta2, eps, wd, t):
    """Forward + backward + AdamW.  ``adam_state`` is a dict name -> (m, v) or
    None for zeros.  Returns (mean_loss, grads, new_params, new_state)."""
    loss, _, _, cache = gpt2_forward(params, tokens, targets, cfg)
    grads = gpt2_backward(params, cache, cfg)
    new_params, new_state = {}, {}
    for name, theta in params.items():
        if adam_state is None:
            m = np.zeros_like(theta)
            v = np.zeros_like(theta)
        else:
            m, v = adam_state[name]
        new_params[name], m, v = adamw_update(theta, grads[name], m, v, lr, beta1,
                                              beta2, eps, wd, t)
        new_state[name] = (m, v)
    return loss, grads, new_params, new_state


# --------------------------------------------------------------------------
# Gradient accumulation and global-norm clipping
# --------------------------------------------------------------------------
# The page "State of the Union [May 3, 2024]" lists both as pending work for
# the GPT-2 miniseries (section "Functional") and gives no formula, so the
# readings are the standard ones:
# * accumulation over k equal micro-batches is the gradient of the mean of
#   their mean losses, (1/k) sum_i grad_i -- the gradient of the mean loss
#   over the concatenated batch;
# * clipping takes the L2 norm n of all parameter gradients as one vector
#   and, when n exceeds max_norm > 0, multiplies every gradient by
#   max_norm / n (no epsilon); max_norm <= 0 leaves them as they are.

def accumulate_grads(grad_list):
    """(1/k) sum of k gradient dicts."""
    k = len(grad_list)
    out = {name: np.zeros_like(g) for name, g in grad_list[0].items()}
    for g in grad_list:
        for name in out:
            out[name] = out[name] + g[name] / k
    return out


def global_grad_norm(grads):
    """L2 norm of all gradients taken as one vector (accumulated in float64)."""
    total = 0.0
    for g in grads.values():
        total += float(np.sum(np.asarray(g, dtype=np.float64) ** 2))
    return math.sqrt(total)


def clip_factor(norm, max_norm):
    """max_norm / norm when norm > max_norm > 0, else 1."""
    return max_norm / norm if (max_norm > 0 and norm > max_norm) else 1.0


def gpt2_step_accumulated(params, micro_batches, cfg: OracleConfig, adam_state, lr, beta1, beta2, eps, wd, t,
                          max_grad_norm=0.0):
    """Forward + backward over each (tokens, targets) micro-batch, accumulated
    gradients, global-norm clipping, AdamW.  Returns (losses, grads, norm,
    new_params, new_state) with grads and norm before clipping."""
    losses, glist = [], []
    for tokens, targets in micro_batches:
        loss, _, _, cache = gpt2_forward(params, tokens, targets, cfg)
        losses.append(loss)
        glist.append(gpt2_backward(params, cache, cfg))
    grads = accumulate_grads(glist)
    norm = global_grad_norm(grads)
    s = clip_factor(norm, max_grad_norm)
    new_params, new_state = {}, {}
    for name, theta in params.items():
        if adam_state is None:
            m = np.zeros_like(theta)
            v = np.zeros_like(theta)
        else:
            m, v = adam_state[name]
        new_params[name], m, v = adamw_update(theta, grads[name] * s, m, v, lr, beta1, beta2, eps, wd, t)
        new_state[name] = (m, v)
    return losses, grads, norm, new_params, new_state

"""Seeded synthetic inputs (token streams, parameter sets, classifier tensors).

This module holds none of the training step's arithmetic: it only draws
random inputs.  It is the one piece the HIP path's drivers (bench, tests) and
the CPU oracle's drivers both use, so the two sides see identical inputs.

Token statistics stand in for the text corpora the pages train on (TinyStories
in "State of the Union [May 3, 2024]", section "Peak memory"; FineWeb on the
modded-nanogpt page): Zipf(s = 1.1) ranks over the 50257 GPT-2 ids with the
end-of-text id 50256 inserted after Geometric(1/512) gaps.
"""

from __future__ import annotations

import math

import numpy as np

GPT2_VOCAB = 50257
GPT2_EOT = 50256


def _zipf_cdf(V: int, s: float) -> np.ndarray:
    w = 1.0 / np.arange(1, V + 1, dtype=np.float64) ** s
    c = np.cumsum(w)
    return c / c[-1]


_CDF_CACHE: dict = {}


def zipf_eot_stream(n: int, seed: int, V: int = GPT2_VOCAB, s: float = 1.1,
                    eot: int = GPT2_EOT, mean_gap: float = 512.0) -> np.ndarray:
    """n token ids: id = Zipf rank - 1 (rank 1 most frequent), truncated to V
    ids; every Geometric(1/mean_gap) tokens the position is overwritten by eot."""
    key = (V, s)
    if key not in _CDF_CACHE:
        _CDF_CACHE[key] = _zipf_cdf(V, s)
    cdf = _CDF_CACHE[key]
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right").astype(np.int64)
    ids = np.minimum(ids, V - 1)
    pos = -1
    while True:
        pos += int(rng.geometric(1.0 / mean_gap))
        if pos >= n:
            break
        ids[pos] = eot
    return ids.astype(np.int32)


def zipf_batch(B: int, T: int, seed: int, V: int = GPT2_VOCAB):
    """(inputs, targets), both int32 [B, T]: a stream of B*T + 1 tokens,
    inputs = stream[:-1], targets = stream[1:]."""
    st = zipf_eot_stream(B * T + 1, seed, V=V, eot=V - 1)
    return st[:-1].reshape(B, T).copy(), st[1:].reshape(B, T).copy()


def uniform_batch(B: int, T: int, V: int, seed: int):
    """(inputs, targets) i.i.d. uniform in [0, V), drawn independently."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.integers(0, V, size=(B, T), dtype=np.int64).astype(np.int32)
    y = rng.integers(0, V, size=(B, T), dtype=np.int64).astype(np.int32)
    return x, y


def param_table(V: int, Vp: int, maxT: int, L: int, C: int):
    """(name, shape) of every parameter tensor in the library's flat order;
    the token table has Vp rows here (rows >= V are padding)."""
    return [
        ("wte", (Vp, C)), ("wpe", (maxT, C)),
        ("ln1w", (L, C)), ("ln1b", (L, C)),
        ("qkvw", (L, 3 * C, C)), ("qkvb", (L, 3 * C)),
        ("attprojw", (L, C, C)), ("attprojb", (L, C)),
        ("ln2w", (L, C)), ("ln2b", (L, C)),
        ("fcw", (L, 4 * C, C)), ("fcb", (L, 4 * C)),
        ("fcprojw", (L, C, 4 * C)), ("fcprojb", (L, C)),
        ("lnfw", (C,)), ("lnfb", (C,)),
    ]


def random_params(V: int, Vp: int, maxT: int, L: int, C: int, seed: int,
                  perturbed: bool = True, pad_value: float = 0.0) -> dict:
    """float32 parameters with GPT-2-like scales.

    perturbed=False: weights N(0, 0.02) (residual projections 0.02/sqrt(2L)),
    biases 0, LayerNorm gains 1, shifts 0.  perturbed=True additionally draws
    biases N(0, 0.02) and gains 1 + N(0, 0.1), shifts N(0, 0.02) so that every
    parameter influences the loss.  Padded token-table rows get pad_value."""
    rng = np.random.Generator(np.random.PCG64(seed))
    resid = 0.02 / math.sqrt(2.0 * max(L, 1))
    out = {}
    for name, shape in param_table(V, Vp, maxT, L, C):
        if name in ("ln1w", "ln2w", "lnfw"):
            a = 1.0 + (rng.standard_normal(shape) * 0.1 if perturbed else 0.0)
            a = np.broadcast_to(a, shape)
        elif name in ("ln1b", "ln2b", "lnfb", "qkvb", "attprojb", "fcb", "fcprojb"):
            a = rng.standard_normal(shape) * 0.02 if perturbed else np.zeros(shape)
        else:
            std = resid if name in ("attprojw", "fcprojw") else 0.02
            a = rng.standard_normal(shape) * std
        a = np.ascontiguousarray(a, dtype=np.float32)
        if name == "wte":
            a[V:] = pad_value
        out[name] = a
    return out


def classifier_inputs(BT: int, C: int, V: int, Vp: int, seed: int):
    """Inputs of the stand-alone classifier: hidden ~ N(0, 1) [BT, C],
    token table ~ N(0, 0.02) [Vp, C] including its padded rows, and labels
    uniform in [0, V).  All float32; the caller rounds to its storage type."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hidden = rng.standard_normal((BT, C), dtype=np.float32)
    wte = (rng.standard_normal((Vp, C), dtype=np.float32) * np.float32(0.02))
    labels = rng.integers(0, V, size=BT, dtype=np.int64).astype(np.int32)
    return hidden, wte, labels


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32.  This is input preparation (the stored precision of a
    bf16 input tensor), not part of the step."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    r = r.astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint32(0x7FC00000)
    return r.view(np.float32)

"""Seeded parameter initialisation, re-derived independently of the library
(TEST INFRASTRUCTURE: only tests, smoke() and bench.py's cpu_baseline use it).

The page "State of the Union [May 3, 2024]" lists "init from random weights
direct in C" among the pending items (section opening the post, paragraph
"Functional").  The distribution is the GPT-2 one: N(0, 0.02) for the token
and position tables, the QKV and the MLP up-projection weights;
N(0, 0.02 / sqrt(2 L)) for the two residual projections; biases 0; LayerNorm
gains 1 and shifts 0; padded token-table rows 0.

Counter-based generator (both sides implement it from this definition):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the n-th output (n = 0, 1, ...) of the stream
  seeded with s is mix(s + (n + 1) * 0x9E3779B97F4A7C15 mod 2^64), where
  mix(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31.
* Element e (row-major index inside its tensor) of tensor number i (its
  position in the parameter order) uses counter c = (i << 40) | e and the two
  stream outputs r0 = out(2c), r1 = out(2c + 1).
* Box-Muller (1958): u1 = ((r0 >> 11) + 1) * 2^-53 in (0, 1],
  u2 = (r1 >> 11) * 2^-53 in [0, 1), z = sqrt(-2 ln u1) cos(2 pi u2),
  evaluated in float64; the parameter is float32(std * z).
"""

from __future__ import annotations

import math

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
MIX_M1 = np.uint64(0xBF58476D1CE4E5B9)
MIX_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z):
    z = z ^ (z >> np.uint64(30))
    z = z * MIX_M1
    z = z ^ (z >> np.uint64(27))
    z = z * MIX_M2
    return z ^ (z >> np.uint64(31))


def splitmix64_stream(seed: int, n):
    """Outputs number n (array of uint64) of the SplitMix64 stream seeded with seed."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (n + np.uint64(1)) * GOLDEN_GAMMA
        return _mix(state)


def normal_for(seed: int, tensor_index: int, count: int, std: float, chunk=1 << 22):
    """float32 N(0, std^2) draws for elements 0..count-1 of one tensor."""
    out = np.empty(count, dtype=np.float32)
    base = np.uint64(tensor_index) << np.uint64(40)
    for s in range(0, count, chunk):
        e = np.arange(s, min(count, s + chunk), dtype=np.uint64)
        c = base | e
        r0 = splitmix64_stream(seed, c * np.uint64(2))
        r1 = splitmix64_stream(seed, c * np.uint64(2) + np.uint64(1))
        u1 = ((r0 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
        u2 = (r1 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
        out[s:s + len(e)] = (std * z).astype(np.float32)
    return out


def gpt2_init_params(shapes, num_layers: int, seed: int, vocab_rows: int | None = None):
    """Initial parameters for the list of (name, shape) in parameter order.

    ``vocab_rows``: if the token table in ``shapes`` has padded rows beyond the
    real vocabulary, rows >= vocab_rows are set to zero."""
    resid_std = 0.02 / math.sqrt(2.0 * num_layers)
    params = {}
    for i, (name, shape) in enumerate(shapes):
        n = int(np.prod(shape))
        if name in ("ln1w", "ln2w", "lnfw"):
            a = np.ones(n, dtype=np.float32)
        elif name.endswith("b") and name not in ("wte",):
            a = np.zeros(n, dtype=np.float32)
        else:
            std = resid_std if name in ("attprojw", "fcprojw") else 0.02
            a = normal_for(seed, i, n, std)
        a = a.reshape(shape)
        if name == "wte" and vocab_rows is not None:
            a[vocab_rows:] = 0.0
        params[name] = a
    return params

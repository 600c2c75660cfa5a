"""Pins of the oracle's seeded initialisation (CPU only): SplitMix64's
published test vectors, Box-Muller statistics, and the GPT-2 init scales."""

import json
import math
import os

import numpy as np

import oracle as O
from oracle.init_rng import normal_for, splitmix64_stream

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vectors():
    with open(os.path.join(GOLDEN, "splitmix64_vectors.json")) as f:
        g = json.load(f)
    for s in g["streams"]:
        n = len(s.get("outputs_hex", s.get("outputs_dec")))
        out = splitmix64_stream(s["seed"], np.arange(n))
        if "outputs_hex" in s:
            assert [format(int(x), "016x") for x in out] == s["outputs_hex"]
        else:
            assert [str(int(x)) for x in out] == s["outputs_dec"]


def test_box_muller_moments():
    z = normal_for(seed=99, tensor_index=3, count=1 << 20, std=1.0).astype(np.float64)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    kurt = ((z - z.mean()) ** 4).mean() / z.var() ** 2
    assert abs(kurt - 3) < 0.05
    # fraction within one sigma ~ 0.6827
    assert abs((np.abs(z) < 1).mean() - 0.682689) < 0.003


def test_box_muller_single_value_closed_form():
    # element 0 of tensor 0, seed 0: counter c = 0, r0 = out(0), r1 = out(1)
    r = splitmix64_stream(0, np.arange(2))
    u1 = ((int(r[0]) >> 11) + 1) * 2.0 ** -53
    u2 = (int(r[1]) >> 11) * 2.0 ** -53
    z = math.sqrt(-2 * math.log(u1)) * math.cos(2 * math.pi * u2)
    assert normal_for(0, 0, 1, 1.0)[0] == np.float32(z)


def test_gpt2_init_scales():
    cfg = O.OracleConfig(vocab_size=512, max_seq_len=64, num_layers=2, num_heads=4, channels=64)
    shapes = O.param_shapes(cfg)
    p = O.gpt2_init_params(shapes, cfg.num_layers, seed=7)
    for name in ("ln1w", "ln2w", "lnfw"):
        assert np.all(p[name] == 1.0)
    for name in ("ln1b", "ln2b", "lnfb", "qkvb", "attprojb", "fcb", "fcprojb"):
        assert np.all(p[name] == 0.0)
    for name, sd in [("wte", 0.02), ("wpe", 0.02), ("qkvw", 0.02), ("fcw", 0.02),
                     ("attprojw", 0.02 / math.sqrt(4)), ("fcprojw", 0.02 / math.sqrt(4))]:
        a = p[name].astype(np.float64)
        assert abs(a.std() - sd) < 0.03 * sd, (name, a.std())
        assert abs(a.mean()) < 5 * sd / math.sqrt(a.size)
    # tensors are independent streams: different tensors, different draws
    assert not np.allclose(p["wte"][:64].reshape(-1)[:100], p["wpe"].reshape(-1)[:100])


def test_padded_rows_are_zero():
    shapes = [("wte", (80, 8))]
    p = O.gpt2_init_params(shapes, 1, seed=3, vocab_rows=70)
    assert np.all(p["wte"][70:] == 0) and np.any(p["wte"][:70] != 0)

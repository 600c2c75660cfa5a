"""Pins of the oracle's FP8 arithmetic (CPU only): the OCP E4M3 / E5M2
rounding against torch's own float8 casts, the grid's closure and encoding
from the format definition, the scaling closed forms, and FP8 linear layers
that reduce exactly to the plain (pinned) ones when their operands already lie
on the grid with unit scale."""

import numpy as np
import pytest
import torch

import oracle as O
from gpt_transformer_lm_amd import synthetic as S

RNG = np.random.Generator(np.random.PCG64(808))
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FMTS = [O.E4M3, O.E5M2]


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


def finite_codes(fmt):
    codes = np.arange(256, dtype=np.int64)
    vals = O.fp8_decode(codes, fmt)
    keep = np.abs(vals) <= fmt.max_finite
    if fmt.name == "e4m3":                     # S.1111.111 is NaN
        keep &= (codes & 0x7F) != 0x7F
    else:                                      # exponent 11111: infinities and NaNs
        keep &= ((codes >> 2) & 31) != 31
    return codes[keep], vals[keep]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_format_constants(fmt):
    codes, vals = finite_codes(fmt)
    assert vals.max() == fmt.max_finite
    assert np.min(vals[vals > 0]) == 2.0 ** (1 - fmt.bias - fmt.man_bits)      # smallest subnormal
    assert len(codes) == (254 if fmt.name == "e4m3" else 248)
    assert O.fp8_decode(0x38 if fmt.name == "e4m3" else 0x3C, fmt) == 1.0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_grid_is_closed_and_encoding_round_trips(fmt):
    codes, vals = finite_codes(fmt)
    assert np.array_equal(O.round_to_fp8(vals, fmt), vals)
    enc = O.fp8_encode(vals, fmt)
    # +0 and -0 both decode to 0; compare on the nonzero codes and the zero
    nz = vals != 0
    assert np.array_equal(enc[nz], codes[nz].astype(np.uint8))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_rounding_matches_torch_float8_casts(fmt):
    x = np.concatenate([RNG.standard_normal(20000) * s for s in (1e-4, 1e-2, 1.0, 30.0)])
    x = x[np.abs(x) < fmt.max_finite * 0.99]
    ours = O.fp8_encode(O.round_to_fp8(x.astype(np.float32), fmt), fmt)
    ref = torch.from_numpy(x.astype(np.float32)).to(TORCH_DT[fmt.name]).view(torch.uint8).numpy()
    z = O.round_to_fp8(x.astype(np.float32), fmt) == 0           # signed zeros: compare values
    assert np.array_equal(ours[~z], ref[~z])
    assert np.all(O.fp8_decode(ref[z], fmt) == 0)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_midpoints_round_to_even(fmt):
    _, vals = finite_codes(fmt)
    v = np.unique(vals[vals >= 0])
    mids = (v[:-1] + v[1:]) / 2
    r = O.round_to_fp8(mids, fmt)
    codes = O.fp8_encode(r, fmt)
    assert np.all(codes[r > 0] % 2 == 0)                          # the even mantissa wins
    assert np.all((r == v[:-1]) | (r == v[1:]))
    ref = torch.from_numpy(mids.astype(np.float32)).to(TORCH_DT[fmt.name]).float().numpy()
    assert np.array_equal(r, ref)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_quantize_scale_closed_forms(fmt):
    x = RNG.standard_normal((17, 33)).astype(np.float32) * 3.7
    q, s = O.quantize(x, fmt)
    amax = np.max(np.abs(x))
    inv, s2 = O.fp8_scales(amax, fmt)
    assert s == s2 and s == np.float32(amax) / np.float32(fmt.max_finite)
    assert np.max(np.abs(q)) == fmt.max_finite                    # the largest element maps to FMAX
    assert np.array_equal(O.quantize(-x, fmt)[0], -q)             # sign symmetric
    # relative error of the dequantised values: half the grid spacing
    deq = q * np.float64(s)
    big = np.abs(x) > amax * 2.0 ** (-fmt.bias + 2)               # normal range
    assert np.max(np.abs(deq[big] - x[big]) / np.abs(x[big])) <= 2.0 ** -(fmt.man_bits + 1) * 1.0001
    qz, sz = O.quantize(np.zeros((3, 4)), fmt)
    assert sz == 1 and np.all(qz == 0)


def test_fp8_linear_reduces_to_linear_on_the_grid():
    """Operands already on the grids with amax = FMAX (unit scales): the FP8
    forward and straight-through backward equal the plain linear layer."""
    _, v4 = finite_codes(O.E4M3)
    _, v5 = finite_codes(O.E5M2)
    v4 = v4[np.abs(v4) <= 8]
    v5 = v5[np.abs(v5) <= 8]
    x = RNG.choice(v4, (12, 16))
    w = RNG.choice(v4, (10, 16))
    dy = RNG.choice(v5, (12, 10))
    x[0, 0], w[0, 0], dy[0, 0] = 448.0, 448.0, 57344.0             # amax = FMAX -> scale 1
    b = RNG.standard_normal(10)
    y, cache = O.fp8_linear_forward(x, w, b)
    assert np.array_equal(y, O.linear_forward(x, w, b))
    dx, dw, db = O.fp8_linear_backward(dy, cache)
    rdx, rdw, rdb = O.linear_backward(dy, x, w)
    assert np.array_equal(dx, rdx) and np.array_equal(dw, rdw) and np.array_equal(db, rdb)


def test_fp8_linear_power_of_two_scales_are_exact():
    """Scaling an on-grid operand by a power of two changes only s."""
    _, v4 = finite_codes(O.E4M3)
    x = RNG.choice(v4[np.abs(v4) <= 4], (8, 32))
    w = RNG.choice(v4[np.abs(v4) <= 4], (6, 32))
    x[0, 0] = w[0, 0] = 448.0
    y1, _ = O.fp8_linear_forward(x, w)
    y2, _ = O.fp8_linear_forward(x * 2.0 ** -20, w * 2.0 ** 7)
    assert np.array_equal(y2, y1 * 2.0 ** -13)


def test_fp8_model_is_close_to_the_plain_model():
    """The FP8 products perturb the loss and gradients by the quantisation
    error only: a few per cent, not a different function."""
    kw = dict(vocab_size=64, max_seq_len=16, num_layers=2, num_heads=4, channels=32)
    c0, c8 = O.OracleConfig(**kw), O.OracleConfig(**kw, fp8=True)
    p = {k: v.astype(np.float64) for k, v in S.random_params(64, 64, 16, 2, 32, 71, perturbed=True).items()}
    tok, tgt = S.uniform_batch(2, 16, 64, seed=72)
    l0, _, _, cache0 = O.gpt2_forward(p, tok, tgt, c0)
    l8, _, _, cache8 = O.gpt2_forward(p, tok, tgt, c8)
    assert l8 != l0 and abs(l8 - l0) / l0 < 1e-2
    g0, g8 = O.gpt2_backward(p, cache0, c0), O.gpt2_backward(p, cache8, c8)
    for k in g0:
        assert rel(g8[k], g0[k]) < 0.15, k


@pytest.mark.parametrize("mistake", ["ties_away_from_zero", "e4m3_bias_8", "no_subnormals"])
def test_planted_rounding_mistakes_are_caught(mistake, monkeypatch):
    """Each slip, planted in the oracle on the CPU, disagrees with torch's casts."""
    import oracle.fp8 as F8
    fmt = O.E4M3
    if mistake == "ties_away_from_zero":
        monkeypatch.setattr(F8.np, "round", lambda a: np.floor(np.asarray(a) + 0.5))
    elif mistake == "e4m3_bias_8":
        fmt = F8.Fp8Format("e4m3", 4, 3, 8, 240.0)
    else:
        orig = F8.round_to_fp8
        monkeypatch.setattr(F8, "round_to_fp8", lambda x, f: np.where(np.abs(orig(x, f)) < 2.0 ** (1 - f.bias), 0.0,
                                                                      orig(x, f)))
    _, v = finite_codes(O.E4M3)
    v = np.unique(v[(v > 0) & (v < 200)])
    x = np.concatenate([(v[:-1] + v[1:]) / 2, RNG.standard_normal(2000) * 0.05]).astype(np.float32)
    ours = F8.round_to_fp8(x, fmt)
    monkeypatch.undo()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert not np.array_equal(ours, ref), mistake

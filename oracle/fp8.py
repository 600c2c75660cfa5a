"""FP8 rounding and FP8 matrix products for the CPU oracle (test
infrastructure; only tests, __graft_entry__.smoke() and bench.py's
cpu_baseline may import the oracle).

The page "NanoGPT (124M) in 90 seconds" (section "How it works", item
"Precision & Hardware") runs the MLP's forward and backward products, the QKV
projection and the head in FP8 and gives no recipe.  The reading here is the
plainest common one:

* formats: the OCP 8-bit floats -- E4M3 (4 exponent bits, bias 7, 3 mantissa
  bits, largest finite 448, no infinities) for activations and weights, E5M2
  (5, bias 15, 2; largest finite 57344) for gradients -- with subnormals, and
  round-to-nearest-even;
* per-tensor scaling from the tensor's own absolute maximum: in float32,
  inv = FMAX / amax and s = amax / FMAX (both 1 when amax = 0); every element
  is mapped to fp8(float32(x * inv)), and a product of two quantised operands
  is multiplied back by s_a * s_b (float32);
* straight-through backward: dX = Q5(dY) Q4(W) and dW = Q5(dY)^T Q4(X), with
  the same quantised W and X as the forward; bias gradients unquantised.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fp8Format:
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    max_finite: float


E4M3 = Fp8Format("e4m3", 4, 3, 7, 448.0)
E5M2 = Fp8Format("e5m2", 5, 2, 15, 57344.0)


def round_to_fp8(x, fmt: Fp8Format):
    """Nearest value of the format's grid, ties to even, subnormals included
    (float64 result).  |x| must not round past the largest finite value."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    emin = 1 - fmt.bias                                 # exponent of the smallest normal
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    ulp = np.exp2(e - fmt.man_bits)                      # spacing of the grid at |x|
    q = np.round(a / ulp) * ulp                          # np.round: half to even
    if np.any(q > fmt.max_finite):
        raise OverflowError(f"{fmt.name}: value beyond the largest finite {fmt.max_finite}")
    return np.copysign(q, x)


def fp8_encode(q, fmt: Fp8Format):
    """Bit pattern (uint8) of values already on the grid (sign | exponent | mantissa)."""
    q = np.asarray(q, dtype=np.float64)
    sign = (np.signbit(q)).astype(np.uint32) << 7
    a = np.abs(q)
    emin = 1 - fmt.bias
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    normal = (a >= 2.0 ** emin)
    efield = np.where(normal, e + fmt.bias, 0).astype(np.int64)
    frac = np.where(normal, a / np.exp2(e) - 1.0, a / 2.0 ** emin)
    mfield = np.round(frac * 2 ** fmt.man_bits).astype(np.int64)
    code = sign | (efield.astype(np.uint32) << fmt.man_bits) | mfield.astype(np.uint32)
    return code.astype(np.uint8)


def fp8_decode(code, fmt: Fp8Format):
    """Value of bit patterns (finite codes only)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    efield = (c >> fmt.man_bits) & ((1 << fmt.exp_bits) - 1)
    mfield = c & ((1 << fmt.man_bits) - 1)
    emin = 1 - fmt.bias
    val = np.where(efield == 0, mfield / 2.0 ** fmt.man_bits * 2.0 ** emin,
                   (1.0 + mfield / 2.0 ** fmt.man_bits) * np.exp2(efield - fmt.bias))
    return sign * val


def fp8_scales(amax, fmt: Fp8Format):
    """(inv, s) in float32: inv = FMAX / amax, s = amax / FMAX; (1, 1) for amax = 0."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(fmt.max_finite) / amax, amax / np.float32(fmt.max_finite)


def quantize(x, fmt: Fp8Format):
    """Per-tensor quantisation: returns (q, s) with q the fp8 grid values of
    float32(x * inv) (float64 array) and s the float32 scale."""
    x32 = np.asarray(x, dtype=np.float32)
    inv, s = fp8_scales(np.max(np.abs(x32)) if x32.size else 0.0, fmt)
    return round_to_fp8(x32 * inv, fmt), s


def fp8_matmul_nt(qa, sa, qb, sb):
    """(qa qb^T) * float32(sa * sb): the product of two quantised operands,
    accumulated exactly here (float64), scaled back."""
    return (np.asarray(qa, np.float64) @ np.asarray(qb, np.float64).T) * np.float64(np.float32(sa * sb))


def fp8_linear_forward(x, w, b=None):
    """y = Q4(x) Q4(w)^T s_x s_w (+ b) for w stored [out, in]; also returns the
    quantised operands for the backward."""
    x2 = x.reshape(-1, x.shape[-1])
    qx, sx = quantize(x2, E4M3)
    qw, sw = quantize(w, E4M3)
    y = fp8_matmul_nt(qx, sx, qw, sw)
    if b is not None:
        y = y + b
    return y.reshape(*x.shape[:-1], w.shape[0]), (qx, sx, qw, sw)


def fp8_linear_backward(dy, cache):
    """Straight-through gradients of fp8_linear_forward:
    dx = Q5(dy) Q4(w) s s,  dW = Q5(dy)^T Q4(x) s s,  db = sum over rows of dy."""
    qx, sx, qw, sw = cache
    dy2 = dy.reshape(-1, dy.shape[-1])
    qd, sd = quantize(dy2, E5M2)
    dx = fp8_matmul_nt(qd, sd, qw.T, sw)                 # [M, K]
    dw = fp8_matmul_nt(qd.T, sd, qx.T, sx)               # [N, K]
    return dx.reshape(*dy.shape[:-1], qw.shape[1]), dw, dy2.sum(axis=0)

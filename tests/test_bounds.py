"""CPU check of the rounding bounds the GPU tests hold the GEMV kernels to
(gpuhelp.error_bound): an fp32 emulation of each kernel's arithmetic, with two
roundings per v_dot2 step (the pessimistic reading of the instruction), stays
within the bound of the exact result on random and on cancelling inputs."""
import numpy as np
import pytest

import oracle
import synth
from gpuhelp import error_bound, half_f64

f32 = np.float32


def _pairs(q):
    """[..., 32] codes -> the v_dot2 steps of a group: per word j the pairs
    (0,4) (1,5) (2,6) (3,7) of elements 8j + i, as index arrays."""
    order = []
    for j in range(4):
        for lo, hi in ((0, 4), (1, 5), (2, 6), (3, 7)):
            order.append((8 * j + lo, 8 * j + hi))
    return order


def _chain(t, x, parity):
    """fp32 chain over the group's pairs of one parity (even: pairs (0,4),(2,6))."""
    acc = np.zeros(t.shape[:-1], f32)
    for a, b in _pairs(None):
        if a % 2 != parity:
            continue
        p = (t[..., a].astype(np.float64) * x[..., a]).astype(f32) + \
            (t[..., b].astype(np.float64) * x[..., b]).astype(f32)     # round, round
        acc = (acc + p.astype(f32)).astype(f32)
    return acc


def emulate(words, scales, x, kind):
    """fp32 emulation of y = W x per kernel kind ("sub" or "exact"), before the
    fp16 rounding.  words [N][K/8], scales fp16 bits [N][G], x fp16 bits [K]."""
    codes = oracle.unpack(words).astype(np.float64)
    N, K = codes.shape
    G = K // 32
    q = codes.reshape(N, G, 32)
    xv = half_f64(x).reshape(1, G, 32)
    s = half_f64(scales).astype(f32)
    if kind == "sub":
        unit = np.where(np.arange(32) % 2 == 0, 2.0 ** -24, 2.0 ** -20)
        def d(qq):
            t = qq * unit
            a, b = _chain(t, xv, 0), _chain(t, xv, 1)
            return (a.astype(np.float64) * 16 + b).astype(f32)
        pd = (d(q).astype(np.float64) - d(np.full_like(q, 7.0))).astype(f32)
        scale = 2.0 ** 20
    else:
        t = q - 7
        pd = (_chain(t, xv, 0).astype(np.float64) + _chain(t, xv, 1)).astype(f32)
        scale = 1.0
    acc = np.zeros(N, f32)
    for g in range(G):
        acc = (pd[:, g].astype(np.float64) * s[:, g] + acc).astype(f32)
    return acc.astype(np.float64) * scale


@pytest.mark.parametrize("kind", ["sub", "exact"])
@pytest.mark.parametrize("case", ["random", "cancelling", "wide_range"])
def test_emulated_kernel_within_bound(kind, case):
    N, K = 64, 1024
    m = synth.Matrix(f"bound/{case}", N, K)
    w, s = m.words(), m.scales()
    x = synth.activations(f"bound/x/{case}", 0, K)
    if case == "cancelling":
        # x alternating in sign with equal magnitudes: sums cancel inside every group
        xv = np.abs(half_f64(x))
        xv[1::2] = -xv[0::2]
        x = synth.to_half_bits(xv)
    elif case == "wide_range":
        xv = half_f64(x) * np.exp2(np.arange(K) % 24 - 12)
        x = synth.to_half_bits(np.clip(xv, -60000, 60000))
    y = emulate(w, s, x, kind)
    y64, _ = oracle.gemv_exact(w, s, x)
    B = error_bound(s, x, kind)[0]
    err = np.abs(y - y64)
    assert np.all(err <= B), (kind, case, float((err / B).max()))
    # the bound is not vacuous: the emulation does round
    assert err.max() > 0


def test_sub_units_are_exact():
    # codes as fp16 subnormals: q * 2^-24 and q * 2^-20 are exact fp16 values, and
    # a product with any finite fp16 x is exact in fp32
    q = np.arange(16, dtype=np.float64)
    for unit in (2.0 ** -24, 2.0 ** -20):
        v = (q * unit).astype(np.float16).astype(np.float64)
        assert np.array_equal(v, q * unit)
    xs = half_f64(np.arange(0, 0x7C00, 97, dtype=np.uint16))
    for unit in (2.0 ** -24, 2.0 ** -20):
        p = np.outer(q * unit, xs)
        assert np.array_equal(p.astype(f32).astype(np.float64), p)

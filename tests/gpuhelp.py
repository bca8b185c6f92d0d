"""Helpers shared by the GPU tests: host<->device transfer of bit patterns and
comparison of GPU outputs with the CPU oracle."""
import numpy as np
import torch

import oracle
import synth


def dev_words(w: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(w, np.uint32).view(np.int32)).cuda()


def dev_half(h: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(h, np.uint16).view(np.int16)).cuda().view(
        torch.float16)


def host_half(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_words(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def half_f64(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


class Report:
    """Largest error found and the tolerance it was held to."""

    def __init__(self):
        self.worst = 0.0

    def note(self, err_over_tol):
        self.worst = max(self.worst, err_over_tol)


def assert_gemv_close(y_gpu_bits, words, scales, X, rows=None, rel=2e-3, report=None,
                      exact=False):
    """Check GPU fp16 outputs against the fp64 oracle.

    y_gpu_bits: [n_rows] or [M][n_rows] fp16 bits of the rows `rows` (all rows if
    None).  Tolerance per input row m: rel * ||x_m||_2 * max_n ||W_n||_2 over the
    checked rows (the benchmark spec's bound; a max over fewer rows is stricter).
    With exact=True the exact (int128) oracle is used as well and at least 99 %
    of outputs must equal the exactly rounded fp16 value, the others within one
    fp16 ulp of it.
    """
    Xs = np.asarray(X, np.uint16)
    X2 = Xs.reshape(-1, Xs.shape[-1])
    y = np.asarray(y_gpu_bits, np.uint16).reshape(X2.shape[0], -1)
    ref = oracle.gemv_f64(words, scales, X2, rows=rows)
    ref = ref.reshape(X2.shape[0], -1)
    wmax = oracle.row_norms(words, scales, rows=rows).max()
    got = half_f64(y)
    for m in range(X2.shape[0]):
        tol = rel * oracle.vec_norm(X2[m]) * wmax
        err = np.abs(got[m] - ref[m])
        # fp16 overflow: beyond the largest finite value plus the tolerance the
        # result must be the infinity of the same sign; near the edge either
        over = np.abs(ref[m]) >= 65520.0 + tol
        edge = ~over & (np.abs(ref[m]) > 65504.0 - tol)
        inf_ok = np.isinf(got[m]) & (np.sign(got[m]) == np.sign(ref[m]))
        assert np.all(inf_ok[over]), f"row m={m}: overflowing outputs are not signed inf"
        err = np.where(over | (edge & inf_ok), 0.0, err)
        bad = np.nonzero(~(err <= tol))[0]
        assert len(bad) == 0, (f"row m={m}: {len(bad)} outputs outside tolerance {tol:.3g}; "
                               f"first n={bad[:5]}, gpu={got[m][bad[:5]]}, ref={ref[m][bad[:5]]}")
        if report is not None and tol > 0:
            report.note(float(err.max() / tol))
    if exact:
        _, y16 = oracle.gemv_exact(words, scales, X2, rows=rows)
        y16 = y16.reshape(X2.shape[0], -1)
        diff = y16 != y
        frac = diff.mean()
        assert frac <= 0.01, f"{frac:.4f} of outputs differ from the exactly rounded fp16"
        ulps = np.abs(y16.view(np.int16).astype(np.int64) - y.view(np.int16).astype(np.int64))
        same_sign = (y16 >> 15) == (y >> 15)
        assert np.all(ulps[diff & same_sign] <= 1), "an output is more than 1 ulp off"
        # sign flips only around zero
        flip = diff & ~same_sign
        assert np.all(np.abs(half_f64(y[flip])) <= 2 ** -14)
    return ref


# ---------------------------------------------------------------------------
# Rounding-error bounds of the GEMV kernels, against the exact result
# ---------------------------------------------------------------------------
#
# u = 2^-24 is the unit roundoff of fp32.  Per 32-weight group g of a row, with
# X_g = sum_{k in g} |x_k| (and its even / odd halves X_e, X_o), a kernel forms
# D_g ~ T_g = sum_{k in g} (q_k - 7) x_k with an error E_g, and the row's output
# as the fp32 sum over groups of s_g * D_g, rounded once to fp16.
#
#  * "fold" (the M = 1 persistent kernel): D_g is the difference of two fp32
#    chains of v_dot2 over t_k x_k with t_k = 1024 + q_k (k even) or 64 + q_k
#    (k odd), the second with every q_k = 7.  Each chain has 8 dot steps per
#    parity; counting two roundings per step, a chain's error is at most
#    16 u times the sum of its terms' magnitudes (|t_k| <= 1039 or 79), the add
#    of the two chains one more rounding, and the subtraction one rounding of
#    at most u |T_g| <= 8 u X_g (doubled to cover the second-order terms):
#        E_g <= 2 * 17 u (1039 X_e + 79 X_o) + 2 u * 8 X_g
#  * "sub" (the M = 1 persistent kernel): the codes enter as fp16 subnormals
#    (q * 2^-24, or q * 2^-20 at odd positions), products exact; two chains of
#    8 v_dot2 steps (two roundings each) over terms of at most 15 |x|, joined by
#    one fma, minus the same function of codes 7 (at most 7 |x| per term), then
#    one rounding of the difference (at most u |T_g| <= 8 u X_g, doubled):
#        E_g <= 17 u * 15 X_g + 17 u * 7 X_g + 2 u * 8 X_g = 390 u X_g
#  * "exact" (every other kernel: q - 7 formed exactly in fp16, one chain of
#    products of at most 8 |x|, or one MFMA over the group):
#        E_g <= 34 u * 8 X_g
# Accumulation over the G groups and a cross-lane reduction of at most 6 steps:
# at most G + 8 further roundings of partial sums bounded by
# sum_g |s_g| (8 X_g + E_g).  Then
#     |y_fp32 - y| <= B = sum_g |s_g| E_g + (G + 8) u sum_g |s_g| (8 X_g + E_g)
# and the fp16 output is within B + ulp16(|y| + B) / 2 of the exact y.

_U = 2.0 ** -24


def group_abs_sums(X):
    """[M][G] sums of |x| per group, and of the even and odd positions."""
    Xa = np.asarray(X, np.uint16)
    x = half_f64(Xa).reshape(Xa.shape[0] if Xa.ndim > 1 else 1, -1)
    a = np.abs(x).reshape(x.shape[0], -1, 32)
    return a.sum(axis=2), a[:, :, 0::2].sum(axis=2), a[:, :, 1::2].sum(axis=2)


def error_bound(scales, X, kind):
    """[M][N] bound B on |y_fp32 - y| for fp16 scales bits [N][G] and X [M][K]."""
    xg, xe, xo = group_abs_sums(X)
    if kind == "fold":
        E = 34 * _U * (1039 * xe + 79 * xo) + 2 * _U * 8 * xg
    elif kind == "sub":
        E = 390 * _U * xg
    elif kind == "exact":
        E = 34 * _U * 8 * xg
    else:
        raise ValueError(kind)
    G = xg.shape[1]
    C = E + (G + 8) * _U * (8 * xg + E)
    s = np.abs(half_f64(np.asarray(scales, np.uint16))).reshape(-1, G)
    return (C @ s.T) * (1 + 2.0 ** -20)


def ulp16(v):
    """Unit in the last place of fp16 at magnitude v (2^-24 below the normal range)."""
    v = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(v)) - 10)


def assert_within_rounding_bound(y_gpu_bits, y_exact64, y_exact16, scales, X, kind,
                                 exact_frac=0.99, what=""):
    """Every output within the kernel's rounding bound of the exact result, and
    at least `exact_frac` of them equal to the exactly rounded fp16 value (the
    others within one fp16 ulp).  Returns (worst error / bound, fraction equal)."""
    y = np.asarray(y_gpu_bits, np.uint16).reshape(np.asarray(y_exact64).shape)
    B = error_bound(scales, X, kind).reshape(y.shape)
    got = half_f64(y)
    ref = np.asarray(y_exact64, np.float64)
    lim = B + 0.5 * ulp16(np.abs(ref) + B)
    err = np.abs(got - ref)
    bad = np.nonzero(~(err <= lim))
    assert len(bad[0]) == 0, (f"{what}: {len(bad[0])} outputs beyond the rounding bound; first "
                              f"{[(int(i), got[i], ref[i], lim[i]) for i in zip(*bad)][:3]}")
    # exactly rounded: the same fp16 value (+0 and -0 count as one)
    ex16 = np.asarray(y_exact16, np.uint16).reshape(y.shape)
    same = (ex16 == y) | (((ex16 | y) & 0x7FFF) == 0)
    frac = float(same.mean())
    assert frac >= exact_frac, f"{what}: only {frac:.4f} of outputs exactly rounded"
    return float((err / lim).max()), frac


def weights_f64(words, scales):
    codes = oracle.unpack(words).astype(np.float64)
    return (codes - 7) * np.repeat(half_f64(scales), 32, axis=1)


def folded_bound(w, s, h_bits, gamma_bits, eps, y_ref, kind="exact"):
    """Per-output bound on |y_folded (fp32, before its rounding) - y_unfolded| for
    the GEMV of a folded RMSNorm (input fp16(h * gamma), outputs scaled by
    1 / rms(h)); kind: the GEMV's dequantisation (error_bound)."""
    K = h_bits.size
    h, g = half_f64(h_bits), half_f64(gamma_bits)
    r = 1.0 / np.sqrt(np.mean(h * h) + eps)
    a = h * g                                           # exact in fp64
    v_bits = synth.to_half_bits(a)                      # the folded GEMV's input
    W = np.abs(weights_f64(w, s))
    # the two fp16 roundings of each input term: fp16(a) * r against fp16(r a)
    t_in = W @ (2.0 ** -10 * r * np.abs(a) + 2.0 ** -25 * (1.0 + r))
    # the folded GEMV's fp32 error on its own input, times r
    t_gemv = r * error_bound(s, v_bits, kind)[0]
    # the fp32 norm scalar: sum of K squares, the mean, the root, the reciprocal, the product
    t_r = (K + 8) * _U * r * (W @ np.abs(half_f64(v_bits)))
    return t_in + t_gemv + t_r

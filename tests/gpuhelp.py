"""Helpers shared by the GPU tests: host<->device transfer of bit patterns and
comparison of GPU outputs with the CPU oracle."""
import numpy as np
import torch

import oracle


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

"""q4f16_1 CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct C implementation (``q4_oracle.c``) of what the
decode GEMV path computes, loaded through ctypes. Only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may use
it; the HIP library never does, and the two share no code.

Definitions (Zero TVM documentation, section "Q4F16 quantization format"):
eight 4-bit codes per uint32 word, nibble ``i`` = ``(word >> 4i) & 0xF``, one
fp16 scale per 32 weights, weight = ``(code - 7) * scale``; y = W x.
The feed-forward glue between the gate/up and down projections ("Decode loop"):
fp16(silu(gate) * up); and the steps around the GEMVs: the token's embedding row,
RMSNorm, the residual add with RMSNorm, the argmax over the logits.

Parity pins for every function here live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liborc.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = C.CDLL(_LIB_PATH)
            p = C.c_void_p
            i64 = C.c_int64
            lib.orc_half_to_f64.argtypes = [C.c_uint16]
            lib.orc_half_to_f64.restype = C.c_double
            lib.orc_bf16_to_f64.argtypes = [C.c_uint16]
            lib.orc_bf16_to_f64.restype = C.c_double
            lib.orc_set_threads.argtypes = [C.c_int]
            lib.orc_set_threads.restype = None
            lib.orc_get_threads.argtypes = []
            lib.orc_get_threads.restype = C.c_int
            lib.orc_f64_to_half.argtypes = [C.c_double]
            lib.orc_f64_to_half.restype = C.c_uint16
            lib.orc_unpack.argtypes = [p, p, i64, i64]
            lib.orc_unpack.restype = None
            lib.orc_pack.argtypes = [p, p, i64, i64]
            lib.orc_pack.restype = None
            lib.orc_roundtrip_mismatches.argtypes = [C.c_uint64, C.c_uint64]
            lib.orc_roundtrip_mismatches.restype = i64
            lib.orc_gemv_f64.argtypes = [p, p, p, i64, i64, i64, p, i64, p]
            lib.orc_gemv_f64.restype = C.c_int
            lib.orc_gemv_exact.argtypes = [p, p, p, i64, i64, i64, p, i64, p, p]
            lib.orc_gemv_exact.restype = C.c_int
            lib.orc_row_norms.argtypes = [p, p, i64, i64, p, i64, p]
            lib.orc_row_norms.restype = C.c_int
            lib.orc_silu_mul.argtypes = [p, p, i64, i64]
            lib.orc_silu_mul.restype = None
            lib.orc_embed_rows.argtypes = [p, p, i64, i64, p, i64, p]
            lib.orc_embed_rows.restype = None
            lib.orc_rmsnorm.argtypes = [p, p, C.c_double, i64, i64, p]
            lib.orc_rmsnorm.restype = None
            lib.orc_add_rmsnorm.argtypes = [p, p, p, C.c_double, i64, i64, p, p]
            lib.orc_add_rmsnorm.restype = None
            lib.orc_argmax.argtypes = [p, i64, i64, p]
            lib.orc_argmax.restype = None
            lib.orc_gemv_format.argtypes = [C.c_int, p, p, p, p, i64, i64, p, i64, p, p]
            lib.orc_gemv_format.restype = C.c_int
            lib.orc_vec_norm.argtypes = [p, i64]
            lib.orc_vec_norm.restype = C.c_double
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return C.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def half_to_f64(h: int) -> float:
    return _load().orc_half_to_f64(int(h))


def bf16_to_f64(h: int) -> float:
    return _load().orc_bf16_to_f64(int(h))


def set_threads(n: int) -> None:
    """Host threads of the GEMV row loops (1: the plain single-threaded oracle)."""
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


def f64_to_half(v: float) -> int:
    return _load().orc_f64_to_half(float(v))


def unpack(words: np.ndarray, K: int | None = None) -> np.ndarray:
    """uint32 [N][K/8] -> uint8 codes [N][K]."""
    w = _c(words, np.uint32)
    w2 = w.reshape(w.shape[0], -1) if w.ndim > 1 else w.reshape(1, -1)
    N, K8 = w2.shape
    out = np.empty((N, 8 * K8), np.uint8)
    _load().orc_unpack(_ptr(w2), _ptr(out), N, 8 * K8)
    return out if w.ndim > 1 else out.reshape(-1)


def pack(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [N][K] (K % 8 == 0) -> uint32 [N][K/8]."""
    c = _c(codes, np.uint8)
    c2 = c.reshape(c.shape[0], -1) if c.ndim > 1 else c.reshape(1, -1)
    N, K = c2.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    out = np.empty((N, K // 8), np.uint32)
    _load().orc_pack(_ptr(c2), _ptr(out), N, K)
    return out if c.ndim > 1 else out.reshape(-1)


def roundtrip_mismatches(w0: int, w1: int) -> int:
    return int(_load().orc_roundtrip_mismatches(w0, w1))


def _rows_arg(rows, N):
    if rows is None:
        return None, N
    r = _c(rows, np.int64).reshape(-1)
    return r, len(r)


def gemv_f64(words, scales, X, rows=None) -> np.ndarray:
    """fp64 y = W x (X may be [K] or [M][K]); returns [n_rows] or [M][n_rows]."""
    w = _c(words, np.uint32)
    s = _c(scales, np.uint16)
    x = _c(X, np.uint16)
    N = w.shape[0]
    K = 8 * w.shape[1]
    xs = x.reshape(-1, K)
    M = xs.shape[0]
    r, nr = _rows_arg(rows, N)
    Y = np.empty((M, nr), np.float64)
    rc = _load().orc_gemv_f64(_ptr(w), _ptr(s), _ptr(xs), M, N, K, _ptr(r), nr, _ptr(Y))
    if rc:
        raise ValueError(f"orc_gemv_f64 failed ({rc})")
    return Y[0] if x.ndim == 1 else Y


def gemv_exact(words, scales, X, rows=None):
    """Exact y = W x rounded once: returns (fp64 values, fp16 bit patterns)."""
    w = _c(words, np.uint32)
    s = _c(scales, np.uint16)
    x = _c(X, np.uint16)
    N = w.shape[0]
    K = 8 * w.shape[1]
    xs = x.reshape(-1, K)
    M = xs.shape[0]
    r, nr = _rows_arg(rows, N)
    Y64 = np.empty((M, nr), np.float64)
    Y16 = np.empty((M, nr), np.uint16)
    rc = _load().orc_gemv_exact(_ptr(w), _ptr(s), _ptr(xs), M, N, K, _ptr(r), nr,
                                _ptr(Y64), _ptr(Y16))
    if rc:
        raise ValueError(f"orc_gemv_exact failed ({rc})")
    if x.ndim == 1:
        return Y64[0], Y16[0]
    return Y64, Y16


def row_norms(words, scales, rows=None) -> np.ndarray:
    w = _c(words, np.uint32)
    s = _c(scales, np.uint16)
    N = w.shape[0]
    K = 8 * w.shape[1]
    r, nr = _rows_arg(rows, N)
    out = np.empty(nr, np.float64)
    if _load().orc_row_norms(_ptr(w), _ptr(s), N, K, _ptr(r), nr, _ptr(out)):
        raise ValueError("orc_row_norms failed")
    return out


def silu_mul(gu, H: int | None = None) -> np.ndarray:
    """fp16 bits [M][2H] (gate | up) -> fp16 bits [M][H] of fp16(silu(gate) * up),
    in fp64 (Zero TVM documentation, "Decode loop": the FFN's SiLU and multiply)."""
    g = _c(gu, np.uint16)
    g2 = g.reshape(-1, g.shape[-1])
    if g2.shape[1] % 2:
        raise ValueError("last axis must be 2H")
    Hh = g2.shape[1] // 2
    out = np.empty((g2.shape[0], Hh), np.uint16)
    _load().orc_silu_mul(_ptr(g2), _ptr(out), g2.shape[0], Hh)
    return out.reshape(g.shape[:-1] + (Hh,))


def embed_rows(words, scales, tokens) -> np.ndarray:
    """fp16 bits [M][K]: the dequantised rows tokens[m] of a q4f16_1 table."""
    w = _c(words, np.uint32)
    sc = _c(scales, np.uint16)
    t = _c(tokens, np.int32).reshape(-1)
    N, K = w.shape[0], 8 * w.shape[1]
    out = np.empty((len(t), K), np.uint16)
    _load().orc_embed_rows(_ptr(w), _ptr(sc), N, K, _ptr(t), len(t), _ptr(out))
    return out


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """fp16 bits of RMSNorm(x) * gamma per row (fp64; eps as the fp32 the kernels take)."""
    xs = _c(x, np.uint16)
    x2 = xs.reshape(-1, xs.shape[-1])
    g = _c(gamma, np.uint16).reshape(-1)
    out = np.empty_like(x2)
    _load().orc_rmsnorm(_ptr(x2), _ptr(g), float(np.float32(eps)), x2.shape[0], x2.shape[1],
                        _ptr(out))
    return out.reshape(xs.shape)


def add_rmsnorm(delta, res_in, gamma, eps: float):
    """(res_out, out) fp16 bits: res_out = fp16(res_in + delta), out = RMSNorm(res_out)."""
    d = _c(delta, np.uint16)
    r = _c(res_in, np.uint16)
    d2 = d.reshape(-1, d.shape[-1])
    r2 = r.reshape(d2.shape)
    g = _c(gamma, np.uint16).reshape(-1)
    res_out = np.empty_like(d2)
    out = np.empty_like(d2)
    _load().orc_add_rmsnorm(_ptr(d2), _ptr(r2), _ptr(g), float(np.float32(eps)), d2.shape[0],
                            d2.shape[1], _ptr(res_out), _ptr(out))
    return res_out.reshape(d.shape), out.reshape(d.shape)


def argmax(x) -> np.ndarray:
    """int32 [M]: largest fp16 value per row, ties to the lowest index, NaN skipped."""
    xs = _c(x, np.uint16)
    x2 = xs.reshape(-1, xs.shape[-1])
    out = np.empty(x2.shape[0], np.int32)
    _load().orc_argmax(_ptr(x2), x2.shape[0], x2.shape[1], _ptr(out))
    return out


# af4g64: bf16 scales and biases (the pages' MLX affine format);
# af4g64_f16: the same with fp16 scales and biases (an extra variant)
FORMATS = {"q3f16_1": 1, "q4f32_1": 2, "af4g64": 3, "af4g64_f16": 4}


def gemv_format(fmt: str, words, scales, biases, x, K: int, rows=None):
    """fp64 y = W x for a format variant (see orc_gemv_format) and the row norms:
    returns (y [n_rows], norms [n_rows]).  x: fp16 bits, or fp32 for q4f32_1."""
    f = FORMATS[fmt]
    w = _c(words, np.uint32)
    sc = _c(scales, np.float32 if f == 2 else np.uint16)
    bi = _c(biases, np.uint16) if biases is not None else None
    xs = _c(x, np.float32 if f == 2 else np.uint16).reshape(-1)
    N = w.shape[0]
    r, nr = _rows_arg(rows, N)
    y = np.empty(nr, np.float64)
    nrm = np.empty(nr, np.float64)
    rc = _load().orc_gemv_format(f, _ptr(w), _ptr(sc), _ptr(bi), _ptr(xs), N, K, _ptr(r), nr,
                                 _ptr(y), _ptr(nrm))
    if rc:
        raise ValueError(f"orc_gemv_format failed ({rc})")
    return y, nrm


def vec_norm(x) -> float:
    xs = _c(x, np.uint16).reshape(-1)
    return float(_load().orc_vec_norm(_ptr(xs), len(xs)))


def tolerance(x_row, row_norms_max: float, rel: float = 2e-3) -> float:
    """Allowed max |y_gpu - y_ref| for one input row: rel * ||x||_2 * max_n ||W_n||_2."""
    return rel * vec_norm(x_row) * row_norms_max

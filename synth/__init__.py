"""Seeded synthetic inputs for the q4f16_1 decode-GEMV workloads.

This module is shared by the CPU oracle and the HIP path. It only draws random
numbers and shapes them into arrays; it holds none of the arithmetic of the
method (no packing, no dequantisation, no dot products).

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; constants as in Vigna's public-domain
splitmix64.c). It is counter-based: draw ``i`` of a stream with key ``k`` is
``mix64(k + (i + 1) * GAMMA)``, so any slice of a stream (for example the rows
of a large matrix that a test samples) is produced without generating the rest.

Streams are named by a text label (e.g. ``"phi3/L07/down/words"``) and a
seed; the label is hashed with 64-bit FNV-1a and mixed with the seed.

Value recipes (the workloads of the q4f16_1 decode path, with group size 32):
  * packed weights: uniformly random uint32 words -- identical in distribution
    to codes uniform in [0, 15] packed eight per word;
  * codes: uint8 uniform in [0, 15] (four bits of a draw each);
  * "uniform" scales: fp16 of ``lo + (hi - lo) * u``;
  * "halfnormal" scales: fp16 of ``|sigma * z| + floor`` with z ~ N(0, 1);
  * activations: fp16 of z ~ N(0, 1).
Normals use the Box--Muller transform on 53-bit uniforms in (0, 1]; the fp64
to fp16 rounding is numpy's (round to nearest even).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 22  # draws per vectorised block (bounds temporary memory)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(label: str, seed: int = 0) -> int:
    """64-bit key of the stream named ``label`` under ``seed``."""
    h = _FNV_OFFSET
    for b in label.encode("utf-8"):
        h = ((h ^ b) * _FNV_PRIME) & _MASK64
    return _mix64_int(h ^ _mix64_int((seed * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019) & _MASK64))


def draws(label: str, seed: int, start: int, count: int) -> np.ndarray:
    """uint64 draws ``start .. start+count-1`` of the stream (label, seed)."""
    key = np.uint64(stream_key(label, seed))
    out = np.empty(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for c0 in range(0, count, _CHUNK):
            c1 = min(count, c0 + _CHUNK)
            idx = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
            out[c0:c1] = _mix64(key + idx * GAMMA)
    return out


def _draw_range_words(label: str, seed: int, w0: int, w1: int) -> np.ndarray:
    """uint32 words w0..w1-1 of a stream; word i is half (i % 2) of draw i // 2,
    low half first (little-endian view of the draws)."""
    d0, d1 = w0 // 2, (w1 + 1) // 2
    d = draws(label, seed, d0, d1 - d0)
    return d.view(np.uint32)[w0 - 2 * d0: w1 - 2 * d0].copy()


def words(label: str, seed: int, count: int) -> np.ndarray:
    """``count`` uniformly random uint32 words."""
    return _draw_range_words(label, seed, 0, count)


def word_rows(label: str, seed: int, n_rows: int, row_words: int, rows) -> np.ndarray:
    """Rows ``rows`` of the [n_rows][row_words] word matrix ``words(label, seed,
    n_rows*row_words)``, generated without the other rows."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), row_words), dtype=np.uint32)
    for i, r in enumerate(rows):
        if not 0 <= r < n_rows:
            raise IndexError(r)
        out[i] = _draw_range_words(label, seed, int(r) * row_words, (int(r) + 1) * row_words)
    return out


def codes(label: str, seed: int, count: int) -> np.ndarray:
    """``count`` uint8 codes uniform in [0, 15]: bits [4c, 4c+3] of draw i give
    code 16*i + c."""
    nd = (count + 15) // 16
    d = draws(label, seed, 0, nd)
    out = np.empty((nd, 16), dtype=np.uint8)
    for c in range(16):
        out[:, c] = ((d >> np.uint64(4 * c)) & np.uint64(15)).astype(np.uint8)
    return out.reshape(-1)[:count].copy()


def unit_open(label: str, seed: int, start: int, count: int) -> np.ndarray:
    """fp64 uniforms in (0, 1]: ((draw >> 11) + 1) * 2**-53."""
    d = draws(label, seed, start, count)
    return ((d >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal(label: str, seed: int, start: int, count: int) -> np.ndarray:
    """fp64 N(0, 1) values start..start+count-1 (Box--Muller, cosine branch;
    value i uses draws 2i and 2i+1)."""
    u = unit_open(label, seed, 2 * start, 2 * count).reshape(count, 2)
    return np.sqrt(-2.0 * np.log(u[:, 0])) * np.cos(2.0 * np.pi * u[:, 1])


def to_half_bits(v) -> np.ndarray:
    """fp64 -> fp16 (round to nearest even), returned as uint16 bit patterns."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def half_bits_to_f64(h) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Tensors of one q4f16_1 matrix / activation
# --------------------------------------------------------------------------

def scales_uniform(label: str, seed: int, count: int, lo: float, hi: float) -> np.ndarray:
    return to_half_bits(lo + (hi - lo) * unit_open(label, seed, 0, count))


def scales_halfnormal(label: str, seed: int, start: int, count: int,
                      sigma: float = 0.01, floor: float = 1e-3) -> np.ndarray:
    return to_half_bits(np.abs(sigma * normal(label, seed, start, count)) + floor)


def activations(label: str, seed: int, count: int) -> np.ndarray:
    return to_half_bits(normal(label, seed, 0, count))


class Matrix:
    """Seeded q4f16_1 weight of logical shape [N][K] given as raw words
    ([N][K/8] uint32) and scales ([N][K/32] fp16 bits), halfnormal scales."""

    def __init__(self, label: str, N: int, K: int, seed: int = 0,
                 sigma: float = 0.01, floor: float = 1e-3):
        if K % 32:
            raise ValueError("K must be a multiple of 32")
        self.label, self.N, self.K, self.seed = label, N, K, seed
        self.sigma, self.floor = sigma, floor

    @property
    def row_words(self) -> int:
        return self.K // 8

    @property
    def row_groups(self) -> int:
        return self.K // 32

    def words(self) -> np.ndarray:
        return words(self.label + "/words", self.seed, self.N * self.row_words).reshape(
            self.N, self.row_words)

    def scales(self) -> np.ndarray:
        return scales_halfnormal(self.label + "/scales", self.seed, 0,
                                 self.N * self.row_groups, self.sigma, self.floor).reshape(
            self.N, self.row_groups)

    def word_rows(self, rows) -> np.ndarray:
        return word_rows(self.label + "/words", self.seed, self.N, self.row_words, rows)

    def scale_rows(self, rows) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64)
        g = self.row_groups
        return np.stack([scales_halfnormal(self.label + "/scales", self.seed, int(r) * g, g,
                                           self.sigma, self.floor) for r in rows]) \
            if len(rows) else np.empty((0, g), np.uint16)

    @property
    def weight_bytes(self) -> int:
        """Packed words plus scales: 18 bytes per 32 weights."""
        return self.N * self.K // 2 + self.N * self.K // 16


# --------------------------------------------------------------------------
# The workloads
# --------------------------------------------------------------------------

# Phi-3-mini constants (Zero TVM docs, "Phi-3 model constants").
PHI3 = dict(D=3072, LAYERS=32, FFN=8192, VOCAB=32064)
# 2B-class decoder shape used for the batched (M = 8) sweep.
TWO_B = dict(D=2048, LAYERS=28, FFN=6144, VOCAB=151936, QKV=4096)


def phi3_layer_shapes():
    """(role, N, K) of the four projections of one Phi-3-mini layer: fused QKV
    without grouped-query attention (3*D), O, fused gate+up (2*FFN), down."""
    D, F = PHI3["D"], PHI3["FFN"]
    return [("qkv", 3 * D, D), ("o", D, D), ("gate_up", 2 * F, D), ("down", D, F)]


def twob_layer_shapes():
    D, F, Q = TWO_B["D"], TWO_B["FFN"], TWO_B["QKV"]
    return [("qkv", Q, D), ("o", D, D), ("gate_up", 2 * F, D), ("down", D, F)]


def sweep_shapes(model: str):
    """Ordered (label, N, K) list of every GEMV of one decode step."""
    if model == "phi3":
        layers, shapes, head = PHI3["LAYERS"], phi3_layer_shapes(), (PHI3["VOCAB"], PHI3["D"])
    elif model == "2b":
        layers, shapes, head = TWO_B["LAYERS"], twob_layer_shapes(), (TWO_B["VOCAB"], TWO_B["D"])
    else:
        raise ValueError(model)
    out = []
    for L in range(layers):
        for role, N, K in shapes:
            out.append((f"{model}/L{L:02d}/{role}", N, K))
    out.append((f"{model}/lm_head", head[0], head[1]))
    return out


def small_config(seed: int = 0):
    """The 256 x 512 correctness GEMV: codes uniform in [0, 15] (uint8 [N][K]),
    scales uniform in [0.005, 0.02] (fp16 bits [N][K/32]), x ~ N(0, 1) (fp16
    bits [K])."""
    N, K = 256, 512
    c = codes("small/codes", seed, N * K).reshape(N, K)
    s = scales_uniform("small/scales", seed, N * K // 32, 0.005, 0.02).reshape(N, K // 32)
    x = activations("small/x", seed, K)
    return c, s, x


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """Bytes a q4f16_1 GEMV must move at least once: packed words, fp16 scales,
    fp16 input rows and fp16 output rows."""
    return N * K // 2 + N * K // 16 + 2 * M * K + 2 * M * N

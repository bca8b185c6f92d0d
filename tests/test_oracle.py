"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Every check compares the oracle with something it does not share code with:
numpy's IEEE binary16 conversions, numpy's float64 matrix product over an
independently decoded weight, hand-worked fixtures (tests/golden), closed forms
and invariants of the definition, and figures the pages print.
"""
import ctypes as C
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT, load_golden_cases, load_page_figures


# ----------------------------------------------------------------- binary16

def test_half_decode_exhaustive_vs_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    lib = oracle._load()
    got = np.array([lib.orc_half_to_f64(int(v)) for v in h])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_half_encode_vs_numpy():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        # every fp16 value and every midpoint between neighbours (ties)
        np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64),
        (np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64) +
         np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2,
        [65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
         5.960464477539063e-08, -0.0, 0.0],
    ])
    vals = np.concatenate([vals, -vals])
    ref = vals.astype(np.float16).view(np.uint16)
    lib = oracle._load()
    got = np.array([lib.orc_f64_to_half(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(vals[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


# -------------------------------------------------------------------- codec

def test_codec_closed_forms():
    # nibble i of a word is (word >> 4i) & 0xF (Zero TVM, "Q4F16 quantization format")
    w = np.array([[0x76543210, 0xFEDCBA98, 0x77777777]], np.uint32)
    c = oracle.unpack(w)
    assert c.tolist() == [list(range(16)) + [7] * 8]
    assert np.array_equal(oracle.pack(c), w)


def test_codec_vs_little_endian_byte_view():
    # Independent decoding: a little-endian uint32 is four bytes, low byte first;
    # byte b of word j holds elements 8j+2b (low nibble) and 8j+2b+1 (high nibble).
    rng = np.random.default_rng(2)
    w = rng.integers(0, 2 ** 32, size=(37, 24), dtype=np.uint64).astype(np.uint32)
    b = w.astype("<u4").view(np.uint8).reshape(37, 24 * 4)
    ref = np.empty((37, 24 * 8), np.uint8)
    ref[:, 0::2] = b & 0xF
    ref[:, 1::2] = b >> 4
    assert np.array_equal(oracle.unpack(w), ref)
    assert np.array_equal(oracle.pack(ref), w)


def test_codec_masks_high_bits_of_codes():
    c = np.array([[0x1F, 0xF0, 0x27, 3, 4, 5, 6, 0xFF]], np.uint8)
    assert oracle.pack(c)[0, 0] == oracle.pack(c & 0xF)[0, 0]


def test_codec_roundtrip_random_and_words():
    c = synth.codes("t/codes", 3, 64 * 96).reshape(64, 96)
    assert np.array_equal(oracle.unpack(oracle.pack(c)), c)
    # every word with a single non-zero nibble, and a 2^22 sub-range
    single = [v << (4 * i) for i in range(8) for v in range(16)]
    w = np.array(single, np.uint32).reshape(-1, 1)
    assert np.array_equal(oracle.pack(oracle.unpack(w)), w)
    assert oracle.roundtrip_mismatches(0xDEAD0000 - (1 << 21), 0xDEAD0000 + (1 << 21)) == 0


@pytest.mark.slow
@pytest.mark.skipif(os.environ.get("Q4_SLOW") != "1", reason="about a minute; set Q4_SLOW=1")
def test_codec_roundtrip_all_words():
    assert oracle.roundtrip_mismatches(0, 1 << 32) == 0


# --------------------------------------------------------------------- GEMV

def _dequant_numpy(words, scales):
    """Independent fp64 dequantisation via the byte view and numpy float16."""
    N, K8 = words.shape
    b = words.astype("<u4").view(np.uint8).reshape(N, K8 * 4)
    q = np.empty((N, K8 * 8), np.int64)
    q[:, 0::2] = b & 0xF
    q[:, 1::2] = b >> 4
    s = scales.view(np.float16).astype(np.float64)
    return (q - 7).astype(np.float64) * np.repeat(s, 32, axis=1)


def _rand_case(seed, N, K, M=1, neg_scales=False):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    s = np.abs(rng.standard_normal((N, K // 32)) * 0.01) + 1e-3
    if neg_scales:
        s *= rng.choice([-1.0, 1.0], size=s.shape)
    s = s.astype(np.float16).view(np.uint16)
    x = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    return w, s, x


@pytest.mark.parametrize("N,K,M", [(1, 32, 1), (7, 64, 1), (33, 160, 3), (64, 256, 8), (5, 1024, 2)])
def test_f64_and_exact_vs_numpy_matmul(N, K, M):
    w, s, x = _rand_case(N * 1000 + K + M, N, K, M, neg_scales=True)
    ref = x.view(np.float16).astype(np.float64) @ _dequant_numpy(w, s).T   # [M][N]
    y64 = oracle.gemv_f64(w, s, x)
    ye, y16 = oracle.gemv_exact(w, s, x)
    scale = np.abs(x.view(np.float16).astype(np.float64)) @ np.abs(_dequant_numpy(w, s)).T
    assert np.all(np.abs(y64 - ref) <= 1e-13 * scale + 1e-300)
    assert np.all(np.abs(ye - ref) <= 1e-13 * scale + 1e-300)
    # the exact result rounded once equals numpy's rounding of the exact fp64 value
    # whenever that fp64 value is itself exact (always true here: |terms| < 2^53 ulps)
    assert np.array_equal(y16, ye.astype(np.float16).view(np.uint16))


def test_small_config_exact_vs_f64_all_rows():
    c, s, x = synth.small_config(0)
    w = oracle.pack(c)
    y64 = oracle.gemv_f64(w, s, x)
    ye, y16 = oracle.gemv_exact(w, s, x)
    assert np.max(np.abs(y64 - ye)) <= 1e-12 * np.max(np.abs(ye))
    ref = x.view(np.float16).astype(np.float64) @ _dequant_numpy(w, s).T
    assert np.allclose(ye, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", load_golden_cases("hand_worked_gemv.txt"), ids=lambda c: c["name"])
def test_hand_worked_fixtures(case):
    y64 = oracle.gemv_f64(case["words"], case["scales"], case["x"])
    ye, y16 = oracle.gemv_exact(case["words"], case["scales"], case["x"])
    assert np.array_equal(y16, case["y16"]), (y16, case["y16"])
    # the fixtures' decimal values are the exact sums before rounding except for
    # the tie cases, whose fp16 results are listed; compare the fp16 decoding
    assert np.array_equal(y16.view(np.float16).astype(np.float64), case["y"])
    assert np.array_equal(np.array([oracle.f64_to_half(v) for v in y64], np.uint16), case["y16"])


def test_closed_form_all_sevens_is_zero():
    N, K = 9, 96
    w = np.full((N, K // 8), 0x77777777, np.uint32)
    _, s, x = _rand_case(5, N, K, 1, neg_scales=True)
    assert np.all(oracle.gemv_f64(w, s, x[0]) == 0.0)
    assert np.all(oracle.gemv_exact(w, s, x[0])[1] == 0)


def test_closed_form_unit_scale_ones_gives_code_sum():
    c = synth.codes("t/cs", 4, 12 * 320).reshape(12, 320)
    w = oracle.pack(c)
    s = np.full((12, 10), 0x3C00, np.uint16)          # 1.0
    x = np.full(320, 0x3C00, np.uint16)               # ones
    expect = (c.astype(np.int64) - 7).sum(axis=1)
    assert np.array_equal(oracle.gemv_f64(w, s, x), expect.astype(np.float64))
    assert np.array_equal(oracle.gemv_exact(w, s, x)[1],
                          expect.astype(np.float16).view(np.uint16))


def test_one_hot_input_selects_one_weight():
    # non-square (N=5, K=96): pins nibble, word and group indexing and orientation
    N, K = 5, 96
    c = synth.codes("t/oh", 6, N * K).reshape(N, K)
    w = oracle.pack(c)
    s = synth.scales_uniform("t/ohs", 6, N * K // 32, 0.005, 0.02).reshape(N, K // 32)
    sv = s.view(np.float16).astype(np.float64)
    for k in range(K):
        x = np.zeros(K, np.uint16)
        x[k] = 0x3C00
        expect = (c[:, k].astype(np.float64) - 7) * sv[:, k // 32]
        assert np.array_equal(oracle.gemv_f64(w, s, x), expect), k
        assert np.array_equal(oracle.gemv_exact(w, s, x)[1],
                              expect.astype(np.float16).view(np.uint16)), k


def test_scale_group_isolation():
    N, K = 4, 128
    c = synth.codes("t/g", 7, N * K).reshape(N, K)
    w = oracle.pack(c)
    x = synth.activations("t/gx", 7, K)
    xv = x.view(np.float16).astype(np.float64)
    for g in range(K // 32):
        s = np.zeros((N, K // 32), np.uint16)
        s[:, g] = 0x3C00
        expect = ((c[:, 32 * g:32 * g + 32].astype(np.float64) - 7) * xv[32 * g:32 * g + 32]).sum(1)
        assert np.allclose(oracle.gemv_exact(w, s, x)[0], expect, rtol=0, atol=1e-12)


def test_invariants_scaling_and_row_permutation():
    w, s, x = _rand_case(8, 40, 256, 1, neg_scales=True)
    y = oracle.gemv_exact(w, s, x[0])[0]
    s2 = (s.view(np.float16).astype(np.float64) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.gemv_exact(w, s2, x[0])[0], 2 * y)
    perm = np.random.default_rng(9).permutation(40)
    assert np.array_equal(oracle.gemv_exact(w[perm], s[perm], x[0])[0], y[perm])
    rows = np.array([39, 0, 17, 17])
    assert np.array_equal(oracle.gemv_f64(w, s, x[0], rows=rows), oracle.gemv_f64(w, s, x[0])[rows])


def test_exact_rejects_inf_and_nan():
    w, s, x = _rand_case(10, 2, 32)
    x = x.copy()
    x[0, 3] = 0x7C00
    with pytest.raises(ValueError):
        oracle.gemv_exact(w, s, x[0])
    assert np.isnan(oracle.gemv_f64(w, s, x[0])).any() or \
        np.isinf(oracle.gemv_f64(w, s, x[0])).any()


def test_tolerance_helpers():
    w, s, x = _rand_case(11, 6, 64)
    ref = _dequant_numpy(w, s)
    assert np.allclose(oracle.row_norms(w, s), np.linalg.norm(ref, axis=1), rtol=1e-14)
    assert np.isclose(oracle.vec_norm(x[0]),
                      np.linalg.norm(x[0].view(np.float16).astype(np.float64)), rtol=1e-14)
    # fp16 output rounding alone stays far inside the tolerance (Cauchy-Schwarz)
    ye, y16 = oracle.gemv_exact(w, s, x[0])
    err = np.abs(y16.view(np.float16).astype(np.float64) - ye).max()
    assert err <= 2e-3 * oracle.vec_norm(x[0]) * oracle.row_norms(w, s).max()


# ------------------------------------------------------- figures of the pages

def test_page_figures_bytes_and_shapes():
    f = load_page_figures()
    assert synth.PHI3["D"] == f["phi3_D"][0][0]
    assert synth.PHI3["LAYERS"] == f["phi3_layers"][0][0]
    assert synth.PHI3["FFN"] == f["phi3_ffn"][0][0]
    assert synth.PHI3["VOCAB"] == f["phi3_vocab"][0][0]
    assert synth.TWO_B["D"] == f["twob_hidden"][0][0]
    assert synth.TWO_B["FFN"] == f["twob_intermediate"][0][0]
    m = synth.Matrix("x", 1, 32)
    assert m.weight_bytes == f["q4f16_1_bytes_per_32"][0][0]
    total = sum(synth.Matrix(l, N, K).weight_bytes for l, N, K in synth.sweep_shapes("phi3"))
    assert total == 2_093_838_336
    assert round(total / 1e9, 2) == f["phi3_token_weight_gb"][0][0]
    for K, iters in f["lane_iters"]:
        assert K / 8 / 64 == iters     # 64 lanes, one uint32 (8 weights) per iteration


def test_sweep_descriptor_lists():
    phi = synth.sweep_shapes("phi3")
    assert len(phi) == 129 and phi[-1][1:] == (32064, 3072)
    assert phi[0][1:] == (9216, 3072) and phi[3][1:] == (3072, 8192)
    two = synth.sweep_shapes("2b")
    assert len(two) == 113 and two[-1][1:] == (151936, 2048)
    w2 = sum(synth.Matrix(l, N, K).weight_bytes for l, N, K in two)
    assert w2 == 967_753_728


# ------------------------------------- planted mistakes must break the pins

MUTATIONS = {
    "sign": ("acc += ((double)(q - 7) * s[k / 32]) * x[k];",
             "acc += ((double)(7 - q) * s[k / 32]) * x[k];"),
    "scale_index": ("acc += ((double)(q - 7) * s[k / 32]) * x[k];",
                    "acc += ((double)(q - 7) * s[k / 8 % (K / 32)]) * x[k];"),
    "dropped_term": ("for (int64_t k = 0; k < K; ++k) {\n          int q = (int)code_at(words, K, n, k);\n          acc +=",
                     "for (int64_t k = 0; k < K - 1; ++k) {\n          int q = (int)code_at(words, K, n, k);\n          acc +="),
    "nibble_order": ("return (w >> (4 * (k % 8))) & 0xFu;", "return (w >> (4 * (7 - k % 8))) & 0xFu;"),
    "transposed": ("uint32_t w = words[n * (K / 8) + k / 8];", "uint32_t w = words[(k / 8) * (K / 8) + n % (K / 8)];"),
    "zero_point_8": ("acc += ((double)(q - 7) * s[k / 32]) * x[k];",
                     "acc += ((double)(q - 8) * s[k / 32]) * x[k];"),
}


def _build_mutant(tmp, name):
    src = open(os.path.join(ROOT, "oracle", "q4_oracle.c")).read()
    a, b = MUTATIONS[name]
    assert a in src, name
    path = os.path.join(tmp, f"m_{name}.c")
    open(path, "w").write(src.replace(a, b))
    so = os.path.join(tmp, f"m_{name}.so")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", so, path, "-lm"])
    lib = C.CDLL(so)
    lib.orc_gemv_f64.argtypes = [C.c_void_p] * 3 + [C.c_int64] * 3 + [C.c_void_p, C.c_int64, C.c_void_p]
    return lib


def _mutant_gemv(lib, w, s, x):
    w = np.ascontiguousarray(w)
    s = np.ascontiguousarray(s)
    x = np.ascontiguousarray(x)
    N, K = w.shape[0], w.shape[1] * 8
    y = np.empty(N)
    lib.orc_gemv_f64(w.ctypes.data, s.ctypes.data, x.ctypes.data, 1, N, K, None, N, y.ctypes.data)
    return y


def _pins_pass(gemv):
    """A subset of the pins above, run against a given gemv(w, s, x) -> fp64 y."""
    ok = True
    for case in load_golden_cases("hand_worked_gemv.txt"):
        y = gemv(case["words"], case["scales"], case["x"])
        ok &= np.array_equal(y.astype(np.float16).view(np.uint16), case["y16"])
    N, K = 5, 96
    c = synth.codes("t/oh", 6, N * K).reshape(N, K)
    w = oracle.pack(c)
    s = synth.scales_uniform("t/ohs", 6, N * K // 32, 0.005, 0.02).reshape(N, K // 32)
    sv = s.view(np.float16).astype(np.float64)
    for k in range(K):
        x = np.zeros(K, np.uint16)
        x[k] = 0x3C00
        ok &= np.array_equal(gemv(w, s, x), (c[:, k].astype(np.float64) - 7) * sv[:, k // 32])
    return bool(ok)


def test_pins_pass_on_the_oracle():
    assert _pins_pass(lambda w, s, x: oracle.gemv_f64(w, s, x))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, name)
        assert not _pins_pass(lambda w, s, x: _mutant_gemv(lib, w, s, x)), name


# ---------------------------------------------------------------- MLP glue pins

def _np_silu_mul(g16, u16):
    """numpy's exp and float16 cast (independent of the oracle's own rounding)."""
    g = g16.view(np.float16).astype(np.float64)
    u = u16.view(np.float16).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        sg = g / (1.0 + np.exp(-g))
    sg = np.where(np.isposinf(g), g, np.where(np.isneginf(g), -0.0, sg))
    with np.errstate(over="ignore", invalid="ignore"):
        return (sg * u).astype(np.float16).view(np.uint16)


def test_silu_mul_every_gate_value_vs_numpy():
    """All 65 536 fp16 gate values against numpy, with up = 1 and with a few other
    up values (any dropped term, wrong sign or swapped half shows here)."""
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for u_val in (1.0, -2.0, 0.5, 3.5, -0.0078125):
        u = np.full(65536, np.float16(u_val)).view(np.uint16)
        gu = np.concatenate([g, u]).reshape(1, -1)
        got = oracle.silu_mul(gu)[0]
        ref = _np_silu_mul(g, u)
        nan = np.isnan(ref.view(np.float16))
        assert np.array_equal(np.isnan(got.view(np.float16)), nan), u_val
        assert np.array_equal(got[~nan], ref[~nan]), u_val


def test_silu_mul_closed_forms_and_layout():
    # silu(0) = 0; large positive gate: silu(g) = g; large negative: -> -0
    H = 4
    gate = np.array([0.0, 20.0, -30.0, 1.0], np.float16)
    up = np.array([5.0, 0.5, 2.0, 2.0], np.float16)
    gu = np.concatenate([gate, up]).view(np.uint16).reshape(1, 2 * H)
    out = oracle.silu_mul(gu)[0].view(np.float16).astype(np.float64)
    assert out[0] == 0.0
    assert out[1] == 10.0
    assert out[2] == 0.0 and np.signbit(out[2])
    # silu(1) * 2 = 2 / (1 + 1/e) = 1.46211715726...: the nearest fp16 (step 2^-10)
    assert out[3] == np.float16(2.0 / (1.0 + np.exp(-1.0)))
    assert abs(out[3] - 1.4621171572600098) <= 2.0 ** -11
    # rows are independent and the halves are [gate | up] per row
    rng = np.random.default_rng(3)
    M, H = 3, 40
    gu = rng.standard_normal((M, 2 * H)).astype(np.float16).view(np.uint16)
    out = oracle.silu_mul(gu)
    for m in range(M):
        assert np.array_equal(out[m], _np_silu_mul(gu[m, :H], gu[m, H:]))
    swapped = np.concatenate([gu[:, H:], gu[:, :H]], axis=1)
    assert not np.array_equal(oracle.silu_mul(swapped), out)


SILU_MUTATIONS = {
    "sign_of_exponent": ("sg = g / (1.0 + exp(-g));", "sg = g / (1.0 + exp(g));"),
    "halves_swapped": ("double u = orc_half_to_f64(GU[m * 2 * H + H + i]);",
                       "double u = orc_half_to_f64(GU[m * 2 * H + i]);"),
    "sigmoid_only": ("OUT[m * H + i] = orc_f64_to_half(sg * u);",
                     "OUT[m * H + i] = orc_f64_to_half(sg / g * u);"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("name", sorted(SILU_MUTATIONS))
def test_silu_pins_catch_planted_mistake(name):
    src = open(os.path.join(ROOT, "oracle", "q4_oracle.c")).read()
    a, b = SILU_MUTATIONS[name]
    assert a in src, name
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "m.c")
        open(path, "w").write(src.replace(a, b))
        so = os.path.join(tmp, "m.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", so,
                               path, "-lm"])
        lib = C.CDLL(so)
        lib.orc_silu_mul.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64]
        g = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
        u = np.full(len(g), np.float16(-2.0)).view(np.uint16)
        gu = np.ascontiguousarray(np.concatenate([g, u]))
        out = np.empty(len(g), np.uint16)
        lib.orc_silu_mul(gu.ctypes.data, out.ctypes.data, 1, len(g))
        ref = _np_silu_mul(g, u)
        ok = ~np.isnan(ref.view(np.float16))
        assert not np.array_equal(out[ok], ref[ok]), name


# ------------------------------------------- embedding, norms and argmax pins

def test_embed_rows_vs_numpy_decode():
    """Rows picked by token id, dequantised as (code - 7) * scale and rounded by
    numpy's float16 cast; out-of-range ids give NaN rows."""
    N, K = 50, 96
    c = synth.codes("t/emb", 1, N * K).reshape(N, K)
    w = oracle.pack(c)
    s = synth.scales_uniform("t/embs", 1, N * K // 32, 0.005, 0.02).reshape(N, K // 32)
    tok = np.array([0, 7, 49, 7, -1, 50], np.int32)
    out = oracle.embed_rows(w, s, tok)
    sv = s.view(np.float16).astype(np.float64)
    for m, t in enumerate(tok):
        if 0 <= t < N:
            ref = ((c[t].astype(np.float64) - 7) * np.repeat(sv[t], 32)).astype(np.float16)
            assert np.array_equal(out[m], ref.view(np.uint16))
        else:
            assert np.all(np.isnan(out[m].view(np.float16)))
    # large scales: products beyond fp16's 11 bits round (to nearest even)
    s2 = np.full((N, K // 32), np.float16(1000.0 + 1.0 / 4)).view(np.uint16)
    out2 = oracle.embed_rows(w, s2, np.array([3], np.int32))[0]
    ref2 = ((c[3].astype(np.float64) - 7) * 1000.25).astype(np.float16).view(np.uint16)
    assert np.array_equal(out2, ref2)


def _np_rmsnorm(x16, g16, eps):
    x = x16.view(np.float16).astype(np.float64)
    g = g16.view(np.float16).astype(np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + float(np.float32(eps)))
    return (x * r * g).astype(np.float16).view(np.uint16)


def test_rmsnorm_vs_numpy_and_closed_forms():
    rng = np.random.default_rng(5)
    M, K = 4, 3072
    x = (rng.standard_normal((M, K)) * 3).astype(np.float16).view(np.uint16)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float16).view(np.uint16)
    for eps in (1e-5, 1e-6, 0.5):
        assert np.array_equal(oracle.rmsnorm(x, g, eps), _np_rmsnorm(x, g, eps))
    # a constant row c with gamma 1: every output is c / sqrt(c^2 + eps)
    c = np.full((1, 256), np.float16(2.0)).view(np.uint16)
    one = np.full(256, np.float16(1.0)).view(np.uint16)
    out = oracle.rmsnorm(c, one, 1e-5)[0].view(np.float16).astype(np.float64)
    assert np.all(out == np.float16(2.0 / np.sqrt(4.0 + float(np.float32(1e-5)))))
    # one-hot row: x_k = a at one k -> a / sqrt(a^2 / K + eps) there, 0 elsewhere
    oh = np.zeros((1, 64), np.float16)
    oh[0, 5] = 3.0
    out = oracle.rmsnorm(oh.view(np.uint16), np.full(64, np.float16(1.0)).view(np.uint16), 0.0)
    out = out[0].view(np.float16).astype(np.float64)
    assert out[5] == np.float16(8.0) and not out[:5].any() and not out[6:].any()


def test_add_rmsnorm_vs_numpy():
    rng = np.random.default_rng(6)
    M, K = 3, 1024
    a = (rng.standard_normal((M, K)) * 50).astype(np.float16).view(np.uint16)
    b = (rng.standard_normal((M, K)) * 0.01).astype(np.float16).view(np.uint16)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float16).view(np.uint16)
    res, out = oracle.add_rmsnorm(b, a, g, 1e-5)
    ref_res = (a.view(np.float16).astype(np.float64) +
               b.view(np.float16).astype(np.float64)).astype(np.float16).view(np.uint16)
    assert np.array_equal(res, ref_res)
    assert np.array_equal(out, _np_rmsnorm(ref_res, g, 1e-5))
    # fp16 overflow of the sum gives inf, as fp16 rounding does
    big = np.full((1, 32), np.float16(60000.0)).view(np.uint16)
    res2, _ = oracle.add_rmsnorm(big, big, np.full(32, np.float16(1.0)).view(np.uint16), 1e-5)
    assert np.all(np.isposinf(res2.view(np.float16)))


def test_argmax_vs_numpy_ties_and_nan():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 32064)).astype(np.float16)
    x[1, [100, 2000, 30000]] = np.float16(60000.0)      # ties: lowest index
    x[2, :] = np.float16(-np.inf)
    x[2, 777] = np.float16(-65504.0)
    x[3, 10] = np.float16(np.nan)
    x[3, 11] = np.float16(30000.0)
    out = oracle.argmax(x.view(np.uint16))
    assert list(out[:4]) == [int(np.argmax(x[0])), 100, 777, 11]
    assert out[4] == int(np.nanargmax(x[4].astype(np.float64)))
    allnan = np.full((1, 8), np.float16(np.nan)).view(np.uint16)
    assert oracle.argmax(allnan)[0] == 0


STEP_MUTATIONS = {
    "embed_zero_point": ("double w = (double)((int)code_at(words, K, t, k) - 7) *",
                         "double w = (double)((int)code_at(words, K, t, k) - 8) *"),
    "rms_mean_not_sum": ("double r = 1.0 / sqrt(ss / (double)K + eps);",
                         "double r = 1.0 / sqrt(ss + eps);"),
    "argmax_last_tie": ("if (best < 0 || v > bv) {", "if (best < 0 || v >= bv) {"),
    "add_drops_delta": ("RES_OUT[i] = orc_f64_to_half(orc_half_to_f64(RES_IN[i]) + orc_half_to_f64(DELTA[i]));",
                        "RES_OUT[i] = orc_f64_to_half(orc_half_to_f64(RES_IN[i]));"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("name", sorted(STEP_MUTATIONS))
def test_step_pins_catch_planted_mistake(name, monkeypatch):
    """Each planted mistake makes one of the pins above fail."""
    src = open(os.path.join(ROOT, "oracle", "q4_oracle.c")).read()
    a, b = STEP_MUTATIONS[name]
    assert a in src, name
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "m.c")
        open(path, "w").write(src.replace(a, b))
        so = os.path.join(tmp, "m.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", so,
                               path, "-lm"])
        real = oracle._load()
        mutant = C.CDLL(so)
        for fn in ("orc_embed_rows", "orc_rmsnorm", "orc_add_rmsnorm", "orc_argmax",
                   "orc_half_to_f64", "orc_f64_to_half", "orc_unpack", "orc_pack"):
            f = getattr(mutant, fn)
            f.argtypes = getattr(real, fn).argtypes
            f.restype = getattr(real, fn).restype
        monkeypatch.setattr(oracle, "_lib", mutant)
        failed = 0
        for pin in (test_embed_rows_vs_numpy_decode, test_rmsnorm_vs_numpy_and_closed_forms,
                    test_add_rmsnorm_vs_numpy, test_argmax_vs_numpy_ties_and_nan):
            try:
                pin()
            except AssertionError:
                failed += 1
        assert failed, name


# ------------------------------------------------------------ format variant pins

def _pack_q3(codes):
    """Independent packer: 32 3-bit codes per group -> three little-endian words
    holding bits [3i, 3i + 3) of one 96-bit value (Python integers)."""
    N, K = codes.shape
    out = np.zeros((N, K // 32 * 3), np.uint32)
    for n in range(N):
        for g in range(K // 32):
            v = 0
            for i in range(32):
                v |= int(codes[n, 32 * g + i]) << (3 * i)
            for j in range(3):
                out[n, 3 * g + j] = (v >> (32 * j)) & 0xFFFFFFFF
    return out


def _format_case(fmt, N=6, K=128, seed=3):
    rng = np.random.default_rng(seed)
    if fmt == "q3f16_1":
        c = rng.integers(0, 8, (N, K)).astype(np.uint8)
        w = _pack_q3(c)
        s16 = (rng.standard_normal((N, K // 32)) * 0.02).astype(np.float16)
        W = (c.astype(np.float64) - 3) * np.repeat(s16.astype(np.float64), 32, axis=1)
        return w, s16.view(np.uint16), None, W
    c = rng.integers(0, 16, (N, K)).astype(np.uint8)
    w = oracle.pack(c)
    if fmt == "q4f32_1":
        s32 = (rng.standard_normal((N, K // 32)) * 0.02).astype(np.float32)
        W = (c.astype(np.float64) - 7) * np.repeat(s32.astype(np.float64), 32, axis=1)
        return w, s32, None, W
    if fmt == "af4g64":
        # bf16 scales and biases: the upper halves of fp32 values, decoded through
        # numpy's float32 view of (bits << 16)
        sb = ((rng.standard_normal((N, K // 64)) * 0.02).astype(np.float32).view(np.uint32)
              >> 16).astype(np.uint16)
        bb = ((rng.standard_normal((N, K // 64)) * 0.1).astype(np.float32).view(np.uint32)
              >> 16).astype(np.uint16)
        sv, bv = _np_bf16(sb), _np_bf16(bb)
        W = (c.astype(np.float64) * np.repeat(sv, 64, axis=1) + np.repeat(bv, 64, axis=1))
        return w, sb, bb, W
    s16 = (rng.standard_normal((N, K // 64)) * 0.02).astype(np.float16)
    b16 = (rng.standard_normal((N, K // 64)) * 0.1).astype(np.float16)
    W = (c.astype(np.float64) * np.repeat(s16.astype(np.float64), 64, axis=1) +
         np.repeat(b16.astype(np.float64), 64, axis=1))
    return w, s16.view(np.uint16), b16.view(np.uint16), W


def _np_bf16(h):
    """bf16 bit patterns -> float64 through numpy's float32 (bits << 16)."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_decode_every_pattern():
    # every bf16 bit pattern against numpy's float32 view of the same bits << 16
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _np_bf16(h)
    got = np.array([oracle.bf16_to_f64(int(v)) for v in h])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))   # -0
    # closed forms: 1.0 = 0x3F80, -2.0 = 0xC000, smallest subnormal 2^-133
    assert oracle.bf16_to_f64(0x3F80) == 1.0 and oracle.bf16_to_f64(0xC000) == -2.0
    assert oracle.bf16_to_f64(0x0001) == 2.0 ** -133


@pytest.mark.parametrize("fmt", ["q3f16_1", "q4f32_1", "af4g64", "af4g64_f16"])
def test_format_gemv_vs_numpy(fmt):
    N, K = 6, 128
    w, s, b, W = _format_case(fmt, N, K)
    rng = np.random.default_rng(9)
    if fmt == "q4f32_1":
        x = rng.standard_normal(K).astype(np.float32)
        xf = x.astype(np.float64)
    else:
        x = rng.standard_normal(K).astype(np.float16).view(np.uint16)
        xf = x.view(np.float16).astype(np.float64)
    y, norms = oracle.gemv_format(fmt, w, s, b, x, K)
    assert np.allclose(y, W @ xf, rtol=1e-12, atol=1e-12)
    assert np.allclose(norms, np.sqrt((W * W).sum(axis=1)), rtol=1e-12)
    # one-hot x picks column k of W exactly
    for k in (0, 31, 32, 63, 64, 127):
        oh = np.zeros(K, np.float32) if fmt == "q4f32_1" else np.zeros(K, np.uint16)
        oh[k] = 1.0 if fmt == "q4f32_1" else 0x3C00
        yk, _ = oracle.gemv_format(fmt, w, s, b, oh, K)
        assert np.array_equal(yk, W[:, k]), (fmt, k)


def test_format_closed_forms():
    K = 64
    # q3f16_1: every code 3 -> zero weights; codes 7 with scale 1 -> weight 4
    c = np.full((2, K), 3, np.uint8)
    c[1] = 7
    s = np.full((2, K // 32), np.float16(1.0)).view(np.uint16)
    x = np.full(K, np.float16(1.0)).view(np.uint16)
    y, _ = oracle.gemv_format("q3f16_1", _pack_q3(c), s, None, x, K)
    assert list(y) == [0.0, 4.0 * K]
    # affine: codes 0, bias b -> b * sum(x); codes 15, scale s, bias 0 -> 15 s sum(x)
    w = oracle.pack(np.zeros((1, K), np.uint8))
    sc = np.full((1, 1), np.float16(0.5)).view(np.uint16)
    bi = np.full((1, 1), np.float16(0.25)).view(np.uint16)
    y, _ = oracle.gemv_format("af4g64_f16", w, sc, bi, x, K)
    assert y[0] == 0.25 * K
    # bf16 0.25 = 0x3E80, 0.5 = 0x3F00 (the same values, other bit patterns)
    y, _ = oracle.gemv_format("af4g64", w, np.full((1, 1), 0x3F00, np.uint16),
                              np.full((1, 1), 0x3E80, np.uint16), x, K)
    assert y[0] == 0.25 * K
    w15 = oracle.pack(np.full((1, K), 15, np.uint8))
    y, _ = oracle.gemv_format("af4g64", w15, np.full((1, 1), 0x3F00, np.uint16),
                              np.zeros((1, 1), np.uint16), x, K)
    assert y[0] == 15 * 0.5 * K


FORMAT_MUTATIONS = {
    "q3_zero_point": ("return ((double)q - 3.0) * s;", "return ((double)q - 4.0) * s;"),
    "q3_bit_order": ("const int64_t bit = 3 * i + b;", "const int64_t bit = 3 * i + (2 - b);"),
    "q4f32_zero_point": ("return ((double)q - 7.0) * (double)s;", "return ((double)q - 8.0) * (double)s;"),
    "affine_group_32": ("const uint16_t sh = ((const uint16_t*)scales)[n * (K / 64) + k / 64];",
                        "const uint16_t sh = ((const uint16_t*)scales)[n * (K / 64) + k / 32 % (K / 64)];"),
    "affine_no_bias": ("return s * (double)q + b;", "return s * (double)q;"),
    # the pages' affine format has bf16 scales and biases: reading them as fp16
    "affine_bf16_read_as_fp16": ("const double s = format == 3 ? orc_bf16_to_f64(sh) : orc_half_to_f64(sh);",
                                 "const double s = orc_half_to_f64(sh);"),
    "affine_bf16_bias_as_fp16": ("const double b = format == 3 ? orc_bf16_to_f64(bh) : orc_half_to_f64(bh);",
                                 "const double b = orc_half_to_f64(bh);"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("name", sorted(FORMAT_MUTATIONS))
def test_format_pins_catch_planted_mistake(name, monkeypatch):
    src = open(os.path.join(ROOT, "oracle", "q4_oracle.c")).read()
    a, b = FORMAT_MUTATIONS[name]
    assert a in src, name
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "m.c")
        open(path, "w").write(src.replace(a, b))
        so = os.path.join(tmp, "m.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", so,
                               path, "-lm"])
        real = oracle._load()
        mutant = C.CDLL(so)
        for fn in ("orc_gemv_format", "orc_pack", "orc_unpack", "orc_half_to_f64",
                   "orc_bf16_to_f64"):
            f = getattr(mutant, fn)
            f.argtypes = getattr(real, fn).argtypes
            f.restype = getattr(real, fn).restype
        monkeypatch.setattr(oracle, "_lib", mutant)
        failed = 0
        for fmt in ("q3f16_1", "q4f32_1", "af4g64", "af4g64_f16"):
            try:
                test_format_gemv_vs_numpy(fmt)
            except AssertionError:
                failed += 1
        try:
            test_format_closed_forms()
        except AssertionError:
            failed += 1
        assert failed, name


def test_thread_count_does_not_change_results():
    # the row loops on several threads compute every row by the same steps
    m = synth.Matrix("t/threads", 300, 1024)
    w, sc = m.words(), m.scales()
    X = synth.activations("t/threads/x", 0, 3 * 1024).reshape(3, 1024)
    rows = np.array([299, 0, 17, 150])
    old = oracle.get_threads()
    try:
        oracle.set_threads(1)
        a = oracle.gemv_f64(w, sc, X), oracle.gemv_exact(w, sc, X), oracle.row_norms(w, sc)
        ar = oracle.gemv_f64(w, sc, X, rows=rows)
        oracle.set_threads(7)
        b = oracle.gemv_f64(w, sc, X), oracle.gemv_exact(w, sc, X), oracle.row_norms(w, sc)
        br = oracle.gemv_f64(w, sc, X, rows=rows)
    finally:
        oracle.set_threads(old)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert np.array_equal(a[1][0], b[1][0]) and np.array_equal(a[1][1], b[1][1])
    assert np.array_equal(ar, br) and np.array_equal(ar, a[0][:, rows])

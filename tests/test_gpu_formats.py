"""The format variants (q3f16_1, q4f32_1, MLX affine 4-bit group 64) through
q4_gemv_format against the oracle's plain decode of the same words, at small
ragged shapes and at the Phi-3 projection shapes."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import dev_half, dev_words, half_f64, host_half

pytestmark = pytest.mark.gpu

FMTS = {"q3f16_1": q4.FMT_Q3F16_1, "q4f32_1": q4.FMT_Q4F32_1, "af4g64": q4.FMT_AF4_G64,
        "af4g64_f16": q4.FMT_AF4_G64_F16}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def make(fmt, N, K, tag):
    """Seeded words (uniform codes), scales, biases and x in the format's layout."""
    lab = f"fmt/{fmt}/{tag}/{N}x{K}"
    if fmt == "q3f16_1":
        words = synth.words(lab + "/w", 0, N * K // 32 * 3).reshape(N, K // 32 * 3)
        scales = synth.scales_halfnormal(lab + "/s", 0, 0, N * K // 32, 0.01, 1e-3).reshape(N, -1)
        biases = None
    elif fmt == "q4f32_1":
        words = synth.words(lab + "/w", 0, N * K // 8).reshape(N, K // 8)
        scales = (np.abs(synth.normal(lab + "/s", 0, 0, N * K // 32)) * 0.01 + 1e-3).astype(
            np.float32).reshape(N, -1)
        biases = None
    elif fmt == "af4g64":
        # bf16 scales |N(0, 0.01)| + 1e-3 and biases 0.05 N(0, 1), as the pages'
        # MLX affine checkpoints store them
        words = synth.words(lab + "/w", 0, N * K // 8).reshape(N, K // 8)
        scales = synth.to_bf16_bits(np.abs(0.01 * synth.normal(lab + "/s", 0, 0, N * K // 64))
                                    + 1e-3).reshape(N, -1)
        biases = synth.to_bf16_bits(0.05 * synth.normal(lab + "/b", 0, 0, N * K // 64)).reshape(N, -1)
    else:
        words = synth.words(lab + "/w", 0, N * K // 8).reshape(N, K // 8)
        scales = synth.scales_halfnormal(lab + "/s", 0, 0, N * K // 64, 0.01, 1e-3).reshape(N, -1)
        biases = synth.to_half_bits(0.05 * synth.normal(lab + "/b", 0, 0, N * K // 64)).reshape(N, -1)
    if fmt == "q4f32_1":
        x = synth.normal(lab + "/x", 0, 0, K).astype(np.float32)
    else:
        x = synth.activations(lab + "/x", 0, K)
    return words, scales, biases, x


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.float32:
        return torch.from_numpy(a).cuda()
    if a.dtype == np.uint32:
        return dev_words(a)
    return dev_half(a)


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("N,K", [(33, 128), (1000, 64 * 3), (9216, 3072), (3072, 8192)])
def test_format_gemv_matches_oracle(fmt, N, K):
    words, scales, biases, x = make(fmt, N, K, "par")
    y = q4.q4_gemv_format(FMTS[fmt], to_dev(words), to_dev(scales), to_dev(x), K,
                          biases=to_dev(biases))
    torch.cuda.synchronize()
    rows = np.arange(N) if N <= 4096 else np.unique(np.linspace(0, N - 1, 2048).astype(np.int64))
    ref, norms = oracle.gemv_format(fmt, words, scales, biases, x, K, rows=rows)
    if fmt == "q4f32_1":
        got = y.cpu().numpy().astype(np.float64)[rows]
        xn = float(np.linalg.norm(x.astype(np.float64)))
        tol = 1e-5 * xn * norms.max()
    else:
        got = half_f64(host_half(y))[rows]
        xn = oracle.vec_norm(x)
        tol = 2e-3 * xn * norms.max()
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert err.max() <= tol, (err.max(), tol)


@pytest.mark.parametrize("load", [0, q4.FMT_LOAD_STAGED, q4.FMT_LOAD_DIRECT])
@pytest.mark.parametrize("N,K", [(257, 128 * 37), (64, 32768), (5, 128), (700, 128 * 20),
                                 (1000, 192), (3000, 3072)])
def test_q3_shapes_both_loads(N, K, load):
    """q3f16_1 through either way of loading the words: several trips per row,
    lanes left idle in the last trip, group counts not a multiple of 4, a row
    count that leaves most of the first wave's rows past the matrix, the largest
    K; both ways give the same bits."""
    words, scales, _, x = make("q3f16_1", N, K, "load")
    args = (to_dev(words), to_dev(scales), to_dev(x), K)
    y = q4.q4_gemv_format(q4.FMT_Q3F16_1 | load, *args)
    other = q4.FMT_LOAD_DIRECT if load == q4.FMT_LOAD_STAGED else q4.FMT_LOAD_STAGED
    y2 = q4.q4_gemv_format(q4.FMT_Q3F16_1 | other, *args)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    rows = np.arange(N) if N <= 4096 else np.unique(np.linspace(0, N - 1, 2048).astype(np.int64))
    ref, norms = oracle.gemv_format("q3f16_1", words, scales, None, x, K, rows=rows)
    got = half_f64(host_half(y))[rows]
    assert np.abs(got - ref).max() <= 2e-3 * oracle.vec_norm(x) * norms.max()


def test_q3_large_takes_the_stage_by_default():
    """Enough rows that every team has eight trips (K = 32768, four trips a row):
    the default choice matches the forced ways and the oracle on sampled rows."""
    N, K = 8300, 32768
    words, scales, _, x = make("q3f16_1", N, K, "big")
    args = (to_dev(words), to_dev(scales), to_dev(x), K)
    ys = [q4.q4_gemv_format(q4.FMT_Q3F16_1 | load, *args)
          for load in (0, q4.FMT_LOAD_STAGED, q4.FMT_LOAD_DIRECT)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))
    rows = np.unique(np.linspace(0, N - 1, 1024).astype(np.int64))
    ref, norms = oracle.gemv_format("q3f16_1", words, scales, None, x, K, rows=rows)
    got = half_f64(host_half(ys[0]))[rows]
    assert np.abs(got - ref).max() <= 2e-3 * oracle.vec_norm(x) * norms.max()


def test_format_load_bits_rejected_off_q3():
    x = torch.zeros(64, dtype=torch.float16, device="cuda")
    w = torch.zeros(4, 8, dtype=torch.int32, device="cuda")
    s = torch.zeros(4, 2, dtype=torch.float16, device="cuda")
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_format(q4.FMT_AF4_G64 | q4.FMT_LOAD_STAGED, w, s, x, 64, biases=s)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_format(q4.FMT_Q3F16_1 | q4.FMT_LOAD_STAGED | q4.FMT_LOAD_DIRECT,
                          w[:, :6], s, x, 64)


@pytest.mark.parametrize("load", [0, q4.FMT_LOAD_STAGED, q4.FMT_LOAD_DIRECT])
def test_q3_words_4_byte_aligned(load):
    """Words 4-byte but not 16-byte aligned (both ways of loading need no
    more): the same results."""
    N, K = 300, 1024
    words, scales, _, x = make("q3f16_1", N, K, "mis")
    flat = torch.zeros(N * (K // 32) * 3 + 4, dtype=torch.int32, device="cuda")
    view = flat[1:1 + words.size]
    view.copy_(to_dev(words).view(-1).view(torch.int32))
    assert view.data_ptr() % 16 != 0
    y = q4.q4_gemv_format(q4.FMT_Q3F16_1 | load, view.view(N, -1), to_dev(scales), to_dev(x), K)
    y2 = q4.q4_gemv_format(q4.FMT_Q3F16_1 | load, to_dev(words), to_dev(scales), to_dev(x), K)
    torch.cuda.synchronize()
    ref, norms = oracle.gemv_format("q3f16_1", words, scales, None, x, K, rows=np.arange(N))
    tol = 2e-3 * oracle.vec_norm(x) * norms.max()
    for out in (y, y2):
        got = half_f64(host_half(out))
        assert np.abs(got - ref).max() <= tol


@pytest.mark.parametrize("fmt", ["af4g64", "af4g64_f16"])
@pytest.mark.parametrize("N,K", [(300, 2560), (77, 11264), (5, 64)])
def test_affine_groups_per_lane(fmt, N, K):
    """The affine format on the q4f16_1 GEMV at row lengths of 5 and 6 groups per
    lane and at one 64-weight group."""
    test_format_gemv_matches_oracle(fmt, N, K)


def test_affine_bf16_is_not_read_as_fp16():
    """The same bits as bf16 and as fp16 scales give different products: the bf16
    format decodes its scales and biases as bf16 (the closed form codes 15, bias
    0: y = 15 s sum(x) with s = 0.5 as bf16 0x3F00, which as fp16 is 1.75)."""
    N, K = 4, 128
    words = np.full((N, K // 8), 0xFFFFFFFF, np.uint32)
    sc = np.full((N, K // 64), 0x3F00, np.uint16)
    bi = np.zeros((N, K // 64), np.uint16)
    x = np.full(K, 0x3C00, np.uint16)            # ones
    yb = q4.q4_gemv_format(q4.FMT_AF4_G64, to_dev(words), to_dev(sc), to_dev(x), K,
                           biases=to_dev(bi))
    yh = q4.q4_gemv_format(q4.FMT_AF4_G64_F16, to_dev(words), to_dev(sc), to_dev(x), K,
                           biases=to_dev(bi))
    torch.cuda.synchronize()
    assert np.all(half_f64(host_half(yb)) == 15 * 0.5 * K)
    assert np.all(half_f64(host_half(yh)) == 15 * 1.75 * K)


def test_format_weight_bytes():
    assert q4.q4_format_weight_bytes(0, 9216, 3072) == 9216 * 96 * 18
    assert q4.q4_format_weight_bytes(q4.FMT_Q3F16_1, 9216, 3072) == 9216 * 96 * 14
    assert q4.q4_format_weight_bytes(q4.FMT_Q4F32_1, 9216, 3072) == 9216 * 96 * 20
    assert q4.q4_format_weight_bytes(q4.FMT_AF4_G64, 9216, 3072) == 9216 * 48 * 36
    assert q4.q4_format_weight_bytes(q4.FMT_AF4_G64, 10, 96) == 0
    assert q4.q4_format_weight_bytes(q4.FMT_AF4_G64_F16, 9216, 3072) == 9216 * 48 * 36

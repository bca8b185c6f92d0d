"""q3f16_1 layers inside the decode step (q4_layer.format = Q4_FMT_Q3F16_1, M = 1):
a list mixing q3f16_1 and q4f16_1 GEMVs through the persistent kernel (range mode,
ordered with tagged hand-over between q3f16_1 layers) and one kernel per GEMV,
every output against the oracle (orc_gemv_format / orc_gemv_f64) under the GEMV
tolerance; closed forms through the persistent kernel: codes all 3 give exactly
zero, unit scales and x = 1 give the exact code sums."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import dev_half, dev_words, half_f64, host_half

pytestmark = pytest.mark.gpu

Q3 = q4.FMT_Q3F16_1
MODES = {"range": 0x10, "ordered": 0x2 | 0x10, "each": 0x1}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def q3_weight(tag, N, K):
    lab = f"q3step/{tag}/{N}x{K}"
    words = synth.words(lab + "/w", 0, N * K // 32 * 3).reshape(N, K // 32 * 3)
    scales = synth.scales_halfnormal(lab + "/s", 0, 0, N * K // 32, 0.01, 1e-3).reshape(N, -1)
    return words, scales


def q4_weight(tag, N, K):
    m = synth.Matrix(f"q3step/{tag}/{N}x{K}", N, K)
    return m.words(), m.scales()


def reference(fmt, words, scales, x_bits):
    """fp64 y and the GEMV tolerance 2e-3 ||x|| max ||W_n||."""
    K = x_bits.size
    if fmt == Q3:
        ref, norms = oracle.gemv_format("q3f16_1", words, scales, None, x_bits, K)
        return ref, 2e-3 * oracle.vec_norm(x_bits) * norms.max()
    ref = oracle.gemv_f64(words, scales, x_bits)
    return ref, 2e-3 * oracle.vec_norm(x_bits) * oracle.row_norms(words, scales).max()


# (format, N, K, x_op): tiles and ragged tails, padded rows (G = 17, 3 groups per
# lane of 8), K = 8192 (4 groups per lane of 64), the glue's doubled x
SHAPES = [(Q3, 1000, 3072, 0), (0, 777, 2048, 0), (Q3, 3072, 8192, 0), (Q3, 130, 544, 0),
          (0, 500, 4096, 0), (Q3, 300, 1024, 1), (Q3, 9216, 3072, 0)]


@pytest.mark.parametrize("mode", sorted(MODES))
def test_mixed_list_matches_oracle(mode):
    host, descs = [], []
    for i, (fmt, N, K, x_op) in enumerate(SHAPES):
        w, s = (q3_weight if fmt == Q3 else q4_weight)(f"mix{i}", N, K)
        xin = synth.activations(f"q3step/x{i}", 0, (2 if x_op else 1) * K)
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        descs.append((dev_words(w), dev_half(s), dev_half(xin), y, x_op, fmt))
        host.append((fmt, w, s, xin, x_op))
    layers = q4.make_layers(descs)
    plan = q4.StepPlan(layers, 1, MODES[mode], keep=descs)
    plan.run()
    torch.cuda.synchronize()
    plan.status()
    for i, ((fmt, w, s, xin, x_op), d) in enumerate(zip(host, descs)):
        x = oracle.silu_mul(xin.reshape(1, -1))[0] if x_op else xin
        ref, tol = reference(fmt, w, s, x)
        got = half_f64(host_half(d[3]))
        assert np.all(np.isfinite(got)), i
        err = np.abs(got - ref).max()
        assert err <= tol, (mode, i, err, tol)


def test_ordered_chain_with_tagged_handover():
    """Each layer's x is the previous layer's y (ordered: the tagged hand-over),
    q3f16_1 and q4f16_1 alternating; each output against the oracle on the input
    the GPU produced."""
    chain = [(Q3, 2048, 1024), (Q3, 1536, 2048), (0, 3072, 1536), (Q3, 1024, 3072),
             (0, 512, 1024)]
    x0 = synth.activations("q3step/chain/x", 0, chain[0][2])
    xs = dev_half(x0)
    descs, host = [], []
    x = xs
    for i, (fmt, N, K) in enumerate(chain):
        w, s = (q3_weight if fmt == Q3 else q4_weight)(f"chain{i}", N, K)
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        descs.append((dev_words(w), dev_half(s), x[:K], y, 0, fmt))
        host.append((fmt, w, s))
        x = y
    plan = q4.StepPlan(q4.make_layers(descs), 1, MODES["ordered"], keep=descs)
    for _ in range(3):
        plan.run()
    torch.cuda.synchronize()
    plan.status()
    xin = x0
    for i, ((fmt, w, s), d) in enumerate(zip(host, descs)):
        K = chain[i][2]
        ref, tol = reference(fmt, w, s, xin[:K])
        got_bits = host_half(d[3])
        err = np.abs(half_f64(got_bits) - ref).max()
        assert err <= tol, (i, err, tol)
        xin = got_bits


@pytest.mark.parametrize("mode", ["range", "ordered"])
def test_closed_forms_through_the_persistent_kernel(mode):
    """Codes all 3 (the zero point): y == 0 exactly, whatever the scales and x.
    Unit scales and x = 1: y_n = sum over the row of (q - 3), exactly."""
    N, K = 300, 256
    zero = np.tile(np.array([0xDB6DB6DB, 0xB6DB6DB6, 0x6DB6DB6D], np.uint32), (N, K // 32))
    _, s = q3_weight("cf", N, K)
    x = synth.activations("q3step/cf/x", 0, K)
    w1, _ = q3_weight("cf1", N, K)
    ones_s = np.full((N, K // 32), 0x3C00, np.uint16)
    ones_x = np.full(K, 0x3C00, np.uint16)
    ys = [torch.full((N,), float("nan"), dtype=torch.float16, device="cuda") for _ in range(2)]
    descs = [(dev_words(zero), dev_half(s), dev_half(x), ys[0], 0, Q3),
             (dev_words(w1), dev_half(ones_s), dev_half(ones_x), ys[1], 0, Q3)]
    plan = q4.StepPlan(q4.make_layers(descs), 1, MODES[mode], keep=descs)
    plan.run()
    torch.cuda.synchronize()
    plan.status()
    assert np.all(half_f64(host_half(ys[0])) == 0.0)
    # the code sums from the oracle's own unpacking of the 3-bit words (unit
    # scales, x = 1: the oracle's y is that sum)
    ref, _ = oracle.gemv_format("q3f16_1", w1, ones_s, None, ones_x, K)
    assert np.array_equal(half_f64(host_half(ys[1])), ref)

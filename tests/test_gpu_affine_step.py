"""MLX affine layers inside the decode step (q4_layer.format = Q4_FMT_AF4_G64 with
bf16 scales and biases, or Q4_FMT_AF4_G64_F16; M = 1): lists mixing them with
q4f16_1 and q3f16_1 GEMVs through the persistent kernel (range mode, ordered with
the tagged hand-over) and one kernel per GEMV, every output against the oracle
(orc_gemv_format / orc_gemv_f64) under the GEMV tolerance, with the share of
exactly rounded outputs; closed forms through the persistent kernel: codes 7 with
b = -7 s give exactly zero, unit scales with b = -7 and x = 1 give the exact sums of
q - 7, zero scales with unit biases give exactly K."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import dev_half, dev_words, half_f64, host_half

pytestmark = pytest.mark.gpu

AF, AH, Q3 = q4.FMT_AF4_G64, q4.FMT_AF4_G64_F16, q4.FMT_Q3F16_1
MODES = {"range": 0x10, "ordered": 0x2 | 0x10, "each": 0x1}
NAMES = {AF: "af4g64", AH: "af4g64_f16", Q3: "q3f16_1"}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def weight(fmt, tag, N, K):
    """(words, scales, biases) in the format's layout, seeded: for the affine formats
    bf16 or fp16 scales s = |N(0, 0.01)| + 1e-3 and biases b = -7.5 s + 0.1 s N(0, 1),
    centred groups as an affine quantiser writes them (b near the group's minimum,
    so s q + b spans it), which keeps a chain of layers from growing."""
    lab = f"afstep/{tag}/{fmt}/{N}x{K}"
    if fmt == Q3:
        w = synth.words(lab + "/w", 0, N * K // 32 * 3).reshape(N, K // 32 * 3)
        s = synth.scales_halfnormal(lab + "/s", 0, 0, N * K // 32, 0.01, 1e-3).reshape(N, -1)
        return w, s, None
    if fmt == 0:
        m = synth.Matrix(lab, N, K)
        return m.words(), m.scales(), None
    w = synth.words(lab + "/w", 0, N * K // 8).reshape(N, K // 8)
    sv = np.abs(0.01 * synth.normal(lab + "/s", 0, 0, N * K // 64)) + 1e-3
    bv = -7.5 * sv + 0.1 * sv * synth.normal(lab + "/b", 0, 0, N * K // 64)
    conv = synth.to_bf16_bits if fmt == AF else synth.to_half_bits
    return w, conv(sv).reshape(N, -1), conv(bv).reshape(N, -1)


def reference(fmt, w, s, b, x_bits):
    """fp64 y and the GEMV tolerance 2e-3 ||x|| max ||W_n||."""
    K = x_bits.size
    if fmt == 0:
        ref = oracle.gemv_f64(w, s, x_bits)
        return ref, 2e-3 * oracle.vec_norm(x_bits) * oracle.row_norms(w, s).max()
    ref, norms = oracle.gemv_format(NAMES[fmt], w, s, b, x_bits, K)
    return ref, 2e-3 * oracle.vec_norm(x_bits) * norms.max()


def to16(v):
    return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


def desc(fmt, w, s, b, x_dev, y, x_op=0):
    d = (dev_words(w), dev_half(s), x_dev, y, x_op, fmt)
    return d + (dev_half(b),) if b is not None else d


# (format, N, K, x_op): tiles and ragged tails, padded rows (K = 576: 18 groups, 3
# per lane of 8), K = 8192 (4 groups per lane of 64), the glue's doubled x, q4f16_1
# and q3f16_1 layers between them
SHAPES = [(AF, 1000, 3072, 0), (AH, 777, 2048, 0), (0, 500, 4096, 0), (AF, 3072, 8192, 0),
          (AF, 130, 576, 0), (Q3, 300, 1024, 0), (AF, 300, 1024, 1), (AH, 129, 192, 0),
          (AF, 9216, 3072, 0)]


@pytest.mark.parametrize("mode", sorted(MODES))
def test_mixed_list_matches_oracle(mode):
    host, descs = [], []
    for i, (fmt, N, K, x_op) in enumerate(SHAPES):
        w, s, b = weight(fmt, f"mix{i}", N, K)
        xin = synth.activations(f"afstep/x{i}", 0, (2 if x_op else 1) * K)
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        descs.append(desc(fmt, w, s, b, dev_half(xin), y, x_op))
        host.append((fmt, w, s, b, xin, x_op))
    plan = q4.StepPlan(q4.make_layers(descs), 1, MODES[mode], keep=descs)
    plan.run()
    torch.cuda.synchronize()
    plan.status()
    for i, ((fmt, w, s, b, xin, x_op), d) in enumerate(zip(host, descs)):
        x = oracle.silu_mul(xin.reshape(1, -1))[0] if x_op else xin
        ref, tol = reference(fmt, w, s, b, x)
        got_bits = host_half(d[3])
        got = half_f64(got_bits)
        assert np.all(np.isfinite(got)), i
        err = np.abs(got - ref).max()
        assert err <= tol, (mode, i, err, tol)
        if fmt in (AF, AH):
            # the fp64 oracle rounded once to fp16 is the exactly rounded value
            # (its error is ~2^-50 relative); the kernel forms s * sum(q x) and
            # b * sum(x) per group in fp32 (a few units of 2^-24 of the group's
            # absolute sums), so nearly every output rounds the same way
            same = float(np.mean(to16(ref) == got_bits))
            assert same >= 0.95, (mode, i, same)


def test_ordered_chain_with_tagged_handover():
    """Each layer's x is the previous layer's y (ordered: the tagged hand-over),
    affine layers between q4f16_1 and q3f16_1 ones; each output against the
    oracle on the input the GPU produced."""
    chain = [(AF, 2048, 1024), (AH, 1536, 2048), (0, 3072, 1536), (AF, 1024, 3072),
             (Q3, 512, 1024), (AF, 640, 512)]
    x0 = synth.activations("afstep/chain/x", 0, chain[0][2])
    x = dev_half(x0)
    descs, host = [], []
    for i, (fmt, N, K) in enumerate(chain):
        w, s, b = weight(fmt, f"chain{i}", N, K)
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        descs.append(desc(fmt, w, s, b, x[:K], y))
        host.append((fmt, w, s, b))
        x = y
    plan = q4.StepPlan(q4.make_layers(descs), 1, MODES["ordered"], keep=descs)
    for _ in range(3):
        plan.run()
    torch.cuda.synchronize()
    plan.status()
    xin = x0
    for i, ((fmt, w, s, b), d) in enumerate(zip(host, descs)):
        K = chain[i][2]
        ref, tol = reference(fmt, w, s, b, xin[:K])
        got_bits = host_half(d[3])
        err = np.abs(half_f64(got_bits) - ref).max()
        assert err <= tol, (i, err, tol)
        xin = got_bits


@pytest.mark.parametrize("mode", ["range", "ordered"])
@pytest.mark.parametrize("fmt", [AF, AH])
def test_closed_forms_through_the_persistent_kernel(mode, fmt):
    """Codes all 7 with b = -7 s (s = 2^-7): y == 0 exactly, whatever x.  Unit
    scales, b = -7 and x = 1: y_n = the row's sum of (q - 7), exactly.  Scales 0,
    biases 1 and x = 1: y_n = K exactly."""
    N, K = 300, 128
    cv = synth.to_bf16_bits if fmt == AF else synth.to_half_bits
    w1, _, _ = weight(fmt, "cf1", N, K)
    x = synth.activations("afstep/cf/x", 0, K)
    w7 = np.full((N, K // 8), 0x77777777, np.uint32)
    full = lambda v: np.full((N, K // 64), int(cv(np.array([v]))[0]), np.uint16)
    ones_x = np.full(K, 0x3C00, np.uint16)
    ys = [torch.full((N,), float("nan"), dtype=torch.float16, device="cuda") for _ in range(3)]
    descs = [desc(fmt, w7, full(2.0 ** -7), full(-7 * 2.0 ** -7), dev_half(x), ys[0]),
             desc(fmt, w1, full(1.0), full(-7.0), dev_half(ones_x), ys[1]),
             desc(fmt, w1, full(0.0), full(1.0), dev_half(ones_x), ys[2])]
    plan = q4.StepPlan(q4.make_layers(descs), 1, MODES[mode], keep=descs)
    plan.run()
    torch.cuda.synchronize()
    plan.status()
    assert np.all(half_f64(host_half(ys[0])) == 0.0)
    codes = oracle.unpack(w1).reshape(N, K).astype(np.int64)
    assert np.array_equal(half_f64(host_half(ys[1])), (codes - 7).sum(axis=1).astype(np.float64))
    assert np.all(half_f64(host_half(ys[2])) == float(K))

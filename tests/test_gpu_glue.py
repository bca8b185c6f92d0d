"""The feed-forward glue between the gate/up and down projections, fp16(silu(gate)
* up): the standalone kernel against the oracle, and the down projection reading
[gate | up] through x_op = X_SILU_MUL (formed while its input is staged) against
the oracle on the values the GPU actually read, in every decode-step mode."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import assert_gemv_close, dev_half, dev_words, half_f64, host_half

pytestmark = pytest.mark.gpu

MODES = {"hazards": q4.STEP_PERSISTENT, "ordered": q4.STEP_ORDERED | q4.STEP_PERSISTENT,
         "launch_each": q4.STEP_LAUNCH_EACH, "auto": 0}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def mat(label, N, K):
    m = synth.Matrix(label, N, K, sigma=2.0 / K, floor=0.5 / K)
    return m, dev_words(m.words()), dev_half(m.scales())


def nan_half(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float16, device="cuda")


def assert_glue_close(got_bits, ref_bits, min_exact=0.999):
    """Within one fp16 unit in the last place of the exactly rounded value (fp32
    against fp64 evaluation can round the other way near a tie), NaN where it is
    NaN, and almost all bitwise equal."""
    got = np.asarray(got_bits, np.uint16).reshape(-1)
    ref = np.asarray(ref_bits, np.uint16).reshape(-1)
    gf = got.view(np.float16).astype(np.float64)
    rf = ref.view(np.float16).astype(np.float64)
    nan = np.isnan(rf)
    assert np.array_equal(np.isnan(gf), nan)
    fin = ~nan
    assert np.array_equal(np.isinf(gf[fin]), np.isinf(rf[fin]))
    both = fin & np.isfinite(rf)
    mag = np.abs(rf[both])
    # fp16 unit in the last place at |ref|: 2^(e - 10) for normals, 2^-24 below
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -14)))
    spacing = 2.0 ** (e - 10)
    assert np.all(np.abs(gf[both] - rf[both]) <= spacing)
    assert (got == ref).mean() >= min_exact


@pytest.mark.parametrize("M,H", [(1, 8), (1, 8192), (3, 1000 * 8)])
def test_silu_mul_matches_oracle(M, H):
    gu = synth.activations(f"glue/gu/{M}x{H}", 0, M * 2 * H).reshape(M, 2 * H)
    g = gu.view(np.float16).astype(np.float32) * 4.0          # spread the gate over +-20
    gu = g.astype(np.float16).view(np.uint16)
    if H >= 16:   # special values in the gate and the up halves
        sp = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, -65504.0, 6e-8, -30.0, 30.0, 1.0],
                      np.float16).view(np.uint16)
        gu[0, :len(sp)] = sp
        gu[0, H:H + len(sp)] = np.array([1.0] * len(sp), np.float16).view(np.uint16)
        gu[0, H + 2] = np.float16(0.0).view(np.uint16)      # inf * 0 -> NaN
    out = q4.q4_silu_mul(dev_half(gu))
    torch.cuda.synchronize()
    assert_glue_close(host_half(out), oracle.silu_mul(gu))


@pytest.mark.parametrize("mode", sorted(MODES))
def test_mlp_gate_up_then_down(mode):
    """gate_up 3072 -> 16384, then down 8192 -> 3072 reading [gate | up]."""
    D, H = 3072, 8192
    mgu, Wgu, Sgu = mat("glue/mlp/gate_up", 2 * H, D)
    mdn, Wdn, Sdn = mat("glue/mlp/down", D, H)
    x = dev_half(synth.activations("glue/mlp/x", 0, D))
    gu, y = nan_half(2 * H), nan_half(D)
    layers = q4.make_layers([(Wgu, Sgu, x, gu), (Wdn, Sdn, gu, y, q4.X_SILU_MUL)])
    q4.q4_decode_step(layers, 1, MODES[mode])
    torch.cuda.synchronize()
    gu_h = host_half(gu)
    assert np.all(np.isfinite(half_f64(gu_h)))
    assert_gemv_close(gu_h, mgu.words(), mgu.scales(), host_half(x))
    h_ref = oracle.silu_mul(gu_h.reshape(1, -1))[0]
    y_h = host_half(y)
    assert np.all(np.isfinite(half_f64(y_h)))
    assert_gemv_close(y_h, mdn.words(), mdn.scales(), h_ref)


def test_fused_glue_equals_standalone_glue_bitwise():
    """The persistent kernel forms the same h as q4_silu_mul: the down projection
    over [gate | up] equals the down projection over q4_silu_mul's output."""
    D, H = 3072, 8192
    mgu, Wgu, Sgu = mat("glue/bit/gate_up", 2 * H, D)
    mdn, Wdn, Sdn = mat("glue/bit/down", D, H)
    x = dev_half(synth.activations("glue/bit/x", 0, D))
    gu, y = nan_half(2 * H), nan_half(D)
    q4.q4_decode_step(q4.make_layers([(Wgu, Sgu, x, gu), (Wdn, Sdn, gu, y, q4.X_SILU_MUL)]), 1,
                      q4.STEP_PERSISTENT)
    h = q4.q4_silu_mul(gu)
    y2 = nan_half(D)
    # one-descriptor lists run as one GEMV kernel unless the persistent one is asked for
    q4.q4_decode_step(q4.make_layers([(Wdn, Sdn, h, y2)]), 1, q4.STEP_PERSISTENT)
    # and the glue from a plain input buffer (no producer in the list); the copy
    # must outlive the call (make_layers keeps only its address)
    gu2, y3 = gu.clone(), nan_half(D)
    q4.q4_decode_step(q4.make_layers([(Wdn, Sdn, gu2, y3, q4.X_SILU_MUL)]), 1,
                      q4.STEP_PERSISTENT)
    torch.cuda.synchronize()
    assert np.array_equal(host_half(y), host_half(y2))
    assert np.array_equal(host_half(y), host_half(y3))
    assert_glue_close(host_half(h), oracle.silu_mul(host_half(gu).reshape(1, -1))[0])


def test_glue_behind_a_counter_wait():
    """Ordered, with a GEMV between gate_up and down: down's producer is not its
    predecessor, so it waits on a completion counter and reads [gate | up] with
    coherent loads instead of tagged pairs."""
    D, H = 3072, 4096
    mgu, Wgu, Sgu = mat("glue/ctr/gate_up", 2 * H, D)
    mmid, Wmid, Smid = mat("glue/ctr/mid", 1000, D)
    mdn, Wdn, Sdn = mat("glue/ctr/down", D, H)
    x = dev_half(synth.activations("glue/ctr/x", 0, D))
    gu, z, y = nan_half(2 * H), nan_half(1000), nan_half(D)
    layers = q4.make_layers([(Wgu, Sgu, x, gu), (Wmid, Smid, x, z),
                             (Wdn, Sdn, gu, y, q4.X_SILU_MUL)])
    q4.q4_decode_step(layers, 1, q4.STEP_ORDERED | q4.STEP_PERSISTENT)
    torch.cuda.synchronize()
    gu_h = host_half(gu)
    assert_gemv_close(gu_h, mgu.words(), mgu.scales(), host_half(x))
    assert_gemv_close(host_half(z), mmid.words(), mmid.scales(), host_half(x))
    assert_gemv_close(host_half(y), mdn.words(), mdn.scales(),
                      oracle.silu_mul(gu_h.reshape(1, -1))[0])


def test_glue_at_small_m():
    """M = 2: the list runs one kernel per GEMV (glue kernel, then the GEMV)."""
    M, D, H = 2, 2048, 3072
    mgu, Wgu, Sgu = mat("glue/m2/gate_up", 2 * H, D)
    mdn, Wdn, Sdn = mat("glue/m2/down", D, H)
    x = dev_half(synth.activations("glue/m2/x", 0, M * D).reshape(M, D))
    gu, y = nan_half(M, 2 * H), nan_half(M, D)
    layers = q4.make_layers([(Wgu, Sgu, x, gu), (Wdn, Sdn, gu, y, q4.X_SILU_MUL)])
    q4.q4_decode_step(layers, M, 0)
    torch.cuda.synchronize()
    gu_h = host_half(gu)
    assert_gemv_close(gu_h, mgu.words(), mgu.scales(), host_half(x))
    assert_gemv_close(host_half(y), mdn.words(), mdn.scales(), oracle.silu_mul(gu_h))

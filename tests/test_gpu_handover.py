"""Dependencies inside one decode-step launch: a GEMV whose x lies inside one
earlier GEMV's y takes it over as epoch-tagged pairs (no completion counter);
other conflicts wait on counters, and a list whose conflicts one wait cannot
cover runs one kernel per GEMV.  Every case is checked against the oracle on the
inputs the GPU actually read, and where two paths run the same arithmetic, for
bitwise agreement between them."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import assert_gemv_close, dev_half, dev_words, half_f64, host_half

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def mat(label, N, K):
    # scales ~ 1/K keep chained activations O(1)
    m = synth.Matrix(label, N, K, sigma=2.0 / K, floor=0.5 / K)
    return m, dev_words(m.words()), dev_half(m.scales())


def nan_half(n):
    return torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")


def run(descs, flags=q4.STEP_PERSISTENT, ws=None):
    # the persistent kernel even where the driver would launch one kernel per GEMV
    layers = q4.make_layers(descs)
    q4.q4_decode_step(layers, 1, flags, ws=ws)
    torch.cuda.synchronize()


def check(m, X, Y):
    y = host_half(Y)
    assert np.all(np.isfinite(half_f64(y)))
    assert_gemv_close(y, m.words(), m.scales(), host_half(X))


@pytest.mark.parametrize("flags", [q4.STEP_PERSISTENT, q4.STEP_ORDERED | q4.STEP_PERSISTENT, 0],
                         ids=["hazards", "ordered", "auto"])
def test_consumers_of_slices(flags):
    """Three GEMVs read the three thirds of one qkv-shaped output (even element
    offsets); in ordered mode each also waits for its predecessor."""
    K = 3072
    mp, Wp, Sp = mat("ho/slices/p", 3 * K, K)
    x = dev_half(synth.activations("ho/slices/x", 0, K))
    yp = nan_half(3 * K)
    descs, mats = [(Wp, Sp, x, yp)], [mp]
    for i in range(3):
        m, W, S = mat(f"ho/slices/{i}", 1000 + 24 * i, K)
        descs.append((W, S, yp[i * K:(i + 1) * K], nan_half(1000 + 24 * i)))
        mats.append(m)
    run(descs, flags)
    for m, (W, S, X, Y) in zip(mats, descs):
        check(m, X, Y)


def test_offsets_into_odd_row_producer():
    """Consumers at two offsets into the output of a producer with one row per
    row-step (rows split over workgroups in pairs) and an odd row count."""
    mp, Wp, Sp = mat("ho/odd/p", 4097, 8192)
    x = dev_half(synth.activations("ho/odd/x", 0, 8192))
    yp = nan_half(4097)
    m1, W1, S1 = mat("ho/odd/1", 777, 4064)
    m2, W2, S2 = mat("ho/odd/2", 513, 4064)
    descs = [(Wp, Sp, x, yp), (W1, S1, yp[8:8 + 4064], nan_half(777)),
             (W2, S2, yp[32:32 + 4064], nan_half(513))]
    run(descs)
    for m, (W, S, X, Y) in zip([mp, m1, m2], descs):
        check(m, X, Y)


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("chained", [False, True], ids=["independent", "second_reads_first"])
def test_reader_of_two_writers(chained, M):
    """x spans the outputs of two GEMVs: one counter wait cannot cover both unless
    the later writer waits for the earlier through counters, so the list runs one
    kernel per GEMV; results are right either way (M = 2: the small-M planner)."""
    K, H = 3072, 1536
    buf = torch.full((M * K,), float("nan"), dtype=torch.float16, device="cuda")
    y1 = buf[:M * H].view(M, H)
    y2 = buf[M * H:].view(M, H)
    m1, W1, S1 = mat("ho/two/1", H, K)
    x1 = dev_half(synth.activations("ho/two/x1", 0, M * K).reshape(M, K))
    if chained:
        m2, W2, S2 = mat("ho/two/2c", H, H)
        x2 = y1
    else:
        m2, W2, S2 = mat("ho/two/2", H, K)
        x2 = dev_half(synth.activations("ho/two/x2", 0, M * K).reshape(M, K))
    m3, W3, S3 = mat("ho/two/3", 2048, K)
    y3 = torch.full((M, 2048), float("nan"), dtype=torch.float16, device="cuda")
    if M == 1:
        descs = [(W1, S1, x1[0], y1[0]), (W2, S2, x2[0], y2[0]), (W3, S3, buf, y3[0])]
    else:
        descs = [(W1, S1, x1, y1), (W2, S2, x2, y2), (W3, S3, buf.view(M, K), y3)]
    layers = q4.make_layers(descs)
    q4.q4_decode_step(layers, M, q4.STEP_PERSISTENT)
    torch.cuda.synchronize()
    for m, (W, S, X, Y) in zip([m1, m2, m3], descs):
        y = host_half(Y)
        assert np.all(np.isfinite(half_f64(y)))
        assert_gemv_close(y, m.words(), m.scales(), host_half(X).reshape(M, -1))


def test_ping_pong_buffers_match_separate_buffers():
    """A chain through two alternating buffers (every step overwrites what the one
    before it read: counter waits) gives the same bits as the same chain through
    separate buffers (tagged hand-over), and the latter matches the oracle."""
    K = 3072
    mats = [mat(f"ho/pp/{i}", K, K) for i in range(6)]
    x0 = synth.activations("ho/pp/x", 0, K)
    A, B = dev_half(x0), nan_half(K)
    bufs = [A, B]
    descs = [(W, S, bufs[i % 2], bufs[(i + 1) % 2]) for i, (m, W, S) in enumerate(mats)]
    run(descs)
    pp_last = host_half(bufs[len(mats) % 2])
    x = dev_half(x0)
    sep = []
    for m, W, S in mats:
        y = nan_half(K)
        sep.append((W, S, x, y))
        x = y
    run(sep)
    assert np.array_equal(pp_last, host_half(sep[-1][3]))
    for (m, _, _), (W, S, X, Y) in zip(mats, sep):
        check(m, X, Y)


def test_repeated_calls_on_one_workspace():
    """Tagged pairs from earlier calls never pass for this call's: repeated calls
    (the workspace left clean, then reused) give the same bits every time."""
    # one Phi-3-shaped layer and the LM head, each x a prefix of the previous y
    shapes = [(9216, 3072), (3072, 3072), (16384, 3072), (3072, 8192), (32064, 3072)]
    x = dev_half(synth.activations("ho/rep/x", 0, 3072))
    descs, mats = [], []
    for i, (N, K) in enumerate(shapes):
        m, W, S = mat(f"ho/rep/{i}", N, K)
        y = nan_half(N)
        descs.append((W, S, x[:K], y))
        mats.append(m)
        x = y
    layers = q4.make_layers(descs)
    P = q4.STEP_PERSISTENT
    need = q4.q4_decode_step_workspace_bytes(layers, 1, P)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    plan = q4.StepPlan(layers, 1, P, ws=ws)
    plan.run()
    plan.status()
    ref = [host_half(d[3]) for d in descs]
    for m, (W, S, X, Y) in zip(mats, descs):
        check(m, X, Y)
    for _ in range(6):
        for d in descs:
            d[3].fill_(float("nan"))
        plan.run()
        plan.status()
        for r, d in zip(ref, descs):
            assert np.array_equal(r, host_half(d[3]))

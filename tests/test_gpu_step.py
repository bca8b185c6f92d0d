"""The decode-step driver (q4_decode_step) in its three modes: one persistent
kernel honouring memory hazards (default), one persistent kernel with every
descriptor waiting for its predecessor (ordered), one kernel per descriptor.
Every output is checked against the oracle on the inputs the GPU actually read."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import assert_gemv_close, dev_half, dev_words, half_f64, host_half, host_words

pytestmark = pytest.mark.gpu

# default: the persistent kernel (STEP_PERSISTENT keeps dependency-heavy lists in
# it; "auto" lets the driver choose)
MODES = {"hazards": q4.STEP_PERSISTENT, "ordered": q4.STEP_ORDERED | q4.STEP_PERSISTENT,
         "launch_each": q4.STEP_LAUNCH_EACH, "auto": 0}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def mat(label, N, K, chain=False):
    kw = dict(sigma=2.0 / K, floor=0.5 / K) if chain else {}
    m = synth.Matrix(label, N, K, **kw)
    return m, dev_words(m.words()), dev_half(m.scales())


def run(descs, flags):
    layers = q4.make_layers(descs)
    q4.q4_decode_step(layers, 1, flags)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("dims", [[3072, 8192, 3072, 6144, 2048, 512, 1024, 256, 3072],
                                  [3072, 9216, 3072, 544, 96, 2048]],
                         ids=["k256", "ragged_k"])
def test_dependent_chain(mode, dims):
    """Each descriptor reads the previous one's output (RAW hazards)."""
    x0 = dev_half(synth.activations("stepchain/x", 0, dims[0]))
    descs, mats = [], []
    x = x0
    for i in range(len(dims) - 1):
        m, W, S = mat(f"stepchain/{i}", dims[i + 1], dims[i], chain=True)
        y = torch.full((dims[i + 1],), float("nan"), dtype=torch.float16, device="cuda")
        descs.append((W, S, x, y))
        mats.append(m)
        x = y
    run(descs, MODES[mode])
    for m, (W, S, X, Y) in zip(mats, descs):
        y = host_half(Y)
        assert np.all(np.isfinite(half_f64(y)))
        assert_gemv_close(y, m.words(), m.scales(), host_half(X))


@pytest.mark.parametrize("mode", sorted(MODES))
def test_write_after_read_and_write_after_write(mode):
    K = 1024
    mA, WA, SA = mat("war/a", K, K)
    mB, WB, SB = mat("war/b", K, K)
    mC, WC, SC = mat("war/c", K, K)
    xa = synth.activations("war/xa", 0, K)
    xb = synth.activations("war/xb", 0, K)
    A = dev_half(xa)
    B = dev_half(xb)
    out = torch.empty(K, dtype=torch.float16, device="cuda")
    # 0: out = WA A   1: A = WB B (overwrites 0's input)   2: out = WC B (overwrites 0's output)
    run([(WA, SA, A, out), (WB, SB, B, A), (WC, SC, B, out)], MODES[mode])
    assert_gemv_close(host_half(A), mB.words(), mB.scales(), xb)
    assert_gemv_close(host_half(out), mC.words(), mC.scales(), xb)
    # and the first descriptor read the original A: recompute it alone
    A2 = dev_half(xa)
    out0 = torch.empty(K, dtype=torch.float16, device="cuda")
    run([(WA, SA, A2, out0)], MODES[mode])
    assert_gemv_close(host_half(out0), mA.words(), mA.scales(), xa)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("shapes", [
    [(1, 32)], [(3, 544), (1000, 32), (257, 96)], [(7, 8192), (64, 64), (5000, 2048)],
    [(32064, 3072)], [(17, 256)] * 9, [(1, 256), (3, 8192), (5, 512), (2049, 2048)],
], ids=["tiny", "ragged", "mixed", "lm_head", "many_small", "k256_ragged_rows"])
def test_independent_lists(mode, shapes):
    descs, mats, xs = [], [], []
    for i, (N, K) in enumerate(shapes):
        m, W, S = mat(f"ind/{i}/{N}x{K}", N, K)
        x = synth.activations(f"ind/x/{i}", 0, K)
        descs.append((W, S, dev_half(x), torch.empty(N, dtype=torch.float16, device="cuda")))
        mats.append(m)
        xs.append(x)
    run(descs, MODES[mode])
    for m, x, (W, S, X, Y) in zip(mats, xs, descs):
        assert_gemv_close(host_half(Y), m.words(), m.scales(), x)


@pytest.mark.parametrize("shapes", [
    [(100, 256), (37, 128)], [(64, 512)] * 300, [(65536, 4096), (3, 32)],
    [(9216, 3072), (3072, 3072), (16384, 3072), (3072, 8192)] * 2 + [(32064, 3072)],
], ids=["most_wgs_idle", "300_gemvs", "tiny_tail", "two_phi3_blocks_lm_head"])
def test_range_mode_repeat(shapes):
    """Lists without dependencies (one stretch of row-steps per workgroup, many
    workgroups with none, or hundreds of GEMVs): every row computed once and
    right, the counters left zero (so runs of the plan need no clearing), and
    repeated runs bitwise equal."""
    descs, mats, xs = [], [], []
    for i, (N, K) in enumerate(shapes):
        m, W, S = mat(f"pool/{i}/{N}x{K}", N, K)
        x = synth.activations(f"pool/x/{i % 7}/{K}", 0, K)
        descs.append((W, S, dev_half(x), torch.full((N,), float("nan"), dtype=torch.float16,
                                                    device="cuda")))
        mats.append(m)
        xs.append(x)
    layers = q4.make_layers(descs)
    n = len(descs)
    flags = q4.STEP_PERSISTENT
    need = q4.q4_decode_step_workspace_bytes(layers, 1, flags)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")   # garbage
    plan = q4.StepPlan(layers, 1, flags, ws=ws)                         # clears the counters
    plan.run()
    plan.status()
    ref = [host_half(d[3]) for d in descs]
    for m, x, y in zip(mats, xs, ref):
        assert_gemv_close(y, m.words(), m.scales(), x)
    assert counters_zero(ws, n)
    for _ in range(3):
        for d in descs:
            d[3].fill_(float("nan"))
        plan.run()
        plan.status()
        for r, d in zip(ref, descs):
            assert np.array_equal(r, host_half(d[3]))
        assert counters_zero(ws, n)


def counters_zero(ws, n):
    """The control block's error word and exit count, and the n completion
    counters after the block, are zero."""
    w = ws.view(torch.int32).cpu().numpy()
    return w[0] == 0 and w[2] == 0 and not w[64:64 + n].any()


@pytest.mark.parametrize("flags", [q4.STEP_PERSISTENT, q4.STEP_ORDERED | q4.STEP_PERSISTENT],
                         ids=["hazards", "ordered"])
def test_plan_runs_repeat_and_leave_counters_zero(flags):
    """The persistent kernel leaves its counters zero and advances the hand-over
    epoch once per launch, so a plan runs again and again on one workspace with
    nothing cleared in between; results stay bitwise the same, and equal those of
    the one-call entry point."""
    dims = [3072, 8192, 3072, 6144, 2048, 512, 1024, 256, 3072]
    x = dev_half(synth.activations("wsclean/x", 0, dims[0]))
    descs = []
    for i in range(len(dims) - 1):
        m, W, S = mat(f"wsclean/{i}", dims[i + 1], dims[i], chain=True)
        y = torch.empty(dims[i + 1], dtype=torch.float16, device="cuda")
        descs.append((W, S, x, y))
        x = y
    layers = q4.make_layers(descs)
    n = len(descs)
    need = q4.q4_decode_step_workspace_bytes(layers, 1, flags)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")   # garbage
    q4.q4_decode_step(layers, 1, flags, ws=ws)                          # plans, clears, runs
    ref = [host_half(d[3]) for d in descs]
    assert counters_zero(ws, n)
    plan = q4.StepPlan(layers, 1, flags, ws=ws)
    for r in range(5):
        for d in descs:
            d[3].fill_(float("nan"))
        plan.run()
        plan.status()
        for a, d in zip(ref, descs):
            assert np.array_equal(a, host_half(d[3]))
        assert counters_zero(ws, n)
        assert int(ws.view(torch.int32)[1]) == r + 1        # the epoch of launch r + 1


def _m_chain(prefix, M, dims):
    x = dev_half(synth.activations(f"{prefix}/x", 0, M * dims[0]).reshape(M, dims[0]))
    descs, mats = [], []
    for i in range(len(dims) - 1):
        m, W, S = mat(f"{prefix}/{i}", dims[i + 1], dims[i], chain=True)
        y = torch.full((M, dims[i + 1]), float("nan"), dtype=torch.float16, device="cuda")
        descs.append((W, S, x, y))
        mats.append(m)
        x = y
    return descs, mats


@pytest.mark.parametrize("M", [2, 3, 5, 8])
@pytest.mark.parametrize("flags", [q4.STEP_PERSISTENT, q4.STEP_ORDERED | q4.STEP_PERSISTENT, 0],
                         ids=["hazards", "ordered", "auto"])
def test_small_m_dependent_chain(M, flags):
    """M rows per GEMV in one persistent kernel: each descriptor reads the previous
    one's Y; ragged rows (N not a multiple of 16, N < 16) and K from 128 to 8192."""
    # K must be a multiple of 128 for the persistent path: the ragged sizes are on N
    dims = [2048, 6144, 2048, 8192, 384, 1024, 128, 2048]
    descs, mats = _m_chain(f"mchain{M}", M, dims)
    # ragged N on independent tails that read the chain's last Y
    x_last = descs[-1][3]
    for N in (300, 17, 5):
        m, W, S = mat(f"mchain{M}/tail{N}", N, dims[-1], chain=True)
        descs.append((W, S, x_last, torch.full((M, N), float("nan"), dtype=torch.float16,
                                                device="cuda")))
        mats.append(m)
    run_m(descs, M, flags)
    for m, (W, S, X, Y) in zip(mats, descs):
        y = host_half(Y)
        assert np.all(np.isfinite(half_f64(y)))
        assert_gemv_close(y, m.words(), m.scales(), host_half(X))


@pytest.mark.parametrize("M", [2, 5, 8])
@pytest.mark.parametrize("flags", [q4.STEP_PERSISTENT, q4.STEP_ORDERED | q4.STEP_PERSISTENT],
                         ids=["hazards", "ordered"])
def test_small_m_partial_scale_blocks(M, flags):
    """Row lengths whose group count is a multiple of 8 but not of 32 (K 256, 768,
    1280, 2304): the last block of a row's scales is partial, and the list's last
    GEMV ends its matrix mid-tile, so a partial block meets the end of the scales."""
    shapes = [(1000, 256), (333, 768), (4097, 1280), (50, 2304), (77, 768)]
    descs, mats, xs = [], [], []
    for i, (N, K) in enumerate(shapes):
        m, W, S = mat(f"mpart{M}/{i}/{N}x{K}", N, K)
        x = synth.activations(f"mpart{M}/x{i}", 0, M * K).reshape(M, K)
        descs.append((W, S, dev_half(x), torch.full((M, N), float("nan"), dtype=torch.float16,
                                                    device="cuda")))
        mats.append(m)
        xs.append(x)
    run_m(descs, M, flags)
    for m, x, (W, S, X, Y) in zip(mats, xs, descs):
        y = host_half(Y)
        assert np.all(np.isfinite(half_f64(y)))
        assert_gemv_close(y, m.words(), m.scales(), x)


def run_m(descs, M, flags):
    layers = q4.make_layers(descs)
    q4.q4_decode_step(layers, M, flags)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [2, 8])
def test_small_m_matches_batched_calls(M):
    """The persistent small-M path and one q4_gemv_batched call per GEMV agree
    within tolerance on an independent list, and the one-kernel-per-GEMV fallback
    (K not a multiple of 128) is taken for a list that needs it."""
    shapes = [(4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144), (777, 8192), (16, 128)]
    Ks = sorted({K for _, K in shapes})
    xs = {K: dev_half(synth.activations(f"mb{M}/x{K}", 0, M * K).reshape(M, K)) for K in Ks}
    descs, mats = [], []
    for i, (N, K) in enumerate(shapes):
        m, W, S = mat(f"mb{M}/{i}", N, K)
        descs.append((W, S, xs[K], torch.empty((M, N), dtype=torch.float16, device="cuda")))
        mats.append(m)
    run_m(descs, M, 0)
    for m, (W, S, X, Y) in zip(mats, descs):
        ref = q4.q4_gemv_batched(W, S, X)
        torch.cuda.synchronize()
        assert_gemv_close(host_half(Y), m.words(), m.scales(), host_half(X))
        assert_gemv_close(host_half(ref), m.words(), m.scales(), host_half(X))
    # a K that is not a multiple of 128 sends the whole list one kernel per GEMV
    m, W, S = mat(f"mb{M}/odd", 64, 544)
    x = dev_half(synth.activations(f"mb{M}/x544", 0, M * 544).reshape(M, 544))
    y = torch.empty((M, 64), dtype=torch.float16, device="cuda")
    run_m(descs + [(W, S, x, y)], M, 0)
    assert_gemv_close(host_half(y), m.words(), m.scales(), host_half(x))


def test_small_m_workspace_left_clean():
    M = 8
    descs, mats = _m_chain("mclean", M, [2048, 6144, 2048, 8192, 2048])
    layers = q4.make_layers(descs)
    need = q4.q4_decode_step_workspace_bytes(layers, M, q4.STEP_PERSISTENT)
    ws = torch.full((need,), 0x33, dtype=torch.uint8, device="cuda")
    plan = q4.StepPlan(layers, M, q4.STEP_PERSISTENT, ws=ws)
    plan.run()
    plan.status()
    ref = [host_half(d[3]) for d in descs]
    n = len(descs)
    assert counters_zero(ws, n)
    for _ in range(3):
        for d in descs:
            d[3].fill_(float("nan"))
        plan.run()
        plan.status()
        for r, d in zip(ref, descs):
            assert np.array_equal(r, host_half(d[3]))
        assert counters_zero(ws, n)
    for m, (W, S, X, Y) in zip(mats, descs):
        assert_gemv_close(host_half(Y), m.words(), m.scales(), host_half(X))


def test_error_word_is_reported_and_cleared():
    """A nonzero error word in the workspace (as a kernel writes it when a bounded
    wait runs out: code | (GEMV + 1) << 8) makes q4_step_status fail with
    Q4_ERR_TIMEOUT naming the wait and the descriptor, and clears the word."""
    m, W, S = mat("errword/0", 256, 512)
    x = dev_half(synth.activations("errword/x", 0, 512))
    descs = [(W, S, x, torch.empty(256, dtype=torch.float16, device="cuda")),
             (W, S, x, torch.empty(256, dtype=torch.float16, device="cuda"))]
    plan = q4.StepPlan(q4.make_layers(descs), 1, q4.STEP_PERSISTENT)
    plan.run()
    plan.status()                                  # a clean run: no error
    plan.ws.view(torch.int32)[0] = 2 | (2 << 8)    # counter wait, layers[1]
    with pytest.raises(q4.Q4Error) as e:
        plan.status()
    assert e.value.code == 7 and "layers[1]" in e.value.detail
    assert "completion counter" in e.value.detail
    assert int(plan.ws.view(torch.int32)[0]) == 0
    plan.status()                                  # cleared

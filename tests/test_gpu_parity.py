"""Parity of the HIP path with the CPU oracle (needs an MI355X).

Every call goes through the C ABI (libq4f16.so via the thin binding); the oracle
gets the same seeded inputs.  Bars: bit-exact for the codec and the closed forms;
the benchmark spec's tolerance max|y_gpu - y_ref| <= 2e-3 * ||x||_2 * max_n ||W_n||_2 for
GEMV outputs (per input row for M > 1), plus "within one fp16 ulp of the exactly
rounded result, and equal to it for >= 99 % of outputs" where stated.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from conftest import load_golden_cases
from gpuhelp import (Report, assert_gemv_close, assert_within_rounding_bound, dev_half, dev_words,
                     half_f64, host_half,
                     host_words)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()
    yield
    torch.cuda.synchronize()


def rand_case(seed, N, K, M=1, neg=False):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    s = np.abs(rng.standard_normal((N, K // 32)) * 0.01) + 1e-3
    if neg:
        s *= rng.choice([-1.0, 1.0], size=s.shape)
    s = s.astype(np.float16).view(np.uint16)
    x = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    return w, s, x


def gemv_gpu(w, s, x, splits=None):
    W, S, X = dev_words(w), dev_half(s), dev_half(x.reshape(-1))
    if splits is None:
        y = q4.q4_gemv(W, S, X)
    else:
        y = q4.q4_gemv_splitk(W, S, X, splits)
    torch.cuda.synchronize()
    return host_half(y)


# ------------------------------------------------------------------- codec

def test_pack_unpack_small_config_bit_exact():
    c, _, _ = synth.small_config(0)
    words = q4.q4_pack(torch.from_numpy(c).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(host_words(words), oracle.pack(c))
    back = q4.q4_unpack(words)
    assert np.array_equal(back.cpu().numpy(), c)


@pytest.mark.parametrize("N,K,offset", [(1, 32, 0), (3, 96, 1), (17, 544, 3), (256, 4096, 0),
                                        (9, 64, 5)])
def test_pack_unpack_shapes_and_misaligned_codes(N, K, offset):
    c = synth.codes(f"codec/{N}/{K}", 1, N * K).reshape(N, K)
    c[0, :min(K, 8)] |= 0xF0                    # high bits are dropped
    buf = torch.zeros(N * K + offset + 16, dtype=torch.uint8, device="cuda")
    dc = buf[offset:offset + N * K].view(N, K)
    dc.copy_(torch.from_numpy(c))
    words = q4.q4_pack(dc)
    torch.cuda.synchronize()
    assert np.array_equal(host_words(words), oracle.pack(c))
    out = torch.zeros(N * K + offset, dtype=torch.uint8, device="cuda")
    q4.q4_unpack(words, out[offset:].view(N, K))
    torch.cuda.synchronize()
    assert np.array_equal(out[offset:].view(N, K).cpu().numpy(), oracle.unpack(oracle.pack(c)))


def test_unpack_pack_roundtrip_all_words_on_device():
    chunk = 1 << 28
    for c0 in range(0, 1 << 32, chunk):
        w = torch.arange(c0, c0 + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
        w = w.view(chunk // 8, 8)
        codes = q4.q4_unpack(w)
        back = q4.q4_pack(codes)
        assert torch.equal(back, w), hex(c0)
        assert int(codes.max()) <= 15
    # the oracle on a sample of the words
    sample = np.random.default_rng(0).integers(0, 2 ** 32, size=(4096, 8), dtype=np.uint64)
    sample = sample.astype(np.uint32)
    codes = q4.q4_unpack(dev_words(sample))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack(sample))


# -------------------------------------------------------------- M == 1 GEMV

def test_small_config_all_rows():
    c, s, x = synth.small_config(0)
    w = oracle.pack(c)
    assert_gemv_close(gemv_gpu(w, s, x), w, s, x, exact=True)


@pytest.mark.parametrize("case", load_golden_cases("hand_worked_gemv.txt"), ids=lambda c: c["name"])
def test_hand_worked_fixtures_bit_exact(case):
    y = gemv_gpu(case["words"], case["scales"], case["x"])
    assert np.array_equal(y, case["y16"])


def test_closed_forms_bit_exact():
    N, K = 300, 3072
    _, s, x = rand_case(1, N, K, neg=True)
    w7 = np.full((N, K // 8), 0x77777777, np.uint32)
    assert np.all(gemv_gpu(w7, s, x) & 0x7FFF == 0)                   # +-0
    c = synth.codes("cf", 2, N * K).reshape(N, K)
    w = oracle.pack(c)
    ones_s = np.full((N, K // 32), 0x3C00, np.uint16)
    ones_x = np.full(K, 0x3C00, np.uint16)
    expect = (c.astype(np.int64) - 7).sum(1).astype(np.float16).view(np.uint16)
    assert np.array_equal(gemv_gpu(w, ones_s, ones_x), expect)
    for splits in (2, 7, 64):
        assert np.array_equal(gemv_gpu(w, ones_s, ones_x, splits), expect)


def test_one_hot_index_mapping_bit_exact():
    N, K = 37, 160                     # non-square, ragged rows, odd group count
    c = synth.codes("oh", 3, N * K).reshape(N, K)
    w = oracle.pack(c)
    s = synth.scales_uniform("ohs", 3, N * K // 32, 0.005, 0.02).reshape(N, K // 32)
    sv = half_f64(s)
    for k in range(K):
        x = np.zeros(K, np.uint16)
        x[k] = 0x3C00
        expect = ((c[:, k].astype(np.float64) - 7) * sv[:, k // 32]).astype(np.float16)
        assert np.array_equal(gemv_gpu(w, s, x), expect.view(np.uint16)), k


@pytest.mark.parametrize("N", [1, 7, 33, 100, 257, 1031])
@pytest.mark.parametrize("K", [32, 64, 96, 544, 1024, 3072])
def test_random_shapes(N, K):
    w, s, x = rand_case(N * 7 + K, N, K, neg=True)
    assert_gemv_close(gemv_gpu(w, s, x), w, s, x, exact=True)


@pytest.mark.parametrize("N", [33, 1000])
@pytest.mark.parametrize("K", [1536, 2560, 5120, 11264])
def test_groups_per_lane_3_5_6(N, K):
    """Row lengths whose groups split into exactly 3, 5, 5 and 6 per lane of a
    row's team (each an instantiation of its own)."""
    w, s, x = rand_case(N + 3 * K, N, K, neg=True)
    assert_gemv_close(gemv_gpu(w, s, x), w, s, x, exact=True)


def test_subnormal_inputs():
    N, K = 64, 512
    w, s, x = rand_case(5, N, K)
    x = x.copy()
    x[0, ::3] = np.arange(1, 0x400, 6, dtype=np.uint16)[: len(x[0, ::3])]   # subnormal x
    s = s.copy()
    s[:, 1] = 0x0200                                                          # subnormal scale
    assert_gemv_close(gemv_gpu(w, s, x), w, s, x)


@pytest.mark.parametrize("N,K", [(64, 32768), (40, 65536)])
def test_long_rows(N, K):
    w, s, x = rand_case(11, N, K)
    assert_gemv_close(gemv_gpu(w, s, x), w, s, x)


@pytest.mark.parametrize("N,K", [(515, 16384), (70, 12320)])
def test_one_slice_longer_than_the_early_staging_loads(N, K):
    """One K slice of more than 4 x 256 blocks of x: the staging loads each thread's
    first four blocks ahead of the weights and the rest in a loop after them."""
    w, s, x = rand_case(17, N, K, neg=True)
    assert_gemv_close(gemv_gpu(w, s, x, 1), w, s, x, exact=True)


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 13, 32, 64])
def test_splitk_matches_oracle_and_is_deterministic(splits):
    N, K = 515, 8192
    w, s, x = rand_case(13, N, K, neg=True)
    y1 = gemv_gpu(w, s, x, splits)
    assert_gemv_close(y1, w, s, x)
    assert np.array_equal(y1, gemv_gpu(w, s, x, splits))


def test_qkv_projection_full():
    m = synth.Matrix("phi3/L00/qkv", 9216, 3072)
    w, s = m.words(), m.scales()
    x = synth.activations("phi3/x3072", 0, 3072)
    rep = Report()
    assert_gemv_close(gemv_gpu(w, s, x), w, s, x, report=rep)
    print(f"qkv: worst error / tolerance = {rep.worst:.2e}")


def test_mlp_projections_full():
    g = synth.Matrix("phi3/L00/gate_up", 16384, 3072)
    d = synth.Matrix("phi3/L00/down", 3072, 8192)
    x1 = synth.activations("phi3/x3072", 0, 3072)
    x2 = synth.activations("phi3/x8192", 0, 8192)
    for m, x in ((g, x1), (d, x2)):
        w, s = m.words(), m.scales()
        assert_gemv_close(gemv_gpu(w, s, x), w, s, x)


def test_run_to_run_determinism():
    w, s, x = rand_case(17, 4099, 3072)
    a = gemv_gpu(w, s, x)
    for _ in range(3):
        assert np.array_equal(a, gemv_gpu(w, s, x))


# --------------------------------------------------------- M in 2..8 GEMV

def batched_gpu(w, s, X):
    Y = q4.q4_gemv_batched(dev_words(w), dev_half(s), dev_half(X))
    torch.cuda.synchronize()
    return host_half(Y)


@pytest.mark.parametrize("M", [2, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(1, 32), (17, 96), (100, 544), (2048, 2048), (513, 6144)])
def test_batched_vs_oracle(M, N, K):
    w, s, X = rand_case(M * 1000 + N + K, N, K, M=M, neg=True)
    Y = batched_gpu(w, s, X)
    assert Y.shape == (M, N)
    assert_gemv_close(Y, w, s, X, exact=(N * K <= 100_000))


@pytest.mark.parametrize("M", [2, 3])
@pytest.mark.parametrize("N,K", [(9216, 3072), (20000, 544)])
def test_batched_vector_rows_equal_single_gemvs(M, N, K):
    """At two and three rows each row of X runs the single-row GEMV's arithmetic, so
    where both run as one K slice every row of Y is bitwise that GEMV's output; and
    every output within the kernel's rounding bound of the exact product (at least
    99 % exactly rounded)."""
    assert q4.q4_workspace_bytes(M, N, K) == 0 and q4.q4_workspace_bytes(1, N, K) == 0
    w, s, X = rand_case(91 + M + N, N, K, M=M, neg=True)
    Y = batched_gpu(w, s, X)
    for m in range(M):
        assert np.array_equal(Y[m], gemv_gpu(w, s, X[m]))
    y64, y16 = oracle.gemv_exact(w, s, X)
    assert_within_rounding_bound(Y, y64, y16, s, X, "exact", exact_frac=0.99,
                                 what=f"M={M} {N}x{K}")


@pytest.mark.parametrize("M", [3, 8])
def test_batched_mixed_slices(M):
    """Few row tiles, so K is split: slices of 16 and 17 groups, some taken as
    eight-group blocks and some one group per lane."""
    N, K = 40, 6400
    w, s, X = rand_case(77 + M, N, K, M=M, neg=True)
    assert_gemv_close(batched_gpu(w, s, X), w, s, X)


def test_batched_scales_2_byte_aligned():
    """Scales not 16-byte aligned: the one-group-per-lane path, same results."""
    N, K, M = 600, 2048, 4
    w, s, X = rand_case(78, N, K, M=M, neg=True)
    big = torch.zeros(s.size + 8, dtype=torch.int16, device="cuda")
    sv = big[1:1 + s.size]
    sv.copy_(dev_half(s).reshape(-1).view(torch.int16))
    assert sv.data_ptr() % 16 != 0
    Y = q4.q4_gemv_batched(dev_words(w), sv.view(torch.float16).view(N, -1), dev_half(X))
    torch.cuda.synchronize()
    assert_gemv_close(host_half(Y), w, s, X)


def test_batched_rows_equal_single_row_calls_within_tolerance():
    w, s, X = rand_case(21, 300, 2048, M=8)
    Y = batched_gpu(w, s, X)
    for m in range(8):
        ym = gemv_gpu(w, s, X[m])
        tol = 2e-3 * oracle.vec_norm(X[m]) * oracle.row_norms(w, s).max()
        assert np.abs(half_f64(Y[m]) - half_f64(ym)).max() <= tol


def test_batched_closed_forms():
    N, K = 64, 1024
    c = synth.codes("bcf", 4, N * K).reshape(N, K)
    w = oracle.pack(c)
    s = np.full((N, K // 32), 0x3C00, np.uint16)
    X = np.full((8, K), 0x3C00, np.uint16)
    X[3] = 0x4000                                  # 2.0 on row 3
    expect = (c.astype(np.int64) - 7).sum(1)
    Y = batched_gpu(w, s, X)
    for m in range(8):
        e = expect * (2 if m == 3 else 1)
        assert np.array_equal(Y[m], e.astype(np.float16).view(np.uint16)), m


# ------------------------------------------------------------ decode step

def test_decode_step_chain_equals_sequential_calls():
    """x of each descriptor is the previous descriptor's y (a dependent chain)."""
    dims = [3072, 9216, 3072, 16384, 8192, 3072]
    ws, ss, ys = [], [], []
    x0 = dev_half(synth.activations("chain/x", 0, dims[0]))
    for i in range(len(dims) - 1):
        # scales ~ 1/K keep every link's output O(1) (codes have mean 7.5, so an
        # unscaled chain grows geometrically until fp16 overflows)
        m = synth.Matrix(f"chain/{i}", dims[i + 1], dims[i], sigma=2.0 / dims[i],
                         floor=0.5 / dims[i])
        ws.append(dev_words(m.words()))
        ss.append(dev_half(m.scales()))
        ys.append(torch.empty(dims[i + 1], dtype=torch.float16, device="cuda"))
    xs = [x0] + ys[:-1]
    layers = q4.make_layers(zip(ws, ss, xs, ys))
    for flags in (0, q4.STEP_LAUNCH_EACH):
        for y in ys:
            y.zero_()
        q4.q4_decode_step(layers, 1, flags)
        torch.cuda.synchronize()
        got = [host_half(y) for y in ys]
        # the same chain through q4_gemv, one call at a time
        x = x0
        for i in range(len(ws)):
            ref = q4.q4_gemv(ws[i], ss[i], x)
            torch.cuda.synchronize()
            assert np.array_equal(host_half(ref), got[i]), (flags, i)
            x = ref
        # and each link against the oracle, on the input the GPU actually used
        for i in range(len(ws)):
            xin = host_half(xs[i])
            assert_gemv_close(got[i], host_words(ws[i]), host_half(ss[i]), xin)


def _sweep(model, M, rows_per=6, flags=0):
    shapes = synth.sweep_shapes(model)
    K_set = sorted({K for _, _, K in shapes})
    xs = {K: synth.activations(f"{model}/x{K}", 0, M * K).reshape(M, K) for K in K_set}
    dx = {K: dev_half(xs[K] if M > 1 else xs[K][0]) for K in K_set}
    mats, descs = [], []
    for label, N, K in shapes:
        m = synth.Matrix(label, N, K)
        W = m.words_torch("cuda")
        S = dev_half(m.scales())
        Y = torch.empty((M, N) if M > 1 else (N,), dtype=torch.float16, device="cuda")
        mats.append(m)
        descs.append((W, S, dx[K], Y))
    layers = q4.make_layers(descs)
    q4.q4_decode_step(layers, M, flags)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rep = Report()
    for m, (W, S, X, Y) in zip(mats, descs):
        rows = np.unique(np.concatenate([rng.integers(0, m.N, rows_per), [0, m.N - 1]]))
        wr, sr = m.word_rows(rows), m.scale_rows(rows)
        # the device holds the same generated inputs
        assert np.array_equal(host_words(W[torch.from_numpy(rows).cuda()]), wr)
        y = host_half(Y).reshape(M, m.N)[:, rows]
        xh = xs[m.K]
        assert_gemv_close(y if M > 1 else y[0], wr, sr, xh if M > 1 else xh[0], report=rep)
    return rep


def test_phi3_decode_sweep_sampled_rows():
    rep = _sweep("phi3", 1)
    print(f"phi3 sweep: worst error / tolerance = {rep.worst:.2e}")


def test_phi3_decode_sweep_launch_each_sampled_rows():
    _sweep("phi3", 1, rows_per=2, flags=q4.STEP_LAUNCH_EACH)


def test_2b_batched_decode_sweep_sampled_rows():
    rep = _sweep("2b", 8, rows_per=4)
    print(f"2b M=8 sweep: worst error / tolerance = {rep.worst:.2e}")


def test_fp16_overflow_gives_signed_inf():
    # outputs beyond the fp16 range round to +-inf (the oracle's reading of the
    # output rounding), everything else stays within tolerance
    N, K = 64, 4096
    c = np.full((N, K), 15, np.uint8)
    c[N // 2:] = 0
    w = oracle.pack(c)
    s = np.full((N, K // 32), 0x4000, np.uint16)        # 2.0
    x = np.full(K, 0x4400, np.uint16)                   # 4.0: |y| = 8 or 7 * 2 * 4 * 4096
    y = gemv_gpu(w, s, x)
    assert np.all(y[: N // 2] == 0x7C00) and np.all(y[N // 2:] == 0xFC00)
    assert_gemv_close(y, w, s, x)


def test_errors_do_not_launch():
    w, s, x = rand_case(3, 16, 64)
    W, S, X = dev_words(w), dev_half(s), dev_half(x[0])
    Y = torch.zeros(16, dtype=torch.float16, device="cuda")
    lib = q4.load()
    import ctypes as C
    rc = lib.q4_gemv(C.c_void_p(W.data_ptr()), C.c_void_p(S.data_ptr()),
                     C.c_void_p(X.data_ptr()), C.c_void_p(Y.data_ptr()), 16, 48, None, 0, None)
    assert rc == 2
    torch.cuda.synchronize()
    assert torch.count_nonzero(Y) == 0
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_splitk(W, S, X, 8, ws=torch.empty(4, dtype=torch.uint8, device="cuda"))

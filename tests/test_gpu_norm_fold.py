"""The folded residual add + RMSNorm + GEMV (q4_gemv_norm).

Factored (the GEMV of the factored-norm decode step): against the oracle's
unfolded composition, element by element: fp16(res_in + delta) exactly as the
oracle rounds it, and every output within a bound derived from what differs --
the input rounded to fp16 before the norm's scaling instead of after it (one fp16
rounding of each input term on each side), the fp32 GEMV, the fp32 norm scalar,
and the output rounding.

Exact (the default decode step's GEMVs): bitwise the separate entry points
(q4_add_rmsnorm, then q4_gemv and q4_silu_mul) wherever q4_gemv runs as one K
slice, and against the oracle in every case: the residual bitwise, the normalised
vector within one fp16 ulp, every output within the M = 1 GEMV's rounding bound of
the exact product of that vector, at least 99 % exactly rounded."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import (assert_within_rounding_bound, dev_half, dev_words, folded_bound, half_f64,
                     host_half, ulp16)

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def case(label, rows, K, with_delta):
    m = synth.Matrix(label, rows, K)
    w, s = m.words(), m.scales()
    res = synth.activations(label + "/res", 0, K)
    delta = synth.to_half_bits(0.5 * synth.normal(label + "/d", 0, 0, K)) if with_delta else None
    gamma = synth.to_half_bits(1.0 + 0.1 * synth.normal(label + "/g", 0, 0, K))
    return w, s, res, delta, gamma


@pytest.mark.parametrize("rows,K,with_delta", [(3000, 3072, True), (257, 544, False),
                                               (64, 8192, True), (9216, 3072, True)])
def test_plain_matches_unfolded_oracle(rows, K, with_delta):
    w, s, res, delta, gamma = case(f"fold/{rows}x{K}", rows, K, with_delta)
    eps = 1e-5
    res_out = torch.empty(K, dtype=torch.float16, device="cuda")
    y = q4.q4_gemv_norm(dev_words(w), dev_half(s), dev_half(res), dev_half(gamma), eps,
                        delta=dev_half(delta) if delta is not None else None, res_out=res_out)
    torch.cuda.synchronize()
    if delta is not None:
        h_ref, xn = oracle.add_rmsnorm(delta, res, gamma, eps)
    else:
        h_ref, xn = res.copy(), oracle.rmsnorm(res, gamma, eps)
    assert np.array_equal(host_half(res_out), h_ref)          # h rounded once, as the oracle
    y_ref = oracle.gemv_f64(w, s, xn)                         # the unfolded step
    B = folded_bound(w, s, h_ref, gamma, np.float32(eps), y_ref)
    got = half_f64(host_half(y))
    lim = B + 0.5 * ulp16(np.abs(y_ref) + B)
    err = np.abs(got - y_ref)
    assert np.all(err <= lim), (float((err / lim).max()), int(np.argmax(err / lim)))
    # the bound is a real constraint: inside the GEMV tolerance (it is a worst case,
    # linear in the terms' magnitudes; the errors measured are far below it)
    tol = 2e-3 * oracle.vec_norm(xn) * oracle.row_norms(w, s).max()
    assert lim.max() < tol
    print(f"folded {rows}x{K}: worst error / bound {float((err / lim).max()):.3f}, "
          f"bound / tolerance {float(lim.max() / tol):.3f}")


@pytest.mark.parametrize("F,K", [(2048, 3072), (100, 1024)])
def test_glu_matches_unfolded_oracle(F, K):
    """gate/up rows folded with the glue: y = fp16(silu(fp16(gate)) * fp16(up))."""
    w, s, res, delta, gamma = case(f"foldglu/{F}x{K}", 2 * F, K, True)
    eps = 1e-5
    y = q4.q4_gemv_norm(dev_words(w), dev_half(s), dev_half(res), dev_half(gamma), eps,
                        delta=dev_half(delta), glu=True)
    torch.cuda.synchronize()
    h_ref, xn = oracle.add_rmsnorm(delta, res, gamma, eps)
    gu_ref = oracle.gemv_f64(w, s, xn)
    B = folded_bound(w, s, h_ref, gamma, np.float32(eps), gu_ref)
    # gate and up are rounded to fp16 before the glue: each within B + half an ulp
    e = B + 0.5 * ulp16(np.abs(gu_ref) + B)
    g, u = gu_ref[:F], gu_ref[F:]
    eg, eu = e[:F], e[F:]
    sg = g / (1.0 + np.exp(-g))
    want = sg * u
    # |d silu / dg| <= 1.0999; the glue in fp32 (a few roundings) and its fp16 output
    lim = (1.1 * np.abs(u) * eg + (np.abs(sg) + 1.1 * eg) * eu + 8 * U * np.abs(want))
    lim = lim + 0.5 * ulp16(np.abs(want) + lim)
    got = half_f64(host_half(y))
    err = np.abs(got - want)
    assert np.all(err <= lim), (float((err / lim).max()), int(np.argmax(err / lim)))


def _within_one_ulp(got, ref):
    g, r = half_f64(np.asarray(got, np.uint16)), half_f64(np.asarray(ref, np.uint16))
    assert np.all(np.abs(g - r) <= ulp16(np.abs(r)))


@pytest.mark.parametrize("rows,K,with_delta,glu", [
    (9216, 3072, True, False),     # Phi-3 qkv: one K slice, bitwise against q4_gemv
    (32064, 3072, True, False),    # the LM head
    (3000, 3072, False, False),    # a ragged row count, no delta
    (16384, 3072, True, True),     # Phi-3 gate/up with the glue
    (257, 544, True, False),       # q4_gemv splits K here: oracle bound only
    (208, 1024, True, True),       # the same with the glue
    (4096, 8192, True, False),     # a long row: several blocks per thread
])
def test_exact_equals_norm_then_gemv(rows, K, with_delta, glu):
    w, s, res, delta, gamma = case(f"foldx/{rows}x{K}", rows, K, with_delta)
    eps = 1e-5
    dw, ds, dres, dg = dev_words(w), dev_half(s), dev_half(res), dev_half(gamma)
    ddel = dev_half(delta) if delta is not None else None
    res_out = torch.empty(K, dtype=torch.float16, device="cuda")
    y = q4.q4_gemv_norm(dw, ds, dres, dg, eps, delta=ddel, res_out=res_out, glu=glu, exact=True)
    # the separate entry points on the same inputs
    if ddel is not None:
        r2, xn = q4.q4_add_rmsnorm(ddel, dres, dg, eps)
    else:
        r2, xn = dres.clone(), q4.q4_rmsnorm(dres, dg, eps)
    full = torch.empty(rows, dtype=torch.float16, device="cuda")
    ws = torch.empty(max(q4.q4_workspace_bytes(1, rows, K), 16), dtype=torch.uint8, device="cuda")
    q4.q4_gemv(dw, ds, xn, full, ws=ws)
    ref_y = q4.q4_silu_mul(full) if glu else full
    torch.cuda.synchronize()
    one_slice = q4.q4_workspace_bytes(1, rows, K) == 0
    h_ref, xn_ref = (oracle.add_rmsnorm(delta, res, gamma, eps) if delta is not None
                     else (res.copy(), oracle.rmsnorm(res, gamma, eps)))
    assert np.array_equal(host_half(res_out), h_ref)
    assert np.array_equal(host_half(r2), h_ref)
    _within_one_ulp(host_half(xn), xn_ref)
    if one_slice:
        assert np.array_equal(host_half(y), host_half(ref_y).reshape(-1)), \
            "not bitwise the composition"
    # the GEMV on the normalised vector the kernels staged, against the exact oracle
    if glu:
        g16 = host_half(full)
        y64, y16 = oracle.gemv_exact(w, s, host_half(xn))
        assert_within_rounding_bound(g16, y64, y16, s, host_half(xn), "exact", exact_frac=0.99,
                                     what="gate/up")
        if one_slice:
            _within_one_ulp(host_half(y), oracle.silu_mul(g16.reshape(1, -1))[0])
    else:
        y64, y16 = oracle.gemv_exact(w, s, host_half(xn))
        assert_within_rounding_bound(host_half(y), y64, y16, s, host_half(xn), "exact",
                                     exact_frac=0.99, what="exact fold")


def test_exact_limit_and_flags():
    K = 32768                      # 1024 groups: 192 KB of exact staging
    x = torch.zeros(K, dtype=torch.float16, device="cuda")
    w = torch.zeros(4, K // 8, dtype=torch.int32, device="cuda")
    s = torch.zeros(4, K // 32, dtype=torch.float16, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_gemv_norm(w, s, x, x, 1e-5, exact=True)
    assert e.value.code == 6
    # the factored form of the same call fits (64 bytes per group) and gives zeros
    y = q4.q4_gemv_norm(w, s, x, x, 1e-5)
    torch.cuda.synchronize()
    assert not bool(torch.any(y != 0))


def test_argument_errors():
    x = torch.zeros(64, dtype=torch.float16, device="cuda")
    w = torch.zeros(4, 8, dtype=torch.int32, device="cuda")
    s = torch.zeros(4, 2, dtype=torch.float16, device="cuda")
    with pytest.raises(q4.Q4Error):        # res_out aliasing res_in
        q4.q4_gemv_norm(w, s, x, x, 1e-5, res_out=x)
    with pytest.raises(q4.Q4Error):        # a negative epsilon
        q4.q4_gemv_norm(w, s, x, x, -1.0)
    with pytest.raises(q4.Q4Error):        # y overlapping res_in
        q4.q4_gemv_norm(w, s, x, x, 1e-5, y=x[:4])

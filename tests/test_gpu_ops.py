"""The operations around the GEMVs (embedding row, RMSNorm, residual add with
RMSNorm, argmax) against the oracle on the same inputs: bit-exact where one
rounding of an exact value decides (embedding, the residual sum, argmax), within
one fp16 unit in the last place where an fp32 sum of squares feeds the rounding."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import dev_half, dev_words, host_half

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def within_one_ulp(got, ref, min_exact=0.99):
    g = np.asarray(got, np.uint16).reshape(-1)
    r = np.asarray(ref, np.uint16).reshape(-1)
    gf = g.view(np.float16).astype(np.float64)
    rf = r.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(gf), np.isnan(rf))
    ok = ~np.isnan(rf)
    mag = np.abs(rf[ok])
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -14))) - 10)
    assert np.all(np.abs(gf[ok] - rf[ok]) <= ulp)
    assert (g == r).mean() >= min_exact


@pytest.mark.parametrize("N,K", [(32064, 3072), (100, 32)])
def test_embed_rows_bit_exact(N, K):
    m = synth.Matrix(f"ops/emb/{N}", N, K)
    W, S = m.words_torch("cuda"), dev_half(m.scales())
    toks = np.array([0, N - 1, 17 % N, 5 % N, -3, N], np.int32)
    out = q4.q4_embed_rows(W, S, torch.from_numpy(toks).cuda())
    torch.cuda.synchronize()
    # the oracle decodes the same words (generated on the host from the same seed)
    ref = oracle.embed_rows(m.words(), m.scales(), toks)
    assert np.array_equal(host_half(out), ref)


@pytest.mark.parametrize("M,K", [(1, 3072), (3, 8192), (2, 8)])
@pytest.mark.parametrize("eps", [1e-5, 0.25])
def test_rmsnorm(M, K, eps):
    x = synth.activations(f"ops/rms/x{M}x{K}", 0, M * K).reshape(M, K)
    g = synth.activations(f"ops/rms/g{K}", 0, K)
    out = q4.q4_rmsnorm(dev_half(x), dev_half(g), eps)
    torch.cuda.synchronize()
    within_one_ulp(host_half(out), oracle.rmsnorm(x, g, eps))


@pytest.mark.parametrize("inplace", [False, True])
def test_add_rmsnorm(inplace):
    M, K = 2, 3072
    d = synth.activations("ops/add/d", 0, M * K).reshape(M, K)
    r = (synth.activations("ops/add/r", 0, M * K).view(np.float16) * np.float16(40)).view(
        np.uint16).reshape(M, K)
    g = synth.activations("ops/add/g", 0, K)
    D, R, G = dev_half(d), dev_half(r), dev_half(g)
    res_out = R if inplace else torch.empty_like(R)
    res_out, out = q4.q4_add_rmsnorm(D, R, G, 1e-5, res_out=res_out)
    torch.cuda.synchronize()
    ref_res, ref_out = oracle.add_rmsnorm(d, r, g, 1e-5)
    assert np.array_equal(host_half(res_out), ref_res)     # the fp16 sum: rounded once
    within_one_ulp(host_half(out), ref_out)


@pytest.mark.parametrize("M,N", [(3, 1001), (4, 5), (2, 8 * 1024 * 4 + 5), (5, 64)])
def test_argmax_shapes(M, N):
    """Rows not 16-byte aligned (N % 8 != 0), rows shorter than a chunk, a tail
    after the chunks, and ties inside one chunk and across threads."""
    rng = np.random.default_rng(N)
    x = rng.standard_normal((M, N)).astype(np.float16)
    x[0, [N // 2, N - 1]] = np.float16(9.0)                   # tie: lowest index
    if N >= 8:
        x[-1, [1, 2, 7]] = np.float16(9.5)                    # ties inside one chunk
    out = q4.q4_argmax(dev_half(x.view(np.uint16)))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.argmax(x.view(np.uint16)))


def test_argmax_bit_exact():
    rng = np.random.default_rng(11)
    M, N = 6, 32064
    x = rng.standard_normal((M, N)).astype(np.float16)
    x[1, [5, 900, 31000]] = np.float16(65504.0)            # ties: lowest index
    x[2, :] = np.float16(-np.inf)                          # all -inf: index 0
    x[3, ::3] = np.float16(np.nan)                         # NaN skipped
    x[4, :] = np.float16(np.nan)                           # all NaN: 0
    x[5, N - 1] = np.float16(100.0)                        # last element
    out = q4.q4_argmax(dev_half(x.view(np.uint16)))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.argmax(x.view(np.uint16)))

"""Decode tokens end to end (q4_decode_token, q4_decode_tokens): the step composed
from the separate entry points, every intermediate kept and checked against the
oracle on the inputs the GPU read; the driver's logits and token bitwise equal to
that composition (with the norms folded into the GEMVs: within fp16 rounding of
it); and graph replays of several steps equal to the same number of single
steps, replay after replay."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import assert_gemv_close, dev_half, dev_words, host_half
from tokhelp import EPS, Weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()


def within_one_ulp(got, ref):
    g = np.asarray(got, np.uint16).reshape(-1).view(np.float16).astype(np.float64)
    r = np.asarray(ref, np.uint16).reshape(-1).view(np.float16).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -14))) - 10)
    assert np.all(np.abs(g - r) <= ulp)


def composed_step(W, token, check):
    """The decode step from the separate entry points, distinct buffers for every
    intermediate; with `check`, each against the oracle. Returns (logits, token)."""
    D, F = W.D, W.F
    f16 = lambda n: torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")
    tok = torch.tensor([token], dtype=torch.int32, device="cuda")
    keep = []
    res = q4.q4_embed_rows(*W.embed, tok).reshape(-1)
    h = q4.q4_rmsnorm(res, W.blocks[0]["attn_norm"] if W.n else W.final_norm, EPS)
    torch.cuda.synchronize()
    if check:
        m = W.mats["embed"]
        ref = oracle.embed_rows(m.words(), m.scales(), np.array([token], np.int32))[0]
        assert np.array_equal(host_half(res), ref)
        g0 = W.blocks[0]["attn_norm"] if W.n else W.final_norm
        within_one_ulp(host_half(h), oracle.rmsnorm(host_half(res), host_half(g0), EPS))
    for b, B in enumerate(W.blocks):
        qkv, attn, gu, dn = f16(3 * D), f16(D), f16(2 * F), f16(D)
        q4.q4_gemv(*B["qkv"], h, qkv)
        v = qkv[2 * D:]
        q4.q4_gemv(*B["o"], v, attn)
        res2, h2 = q4.q4_add_rmsnorm(attn, res, B["ffn_norm"], EPS)
        q4.q4_gemv(*B["gate_up"], h2, gu)
        hf = q4.q4_silu_mul(gu)
        q4.q4_gemv(*B["down"], hf, dn)
        nxt = W.blocks[b + 1]["attn_norm"] if b + 1 < W.n else W.final_norm
        res3, h3 = q4.q4_add_rmsnorm(dn, res2, nxt, EPS)
        torch.cuda.synchronize()
        if check:
            mm = lambda name: W.mats[f"{b}/{name}"]
            assert_gemv_close(host_half(qkv), mm("qkv").words(), mm("qkv").scales(), host_half(h))
            assert_gemv_close(host_half(attn), mm("o").words(), mm("o").scales(), host_half(v))
            r_ref, h_ref = oracle.add_rmsnorm(host_half(attn), host_half(res),
                                              host_half(B["ffn_norm"]), EPS)
            assert np.array_equal(host_half(res2), r_ref)
            within_one_ulp(host_half(h2), h_ref)
            assert_gemv_close(host_half(gu), mm("gate_up").words(), mm("gate_up").scales(),
                              host_half(h2))
            within_one_ulp(host_half(hf), oracle.silu_mul(host_half(gu).reshape(1, -1))[0])
            assert_gemv_close(host_half(dn), mm("down").words(), mm("down").scales(),
                              host_half(hf))
            r_ref, h_ref = oracle.add_rmsnorm(host_half(dn), host_half(res2), host_half(nxt), EPS)
            assert np.array_equal(host_half(res3), r_ref)
            within_one_ulp(host_half(h3), h_ref)
        keep += [qkv, attn, gu, dn, hf, res2, h2]
        res, h = res3, h3
    logits = f16(W.V)
    q4.q4_gemv(*W.lm_head, h, logits)
    out = q4.q4_argmax(logits)
    torch.cuda.synchronize()
    lg = host_half(logits)
    if check:
        m = W.mats["lm_head"]
        assert_gemv_close(lg, m.words(), m.scales(), host_half(h))
    # the argmax always against the oracle on the logits the GPU produced
    assert int(out.cpu()[0]) == int(oracle.argmax(lg.reshape(1, -1))[0])
    return lg, int(out.cpu()[0])


@pytest.fixture(scope="module")
def small():
    return Weights("small", 3, 256, 512, 1000)


@pytest.fixture(scope="module")
def mid():
    """D 1024, FFN 2048, vocabulary 3000: every normed projection needs a split-K
    pass, so the driver runs each residual add + RMSNorm as its own kernel (and the
    glue after the gate/up GEMV)."""
    return Weights("mid", 2, 1024, 2048, 3000)


@pytest.fixture(scope="module")
def mixed():
    """D 2048, FFN 2048, vocabulary 1000: qkv and gate/up fold their norms, the LM
    head (split-K) takes the separate norm kernel."""
    return Weights("mixed", 2, 2048, 2048, 1000)


@pytest.mark.parametrize("model", ["small", "mid", "mixed"])
def test_step_matches_composition_and_oracle(request, model):
    W = request.getfixturevalue(model)
    split = lambda N, K: q4.q4_workspace_bytes(1, N, K) > 0
    if model == "mid":      # the premise: the separate norm kernels run
        assert split(3 * W.D, W.D) and split(2 * W.F, W.D) and split(W.V, W.D)
    if model == "mixed":
        assert not split(3 * W.D, W.D) and not split(2 * W.F, W.D) and split(W.V, W.D)
    lg_ref, t_ref = composed_step(W, 17, check=True)
    tin = torch.tensor([17], dtype=torch.int32, device="cuda")
    tout = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    logits = torch.empty(W.V, dtype=torch.float16, device="cuda")
    q4.q4_decode_token(W.model, tin, tout, logits)
    torch.cuda.synchronize()
    assert np.array_equal(host_half(logits), lg_ref)
    assert int(tout.cpu()[0]) == t_ref


@pytest.fixture(scope="module")
def wide():
    """Phi-3 width (D 3072, FFN 8192): wide enough that no projection needs a
    split-K pass, so the driver runs the glue and the norms inside the GEMVs."""
    return Weights("wide", 2, 3072, 8192, 2048, host=False)


@pytest.mark.parametrize("model", ["small", "wide"])
@pytest.mark.parametrize("graph", [True, False], ids=["graph", "eager"])
@pytest.mark.parametrize("folded", [False, True], ids=["norms", "folded"])
def test_multi_step_equals_single_steps(request, model, graph, folded):
    W = request.getfixturevalue(model)
    Wm = W.fmodel if folded else W.model
    steps = 6
    # single steps, host round trip between them
    ws = torch.empty(q4.q4_decode_token_workspace_bytes(Wm), dtype=torch.uint8, device="cuda")
    seq = [5]
    for _ in range(steps):
        tin = torch.tensor([seq[-1]], dtype=torch.int32, device="cuda")
        tout = torch.empty(1, dtype=torch.int32, device="cuda")
        q4.q4_decode_token(Wm, tin, tout, ws=ws)
        torch.cuda.synchronize()
        seq.append(int(tout.cpu()[0]))
    # the same steps in one call, twice (a graph is replayed again), with eager
    # work and synchronisation in between
    tokens = torch.full((steps + 1,), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    g = q4.TokensGraph(Wm, tokens, ws=ws, stream=stream) if graph else None
    try:
        for rep in range(3):
            tokens.fill_(-1)
            tokens[0] = seq[0]
            torch.cuda.synchronize()
            if graph:
                g.run(steps, stream=stream)
            else:
                q4.q4_decode_tokens(Wm, tokens, steps, ws=ws, stream=stream)
            torch.cuda.synchronize()
            assert tokens.cpu().tolist() == seq, rep
            junk = torch.randn(1 << 16, device="cuda").sum()    # eager work between replays
            torch.cuda.synchronize()
            del junk
    finally:
        if g is not None:
            g.close()
    # and the sequence is a chain of argmaxes: recompute the last step by composition
    if not folded:
        lg, t = composed_step(W, seq[-2], check=False)
        assert t == seq[-1]


@pytest.mark.parametrize("model", ["small", "wide"])
def test_factored_norm_close_to_composition(request, model):
    """Norms folded into the GEMVs they feed: the logits within fp16 rounding of
    the unfolded composition's, and the token the oracle's argmax of the folded
    logits."""
    W = request.getfixturevalue(model)
    for token in (17, 901):
        lg_ref, _ = composed_step(W, token, check=False)
        tin = torch.tensor([token], dtype=torch.int32, device="cuda")
        tout = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        logits = torch.empty(W.V, dtype=torch.float16, device="cuda")
        q4.q4_decode_token(W.fmodel, tin, tout, logits)
        torch.cuda.synchronize()
        got = host_half(logits).view(np.float16).astype(np.float64)
        ref = lg_ref.view(np.float16).astype(np.float64)
        assert np.all(np.isfinite(got))
        # Folding changes one fp16 rounding per normalised input (the vector is
        # rounded after the gamma product instead of after the full
        # normalisation), ~2^-11 relative per element; with random-sign terms a
        # GEMV output moves by the same relative order, and over these few blocks
        # the logits stayed within 2^-10 of the largest one (measured); the bound
        # is 2^-8 of it.
        assert np.abs(got - ref).max() <= 2.0 ** -8 * np.abs(ref).max()
        assert int(tout.cpu()[0]) == int(oracle.argmax(host_half(logits).reshape(1, -1))[0])


def test_phi3_shaped_step():
    """Two blocks at Phi-3 sizes (D 3072, FFN 8192, vocabulary 32064): the driver's
    logits equal the composition's bitwise; the token is the oracle's argmax of them."""
    W = Weights("phi3", 2, 3072, 8192, 32064, host=False)
    lg_ref, t_ref = composed_step(W, 1234, check=False)
    tin = torch.tensor([1234], dtype=torch.int32, device="cuda")
    tout = torch.empty(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(W.V, dtype=torch.float16, device="cuda")
    q4.q4_decode_token(W.model, tin, tout, logits)
    torch.cuda.synchronize()
    assert np.array_equal(host_half(logits), lg_ref)
    assert int(tout.cpu()[0]) == t_ref
    assert np.all(np.isfinite(host_half(logits).view(np.float16)))

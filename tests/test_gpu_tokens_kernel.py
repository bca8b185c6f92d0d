"""The whole-token persistent kernel (q4_tokens_plan_init, q4_tokens_run): every
stage of the last step checked against the oracle on the inputs the GPU handed
over (the tagged pairs stay in the workspace): o and down as GEMVs of their
tagged input under the kernel's rounding bound; the normalised stages (qkv,
gate/up with the SiLU-multiply, the LM head) against the oracle's unfolded
add + RMSNorm + GEMV of the residual stream rebuilt on the host from the same
tagged values, under the folded-norm bound; the token the oracle's argmax of the
logits.  Several steps in one launch equal the same steps one launch each, and
the logits agree with the multi-kernel factored-norm step within rounding."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import (assert_within_rounding_bound, folded_bound, half_f64, host_half, ulp16)
from tokhelp import EPS, Weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4.load()
    oracle.set_threads(min(16, __import__("os").cpu_count() or 1))


@pytest.fixture(scope="module")
def small():
    return Weights("small", 3, 256, 512, 1000)


@pytest.fixture(scope="module")
def wide():
    """Phi-3 widths (D 3072, FFN 8192) with two blocks and a short vocabulary."""
    return Weights("wide", 2, 3072, 8192, 2048)


def run_tokens(W, token, steps=1, plan=None, logits=True):
    plan = plan or q4.TokensPlan(W.fmodel)
    tokens = torch.full((steps + 1,), -1, dtype=torch.int32, device="cuda")
    tokens[0] = token
    lg = torch.empty(W.V, dtype=torch.float16, device="cuda") if logits else None
    plan.run(tokens, steps, logits=lg)
    torch.cuda.synchronize()
    plan.status()
    return plan, tokens.cpu().tolist(), (host_half(lg) if logits else None)


def check_normed(m, h_bits, gamma_bits, got_bits, rows=None, what=""):
    """A folded-norm GEMV's outputs against the oracle's unfolded RMSNorm + GEMV."""
    w, s = m.words(), m.scales()
    if rows is not None:
        w, s = w[rows], s[rows]
    xn = oracle.rmsnorm(h_bits, gamma_bits, EPS)
    y_ref = oracle.gemv_f64(w, s, xn)
    B = folded_bound(w, s, h_bits, gamma_bits, np.float32(EPS), y_ref, kind="sub")
    lim = B + 0.5 * ulp16(np.abs(y_ref) + B)
    err = np.abs(half_f64(got_bits) - y_ref)
    assert np.all(err <= lim), (what, float((err / lim).max()), int(np.argmax(err / lim)))
    return float((err / lim).max())


def check_glu(m, h_bits, gamma_bits, got_bits, F, what=""):
    """gate/up folded with the glue: fp16(silu(fp16(gate)) * fp16(up))."""
    w, s = m.words(), m.scales()
    xn = oracle.rmsnorm(h_bits, gamma_bits, EPS)
    gu = oracle.gemv_f64(w, s, xn)
    B = folded_bound(w, s, h_bits, gamma_bits, np.float32(EPS), gu, kind="sub")
    e = B + 0.5 * ulp16(np.abs(gu) + B)
    g, u, eg, eu = gu[:F], gu[F:], e[:F], e[F:]
    sg = g / (1.0 + np.exp(-g))
    want = sg * u
    lim = 1.1 * np.abs(u) * eg + (np.abs(sg) + 1.1 * eg) * eu + 8 * 2.0 ** -24 * np.abs(want)
    lim = lim + 0.5 * ulp16(np.abs(want) + lim)
    err = np.abs(half_f64(got_bits) - want)
    assert np.all(err <= lim), (what, float((err / lim).max()), int(np.argmax(err / lim)))


def check_step(W, plan, token, logits):
    """Every stage of the last step run with `plan` (input token `token`)."""
    D, F = W.D, W.F
    act = plan.activation
    m = W.mats
    epochs = set()
    res = oracle.embed_rows(m["embed"].words(), m["embed"].scales(),
                            np.array([token], np.int32))[0]
    for b in range(W.n):
        g_attn = host_half(W.blocks[b]["attn_norm"])
        g_ffn = host_half(W.blocks[b]["ffn_norm"])
        if b > 0:
            res, _ = oracle.add_rmsnorm(act(q4.TOKENS_DOWN, b - 1), res, g_attn, EPS)
            epochs |= set(plan.last_epochs.tolist())
        v = act(q4.TOKENS_V, b)
        epochs |= set(plan.last_epochs.tolist())
        check_normed(m[f"{b}/qkv"], res, g_attn, v, rows=np.arange(2 * D, 3 * D),
                     what=f"qkv v rows, block {b}")
        if b == W.n - 1:
            check_normed(m[f"{b}/qkv"], res, g_attn, act(q4.TOKENS_QK),
                         rows=np.arange(0, 2 * D), what=f"qkv q/k rows, block {b}")
        o = act(q4.TOKENS_O, b)
        epochs |= set(plan.last_epochs.tolist())
        y64, y16 = oracle.gemv_exact(m[f"{b}/o"].words(), m[f"{b}/o"].scales(), v)
        assert_within_rounding_bound(o, y64, y16, m[f"{b}/o"].scales(), v, "sub",
                                     exact_frac=0.97, what=f"o, block {b}")
        res, _ = oracle.add_rmsnorm(o, res, g_ffn, EPS)
        h = act(q4.TOKENS_H, b)
        epochs |= set(plan.last_epochs.tolist())
        check_glu(m[f"{b}/gate_up"], res, g_ffn, h, F, what=f"gate/up, block {b}")
        dn = act(q4.TOKENS_DOWN, b)
        epochs |= set(plan.last_epochs.tolist())
        y64, y16 = oracle.gemv_exact(m[f"{b}/down"].words(), m[f"{b}/down"].scales(), h)
        assert_within_rounding_bound(dn, y64, y16, m[f"{b}/down"].scales(), h, "sub",
                                     exact_frac=0.97, what=f"down, block {b}")
    if W.n:
        res, _ = oracle.add_rmsnorm(act(q4.TOKENS_DOWN, W.n - 1), res, host_half(W.final_norm),
                                    EPS)
    check_normed(m["lm_head"], res, host_half(W.final_norm), logits, what="LM head")
    # every tagged pair of the step carries the step's one epoch
    assert len(epochs) <= 1 and 0 not in epochs, epochs


@pytest.mark.parametrize("model", ["small", "wide"])
def test_every_stage_against_the_oracle(request, model):
    W = request.getfixturevalue(model)
    for token in (17, 901):
        plan, toks, lg = run_tokens(W, token)
        check_step(W, plan, token, lg)
        assert toks[1] == int(oracle.argmax(lg.reshape(1, -1))[0])


def test_last_step_of_several_against_the_oracle(small):
    """Four steps in one launch: the last step's stages from the third token."""
    W = small
    plan, toks, lg = run_tokens(W, 5, steps=4)
    check_step(W, plan, toks[3], lg)
    assert toks[4] == int(oracle.argmax(lg.reshape(1, -1))[0])


@pytest.mark.parametrize("model", ["small", "wide"])
def test_steps_in_one_launch_equal_single_launches(request, model):
    W = request.getfixturevalue(model)
    plan = q4.TokensPlan(W.fmodel)
    seq = [7]
    for _ in range(6):
        _, toks, _ = run_tokens(W, seq[-1], plan=plan, logits=False)
        seq.append(toks[1])
    for rep in range(3):      # the same plan again: the epoch carries over
        _, toks, _ = run_tokens(W, 7, steps=6, plan=plan, logits=False)
        assert toks == seq, rep


@pytest.mark.parametrize("model", ["small", "wide"])
def test_logits_close_to_the_multi_kernel_factored_step(request, model):
    """Same factored-norm step as q4_decode_token with Q4_MODEL_FACTORED_NORM; the
    dot products are summed in another order, so within rounding, not bitwise."""
    W = request.getfixturevalue(model)
    for token in (3, 250):
        _, toks, lg = run_tokens(W, token)
        tin = torch.tensor([token], dtype=torch.int32, device="cuda")
        tout = torch.empty(1, dtype=torch.int32, device="cuda")
        ref = torch.empty(W.V, dtype=torch.float16, device="cuda")
        q4.q4_decode_token(W.fmodel, tin, tout, ref)
        torch.cuda.synchronize()
        a, r = half_f64(lg), half_f64(host_half(ref))
        assert np.all(np.isfinite(a))
        assert np.abs(a - r).max() <= 2.0 ** -9 * np.abs(r).max()


def test_phi3_shaped_model():
    """Two blocks at Phi-3 sizes with the full vocabulary (32064 logits): every
    stage against the oracle, two steps in one launch."""
    W = Weights("phi3k", 2, 3072, 8192, 32064)
    plan, toks, lg = run_tokens(W, 1234, steps=2)
    check_step(W, plan, toks[1], lg)
    assert toks[2] == int(oracle.argmax(lg.reshape(1, -1))[0])


def test_out_of_vocabulary_token_gives_nan_logits_and_token_0(small):
    """An embedding row outside the table is NaN (as q4_embed_rows): every logit
    is NaN and the argmax of a NaN row is 0."""
    W = small
    _, toks, lg = run_tokens(W, W.V + 5)
    assert np.all(np.isnan(half_f64(lg)))
    assert toks[1] == 0


def test_error_word_names_the_stage(small):
    """A bounded wait that ran out (the word written from the host here) is
    reported once, naming the whole-token kernel and the stage, then cleared."""
    plan = q4.TokensPlan(small.fmodel)
    word = torch.tensor([0x84 | (3 << 8)], dtype=torch.int32, device="cuda")
    plan.ws[:4].copy_(word.view(torch.uint8))
    torch.cuda.synchronize()
    with pytest.raises(q4.Q4Error) as ei:
        plan.status()
    assert ei.value.code == 7
    assert "whole-token kernel" in str(ei.value) and "stage 2" in str(ei.value)
    plan.status()


def test_shape_limits_and_arguments(small):
    W = small
    big = Weights("big", 1, 4128, 256, 64, host=False)
    assert q4.q4_tokens_workspace_bytes(big.fmodel) == 0
    with pytest.raises(q4.Q4Error):
        q4.TokensPlan(big.fmodel)
    plan = q4.TokensPlan(W.fmodel)
    with pytest.raises(q4.Q4Error):
        plan.run(None, 1)
    tokens = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(q4.Q4Error):
        plan.run(tokens, -1)
    assert plan.offset(q4.TOKENS_V, W.n) == -1
    assert plan.offset(9) == -1


def test_no_blocks_and_odd_vocabulary():
    """A model with no blocks (the LM head reads the normalised embedding row
    itself) and an odd vocabulary (the last logit pair half filled): the logits
    against the oracle, the token the oracle's argmax, three steps equal to three
    single launches."""
    W = Weights("noblk", 0, 256, 512, 999)
    plan, toks, lg = run_tokens(W, 42)
    check_step(W, plan, 42, lg)
    assert toks[1] == int(oracle.argmax(lg.reshape(1, -1))[0])
    seq = [42]
    for _ in range(3):
        _, t, _ = run_tokens(W, seq[-1], plan=plan, logits=False)
        seq.append(t[1])
    _, t3, _ = run_tokens(W, 42, steps=3, plan=plan, logits=False)
    assert t3 == seq

"""q4_gemv_batched_noalloc: the allocation-free variant of q4_gemv_batched.

Its split-K partials live in the library's static device array instead of a
caller workspace.  Two calls in a row (the second smaller, so stale partials of
the first would show) must equal q4_gemv_batched with a workspace bit for bit
and the oracle within the GEMV tolerance; a shape whose partials exceed the
array is refused before anything is enqueued.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
import bit_weight_streaming_q4f16_amd as q4
from gpuhelp import assert_gemv_close, dev_half, dev_words, host_half

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    q4.load()


def _case(label, M, N, K):
    m = synth.Matrix(label, N, K)
    X = synth.activations(label + "/X", 0, M * K).reshape(M, K)
    return m.words(), m.scales(), X


def _run_both(w, s, X):
    M, K = X.shape
    N = w.shape[0]
    need = q4.q4_workspace_bytes(M, N, K)
    assert 0 < need <= q4.Q4_NOALLOC_SCRATCH_BYTES, "the shape must use split-K partials"
    dw, ds, dX = dev_words(w), dev_half(s), dev_half(X)
    Y_ref = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    Y_na = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    q4.q4_gemv_batched(dw, ds, dX, Y_ref)
    q4.q4_gemv_batched_noalloc(dw, ds, dX, Y_na)
    torch.cuda.synchronize()
    return host_half(Y_ref), host_half(Y_na)


def test_two_calls_in_a_row_second_smaller():
    cases = [("noalloc/a", 8, 1200, 4096), ("noalloc/b", 3, 200, 2048)]
    for label, M, N, K in cases:
        print(f"case {label} M={M} N={N} K={K}", flush=True)
        w, s, X = _case(label, M, N, K)
        y_ref, y_na = _run_both(w, s, X)
        assert np.array_equal(y_na, y_ref), f"{label}: differs from q4_gemv_batched"
        assert_gemv_close(y_na, w, s, X)


def test_m1_split_k():
    print("case noalloc/m1 M=1 N=96 K=8192", flush=True)
    w, s, X = _case("noalloc/m1", 1, 96, 8192)
    y_ref, y_na = _run_both(w, s, X)
    assert np.array_equal(y_na, y_ref)
    assert_gemv_close(y_na, w, s, X)


def test_oversized_plan_refused():
    # partials of 4 * splits * M * N bytes beyond the array: refused on the host,
    # before any launch (the pointers are never dereferenced)
    M, N, K = 8, 65536, 32768
    assert q4.q4_workspace_bytes(M, N, K) > q4.Q4_NOALLOC_SCRATCH_BYTES
    lib = q4.load()
    base = 1 << 44
    rc = lib.q4_gemv_batched_noalloc(C.c_void_p(base), C.c_void_p(base + (1 << 36)),
                                     C.c_void_p(base + (2 << 36)), C.c_void_p(base + (3 << 36)),
                                     M, N, K, None)
    assert rc == 4, rc
    assert b"static scratch" in lib.q4_last_error()

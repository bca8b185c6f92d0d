"""Python binding of the q4f16_1 decode library (include/q4f16.h).

Argument marshalling only: every function takes torch tensors on the GPU,
checks dtype / device / contiguity / shape, and calls the C ABI entry point of
the same name on the current HIP stream.  Every step of the computation runs in
the HIP kernels of libq4f16.so; there is no fallback.  If the library is not
built, loading fails with an error that says how to build it.

Tensor conventions: packed words are int32 tensors holding uint32 bit patterns
([N][K/8]); scales, activations and outputs are float16 tensors ([N][K/32],
[K] or [M][K], [N] or [M][N]); codes are uint8 ([N][K]).
"""
from __future__ import annotations

import ctypes as C
import os
import threading

__all__ = [
    "Q4Error", "load", "lib_path", "q4_version", "q4_pack", "q4_unpack", "q4_gemv",
    "q4_gemv_splitk", "q4_gemv_batched", "q4_gemv_batched_noalloc", "q4_workspace_bytes", "q4_splitk_workspace_bytes",
    "q4_decode_step", "q4_decode_step_workspace_bytes", "q4_probe_read", "q4_probe_copy",
    "Layer", "STEP_LAUNCH_EACH", "STEP_ORDERED", "StepPlan", "make_layers",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "_lib", "libq4f16.so")
_lock = threading.Lock()
_lib = None

Q4_NOALLOC_SCRATCH_BYTES = 4 * 1024 * 1024   # include/q4f16.h
STEP_LAUNCH_EACH = 0x1
STEP_ORDERED = 0x2
STEP_PERSISTENT = 0x10
X_PLAIN = 0
X_SILU_MUL = 1
FMT_Q3F16_1 = 1
FMT_Q4F32_1 = 2
FMT_AF4_G64 = 3       # bf16 scales and biases (the pages' MLX affine format)
FMT_AF4_G64_F16 = 4   # the same with fp16 scales and biases (extra variant)
FMT_LOAD_STAGED = 0x100   # OR-ed into FMT_Q3F16_1: force one way of loading
FMT_LOAD_DIRECT = 0x200
MODEL_FACTORED_NORM = 0x1   # q4_model.options: norms folded into the GEMVs they feed
NORM_GLU = 0x1              # q4_gemv_norm flags
NORM_EXACT = 0x2

STATUS = {0: "Q4_OK", 1: "Q4_ERR_NULL", 2: "Q4_ERR_SHAPE", 3: "Q4_ERR_ALIGN",
          4: "Q4_ERR_WORKSPACE", 5: "Q4_ERR_DEVICE", 6: "Q4_ERR_UNSUPPORTED", 7: "Q4_ERR_TIMEOUT"}


class Q4Error(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        self.name = STATUS.get(code, f"Q4_ERR_{code}")
        self.detail = detail
        super().__init__(f"{self.name}: {detail}")


class Layer(C.Structure):
    """q4_layer: one GEMV of a decode step (device pointers and sizes)."""
    _fields_ = [("words", C.c_void_p), ("scales", C.c_void_p), ("x", C.c_void_p),
                ("y", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64),
                ("x_op", C.c_uint32), ("format", C.c_uint32), ("biases", C.c_void_p)]


class Weight(C.Structure):
    """q4_weight: one q4f16_1 matrix in device memory."""
    _fields_ = [("words", C.c_void_p), ("scales", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64)]


class Block(C.Structure):
    """q4_block: one transformer block (attention at a single position)."""
    _fields_ = [("qkv", Weight), ("o", Weight), ("gate_up", Weight), ("down", Weight),
                ("attn_norm", C.c_void_p), ("ffn_norm", C.c_void_p)]


class ModelDesc(C.Structure):
    """q4_model."""
    _fields_ = [("n_blocks", C.c_int64), ("D", C.c_int64), ("F", C.c_int64), ("V", C.c_int64),
                ("embed", Weight), ("blocks", C.c_void_p), ("final_norm", C.c_void_p),
                ("lm_head", Weight), ("eps", C.c_float), ("options", C.c_uint32)]


def lib_path() -> str:
    return _LIB


def load():
    """Load libq4f16.so (built by __graft_entry__.build() or
    ``python -m bit_weight_streaming_q4f16_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: build it with "
                               "`python -m bit_weight_streaming_q4f16_amd.build`")
        lib = C.CDLL(_LIB)
        p, i64, sz, i32 = C.c_void_p, C.c_int64, C.c_size_t, C.c_int
        sigs = {
            "q4_status_str": ([i32], C.c_char_p),
            "q4_last_error": ([], C.c_char_p),
            "q4_version": ([], i32),
            "q4_pack": ([p, p, i64, i64, p], i32),
            "q4_unpack": ([p, p, i64, i64, p], i32),
            "q4_gemv": ([p, p, p, p, i64, i64, p, sz, p], i32),
            "q4_gemv_splitk": ([p, p, p, p, i64, i64, i64, p, sz, p], i32),
            "q4_gemv_batched": ([p, p, p, p, i64, i64, i64, p, sz, p], i32),
            "q4_gemv_batched_noalloc": ([p, p, p, p, i64, i64, i64, p], i32),
            "q4_workspace_bytes": ([i64, i64, i64], sz),
            "q4_splitk_workspace_bytes": ([i64, i64, i64], sz),
            "q4_last_error_detail": ([], C.c_char_p),
            "q4_step_plan_bytes": ([i64], sz),
            "q4_decode_step_workspace_bytes": ([p, i64, i64, C.c_uint32], sz),
            "q4_step_plan_init": ([p, i64, i64, C.c_uint32, p, sz, p, sz, p], i32),
            "q4_step_run": ([p, p, sz, p], i32),
            "q4_step_status": ([p, p], i32),
            "q4_decode_step": ([p, i64, i64, p, sz, p], i32),
            "q4_decode_step_flags": ([p, i64, i64, C.c_uint32, p, sz, p], i32),
            "q4_silu_mul": ([p, p, i64, i64, p], i32),
            "q4_embed_rows": ([p, p, i64, i64, p, i64, p, p], i32),
            "q4_rmsnorm": ([p, p, C.c_float, i64, i64, p, p], i32),
            "q4_add_rmsnorm": ([p, p, p, C.c_float, i64, i64, p, p, p], i32),
            "q4_argmax": ([p, i64, i64, p, p], i32),
            "q4_gemv_norm": ([p, p, p, p, p, C.c_float, p, p, i64, i64, C.c_uint32, p], i32),
            "q4_gemv_format": ([C.c_uint32, p, p, p, p, p, i64, i64, p], i32),
            "q4_format_weight_bytes": ([C.c_uint32, i64, i64], sz),
            "q4_decode_token_workspace_bytes": ([p], sz),
            "q4_decode_token": ([p, p, p, p, p, sz, p], i32),
            "q4_decode_tokens": ([p, p, i64, p, sz, p], i32),
            "q4_tokens_graph_create": ([p, p, p, sz, p, C.POINTER(p)], i32),
            "q4_tokens_graph_run": ([p, i64, p], i32),
            "q4_tokens_graph_destroy": ([p], i32),
            "q4_tokens_plan_bytes": ([], sz),
            "q4_tokens_workspace_bytes": ([p], sz),
            "q4_tokens_plan_init": ([p, p, sz, p, sz, p], i32),
            "q4_tokens_run": ([p, p, i64, p, p], i32),
            "q4_tokens_ws_offset": ([p, C.c_uint32, i64], i64),
            "q4_probe_read": ([p, sz, p, i64, p], i32),
            "q4_probe_copy": ([p, p, sz, p], i32),
        }
        for name, (args, res) in sigs.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
        return lib


def _check(rc: int):
    if rc != 0:
        raise Q4Error(rc, load().q4_last_error_detail().decode())


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t, name, dtype):
    if t is None:
        raise Q4Error(1, f"{name} is None")
    if not t.is_cuda:
        raise Q4Error(5, f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise Q4Error(2, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise Q4Error(2, f"{name} must be contiguous")
    return t


def _ws(nbytes, ws, device):
    torch = _torch()
    if nbytes == 0:
        return ws, (ws.numel() * ws.element_size() if ws is not None else 0)
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def q4_version() -> int:
    return load().q4_version()


def q4_pack(codes, words=None, stream=None):
    """codes uint8 [N][K] -> words int32 [N][K/8] (uint32 bit patterns)."""
    torch = _torch()
    _dev(codes, "codes", torch.uint8)
    N, K = codes.shape
    if words is None:
        words = torch.empty((N, K // 8), dtype=torch.int32, device=codes.device)
    _dev(words, "words", torch.int32)
    _check(load().q4_pack(_ptr(codes), _ptr(words), N, K, _stream(stream)))
    return words


def q4_unpack(words, codes=None, stream=None):
    """words int32 [N][K/8] -> codes uint8 [N][K]."""
    torch = _torch()
    _dev(words, "words", torch.int32)
    N, K8 = words.shape
    if codes is None:
        codes = torch.empty((N, 8 * K8), dtype=torch.uint8, device=words.device)
    _dev(codes, "codes", torch.uint8)
    _check(load().q4_unpack(_ptr(words), _ptr(codes), N, 8 * K8, _stream(stream)))
    return codes


def q4_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().q4_workspace_bytes(M, N, K))


def q4_splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    return int(load().q4_splitk_workspace_bytes(M, N, splits))


def _gemv_shapes(words, scales):
    torch = _torch()
    _dev(words, "words", torch.int32)
    _dev(scales, "scales", torch.float16)
    N, K8 = words.shape
    K = 8 * K8
    if tuple(scales.shape) != (N, K // 32):
        raise Q4Error(2, f"scales shape {tuple(scales.shape)} != {(N, K // 32)}")
    return N, K


def q4_gemv(words, scales, x, y=None, ws=None, stream=None):
    """y[N] = dequant(words, scales) @ x[K] (fp16 out, fp32 accumulation)."""
    torch = _torch()
    N, K = _gemv_shapes(words, scales)
    _dev(x, "x", torch.float16)
    if x.numel() != K:
        raise Q4Error(2, f"x has {x.numel()} elements, K = {K}")
    if y is None:
        y = torch.empty(N, dtype=torch.float16, device=words.device)
    _dev(y, "y", torch.float16)
    ws, wsb = _ws(q4_workspace_bytes(1, N, K), ws, words.device)
    _check(load().q4_gemv(_ptr(words), _ptr(scales), _ptr(x), _ptr(y), N, K, _ptr(ws), wsb,
                          _stream(stream)))
    return y


def q4_gemv_splitk(words, scales, x, splits: int, y=None, ws=None, stream=None):
    torch = _torch()
    N, K = _gemv_shapes(words, scales)
    _dev(x, "x", torch.float16)
    if y is None:
        y = torch.empty(N, dtype=torch.float16, device=words.device)
    _dev(y, "y", torch.float16)
    ws, wsb = _ws(q4_splitk_workspace_bytes(1, N, splits), ws, words.device)
    _check(load().q4_gemv_splitk(_ptr(words), _ptr(scales), _ptr(x), _ptr(y), N, K, splits,
                                 _ptr(ws), wsb, _stream(stream)))
    return y


def q4_gemv_batched(words, scales, X, Y=None, ws=None, stream=None):
    """Y[M][N] = X[M][K] @ dequant(words, scales)^T for M <= 8."""
    torch = _torch()
    N, K = _gemv_shapes(words, scales)
    _dev(X, "X", torch.float16)
    if X.dim() != 2 or X.shape[1] != K:
        raise Q4Error(2, f"X shape {tuple(X.shape)} must be [M][{K}]")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=words.device)
    _dev(Y, "Y", torch.float16)
    ws, wsb = _ws(q4_workspace_bytes(M, N, K), ws, words.device)
    _check(load().q4_gemv_batched(_ptr(words), _ptr(scales), _ptr(X), _ptr(Y), M, N, K,
                                  _ptr(ws), wsb, _stream(stream)))
    return Y


def q4_gemv_batched_noalloc(words, scales, X, Y=None, stream=None):
    """q4_gemv_batched without a workspace: split-K partials in the library's
    static device array (nothing is allocated by the call; Y is allocated here
    only when not given)."""
    torch = _torch()
    N, K = _gemv_shapes(words, scales)
    _dev(X, "X", torch.float16)
    if X.dim() != 2 or X.shape[1] != K:
        raise Q4Error(2, f"X shape {tuple(X.shape)} must be [M][{K}]")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=words.device)
    _dev(Y, "Y", torch.float16)
    _check(load().q4_gemv_batched_noalloc(_ptr(words), _ptr(scales), _ptr(X), _ptr(Y), M, N, K,
                                          _stream(stream)))
    return Y


def make_layers(descs):
    """descs: iterable of (words, scales, x, y), (words, scales, x, y, x_op),
    (words, scales, x, y, x_op, format) or (words, scales, x, y, x_op, format,
    biases) tensors -> ctypes array of Layer.  K follows from the words' row
    length: 8 per word (q4f16_1, the affine formats) or 32 per three words
    (format FMT_Q3F16_1).  biases: the affine formats' [N][K/64] tensor."""
    descs = list(descs)
    arr = (Layer * len(descs))()
    for i, d in enumerate(descs):
        w, s, x, y = d[:4]
        x_op = d[4] if len(d) > 4 else X_PLAIN
        fmt = d[5] if len(d) > 5 else 0
        b = d[6] if len(d) > 6 else None
        N, RW = w.shape
        K = RW * 32 // 3 if fmt == FMT_Q3F16_1 else 8 * RW
        arr[i] = Layer(w.data_ptr(), s.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, x_op, fmt,
                       None if b is None else b.data_ptr())
    return arr


def q4_decode_step_workspace_bytes(layers, M: int = 1, flags: int = 0) -> int:
    return int(load().q4_decode_step_workspace_bytes(layers, len(layers), M, flags))


def q4_decode_step(layers, M: int = 1, flags: int = 0, ws=None, ws_bytes=None, stream=None,
                   check: bool = True):
    """Plan and run the GEMVs of a Layer array (see make_layers) in order, in one
    call (q4_decode_step_flags); returns the workspace.  check: then wait for the
    stream and raise if a persistent kernel's bounded wait ran out
    (q4_step_status)."""
    torch = _torch()
    need = q4_decode_step_workspace_bytes(layers, M, flags)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    wsb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().q4_decode_step_flags(layers, len(layers), M, flags, _ptr(ws), wsb,
                                       _stream(stream)))
    if check:
        q4_step_status(ws, stream)
    return ws


def q4_step_status(ws, stream=None):
    """Wait for the stream and raise Q4Error(Q4_ERR_TIMEOUT) if a bounded wait in a
    persistent decode-step kernel ran out since the last check."""
    _check(load().q4_step_status(_ptr(ws), _stream(stream)))


class StepPlan:
    """A planned decode-step list (q4_step_plan_init): the plan in host memory, the
    workspace on the device, the descriptors kept alive.  run() enqueues one step
    (q4_step_run), status() checks the error word (q4_step_status)."""

    def __init__(self, layers, M: int = 1, flags: int = 0, ws=None, stream=None, keep=None):
        torch = _torch()
        lib = load()
        n = len(layers)
        self.layers, self.keep, self.M, self.flags = layers, keep, M, flags
        self.plan = C.create_string_buffer(int(lib.q4_step_plan_bytes(n)))
        self.ws_bytes = q4_decode_step_workspace_bytes(layers, M, flags)
        if ws is None:
            ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")
        self.ws = ws
        self._ws_ptr = _ptr(ws)
        self._ws_len = ws.numel() * ws.element_size()
        _check(lib.q4_step_plan_init(layers, n, M, flags, self.plan, len(self.plan),
                                     self._ws_ptr, self._ws_len, _stream(stream)))

    def run(self, stream=None):
        _check(load().q4_step_run(self.plan, self._ws_ptr, self._ws_len, _stream(stream)))

    def run_raw(self, stream_ptr):
        """q4_step_run with the stream given as a ctypes pointer (no Python-side
        conversions: what the host spends per step is the C call)."""
        return load().q4_step_run(self.plan, self._ws_ptr, self._ws_len, stream_ptr)

    def status(self, stream=None):
        q4_step_status(self.ws, stream)


def q4_silu_mul(gu, out=None, stream=None):
    """fp16 [M][2H] (gate | up) -> fp16 [M][H] = fp16(silu(gate) * up)."""
    torch = _torch()
    g = gu if gu.dim() == 2 else gu.reshape(1, -1)
    M, H2 = g.shape
    H = H2 // 2
    if out is None:
        out = torch.empty((M, H) if gu.dim() == 2 else (H,), dtype=torch.float16, device=gu.device)
    _check(load().q4_silu_mul(_ptr(gu), _ptr(out), M, H, _stream(stream)))
    return out


def q4_embed_rows(words, scales, tokens, out=None, stream=None):
    """Dequantised rows tokens[m] (int32 device tensor) of a q4f16_1 table."""
    torch = _torch()
    N, K = words.shape[0], 8 * words.shape[1]
    M = tokens.numel()
    if out is None:
        out = torch.empty((M, K), dtype=torch.float16, device=words.device)
    _check(load().q4_embed_rows(_ptr(words), _ptr(scales), N, K, _ptr(tokens), M, _ptr(out),
                                _stream(stream)))
    return out


def q4_rmsnorm(x, gamma, eps: float, out=None, stream=None):
    torch = _torch()
    K = gamma.numel()
    M = x.numel() // K
    if out is None:
        out = torch.empty_like(x)
    _check(load().q4_rmsnorm(_ptr(x), _ptr(gamma), float(eps), M, K, _ptr(out), _stream(stream)))
    return out


def q4_add_rmsnorm(delta, res_in, gamma, eps: float, res_out=None, out=None, stream=None):
    """(res_out, out): res_out = res_in + delta, out = RMSNorm(res_out) * gamma."""
    torch = _torch()
    K = gamma.numel()
    M = delta.numel() // K
    if res_out is None:
        res_out = torch.empty_like(res_in)
    if out is None:
        out = torch.empty_like(res_in)
    _check(load().q4_add_rmsnorm(_ptr(delta), _ptr(res_in), _ptr(gamma), float(eps), M, K,
                                 _ptr(res_out), _ptr(out), _stream(stream)))
    return res_out, out


def q4_gemv_norm(words, scales, res_in, gamma, eps: float, delta=None, res_out=None, y=None,
                 glu: bool = False, exact: bool = False, stream=None):
    """y = W . RMSNorm(fp16(res_in + delta)) * gamma in one kernel (q4_gemv_norm);
    exact: the normalised input staged as q4_rmsnorm forms it, else the norm's
    scalar applied after the product; glu: W holds gate | up rows and
    y = fp16(silu(gate) * up)."""
    torch = _torch()
    rows, K = words.shape[0], 8 * words.shape[1]
    N = rows // 2 if glu else rows
    if y is None:
        y = torch.empty(N, dtype=torch.float16, device=words.device)
    _check(load().q4_gemv_norm(_ptr(words), _ptr(scales), _ptr(res_in), _ptr(delta), _ptr(gamma),
                               float(eps), _ptr(res_out), _ptr(y), N, K,
                               (NORM_GLU if glu else 0) | (NORM_EXACT if exact else 0),
                               _stream(stream)))
    return y


def q4_argmax(x, out=None, stream=None):
    """int32 [M]: index of the largest value per row (ties: lowest; NaN skipped)."""
    torch = _torch()
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    M, N = x2.shape
    if out is None:
        out = torch.empty(M, dtype=torch.int32, device=x.device)
    _check(load().q4_argmax(_ptr(x), M, N, _ptr(out), _stream(stream)))
    return out


def _weight(ws):
    w, sc = ws
    return Weight(w.data_ptr(), sc.data_ptr(), w.shape[0], 8 * w.shape[1])


class Model:
    """A q4_model for q4_decode_token(s): keeps every tensor it points at alive.

    embed, lm_head: (words, scales); blocks: sequence of dicts with keys qkv, o,
    gate_up, down ((words, scales) each), attn_norm, ffn_norm (fp16 tensors)."""

    def __init__(self, embed, blocks, final_norm, lm_head, eps: float = 1e-5, options: int = 0):
        self._keep = [embed, blocks, final_norm, lm_head]
        blocks = list(blocks)
        self.blocks = (Block * max(len(blocks), 1))()
        for i, b in enumerate(blocks):
            self.blocks[i] = Block(_weight(b["qkv"]), _weight(b["o"]), _weight(b["gate_up"]),
                                   _weight(b["down"]), b["attn_norm"].data_ptr(),
                                   b["ffn_norm"].data_ptr())
        D = embed[0].shape[1] * 8
        F = blocks[0]["down"][0].shape[1] * 8 if blocks else 32
        V = embed[0].shape[0]
        self.desc = ModelDesc(len(blocks), D, F, V, _weight(embed),
                              C.cast(self.blocks, C.c_void_p).value if blocks else None,
                              final_norm.data_ptr(), _weight(lm_head), eps, options)
        self.D, self.F, self.V = D, F, V

    def ref(self):
        return C.byref(self.desc)


def q4_decode_token_workspace_bytes(model: Model) -> int:
    return int(load().q4_decode_token_workspace_bytes(model.ref()))


def q4_decode_token(model: Model, token_in, token_out, logits=None, ws=None, stream=None):
    """One decode step: token_in[0] -> token_out[0] (int32 device tensors)."""
    torch = _torch()
    need = q4_decode_token_workspace_bytes(model)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _check(load().q4_decode_token(model.ref(), _ptr(token_in), _ptr(token_out), _ptr(logits),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4_decode_tokens(model: Model, tokens, steps: int, ws=None, stream=None):
    """`steps` decode steps: tokens[i] -> tokens[i + 1] (int32 device tensor)."""
    torch = _torch()
    need = q4_decode_token_workspace_bytes(model)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _check(load().q4_decode_tokens(model.ref(), _ptr(tokens), steps, _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return ws


class TokensGraph:
    """q4_tokens_graph: one decode step captured on `stream` (not the null stream)
    and replayed per token by run(); close() destroys it (after the caller has
    synchronised the streams it ran on)."""

    def __init__(self, model: Model, tokens, ws=None, stream=None):
        torch = _torch()
        self.model, self.tokens = model, tokens
        need = q4_decode_token_workspace_bytes(model)
        self.ws = ws if ws is not None else torch.empty(need, dtype=torch.uint8, device="cuda")
        h = C.c_void_p()
        _check(load().q4_tokens_graph_create(model.ref(), _ptr(tokens), _ptr(self.ws),
                                             self.ws.numel(), _stream(stream), C.byref(h)))
        self.handle = h

    def run(self, steps: int, stream=None):
        _check(load().q4_tokens_graph_run(self.handle, steps, _stream(stream)))

    def close(self):
        if self.handle:
            _check(load().q4_tokens_graph_destroy(self.handle))
            self.handle = None


TOKENS_QK, TOKENS_V, TOKENS_O, TOKENS_H, TOKENS_DOWN, TOKENS_LOGITS = range(6)


def q4_tokens_workspace_bytes(model: Model) -> int:
    return int(load().q4_tokens_workspace_bytes(model.ref()))


class TokensPlan:
    """The whole-token persistent kernel (q4_tokens_plan_init): the plan in host
    memory, the workspace on the device.  run() enqueues `steps` decode steps
    (q4_tokens_run), status() checks the error word (q4_step_status), and
    activation() reads one of the last step's activations back from the
    workspace (q4_tokens_ws_offset)."""

    def __init__(self, model: Model, ws=None, stream=None):
        torch = _torch()
        lib = load()
        self.model = model
        self.plan = C.create_string_buffer(int(lib.q4_tokens_plan_bytes()))
        need = q4_tokens_workspace_bytes(model)
        if need == 0:
            _check(lib.q4_tokens_plan_init(model.ref(), self.plan, len(self.plan), None, 0,
                                           _stream(stream)))
        self.ws = ws if ws is not None else torch.empty(need, dtype=torch.uint8, device="cuda")
        _check(lib.q4_tokens_plan_init(model.ref(), self.plan, len(self.plan), _ptr(self.ws),
                                       self.ws.numel(), _stream(stream)))

    def run(self, tokens, steps: int, logits=None, stream=None):
        _check(load().q4_tokens_run(self.plan, _ptr(tokens), steps, _ptr(logits),
                                    _stream(stream)))

    def run_raw(self, tokens_ptr, steps: int, stream_ptr):
        """q4_tokens_run with ctypes pointers (what the host spends is the C call)."""
        return load().q4_tokens_run(self.plan, tokens_ptr, steps, None, stream_ptr)

    def status(self, stream=None):
        q4_step_status(self.ws, stream)

    def offset(self, what: int, block: int = 0) -> int:
        return int(load().q4_tokens_ws_offset(self.plan, what, block))

    def activation(self, what: int, block: int = 0):
        """The last step's values of one stage as fp16 bits (numpy uint16): q/k rows,
        logits, or a block's tagged pairs unpacked (epochs in self.last_epochs)."""
        import numpy as np
        off = self.offset(what, block)
        if off < 0:
            raise Q4Error(2, f"no activation {what} for block {block}")
        D, F, V = self.model.D, self.model.F, self.model.V
        n = {TOKENS_QK: 2 * D, TOKENS_LOGITS: V, TOKENS_V: D, TOKENS_O: D, TOKENS_H: F,
             TOKENS_DOWN: D}[what]
        if what in (TOKENS_QK, TOKENS_LOGITS):
            return self.ws[off: off + 2 * n].cpu().numpy().view(np.uint16).copy()
        words = self.ws[off: off + 4 * n].cpu().numpy().view(np.uint32).reshape(-1, 2)
        self.last_epochs = words[:, 1].copy()
        return words[:, 0].copy().view(np.uint16)[:n]


def q4_gemv_format(fmt: int, words, scales, x, K: int, biases=None, y=None, stream=None):
    """y = W x for a format variant (FMT_*); words: int32 tensor of the format's
    layout with N rows; K the logical row length."""
    torch = _torch()
    N = words.shape[0]
    if y is None:
        y = torch.empty(N, dtype=torch.float32 if (fmt & 0xFF) == FMT_Q4F32_1 else torch.float16,
                        device=words.device)
    _check(load().q4_gemv_format(fmt, _ptr(words), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y),
                                 N, K, _stream(stream)))
    return y


def q4_format_weight_bytes(fmt: int, N: int, K: int) -> int:
    return int(load().q4_format_weight_bytes(fmt, N, K))


def q4_probe_read(buf, sink, blocks: int = 0, stream=None):
    _check(load().q4_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), blocks,
                                _stream(stream)))


def q4_probe_copy(src, dst, stream=None):
    _check(load().q4_probe_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                                _stream(stream)))

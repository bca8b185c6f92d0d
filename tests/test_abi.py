"""The C-ABI library: it loads, exports every symbol include/q4f16.h declares,
and rejects bad arguments on the host before touching a device (no GPU needed,
no compute call)."""
import ctypes as C
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

import bit_weight_streaming_q4f16_amd as q4

HEADER = os.path.join(ROOT, "include", "q4f16.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"Q4_API\s+[\w\s\*]*?\b(q4_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q4.lib_path()):
        from bit_weight_streaming_q4f16_amd import build
        build.build()
    return q4.load()


def test_header_declares_the_path():
    syms = declared_symbols()
    for name in ["q4_pack", "q4_unpack", "q4_gemv", "q4_gemv_splitk", "q4_gemv_batched",
                 "q4_decode_step", "q4_workspace_bytes", "q4_status_str", "q4_last_error_detail",
                 "q4_step_plan_bytes", "q4_step_plan_init", "q4_step_run", "q4_step_status"]:
        assert name in syms


# HIP runtime calls that allocate or free device or pinned memory, create
# streams, or wait for the whole device: no entry point may make them
FORBIDDEN = ("hipMalloc", "hipFree", "hipHostMalloc", "hipHostFree", "hipHostRegister",
             "hipMallocAsync", "hipFreeAsync", "hipMallocManaged", "hipExtMallocWithFlags",
             "hipDeviceSynchronize", "hipStreamCreate", "hipStreamCreateWithFlags",
             "hipStreamCreateWithPriority", "hipStreamDestroy", "hipMemset", "hipMemsetAsync",
             "hipMemcpy", "hipEventSynchronize", "hipDeviceReset")


def test_library_links_no_allocation_or_device_wide_wait(lib):
    """The library imports no HIP routine that allocates, frees, creates a stream
    or synchronises the device: no call path can (hipStreamSynchronize and
    hipMemcpyAsync are there for q4_step_status alone, which waits for one
    stream to read the error word)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", q4.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    imported = {l.split()[-1].split("@")[0] for l in out.splitlines() if l.strip()}
    hip = {f for f in imported if f.startswith("hip")}
    assert not (hip & set(FORBIDDEN)), sorted(hip & set(FORBIDDEN))
    assert hip <= {"hipDeviceGetAttribute", "hipFuncSetAttribute", "hipGetDevice",
                   "hipGetErrorString", "hipGetLastError", "hipGetSymbolAddress",
                   "hipGraphDestroy", "hipGraphExecDestroy", "hipGraphInstantiate",
                   "hipGraphLaunch", "hipLaunchCooperativeKernel", "hipLaunchKernel",
                   "hipMemcpyAsync", "hipOccupancyMaxActiveBlocksPerMultiprocessor",
                   "hipStreamBeginCapture", "hipStreamEndCapture", "hipStreamSynchronize"}, hip


CITES = ("Zero TVM", "everything-webgpu", "Splash", "Model Artifact Manifest",
         "MobileTransformers", "callers that cannot")


def test_every_export_cites_a_passage_or_its_callers():
    """The comment above each declaration in the header cites a page (by its
    title, with the section) or, for the allocation-free entry point, names the
    callers it is for.  Declarations with no comment of their own share the one
    above them."""
    text = open(HEADER).read()
    decls = [(m.start(), m.end(), m.group(1)) for m in
             re.finditer(r"Q4_API\s+[\w\s\*]*?\b(q4_\w+)\s*\(", text)]
    assert len(decls) >= 30
    prev_end, window = 0, ""
    for start, end, name in decls:
        gap = text[prev_end:start]
        if "/*" in gap:
            window = " ".join(gap.replace("*", " ").split())
        assert any(k in window for k in CITES), name
        prev_end = text.index(";", end)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", q4.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [s for s in declared_symbols() if s not in exported]
    assert not missing, missing
    for s in declared_symbols():
        assert hasattr(lib, s)
    # nothing but the C ABI leaks out under a q4_ prefix
    extra = [s for s in exported if s.startswith("q4_") and s not in declared_symbols()]
    assert not extra, extra


def test_layer_struct_matches_header():
    # four pointers, two int64, two uint32, the biases pointer
    assert C.sizeof(q4.Layer) == 64
    text = open(HEADER).read()
    body = re.search(r"typedef struct q4_layer \{(.*?)\} q4_layer;", text, re.S).group(1)
    fields = re.findall(r"\b(words|scales|x|y|N|K|x_op|format|biases)\s*;", body)
    assert fields == [f[0] for f in q4.Layer._fields_]
    for name, val in (("Q4_X_PLAIN", q4.X_PLAIN), ("Q4_X_SILU_MUL", q4.X_SILU_MUL)):
        m = re.search(r"#define %s (\w+)u" % name, text)
        assert m and int(m.group(1), 0) == val, name


def test_status_strings(lib):
    for code, name in q4.STATUS.items():
        assert lib.q4_status_str(code).decode() == name
    assert lib.q4_status_str(99).decode() == "Q4_ERR_UNKNOWN"
    assert lib.q4_version() >= 100


P = C.c_void_p
A = P(0x10000)      # aligned fake device addresses: never dereferenced by these calls
B = P(0x20000)
X = P(0x30000)
Y = P(0x40000)


def _err(lib):
    return lib.q4_last_error_detail().decode()


def test_gemv_argument_errors(lib):
    f = lib.q4_gemv
    assert f(None, B, X, Y, 16, 64, None, 0, None) == 1 and "words" in _err(lib)
    assert f(A, None, X, Y, 16, 64, None, 0, None) == 1 and "scales" in _err(lib)
    assert f(A, B, None, Y, 16, 64, None, 0, None) == 1 and "x" in _err(lib)
    assert f(A, B, X, None, 16, 64, None, 0, None) == 1 and "y" in _err(lib)
    assert f(A, B, X, Y, 0, 64, None, 0, None) == 2 and "N = 0" in _err(lib)
    assert f(A, B, X, Y, 16, 48, None, 0, None) == 2 and "K = 48" in _err(lib)
    assert f(A, B, X, Y, 16, 0, None, 0, None) == 2
    assert f(A, B, X, Y, 16, -32, None, 0, None) == 2
    assert f(P(0x10004), B, X, Y, 16, 64, None, 0, None) == 3 and "words" in _err(lib)
    assert f(A, B, P(0x30008), Y, 16, 64, None, 0, None) == 3 and "x" in _err(lib)
    assert f(A, P(0x20001), X, Y, 16, 64, None, 0, None) == 3 and "scales" in _err(lib)
    assert f(A, B, X, P(0x40001), 16, 64, None, 0, None) == 3 and "y" in _err(lib)
    # output overlapping an input
    assert f(A, B, X, P(0x10000 + 64), 16, 64, None, 0, None) == 2 and "overlap" in _err(lib)
    assert f(A, B, X, Y, 1 << 40, 64, None, 0, None) == 6


def test_batched_and_splitk_argument_errors(lib):
    assert lib.q4_gemv_batched(A, B, X, Y, 0, 16, 64, None, 0, None) == 2 and "M = 0" in _err(lib)
    assert lib.q4_gemv_batched(A, B, X, Y, 9, 16, 64, None, 0, None) == 2
    assert lib.q4_gemv_splitk(A, B, X, Y, 16, 64, 0, None, 0, None) == 2
    assert lib.q4_gemv_splitk(A, B, X, Y, 16, 64, 3, None, 0, None) == 2   # 3 > K/32
    assert lib.q4_gemv_splitk(A, B, X, Y, 16, 8192, 65, None, 0, None) == 2
    assert lib.q4_splitk_workspace_bytes(1, 100, 4) == 1600
    assert lib.q4_splitk_workspace_bytes(8, 100, 4) == 12800
    assert lib.q4_splitk_workspace_bytes(1, 100, 1) == 0
    assert lib.q4_workspace_bytes(1, 16, 48) == 0


def test_gemv_norm_argument_errors(lib):
    f = lib.q4_gemv_norm
    G = P(0x50000)
    # flags and pointers are checked before any device query: no GPU needed
    assert f(A, B, X, None, G, 1e-5, None, Y, 16, 64, 4, None) == 2 and "flags" in _err(lib)
    assert f(A, B, X, None, None, 1e-5, None, Y, 16, 64, 2, None) == 1
    text = open(HEADER).read()
    for name, val in (("Q4_NORM_GLU", q4.NORM_GLU), ("Q4_NORM_EXACT", q4.NORM_EXACT)):
        m = re.search(r"#define %s (\w+)u" % name, text)
        assert m and int(m.group(1), 0) == val, name


def test_noalloc_gemv_argument_errors(lib):
    f = lib.q4_gemv_batched_noalloc
    f.argtypes = [C.c_void_p] * 4 + [C.c_int64] * 3 + [C.c_void_p]
    f.restype = C.c_int
    # argument errors come before any device query: they need no GPU
    assert f(None, B, X, Y, 1, 16, 64, None) == 1 and "words" in _err(lib)
    assert f(A, B, X, Y, 9, 16, 64, None) == 2 and "M = 9" in _err(lib)
    assert f(A, B, X, Y, 1, 16, 48, None) == 2
    assert f(A, B, P(0x30008), Y, 1, 16, 64, None) == 3


def test_codec_argument_errors(lib):
    assert lib.q4_pack(None, A, 4, 64, None) == 1
    assert lib.q4_pack(X, None, 4, 64, None) == 1
    assert lib.q4_pack(X, A, 4, 40, None) == 2
    assert lib.q4_pack(X, P(0x10004), 4, 64, None) == 3
    assert lib.q4_unpack(A, None, 4, 64, None) == 1
    assert lib.q4_unpack(P(0x10008), X, 4, 64, None) == 3


def test_decode_step_validates_every_descriptor_first(lib):
    layers = (q4.Layer * 3)()
    layers[0] = q4.Layer(0x10000, 0x20000, 0x30000, 0x40000, 16, 64)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x40000, 0x70000, 16, 64)
    layers[2] = q4.Layer(0x80000, 0x90000, 0x70000, 0xA0000, 16, 40)   # bad K
    assert lib.q4_decode_step_flags(layers, 3, 1, 0, None, 0, None) == 2
    assert "layers[2]" in _err(lib)
    assert lib.q4_decode_step_flags(None, 3, 1, 0, None, 0, None) == 1
    assert lib.q4_decode_step_flags(layers, 0, 1, 0, None, 0, None) == 2
    assert lib.q4_decode_step_flags(layers, 2, 9, 0, None, 0, None) == 2
    assert lib.q4_decode_step_flags(layers, 2, 1, 0x80, None, 0, None) == 2 and "flags" in _err(lib)


def test_decode_step_x_op_errors(lib):
    layers = (q4.Layer * 2)()
    layers[0] = q4.Layer(0x10000, 0x20000, 0x30000, 0x40000, 16, 64, 0, 0)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x40000, 0x70000, 16, 64, 2, 0)   # unknown x_op
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 2
    assert "layers[1]" in _err(lib) and "x_op" in _err(lib)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x40000, 0x70000, 16, 64, 1, 7)   # unknown format
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 2 and "format" in _err(lib)
    # q3f16_1 at M > 1
    layers[1] = q4.Layer(0x50000, 0x60000, 0x90000, 0xA0000, 16, 64, 0, q4.FMT_Q3F16_1)
    assert lib.q4_decode_step_flags(layers, 2, 2, 0, None, 0, None) == 6 and "M = 1" in _err(lib)
    # q3f16_1 words need 4-byte alignment only; 2-byte aligned words fail
    layers[1] = q4.Layer(0x50002, 0x60000, 0x90000, 0xA0000, 16, 64, 0, q4.FMT_Q3F16_1)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 3 and "4-byte" in _err(lib)
    # with the glue, x spans 2K: a y inside that span overlaps it
    layers[1] = q4.Layer(0x50000, 0x60000, 0x80000, 0x80000 + 2 * 64 + 16, 16, 64, 1, 0)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 2 and "overlap" in _err(lib)


def test_decode_step_affine_layer_errors(lib):
    """The affine formats in a layer list: biases required (and only for them), K a
    multiple of 64, M = 1, 2-byte aligned biases, no overlap of y with the biases."""
    layers = (q4.Layer * 2)()
    layers[0] = q4.Layer(0x10000, 0x20000, 0x30000, 0x40000, 16, 128, 0, 0)
    AF = q4.FMT_AF4_G64
    layers[1] = q4.Layer(0x50000, 0x60000, 0x30000, 0x70000, 16, 128, 0, AF, None)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 1 and "biases" in _err(lib)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x30000, 0x70000, 16, 128, 0, 0, 0x68000)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 2 and "biases" in _err(lib)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x30000, 0x70000, 16, 96, 0, AF, 0x68000)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 2 and "64" in _err(lib)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x90000, 0xA0000, 16, 128, 0, AF, 0x68000)
    assert lib.q4_decode_step_flags(layers, 2, 2, 0, None, 0, None) == 6 and "M = 1" in _err(lib)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x30000, 0x70000, 16, 128, 0, q4.FMT_AF4_G64_F16,
                         0x68001)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 3 and "biases" in _err(lib)
    # y inside the biases ([16][2] bf16 = 64 bytes from 0x68000)
    layers[1] = q4.Layer(0x50000, 0x60000, 0x30000, 0x68020, 16, 128, 0, AF, 0x68000)
    assert lib.q4_decode_step_flags(layers, 2, 1, 0, None, 0, None) == 2 and "overlap" in _err(lib)


def test_silu_mul_argument_errors(lib):
    f = lib.q4_silu_mul
    assert f(None, Y, 1, 64, None) == 1
    assert f(X, None, 1, 64, None) == 1
    assert f(X, Y, 0, 64, None) == 2
    assert f(X, Y, 1, 60, None) == 2 and "H" in _err(lib)
    assert f(P(0x30008), Y, 1, 64, None) == 3
    assert f(X, P(0x40008), 1, 64, None) == 3
    assert f(X, P(0x30000 + 128), 1, 64, None) == 2 and "overlap" in _err(lib)
    assert f(X, Y, 1 << 20, 1 << 12, None) == 6


def test_probe_argument_errors(lib):
    assert lib.q4_probe_read(None, 16, A, 0, None) == 1
    assert lib.q4_probe_read(A, 20, X, 0, None) == 2
    assert lib.q4_probe_copy(A, P(0x10010), 64, None) == 2       # overlap
    assert lib.q4_probe_copy(A, P(0x20008), 64, None) == 3


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(q4, "_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(q4, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        q4.load()


STRUCTS = {"q4_layer": "Layer", "q4_weight": "Weight", "q4_block": "Block", "q4_model": "ModelDesc"}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_struct_layouts_match_the_header(tmp_path):
    """sizeof and every field offset of the header's structs, as gcc lays them out,
    equal the binding's ctypes mirrors."""
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "q4f16.h"', 'int main(void) {']
    for cname, pyname in STRUCTS.items():
        py = getattr(q4, pyname)
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), "-o", str(exe), str(src)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}
    for cname, pyname in STRUCTS.items():
        py = getattr(q4, pyname)
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_token_argument_errors(lib):
    m = q4.ModelDesc()
    assert lib.q4_decode_token(None, X, Y, None, A, 1 << 20, None) == 1
    m.n_blocks, m.D, m.F, m.V = 0, 48, 64, 10      # D not a multiple of 32
    assert lib.q4_decode_token(C.byref(m), X, Y, None, A, 1 << 20, None) == 2 and "D" in _err(lib)
    m.D, m.n_blocks = 64, 1
    assert lib.q4_decode_token(C.byref(m), X, Y, None, A, 1 << 20, None) == 2   # blocks NULL
    assert "blocks" in _err(lib)
    m.n_blocks = 0
    assert lib.q4_decode_token(C.byref(m), X, Y, None, A, 1 << 20, None) == 1   # weights NULL
    m.embed = q4.Weight(0x10000, 0x20000, 10, 64)
    m.lm_head = q4.Weight(0x30000, 0x40000, 11, 64)                            # wrong N
    m.final_norm = 0x50000
    assert lib.q4_decode_token(C.byref(m), X, Y, None, A, 1 << 20, None) == 2
    assert "lm_head" in _err(lib)
    m.lm_head = q4.Weight(0x30000, 0x40000, 10, 64)
    assert lib.q4_decode_tokens(C.byref(m), None, 4, A, 1 << 20, None) == 1
    assert lib.q4_decode_tokens(C.byref(m), X, -1, A, 1 << 20, None) == 2
    h = C.c_void_p()
    assert lib.q4_tokens_graph_create(C.byref(m), X, A, 1 << 20, None, C.byref(h)) == 2
    assert "null stream" in _err(lib) and not h.value
    assert lib.q4_tokens_graph_run(None, 4, None) == 1
    assert lib.q4_tokens_graph_destroy(None) == 0
    assert lib.q4_decode_token_workspace_bytes(None) == 0

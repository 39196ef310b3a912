"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, sizes the packed triple as documented, and rejects bad
arguments before touching any device (no compute call needs a GPU here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slim.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slim_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from sparse_int4_gemm_amd import _lib
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for f in ("slim_pack", "slim_linear", "slim_linear_batched", "slim_linear_workspace_bytes"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"libslim.so does not export {name}"
    from sparse_int4_gemm_amd import _lib
    assert set(_declared_functions()) == set(_lib.EXPORTED)


def test_sizes(lib):
    from sparse_int4_gemm_amd import _lib
    assert lib.slim_version() == 1
    assert _lib.slim_values_bytes(4096, 4096) == 4096 * 4096 // 4
    assert _lib.slim_meta_bytes(4096, 11008) == 4096 * 11008 // 8
    assert _lib.slim_scales_bytes(11008, 4096) == 11008 * 32 * 2
    assert _lib.slim_values_bytes(16, 100) == 0          # K not a multiple of 128
    assert _lib.slim_scales_bytes(16, 128, 64) == 0       # only group 128
    ws = _lib.slim_linear_workspace_bytes(16, 4096, 4096, 416)
    assert ws % 256 == 0 and ws >= 16 * 416 * 4
    # Every shape the calls accept has a size, degenerate ones included.
    for M, N, K, r in [(0, 4096, 4096, 416), (1, 16, 128, 0), (256, 4096, 4096, 416), (2048, 4096, 11008, 416),
                       (100000, 16, 128, 32), (17, 11008, 4096, 416)]:
        w = _lib.slim_linear_workspace_bytes(M, N, K, r)
        assert w % 256 == 0 and w >= M * r * 2


def test_status_strings(lib):
    for s in range(4):
        assert lib.slim_status_string(s)
    assert lib.slim_status_string(99) == b"unknown slim_status"


# Fake, aligned, never-dereferenced addresses: every call below must fail in
# validation, before any HIP call.
P = 0x10000


def _lin(lib, **kw):
    a = dict(X=P, M=16, N=512, K=512, v=P, m=P, s=P, group=128, L=P, R=P, r=32, Y=P,
             ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.slim_linear(a["X"], a["M"], a["N"], a["K"], a["v"], a["m"], a["s"], a["group"],
                           a["L"], a["R"], a["r"], a["Y"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(group=64), 2), (dict(K=500), 1), (dict(K=0), 1), (dict(N=100), 1), (dict(N=0), 1),
    (dict(M=-1), 1), (dict(r=33), 1), (dict(r=-32), 1), (dict(X=None), 1), (dict(Y=None), 1),
    (dict(v=None), 1), (dict(L=None), 1), (dict(X=P + 2), 1), (dict(wsb=16), 1), (dict(ws=None), 1),
])
def test_linear_rejects_bad_arguments(lib, kw, code):
    assert _lin(lib, **kw) == code
    assert lib.slim_last_error()


def test_linear_empty_is_noop(lib):
    assert _lin(lib, M=0, X=None, Y=None) == 0


def test_pack_rejects_bad_arguments(lib):
    assert lib.slim_pack(P, 16, 100, 128, P, P, P, None) == 1
    assert lib.slim_pack(P, 16, 128, 32, P, P, P, None) == 2
    assert lib.slim_pack(None, 16, 128, 128, P, P, P, None) == 1
    assert lib.slim_pack(P, 0, 128, 128, P, P, P, None) == 1
    assert lib.slim_pack(P + 4, 16, 128, 128, P, P, P, None) == 1


def test_batched_rejects_overlapping_outputs(lib):
    st = lib.slim_linear_batched(2, 16, 512, 512, 32, 128, P, 0, P, 512 * 128, P, 512 * 64,
                                 P, 512 * 4, P, 512 * 32, P, 32 * 512, P, 100, P, 1 << 24, None)
    assert st == 1


def test_adapter_sizes(lib):
    from sparse_int4_gemm_amd import _lib
    assert _lib.slim_adapter_codes_bytes(416, 4096) == 416 * 2048
    assert _lib.slim_adapter_scales_bytes(416, 4096, 128) == 416 * 32 * 2
    assert _lib.slim_adapter_scales_bytes(4096, 416, 32) == 4096 * 13 * 2
    assert _lib.slim_adapter_scales_bytes(4096, 416, 128) == 0      # 416 is not a multiple of 128
    assert _lib.slim_adapter_scales_bytes(16, 128, 64) == 0         # only groups 32 and 128
    assert _lib.slim_adapter_codes_bytes(0, 128) == 0
    assert _lib.slim_linear_qa_workspace_bytes(1, 4096, 4096, 0) == 0
    for M, N, K, r in [(1, 4096, 4096, 416), (16, 11008, 4096, 416), (2048, 4096, 11008, 416), (0, 16, 128, 32)]:
        w = _lib.slim_linear_qa_workspace_bytes(M, N, K, r)
        assert w % 256 == 0
        # Room for the fp16 path's workspace plus fp16 copies of both factors.
        assert w >= _lib.slim_linear_workspace_bytes(M, N, K, r) + 2 * r * K + 2 * N * r


@pytest.mark.parametrize("args,code", [
    ((P, 16, 128, 64, P, P), 2), ((P, 16, 80, 32, P, P), 1), ((P, 16, 100, 128, P, P), 1),
    ((None, 16, 128, 128, P, P), 1), ((P, 0, 128, 128, P, P), 1), ((P, 16, 128, 128, P + 8, P), 1),
    ((P, 16, 128, 128, P, None), 1),
])
def test_pack_adapter_rejects_bad_arguments(lib, args, code):
    assert lib.slim_pack_adapter(*args, None) == code
    assert lib.slim_last_error()


def _lin_qa(lib, **kw):
    a = dict(X=P, M=1, N=512, K=512, v=P, m=P, s=P, group=128, lq=P, ls=P, rq=P, rs=P, r=32, Y=P,
             ws=P, wsb=1 << 24, stream=None)
    a.update(kw)
    return lib.slim_linear_qa(a["X"], a["M"], a["N"], a["K"], a["v"], a["m"], a["s"], a["group"],
                              a["lq"], a["ls"], a["rq"], a["rs"], a["r"], a["Y"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(group=64), 2), (dict(r=0), 1), (dict(r=48), 1), (dict(K=500), 1), (dict(N=100), 1), (dict(M=-1), 1),
    (dict(lq=None), 1), (dict(ls=None), 1), (dict(rq=None), 1), (dict(rs=None), 1), (dict(rs=P + 2), 1),
    (dict(X=None), 1), (dict(wsb=256), 1), (dict(ws=None), 1),
])
def test_linear_qa_rejects_bad_arguments(lib, kw, code):
    assert _lin_qa(lib, **kw) == code
    assert lib.slim_last_error()


def test_linear_qa_empty_is_noop(lib):
    assert _lin_qa(lib, M=0, X=None, Y=None) == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: with the library missing, loading (and so every call)
    raises instead of computing anything elsewhere."""
    import subprocess
    import sys
    code = ("import sparse_int4_gemm_amd as s\n"
            "try:\n    s._lib.load()\nexcept ImportError as e:\n    print('ImportError', e)\n")
    env = dict(os.environ, SLIM_LIB=str(tmp_path / "absent.so"), PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300)
    assert "ImportError" in out.stdout, out.stdout + out.stderr


def test_transposed_sizes(lib):
    from sparse_int4_gemm_amd import _lib
    assert _lib.slim_transposed_values_bytes(4096, 11008) == 4096 * 11008
    assert _lib.slim_transposed_meta_bytes(4096, 11008) == 4096 * 11008 // 8
    assert _lib.slim_transposed_values_bytes(40, 128) == 0          # N not a multiple of 16
    assert _lib.slim_transposed_meta_bytes(16, 100) == 0            # K not a multiple of 128
    assert _lib.slim_transposed_values_bytes(0, 128) == 0


@pytest.mark.parametrize("args,code", [
    ((P, P, P, 16, 128, 64, P, P), 2), ((P, P, P, 40, 128, 128, P, P), 1), ((P, P, P, 16, 100, 128, P, P), 1),
    ((P, P, P, 0, 128, 128, P, P), 1), ((None, P, P, 16, 128, 128, P, P), 1), ((P, P, P, 16, 128, 128, P, None), 1),
    ((P, P + 4, P, 16, 128, 128, P, P), 1), ((P, P, P, 16, 128, 128, P + 2, P), 1),
    ((P, P, P, 1 << 23, 1 << 22, 128, P, P), 1),
])
def test_pack_transposed_rejects_bad_arguments(lib, args, code):
    assert lib.slim_pack_transposed(*args, None) == code
    assert lib.slim_last_error()


def test_wait_limit_knob(lib):
    """The bounded-wait knob is host state: set, read back, restore."""
    prev = lib.slim_set_wait_limit(0)
    assert lib.slim_set_wait_limit(5) == 0
    assert lib.slim_set_wait_limit(-1) == 5
    assert lib.slim_set_wait_limit(prev) == 1 << 18
    assert lib.slim_set_wait_limit(-1) == prev


def test_giveups_rejects_bad_arguments(lib):
    import ctypes
    n = ctypes.c_uint64(7)
    assert lib.slim_linear_giveups(None, 0, ctypes.byref(n), None) == 1
    assert lib.slim_linear_giveups(ctypes.c_void_p(16), 0, None, None) == 1
    assert lib.slim_linear_giveups(ctypes.c_void_p(24), 0, ctypes.byref(n), None) == 1
    assert n.value == 7


def test_a8_rejects_bad_arguments(lib):
    import ctypes
    p = ctypes.c_void_p(256)
    assert lib.slim_quantize_input(p, 4, 100, p, p, None) == 1          # K % 8
    assert lib.slim_quantize_input(None, 4, 128, p, p, None) == 1       # NULL X
    assert lib.slim_quantize_input(p, 0, 128, None, None, None) == 0    # M = 0: no-op
    ws = lib.slim_linear_a8_workspace_bytes(16, 256, 512, 32)
    assert ws >= lib.slim_linear_workspace_bytes(16, 256, 512, 32) + 16 * 512 * 2
    args = [p, p, 16, 256, 512, p, p, p, 128, p, p, 32, p, p, ws, None]
    bad = list(args); bad[1] = None                                       # NULL scales
    assert lib.slim_linear_a8(*bad) == 1
    bad = list(args); bad[8] = 64                                         # group
    assert lib.slim_linear_a8(*bad) == 2
    bad = list(args); bad[14] = ws - 256                                  # workspace too small
    assert lib.slim_linear_a8(*bad) == 1

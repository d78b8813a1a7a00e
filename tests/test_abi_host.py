"""Host-side checks of the C-ABI libraries (no GPU): the product library and
the test-support library load, each exports exactly the functions its
headers declare, and both reject bad arguments with the documented status
codes before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

from combine_fp32_router_amd import binding as B
from combine_fp32_router_amd import harness as HN

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("moe_route.h", "moe_recv.h")]
HARNESS_HEADERS = [os.path.join(ROOT, "include", "moe_harness.h")]

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_route.so is not built; run __graft_entry__.build()")
    return B.load()


@pytest.fixture(scope="module")
def hlib():
    if not os.path.exists(HN.LIB_PATH):
        pytest.fail("libmoe_harness.so is not built; run __graft_entry__.build()")
    return HN.load()


def declared_functions(headers=HEADERS):
    names = []
    for h in headers:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def exported_functions(path):
    """Names of the moe_* functions a shared library defines (nm -D)."""
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return sorted({ln.split()[-1] for ln in out.splitlines()
                   if ln.split()[-1].startswith("moe_") and " T " in ln})


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"moe_route_topk", "moe_dispatch_layout", "moe_dispatch_pack", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert set(names) == set(B.EXPORTS)
    # the product library exports exactly its headers' functions
    assert exported_functions(B.LIB_PATH) == sorted(names)


def test_harness_library_exports(hlib):
    names = declared_functions(HARNESS_HEADERS)
    assert set(names) == set(HN.EXPORTS)
    for n in names:
        assert hasattr(hlib, n), f"{n} declared but not exported"
    assert exported_functions(HN.LIB_PATH) == sorted(names)
    assert not set(names) & set(exported_functions(B.LIB_PATH))


def test_status_strings(lib):
    for s in range(8):
        assert B.status_string(s).startswith("MOE_")
    assert B.status_string(99) == "unknown moe status"


def test_row_bytes(lib):
    assert B.moe_row_bytes(7168, 0) == 14336
    assert B.moe_row_bytes(7168, 1) == 7168
    assert B.moe_row_bytes(7168, 2) == 3584
    assert B.moe_row_bytes(7168, 3) == 7168
    assert B.moe_row_bytes(16, 4) == -1


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced (validation fails first)
ODD = ctypes.c_void_p(0x10002)


def test_route_validation(lib):
    f = lib.moe_route_topk
    assert f(FAKE, -1, 8, 2, FAKE, FAKE, None) == MOE_ERR_SHAPE
    assert f(FAKE, 4, 8, 9, FAKE, FAKE, None) == MOE_ERR_SHAPE      # k > E
    assert f(FAKE, 4, 8, 0, FAKE, FAKE, None) == MOE_ERR_SHAPE
    assert f(FAKE, 4, 2000, 8, FAKE, FAKE, None) == MOE_ERR_SHAPE   # E > 1024
    assert f(FAKE, 4, 64, 17, FAKE, FAKE, None) == MOE_ERR_SHAPE    # k > 16
    assert f(FAKE, 2 ** 28, 64, 8, FAKE, FAKE, None) == MOE_ERR_SHAPE  # T*k >= 2^31
    assert f(None, 4, 8, 2, FAKE, FAKE, None) == MOE_ERR_NULL
    assert f(ODD, 4, 8, 2, FAKE, FAKE, None) == MOE_ERR_ALIGN
    assert f(None, 0, 8, 2, None, None, None) == MOE_OK             # T == 0: nothing launched


def test_layout_validation_and_workspace_query(lib):
    f = lib.moe_dispatch_layout
    n = ctypes.c_size_t(0)
    assert f(None, 4096, 256, 8, 32, 0, None, None, None, None, None, None, None,
             ctypes.byref(n), None) == MOE_OK
    assert n.value >= 256 * 4 and n.value % 256 == 0
    assert B.layout_workspace_bytes(4096, 256, 8, 32) == n.value
    args = [FAKE] * 6
    assert f(FAKE, 16, 8, 2, 3, 0, *args, FAKE, ctypes.byref(n), None) == MOE_ERR_SHAPE  # E % R
    assert f(FAKE, 16, 8, 2, 0, 0, *args, FAKE, ctypes.byref(n), None) == MOE_ERR_SHAPE  # R < 1
    assert f(FAKE, 16, 8, 2, 2, 0, *args, FAKE, None, None) == MOE_ERR_NULL
    small = ctypes.c_size_t(8)
    assert f(FAKE, 16, 8, 2, 2, 0, *args, FAKE, ctypes.byref(small), None) == MOE_ERR_WORKSPACE
    big = ctypes.c_size_t(1 << 20)
    assert f(FAKE, 16, 8, 2, 2, 0, *args, ODD, ctypes.byref(big), None) == MOE_ERR_ALIGN
    assert f(FAKE, 16, 8, 2, 2, 0, None, *args[1:], FAKE, ctypes.byref(big), None) == MOE_ERR_NULL


def test_pack_combine_validation(lib):
    # every call below fails validation (or has no work), so nothing launches
    p, c = lib.moe_dispatch_pack, lib.moe_combine
    S = FAKE  # a scale array
    assert p(FAKE, 4, 24, 2, FAKE, 0, FAKE, None, None) == MOE_ERR_SHAPE      # H % 16
    assert p(FAKE, 4, 0, 2, FAKE, 0, FAKE, None, None) == MOE_ERR_SHAPE
    assert p(FAKE, 4, 1 << 17, 2, FAKE, 0, FAKE, None, None) == MOE_ERR_SHAPE  # H > 65536
    assert p(FAKE, 4, 32, 2, FAKE, 4, FAKE, S, None) == MOE_ERR_SHAPE      # unknown quant
    assert p(FAKE, 4, 48, 2, FAKE, 2, FAKE, S, None) == MOE_ERR_SHAPE      # int4 needs H % 32
    assert c(FAKE, S, 2, FAKE, FAKE, 4, 48, 2, FAKE, None) == MOE_ERR_SHAPE
    assert p(FAKE, 4, 32, 0, FAKE, 0, FAKE, None, None) == MOE_ERR_SHAPE      # k < 1
    assert p(None, 4, 32, 2, FAKE, 0, FAKE, None, None) == MOE_ERR_NULL
    assert p(ctypes.c_void_p(0x10008), 4, 32, 2, FAKE, 0, FAKE, None, None) == MOE_ERR_ALIGN
    assert p(None, 0, 32, 2, None, 0, None, None, None) == MOE_OK
    for q in (1, 2, 3):  # quantised rows need their scale array
        assert p(FAKE, 4, 32, 2, FAKE, q, FAKE, None, None) == MOE_ERR_NULL
        assert p(FAKE, 4, 32, 2, FAKE, q, FAKE, ODD, None) == MOE_ERR_ALIGN
        assert c(FAKE, None, q, FAKE, FAKE, 4, 32, 2, FAKE, None) == MOE_ERR_NULL
        assert c(FAKE, ODD, q, FAKE, FAKE, 4, 32, 2, FAKE, None) == MOE_ERR_ALIGN
    assert c(FAKE, S, 1, FAKE, FAKE, 4, 24, 2, FAKE, None) == MOE_ERR_SHAPE
    # the streaming-store flag belongs to the pack calls only; other bits are refused
    STREAM = B.MOE_PACK_STREAM
    assert p(FAKE, 4, 24, 2, FAKE, 0 | STREAM, FAKE, None, None) == MOE_ERR_SHAPE  # H % 16
    assert p(FAKE, 4, 32, 2, FAKE, 1 | STREAM, FAKE, None, None) == MOE_ERR_NULL   # scales
    assert p(FAKE, 4, 32, 2, FAKE, 4 | STREAM, FAKE, S, None) == MOE_ERR_SHAPE
    assert p(FAKE, 4, 32, 2, FAKE, 0x200, FAKE, None, None) == MOE_ERR_SHAPE
    assert c(FAKE, S, 1 | STREAM, FAKE, FAKE, 4, 32, 2, FAKE, None) == MOE_ERR_SHAPE  # combine
    assert c(FAKE, S, 1, None, FAKE, 4, 32, 2, FAKE, None) == MOE_ERR_NULL
    assert c(FAKE, S, 1, FAKE, FAKE, 4, 32, 2, ctypes.c_void_p(0x10004), None) == MOE_ERR_ALIGN
    assert c(None, None, 1, None, None, 0, 32, 2, None, None) == MOE_OK


def test_harness_validation(hlib):
    s = hlib.moe_expert_standin
    S = FAKE
    assert s(FAKE, None, 0, FAKE, 8, -1, 32, 0, FAKE, None, None) == MOE_ERR_SHAPE
    assert s(FAKE, None, 0, FAKE, 8, 10, 24, 0, FAKE, None, None) == MOE_ERR_SHAPE
    assert s(None, None, 0, FAKE, 8, 10, 32, 0, FAKE, None, None) == MOE_ERR_NULL
    assert s(FAKE, None, 1, FAKE, 8, 10, 32, 0, FAKE, None, None) == MOE_ERR_NULL   # in scales
    assert s(FAKE, None, 0, FAKE, 8, 10, 32, 2, FAKE, None, None) == MOE_ERR_NULL   # out scales
    assert s(FAKE, S, 1, FAKE, 8, 10, 32, 1, FAKE, ODD, None) == MOE_ERR_ALIGN
    assert s(None, None, 0, None, 8, 0, 32, 0, None, None, None) == MOE_OK
    sp = hlib.moe_stream_probe
    assert sp(FAKE, FAKE, 15, 0, None) == MOE_ERR_SHAPE
    assert sp(FAKE, FAKE, 16, 3, None) == MOE_ERR_SHAPE                     # unknown mode
    assert sp(FAKE, FAKE, 1 << 40, 0, None) == MOE_ERR_SHAPE
    assert sp(None, FAKE, 16, 1, None) == MOE_ERR_NULL
    assert sp(ODD, FAKE, 16, 2, None) == MOE_ERR_ALIGN
    assert sp(FAKE, ctypes.c_void_p(0x10004), 16, 0, None) == MOE_ERR_ALIGN  # copy: 16 B
    assert sp(None, None, 0, 0, None) == MOE_OK


def test_layout_chunks_validation(lib):
    f = lib.moe_dispatch_layout_chunks
    n = ctypes.c_size_t(0)
    assert f(None, 16384, 4096, 256, 8, 32, 0, None, None, None, None, None, None, None, None,
             ctypes.byref(n), None) == MOE_OK
    one = ctypes.c_size_t(0)
    lib.moe_dispatch_layout(None, 4096, 256, 8, 32, 0, None, None, None, None, None, None, None,
                            ctypes.byref(one), None)
    assert n.value >= 4 * one.value - 3 * 255  # four chunks' histograms
    args = [FAKE] * 6
    big = ctypes.c_size_t(1 << 24)
    assert f(FAKE, 16, 0, 8, 2, 2, 0, None, *args, FAKE, ctypes.byref(big), None) == MOE_ERR_SHAPE
    assert f(FAKE, 16, -1, 8, 2, 2, 0, None, *args, FAKE, ctypes.byref(big), None) == MOE_ERR_SHAPE
    assert f(FAKE, 70000, 1, 8, 2, 2, 0, None, *args, FAKE, ctypes.byref(big), None) == MOE_ERR_SHAPE
    assert f(FAKE, 16, 4, 8, 2, 2, 0, ODD, *args, FAKE, ctypes.byref(big), None) == MOE_ERR_ALIGN
    assert f(FAKE, 16, 4, 8, 2, 2, 0, None, *args, FAKE, None, None) == MOE_ERR_NULL


def test_recv_validation(lib, hlib):
    lay, rg, ug, ex = (lib.moe_recv_layout, lib.moe_recv_regroup, lib.moe_recv_ungroup,
                       hlib.moe_exchange_blocks)
    assert lay(FAKE, 16, 3, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_SHAPE   # E % R
    assert lay(FAKE, 2048, 8, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_SHAPE  # E > 1024
    assert lay(FAKE, 16, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_SHAPE
    assert lay(FAKE, 16, 4, -1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_SHAPE
    assert lay(FAKE, 16, 4, 2 ** 31, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MOE_ERR_SHAPE
    assert lay(FAKE, 16, 4, 64, FAKE, None, FAKE, FAKE, FAKE, None) == MOE_ERR_NULL
    assert lay(FAKE, 16, 4, 64, FAKE, FAKE, FAKE, FAKE, None, None) == MOE_ERR_NULL
    assert lay(FAKE, 16, 4, 64, FAKE, FAKE, ODD, FAKE, FAKE, None) == MOE_ERR_ALIGN
    S = FAKE
    for f in (rg, ug):
        # (in, in_scales, max_rows, H, quant, map, out, out_scales, stream)
        assert f(FAKE, None, 64, 24, 0, FAKE, FAKE, None, None) == MOE_ERR_SHAPE   # H % 16
        assert f(FAKE, S, 64, 32, 4, FAKE, FAKE, S, None) == MOE_ERR_SHAPE   # quant
        assert f(FAKE, None, -1, 32, 0, FAKE, FAKE, None, None) == MOE_ERR_SHAPE
        assert f(FAKE, None, 2 ** 31, 32, 0, FAKE, FAKE, None, None) == MOE_ERR_SHAPE
        assert f(FAKE, None, 64, 32, 0, None, FAKE, None, None) == MOE_ERR_NULL
        assert f(FAKE, None, 64, 32, 0, FAKE, ctypes.c_void_p(0x10008), None,
                 None) == MOE_ERR_ALIGN
        assert f(FAKE, None, 64, 32, 0, ODD, FAKE, None, None) == MOE_ERR_ALIGN
        assert f(FAKE, None, 64, 32, 1, FAKE, FAKE, S, None) == MOE_ERR_NULL    # in scales
        assert f(FAKE, S, 64, 32, 1, FAKE, FAKE, None, None) == MOE_ERR_NULL    # out scales
        assert f(FAKE, S, 64, 32, 3, FAKE, FAKE, ODD, None) == MOE_ERR_ALIGN
        assert f(None, None, 0, 32, 0, None, None, None, None) == MOE_OK
    # (send, send_scales, source_rows, recv, recv_scales, max_rows, H, quant, so, E, R, ro,
    #  reverse, stream)
    assert ex(FAKE, None, -1, FAKE, None, 64, 32, 0, FAKE, 16, 4, FAKE, 0, None) == MOE_ERR_SHAPE
    assert ex(FAKE, None, 2 ** 29, FAKE, None, 64, 32, 0, FAKE, 16, 4, FAKE, 0,
              None) == MOE_ERR_SHAPE
    assert ex(FAKE, None, 16, FAKE, None, 64, 32, 0, FAKE, 16, 4, None, 0, None) == MOE_ERR_NULL
    assert ex(ODD, None, 16, FAKE, None, 64, 32, 0, FAKE, 16, 4, FAKE, 0, None) == MOE_ERR_ALIGN
    assert ex(FAKE, None, 16, FAKE, S, 64, 32, 1, FAKE, 16, 4, FAKE, 0, None) == MOE_ERR_NULL
    assert ex(FAKE, S, 16, FAKE, ODD, 64, 32, 2, FAKE, 16, 4, FAKE, 1, None) == MOE_ERR_ALIGN


def test_route_layout_validation(lib):
    f = lib.moe_route_layout_chunks
    n = ctypes.c_size_t(0)
    assert f(None, 16384, 2048, 256, 8, 32, 0, None, None, None, None, None, None, None, None,
             None, None, ctypes.byref(n), None) == MOE_OK
    # the router writes one histogram row per 64-token group: 32 rows per chunk
    assert n.value == 8 * 32 * 256 * 4
    assert n.value == B.route_layout_workspace_bytes(16384, 2048, 256, 8, 32)
    # k = 6 does not tile into whole groups: the separate calls' workspace
    assert (B.route_layout_workspace_bytes(700, 256, 200, 6, 5) ==
            B.layout_chunks_workspace_bytes(700, 256, 200, 6, 5))
    big = ctypes.c_size_t(1 << 24)
    args = [FAKE] * 6
    assert f(FAKE, 16, 4, 8, 9, 2, 0, None, FAKE, FAKE, *args, FAKE, ctypes.byref(big),
             None) == MOE_ERR_SHAPE                                        # k > E
    assert f(FAKE, 16, 4, 8, 2, 3, 0, None, FAKE, FAKE, *args, FAKE, ctypes.byref(big),
             None) == MOE_ERR_SHAPE                                        # E % R
    assert f(FAKE, 16, 0, 8, 2, 2, 0, None, FAKE, FAKE, *args, FAKE, ctypes.byref(big),
             None) == MOE_ERR_SHAPE                                        # chunk_tokens
    assert f(None, 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, *args, FAKE, ctypes.byref(big),
             None) == MOE_ERR_NULL                                         # logits
    assert f(FAKE, 16, 4, 8, 2, 2, 0, None, FAKE, None, *args, FAKE, ctypes.byref(big),
             None) == MOE_ERR_NULL                                         # topk_w
    assert f(FAKE, 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, *args, FAKE, None, None) == MOE_ERR_NULL
    small = ctypes.c_size_t(8)
    assert f(FAKE, 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, *args, FAKE, ctypes.byref(small),
             None) == MOE_ERR_WORKSPACE
    assert f(ctypes.c_void_p(0x10002), 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, *args, FAKE,
             ctypes.byref(big), None) == MOE_ERR_ALIGN


def test_route_layout_noalloc_validation(lib):
    """The no-allocation variant checks what the workspace call checks and
    refuses, before touching the GPU, a call whose histogram scratch would
    not fit the static buffer."""
    f = lib.moe_route_layout_chunks_noalloc
    MOE_ERR_SCRATCH = 7
    args = [FAKE] * 6
    assert f(FAKE, 16, 4, 8, 9, 2, 0, None, FAKE, FAKE, *args, None) == MOE_ERR_SHAPE  # k > E
    assert f(FAKE, 16, 4, 8, 2, 3, 0, None, FAKE, FAKE, *args, None) == MOE_ERR_SHAPE  # E % R
    assert f(FAKE, 16, 0, 8, 2, 2, 0, None, FAKE, FAKE, *args, None) == MOE_ERR_SHAPE
    assert f(None, 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, *args, None) == MOE_ERR_NULL
    assert f(FAKE, 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, None, *args[1:], None) == MOE_ERR_NULL
    assert f(ODD, 16, 4, 8, 2, 2, 0, None, FAKE, FAKE, *args, None) == MOE_ERR_ALIGN
    # E = 1024, 1024-token chunks: 64 router groups of 16 tokens, 256 KiB of
    # histogram per chunk; 16 chunks fill the 4 MiB buffer exactly, 17 do not fit
    for chunks, want in ((16, None), (17, MOE_ERR_SCRATCH)):
        T = 1024 * chunks
        need = B.route_layout_workspace_bytes(T, 1024, 1024, 8, 8)
        assert need == chunks * 64 * 1024 * 4
        if want is not None:
            assert need > B.MOE_NOALLOC_SCRATCH_BYTES
            assert f(FAKE, T, 1024, 1024, 8, 8, 0, None, FAKE, FAKE, *args, None) == want
        else:
            assert need == B.MOE_NOALLOC_SCRATCH_BYTES
    assert B.status_string(MOE_ERR_SCRATCH).startswith("MOE_ERR_SCRATCH")


def test_combine_pack_validation(lib):
    f = lib.moe_combine_pack
    MOE_ERR_ALIAS = 6
    A = ctypes.c_void_p(0x20000)
    S, T = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000)  # two scale arrays
    # recv, recv_scales, pos_c, w, Tc, out, x, pos_p, Tp, send, send_scales, H, k, quant, stream
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, T, 24, 2, 0, None) == MOE_ERR_SHAPE
    assert f(FAKE, S, FAKE, FAKE, -1, FAKE, FAKE, FAKE, 4, A, T, 32, 2, 0, None) == MOE_ERR_SHAPE
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, -1, A, T, 32, 2, 0, None) == MOE_ERR_SHAPE
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, T, 48, 2, 2, None) == MOE_ERR_SHAPE
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, T, 32, 2, 4, None) == MOE_ERR_SHAPE
    assert f(FAKE, S, FAKE, FAKE, 1 << 30, FAKE, FAKE, FAKE, 1 << 30, A, T, 32, 1, 0,
             None) == MOE_ERR_SHAPE                                    # Tc + Tp >= 2^31
    assert f(None, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, T, 32, 2, 0, None) == MOE_ERR_NULL
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, None, T, 32, 2, 0, None) == MOE_ERR_NULL
    assert f(FAKE, None, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, T, 32, 2, 1,
             None) == MOE_ERR_NULL                                     # combine's scales
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, ODD, 32, 2, 3,
             None) == MOE_ERR_ALIGN                                    # pack's scales
    assert f(FAKE, S, FAKE, FAKE, 4, ctypes.c_void_p(0x10008), FAKE, FAKE, 4, A, T, 32, 2, 0,
             None) == MOE_ERR_ALIGN
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, ODD, 4, A, T, 32, 2, 0, None) == MOE_ERR_ALIGN
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, FAKE, T, 32, 2, 0,
             None) == MOE_ERR_ALIAS                                    # send == recv
    assert f(FAKE, S, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 4, A, S, 32, 2, 1,
             None) == MOE_ERR_ALIAS                                    # one scale array
    assert f(None, None, None, None, 0, None, None, None, 0, None, None, 32, 2, 0,
             None) == MOE_OK
    assert B.status_string(MOE_ERR_ALIAS).startswith("MOE_ERR_ALIAS")


def test_combine_pack_partial_overlaps(lib):
    """Overlapping (not only equal) ranges between what the pack writes and
    what the combine touches, and between the combine's output and the pack's
    inputs, are refused.  (Only argument sets that validation rejects are
    used: nothing here may reach a launch.)"""
    f = lib.moe_combine_pack
    MOE_ERR_ALIAS = 6
    V = ctypes.c_void_p
    Tc = Tp = 4
    H, k = 32, 2
    rb = 2 * H                         # bf16 row bytes
    recv, out, x = 0x100000, 0x200000, 0x300000
    pos_c, w, pos_p = 0x400000, 0x500000, 0x600000

    def call(send, quant=0, S=None, T=None, o=out):
        return f(V(recv), S, V(pos_c), V(w), Tc, V(o), V(x), V(pos_p), Tp, V(send), T, H, k,
                 quant, None)

    assert call(recv + Tc * k * rb - 16) == MOE_ERR_ALIAS      # send overlaps recv's tail
    assert call(recv - Tp * k * rb + 16) == MOE_ERR_ALIAS      # send runs into recv's head
    assert call(out + 64) == MOE_ERR_ALIAS                     # send inside the output
    assert call(pos_c - Tp * k * rb + 16) == MOE_ERR_ALIAS     # send runs into pos_c
    assert call(w + 16) == MOE_ERR_ALIAS                       # send over the weights
    assert call(0x700000, o=x + 16) == MOE_ERR_ALIAS           # out overlaps x
    assert call(0x700000, o=pos_p - 16) == MOE_ERR_ALIAS       # out runs into pos_p
    S = 0x800000
    assert call(0x700000, 1, V(S), V(S + 4 * Tc * k - 4)) == MOE_ERR_ALIAS  # scales by 4 B
    assert call(0x700000, 1, V(S), V(recv + 16)) == MOE_ERR_ALIAS  # pack scales into recv


def test_binding_refuses_host_tensors(lib):
    """The binding marshals device tensors only: host tensors are an error,
    never a silent CPU path."""
    import torch
    T, E, k, H = 4, 8, 2, 16
    logits = torch.zeros((T, E), dtype=torch.float32)
    idx = torch.zeros((T, k), dtype=torch.int32)
    w = torch.zeros((T, k), dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        B.moe_route_topk(logits, k, idx, w)
    recv = torch.zeros((T * k, 2 * H), dtype=torch.uint8)
    pos = torch.zeros((T, k), dtype=torch.int32)
    out = torch.zeros((T, H), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        B.moe_combine(recv, None, 0, pos, w, T, H, k, out)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every call raises: nothing falls back."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libmoe_route.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.load()
    with pytest.raises(RuntimeError, match="not built"):
        B.moe_row_bytes(7168, 1)


def test_slot_count_check_does_not_overflow(lib, hlib):
    """T*k >= 2^31 is refused without forming T*k: with T = 2^62 and k = 16
    the product wraps to 0 in int64, which a multiplying check would let
    through.  Every entry point that takes a token or row count returns
    MOE_ERR_SHAPE before looking at its (NULL) pointers or launching."""
    T = 2 ** 62
    n = ctypes.c_size_t(0)
    assert lib.moe_route_topk(None, T, 64, 16, None, None, None) == MOE_ERR_SHAPE
    assert lib.moe_dispatch_layout(None, T, 64, 16, 8, 0, None, None, None, None, None, None,
                                   None, ctypes.byref(n), None) == MOE_ERR_SHAPE
    assert lib.moe_dispatch_layout_chunks(None, T, 4096, 64, 16, 8, 0, None, None, None, None,
                                          None, None, None, None, ctypes.byref(n),
                                          None) == MOE_ERR_SHAPE
    assert lib.moe_route_layout_chunks(None, T, 4096, 64, 16, 8, 0, None, None, None, None,
                                       None, None, None, None, None, None, ctypes.byref(n),
                                       None) == MOE_ERR_SHAPE
    assert lib.moe_dispatch_pack(None, T, 32, 16, None, 0, None, None, None) == MOE_ERR_SHAPE
    assert lib.moe_combine(None, None, 0, None, None, T, 32, 16, None, None) == MOE_ERR_SHAPE
    assert lib.moe_combine_pack(None, None, None, None, T, None, None, None, 0, None, None, 32,
                                16, 0, None) == MOE_ERR_SHAPE
    assert hlib.moe_exchange_blocks(None, None, T, None, None, 0, 32, 0, None, 64, 16, None, 0,
                                    None) == MOE_ERR_SHAPE


def test_grid_work_item_limit(lib):
    """A launch's grid dimension holds fewer than 2^32 work-items: one token
    past the limit is refused with MOE_ERR_SHAPE before any pointer is read;
    the limit itself passes the shape checks (and stops at the NULL
    pointers, so nothing is launched)."""
    lim = (2 ** 32 - 1) // 896  # pack / combine at H = 7168 bf16: 896 threads per token
    assert lim == 4_793_490
    p, c, cp = lib.moe_dispatch_pack, lib.moe_combine, lib.moe_combine_pack
    assert p(None, lim + 1, 7168, 1, None, 0, None, None, None) == MOE_ERR_SHAPE
    assert p(None, lim, 7168, 1, None, 0, None, None, None) == MOE_ERR_NULL
    assert c(None, None, 0, None, None, lim + 1, 7168, 1, None, None) == MOE_ERR_SHAPE
    assert c(None, None, 0, None, None, lim, 7168, 1, None, None) == MOE_ERR_NULL
    assert cp(None, None, None, None, lim // 2, None, None, None, lim // 2 + 2, None, None, 7168,
              1, 0, None) == MOE_ERR_SHAPE
    assert cp(None, None, None, None, lim // 2, None, None, None, lim // 2, None, None, 7168,
              1, 0, None) == MOE_ERR_NULL
    rlim = (2 ** 32 - 1) // 256 * 16  # router, E <= 256: 16 tokens per 256-thread workgroup
    assert lib.moe_route_topk(None, rlim + 1, 256, 1, None, None, None) == MOE_ERR_SHAPE
    assert lib.moe_route_topk(None, rlim, 256, 1, None, None, None) == MOE_ERR_NULL
    n = ctypes.c_size_t(0)
    assert lib.moe_route_layout_chunks(None, rlim + 1, 4096, 256, 1, 8, 0, None, None, None,
                                       None, None, None, None, None, None, None,
                                       ctypes.byref(n), None) == MOE_ERR_SHAPE
    g = lib.moe_recv_regroup
    assert g(None, None, lim + 1, 7168, 0, None, None, None, None) == MOE_ERR_SHAPE
    assert g(None, None, lim, 7168, 0, None, None, None, None) == MOE_ERR_NULL

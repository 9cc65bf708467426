"""Host-side checks of the C ABI (no GPU needed).

The library must load, export exactly the functions include/lse.h declares,
and reject bad arguments with the documented status codes before it touches
the HIP runtime (every call below fails validation, so nothing is launched).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("lse.h", "lse_testing.h")]

LSE_OK, LSE_ERR_NULL, LSE_ERR_SHAPE, LSE_ERR_WORKSPACE, LSE_ERR_OVERLAP = 0, 1, 2, 3, 4
LSE_ERR_UNSUPPORTED = 6
FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every call here fails validation
FAKE2 = ctypes.c_void_p(0x900000000)


def declared_functions():
    assert sorted(HEADERS) == sorted(
        os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include")))
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keywords = {"sizeof", "defined"}
    return sorted(set(n for n in names if n not in keywords))


@pytest.fixture(scope="module")
def lib():
    from log_softmax_reductions_amd import _lib
    return _lib.load()


def test_exports_match_header(lib):
    import subprocess
    from log_softmax_reductions_amd import _lib
    declared = declared_functions()
    assert len(declared) == 27
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines()
                      if l.split()[-2] in ("T", "W") and not l.split()[-1].startswith("_"))
    assert exported == declared
    assert set(_lib.SIGNATURES) == set(declared)


def test_status_strings(lib):
    assert lib.lse_status_string(0) == b"LSE_OK"
    assert lib.lse_status_string(3) == b"LSE_ERR_WORKSPACE"
    assert lib.lse_abi_version() == 1


def test_axis0_validation(lib):
    assert lib.lse_reduce_axis0(FAKE, FAKE2, 0, 5, None) == LSE_ERR_SHAPE
    assert lib.lse_reduce_axis0(FAKE, FAKE2, 3, -1, None) == LSE_ERR_SHAPE
    assert lib.lse_reduce_axis0(None, FAKE2, 3, 5, None) == LSE_ERR_NULL
    assert lib.lse_reduce_axis0(FAKE, None, 3, 5, None) == LSE_ERR_NULL
    assert lib.lse_reduce_axis0(FAKE, FAKE2, 1 << 40, 1 << 40, None) == LSE_ERR_SHAPE
    # out inside x's range
    assert lib.lse_reduce_axis0(FAKE, ctypes.c_void_p(0x100010), 4, 64, None) == LSE_ERR_OVERLAP
    assert b"overlaps" in lib.lse_last_error()
    # inner == 0 is a no-op that succeeds without touching anything
    assert lib.lse_reduce_axis0(None, None, 3, 0, None) == LSE_OK


def test_axis_and_softmax_validation(lib):
    assert lib.lse_reduce_axis(FAKE, FAKE2, 2, 0, 5, None) == LSE_ERR_SHAPE
    assert lib.lse_reduce_axis(FAKE, FAKE2, -1, 3, 5, None) == LSE_ERR_SHAPE
    assert lib.lse_reduce_axis(None, FAKE2, 2, 3, 5, None) == LSE_ERR_NULL
    assert lib.lse_reduce_axis(FAKE, ctypes.c_void_p(0x100004), 2, 3, 5, None) == LSE_ERR_OVERLAP
    assert lib.lse_reduce_axis(None, None, 0, 3, 5, None) == LSE_OK        # empty: no-op
    assert lib.log_softmax_axis(FAKE, FAKE, 2, 3, 5, None) == LSE_ERR_OVERLAP
    assert lib.log_softmax_axis(FAKE, FAKE2, 1 << 40, 1 << 20, 1 << 10, None) == LSE_ERR_SHAPE
    assert lib.softmax_rows(None, FAKE2, 4, 8, None, 0, None) == LSE_ERR_NULL
    assert lib.softmax_rows(FAKE, FAKE2, 16, 393216, None, 0, None) == LSE_ERR_WORKSPACE
    assert b"softmax_rows" in lib.lse_last_error()


def test_strided_validation(lib):
    ax, lsm = lib.lse_reduce_axis_strided, lib.log_softmax_axis_strided
    # negative strides
    assert ax(FAKE, FAKE2, 2, 3, 8, -1, 8, 8, None) == LSE_ERR_SHAPE
    assert lsm(FAKE, FAKE2, 2, 3, 8, 24, 8, 24, -8, None) == LSE_ERR_SHAPE
    # output planes that would collide: y stride over R smaller than inner
    assert lsm(FAKE, FAKE2, 2, 3, 8, 24, 8, 24, 4, None) == LSE_ERR_SHAPE
    assert b"overlap" in lib.lse_last_error()
    # output outer blocks that would collide: (R - 1) * 8 + 8 = 24 > 20
    assert lsm(FAKE, FAKE2, 2, 3, 8, 24, 8, 20, 8, None) == LSE_ERR_SHAPE
    assert ax(FAKE, FAKE2, 2, 3, 8, 24, 8, 7, None) == LSE_ERR_SHAPE
    # extents that overflow
    assert ax(FAKE, FAKE2, 4, 3, 8, 1 << 61, 8, 8, None) == LSE_ERR_SHAPE
    # padded x (plane pitch 10 > inner 8) whose range reaches the output
    span_x = (2 - 1) * 40 + (3 - 1) * 10 + 8
    assert ax(FAKE, ctypes.c_void_p(0x100000 + 4 * (span_x - 1)), 2, 3, 8, 40, 10, 8,
              None) == LSE_ERR_OVERLAP
    assert lsm(FAKE, FAKE, 2, 3, 8, 24, 8, 24, 8, None) == LSE_ERR_OVERLAP
    assert lsm(None, FAKE2, 2, 3, 8, 24, 8, 24, 8, None) == LSE_ERR_NULL
    assert ax(None, None, 0, 3, 8, 24, 8, 8, None) == LSE_OK        # empty: no-op
    # rows with a leading dimension
    rs = lib.log_softmax_rows_strided
    assert rs(FAKE, FAKE2, 4, 8, 7, 8, None, 0, None) == LSE_ERR_SHAPE
    assert rs(FAKE, FAKE2, 4, 8, 8, 7, None, 0, None) == LSE_ERR_SHAPE
    assert rs(FAKE, FAKE2, 4, 8, 1 << 61, 8, None, 0, None) == LSE_ERR_SHAPE
    # x rows every 16 floats, y rows 8 floats into x's first row: interleaved ranges
    assert rs(FAKE, ctypes.c_void_p(0x100000 + 32), 4, 8, 16, 16, None, 0, None) == LSE_ERR_OVERLAP
    assert lib.softmax_rows_strided(FAKE, FAKE2, 16, 393216, 393220, 393216, None, 0,
                                    None) == LSE_ERR_WORKSPACE
    assert rs(None, None, 0, 8, 8, 8, None, 0, None) == LSE_OK


def test_axis_workspace_validation(lib):
    wb = lib.lse_axis_workspace_bytes
    # few outputs over many planes: pairs per (column, chunk), plus (M, log S)
    # per column for log_softmax; 244 chunks of 4099 planes for (1e6, 4)
    assert wb(1, 1000000, 4, 0) == 4 * 244 * 8
    assert wb(1, 1000000, 4, 1) == 4 * 244 * 8 + 4 * 8
    assert wb(128, 64, 15876, 0) == 0 and wb(128, 64, 15876, 1) == 0   # many outputs
    assert wb(1, 63, 64, 0) == 0                                        # too few planes
    assert wb(0, 10, 10, 0) == 0 and wb(-1, 10, 10, 0) == 0 and wb(1, 1 << 40, 1 << 40, 0) == 0
    # long last-axis rows: the split rows' workspace
    assert wb(1, 100000000, 1, 1) >= lib.log_softmax_rows_workspace_bytes(1, 100000000)
    assert wb(4, 100000, 1, 0) >= 4 * 7 * 8
    ax, ax0 = lib.lse_reduce_axis_strided_ws, lib.lse_reduce_axis0_ws
    lsm = lib.log_softmax_axis_strided_ws
    need = wb(1, 1000000, 4, 0)
    far = ctypes.c_void_p(0x7000000000)
    assert ax(FAKE, FAKE2, 1, 1000000, 4, 4000000, 4, 4, None, 0, None) == LSE_ERR_WORKSPACE
    assert ax(FAKE, FAKE2, 1, 1000000, 4, 4000000, 4, 4, far, need - 1, None) == LSE_ERR_WORKSPACE
    assert ax(FAKE, FAKE2, 1, 1000000, 4, 4000000, 4, 4, FAKE, need, None) == LSE_ERR_OVERLAP
    assert ax(FAKE, FAKE2, 1, 1000000, 4, 4000000, 4, 4, FAKE2, need, None) == LSE_ERR_OVERLAP
    assert ax(FAKE, FAKE2, 1, 0, 4, 0, 4, 4, far, need, None) == LSE_ERR_SHAPE
    assert ax(None, FAKE2, 1, 1000000, 4, 4000000, 4, 4, far, need, None) == LSE_ERR_NULL
    assert ax0(FAKE, FAKE2, 1000000, 4, None, 0, None) == LSE_ERR_WORKSPACE
    assert ax0(FAKE, FAKE2, -1, 4, None, 0, None) == LSE_ERR_SHAPE
    need_y = wb(1, 1000000, 4, 1)
    assert lsm(FAKE, FAKE2, 1, 1000000, 4, 4000000, 4, 4000000, 4, far, need_y - 1,
               None) == LSE_ERR_WORKSPACE
    assert lsm(FAKE, FAKE2, 1, 1000000, 4, 4000000, 4, 4000000, 3, far, need_y,
               None) == LSE_ERR_SHAPE
    assert ax(None, None, 0, 3, 8, 24, 8, 8, None, 0, None) == LSE_OK     # empty: no-op


def test_rows_validation(lib):
    assert lib.log_softmax_rows(FAKE, FAKE2, -1, 8, None, 0, None) == LSE_ERR_SHAPE
    assert lib.log_softmax_rows(FAKE, FAKE2, 4, 0, None, 0, None) == LSE_ERR_SHAPE
    assert lib.log_softmax_rows(None, FAKE2, 4, 8, None, 0, None) == LSE_ERR_NULL
    assert lib.log_softmax_rows(FAKE, FAKE, 4, 8, None, 0, None) == LSE_ERR_OVERLAP
    # a split row needs a workspace of the advertised size
    need = lib.log_softmax_rows_workspace_bytes(16, 393216)
    assert need == 256 + 16 * 12 * 8
    assert lib.log_softmax_rows(FAKE, FAKE2, 16, 393216, None, 0, None) == LSE_ERR_WORKSPACE
    assert lib.log_softmax_rows(FAKE, FAKE2, 16, 393216, ctypes.c_void_p(0x7000000000), need - 1,
                                None) == LSE_ERR_WORKSPACE
    assert lib.log_softmax_rows_workspace_bytes(128, 4096) == 0
    assert lib.log_softmax_rows(None, None, 0, 8, None, 0, None) == LSE_OK


def test_rows_plan(lib):
    from log_softmax_reductions_amd import log_softmax_rows_plan
    assert log_softmax_rows_plan(393216) == (12, 32768)
    assert log_softmax_rows_plan(4096) == (1, 4096)
    assert log_softmax_rows_plan(16384) == (1, 16384)
    assert log_softmax_rows_plan(32768) == (1, 32768)
    for cols in (32769, 40000, 100001, 393216, 1 << 22):
        k, chunk = log_softmax_rows_plan(cols)
        assert k > 1 and chunk % 4 == 0 and chunk <= 32768
        assert (k - 1) * chunk < cols <= k * chunk


def test_partial_merge_validation(lib):
    assert lib.lse_rows_num_chunks(100, 7) == 15
    assert lib.lse_rows_num_chunks(0, 7) == -1
    assert lib.lse_rows_partial(FAKE, 4, 100, 0, FAKE2, None) == LSE_ERR_SHAPE
    assert lib.lse_rows_partial(None, 4, 100, 7, FAKE2, None) == LSE_ERR_NULL
    assert lib.lse_rows_merge(FAKE, 4, 0, FAKE2, None) == LSE_ERR_SHAPE
    assert lib.lse_rows_merge(None, 4, 3, FAKE2, None) == LSE_ERR_NULL


def test_partial_chunks_per_row_limit(lib):
    """One row's chunks run in one dispatch: more than 2^32 / 512 of them is a
    shape error, found before anything is launched."""
    assert lib.lse_rows_partial(FAKE, 1, 9_000_000, 1, FAKE2, None) == LSE_ERR_SHAPE
    assert b"exceed one launch" in lib.lse_last_error()


def test_rows_pointer_alignment(lib):
    """Row calls take float pointers on 4-byte boundaries (any 16-byte offset
    is fine); anything else is a shape error before any launch."""
    odd = ctypes.c_void_p(0x100000 + 2)
    assert lib.log_softmax_rows(odd, FAKE2, 4, 8, None, 0, None) == LSE_ERR_SHAPE
    assert b"4-byte aligned" in lib.lse_last_error()
    assert lib.softmax_rows(FAKE, ctypes.c_void_p(0x900000000 + 1), 4, 8, None, 0,
                            None) == LSE_ERR_SHAPE
    assert lib.lse_rows_partial(odd, 4, 8, 4, FAKE2, None) == LSE_ERR_SHAPE


def test_noalloc_validation(lib):
    """The static-scratch call refuses, before any launch, more row-chunk pairs
    than its scratch holds, and the usual shape errors."""
    assert lib.log_softmax_rows_noalloc(FAKE, FAKE2, 10921, 393216, None) == LSE_ERR_WORKSPACE
    assert b"131040" in lib.lse_last_error()
    assert lib.log_softmax_rows_noalloc(FAKE, FAKE2, 4, 0, None) == LSE_ERR_SHAPE
    assert lib.log_softmax_rows_noalloc(None, FAKE2, 4, 8, None) == LSE_ERR_NULL
    assert lib.log_softmax_rows_noalloc(FAKE, FAKE, 4, 8, None) == LSE_ERR_OVERLAP


def test_chain_validation(lib):
    args = lambda K=3, Cin=8, Cout=64, G=16, ws=FAKE2, wsb=1 << 30: (
        FAKE, FAKE, None, None, None, 2, Cin, 10, 10, Cout, K, G, ctypes.c_float(1e-5),
        ctypes.c_void_p(0x5000000000), ws, wsb, None)
    assert lib.fused_conv_gn_act_lse(*args(K=5)) == LSE_ERR_UNSUPPORTED
    assert lib.fused_conv_gn_act_lse(*args(Cin=3)) == LSE_ERR_UNSUPPORTED
    assert lib.fused_conv_gn_act_lse(*args(G=3)) == LSE_ERR_SHAPE          # 64 % 3 != 0
    assert lib.fused_conv_gn_act_lse(*args(G=32)) == LSE_ERR_UNSUPPORTED   # 2-channel groups
    assert lib.fused_conv_gn_act_lse(*args(ws=None)) == LSE_ERR_WORKSPACE
    assert lib.fused_conv_gn_act_lse(*args(wsb=16)) == LSE_ERR_WORKSPACE
    # out or the workspace on top of w, b, gamma or beta
    for i in (1, 2, 3, 4):
        a = list(args())
        a[i] = ctypes.c_void_p(0x5000000000 + 64)          # inside out
        assert lib.fused_conv_gn_act_lse(*a) == LSE_ERR_OVERLAP
        a[i] = ctypes.c_void_p(0x900000000 + 256)          # inside the workspace
        assert lib.fused_conv_gn_act_lse(*a) == LSE_ERR_OVERLAP
    need = lib.fused_conv_gn_act_lse_workspace_bytes(128, 8, 128, 128, 64, 3, 16)
    # mean and rstd (N x G floats each), a 256-byte header, one 8-byte word per
    # (n, tile, g), one 8-byte arrival word per sample, one 4-byte queue slot
    # per tile pair (32 per sample)
    assert need == 2 * 128 * 16 * 4 + 256 + 128 * 63 * 16 * 8 + 128 * 8 + 128 * 32 * 4


def test_last_error_is_per_thread(lib):
    """Each host thread sees the detail of its own last failure."""
    import threading
    seen = {}

    def worker(i):
        rows = -1 - i
        assert lib.log_softmax_rows(FAKE, FAKE2, rows, 8, None, 0, None) == LSE_ERR_SHAPE
        for _ in range(200):
            pass
        seen[i] = lib.lse_last_error().decode()

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    for i in range(8):
        assert f"rows = {-1 - i}" in seen[i], seen[i]

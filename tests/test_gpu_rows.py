"""GPU parity of log_softmax_rows, lse_rows_partial and lse_rows_merge (through
the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _lsm(x_dev, ws=None):
    y = L.log_softmax_rows(x_dev, ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_rows_small_workload(orc):
    """(128, 4096) with 1% x50 outliers and 1% -inf entries."""
    x = inputs.make("rows_small", DEV)
    y = _lsm(x)
    ref, _ = orc.log_softmax_rows(x.cpu().numpy())
    s = compare(y, ref, what="rows_small")
    print("rows_small", s)


@pytest.mark.parametrize("cols", [1, 3, 4, 63, 64, 65, 1000, 1024, 1025, 4097, 16383, 16384,
                                  16385, 20000, 32767, 32768, 32769, 49153, 100001, 131072])
@pytest.mark.parametrize("rows", [1, 3, 7])
def test_rows_shapes(orc, rows, cols):
    x = inputs.normal((rows, cols), seed=rows * 1000003 + cols, sigma=4.0, device=DEV)
    ref, _ = orc.log_softmax_rows(x.cpu().numpy())
    compare(_lsm(x), ref, what=f"rows={rows} cols={cols}")


@pytest.mark.parametrize("cols", [4096, 65536])
def test_rows_misaligned(orc, cols):
    buf = inputs.normal((3 * cols + 1,), seed=cols, device=DEV)
    x = buf[1:].view(3, cols)
    ref, _ = orc.log_softmax_rows(x.cpu().numpy())
    compare(_lsm(x), ref, what="misaligned")


SHORT_COLS = [1, 2, 3, 4, 5, 8, 10, 16, 17, 32, 64, 100, 128, 255, 256, 257, 512, 999, 1000,
              1024]


@pytest.mark.parametrize("cols", [4, 8, 16, 32, 64, 128, 256, 1000, 1024, 3, 10, 17, 255, 999])
@pytest.mark.parametrize("softmax", [False, True])
def test_rows_short_special_values(orc, cols, softmax):
    """Rows of at most 1024 columns run one segment of lanes per row (several
    rows per wave below 256 columns): special values in neighbouring rows of
    one wave, a partial last workgroup (9 rows), aligned (cols % 4 == 0) and
    scalar rows; the row logsumexp through lse_reduce_axis on the same rows."""
    x = inputs.normal((9, cols), seed=cols + 7, device=DEV).cpu()
    x[0, :] = -float("inf")                       # all -inf
    x[1, cols // 2] = float("inf")                # +inf
    x[2, cols - 1] = float("nan")                 # NaN
    x[3, :] = -float("inf"); x[3, 0] = 2.5        # one finite entry
    x[4, :] = 3.0                                 # equal values
    x[5, 1] = 1e30                                # huge
    x[6, ::2] = -float("inf")
    xd = x.to(DEV)
    if softmax:
        y = L.softmax_rows(xd)
        torch.cuda.synchronize()
        compare(y.cpu().numpy(), orc.softmax_rows(x.numpy()), what=f"short softmax {cols}",
                rtol=1e-5, atol=1e-37)
    else:
        ref, _ = orc.log_softmax_rows(x.numpy())
        compare(_lsm(xd), ref, what=f"short rows {cols}")
        out = L.lse_reduce_axis(xd, 1)
        torch.cuda.synchronize()
        compare(out.cpu().numpy(), orc.lse_axis(x.numpy().reshape(9, cols, 1)).reshape(9),
                what=f"short row lse {cols}")


@pytest.mark.parametrize("cols", SHORT_COLS)
@pytest.mark.parametrize("layout", ["packed", "pitch", "offset"])
def test_rows_short_ragged(orc, cols, layout):
    """1037 short rows (a ragged last wave at every segment width): packed,
    at a pitch of cols + 3 (a column slice), and at a 4-byte offset; the
    log_softmax rows, the softmax rows and the row logsumexp against the
    oracle, and the values around each output left alone."""
    rows = 1037
    pad, off = {"packed": (0, 0), "pitch": (3, 0), "offset": (0, 1)}[layout]
    buf = inputs.normal((rows * (cols + pad) + off,), seed=cols * 3 + pad + off, sigma=3.0,
                        device=DEV)
    x = buf[off:].view(rows, cols + pad)[:, :cols]
    xc = x.cpu().numpy()
    ref, _ = orc.log_softmax_rows(xc)
    compare(_lsm(x), ref, what=f"short ragged {layout} {cols}")
    ybuf = torch.full((rows * (cols + pad) + off,), 7.0, device=DEV)
    y = ybuf[off:].view(rows, cols + pad)[:, :cols]
    L.softmax_rows(x, y)
    obuf = torch.full((2 * rows + 1,), 7.0, device=DEV)
    out = obuf[1:].view(rows, 2)[:, 0]            # every other float, one float in
    L.lse_reduce_axis(x, 1, out=out)
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), orc.softmax_rows(xc), what=f"short ragged softmax {layout} {cols}",
            rtol=1e-5, atol=1e-37)
    compare(out.cpu().numpy(), orc.lse_axis(xc.reshape(rows, cols, 1)).reshape(rows),
            what=f"short ragged lse {layout} {cols}")
    if pad:
        assert (ybuf[off:].view(rows, cols + pad)[:, cols:] == 7.0).all()
    assert ybuf[:off].eq(7.0).all() and obuf[0].item() == 7.0
    assert (obuf[1:].view(rows, 2)[:, 1] == 7.0).all()


@pytest.mark.parametrize("rows,cols,off", [(3000, 1025, 0), (2000, 1500, 1), (1000, 2048, 0),
                                           (500, 2049, 0), (700, 3001, 1), (600, 3072, 0),
                                           (500, 4095, 0), (400, 4096, 1), (300, 4096, 0),
                                           (40, 50257, 0), (30, 50257, 1), (2000, 16385, 0)])
def test_row_logsumexp_segments_and_split(orc, rows, cols, off):
    """Last-axis logsumexp: rows up to 2048 values in wave-wide segments (up
    to 32 values per lane), up to 4096 off the 16-byte grid or up to 3072
    aligned (64 per lane; aligned 4096 keeps the workgroup kernel), longer rows
    off the 16-byte grid (odd lengths, a 4-byte offset) split into chunk pairs
    whatever the number of rows."""
    buf = inputs.normal((rows * cols + off,), seed=rows + cols + off, sigma=3.0, device=DEV)
    x = buf[off:].view(rows, cols)
    x[1, 7] = float("inf")
    x[2, :] = -float("inf")
    x[3, cols - 1] = float("nan")
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    ref = orc.lse_axis(x.cpu().numpy().reshape(rows, cols, 1)).reshape(rows)
    compare(out.cpu().numpy(), ref, what=f"row lse {rows}x{cols}+{off}")


def test_rows_short_many_rows(orc):
    """200003 rows of 256 and 2000003 rows of 10: every row's log_softmax
    sums to 1, sampled rows (first, last, partial last workgroup) against the
    oracle, logsumexp and log_softmax."""
    for rows, cols in ((200003, 256), (2000003, 10)):
        x = inputs.normal((rows, cols), seed=11 + cols, sigma=3.0, device=DEV)
        y = L.log_softmax_rows(x)
        out = L.lse_reduce_axis(x, 1)
        torch.cuda.synchronize()
        assert (torch.logsumexp(y.double(), 1)).abs().max().item() < 1e-5
        idx = [0, 1, 2, 3, 4, rows // 2, rows - 4, rows - 3, rows - 2, rows - 1]
        xs = x[idx].cpu().numpy()
        ref, _ = orc.log_softmax_rows(xs)
        compare(y[idx].cpu().numpy(), ref, what=f"short many rows {cols}")
        compare(out[idx].cpu().numpy(), orc.lse_axis(xs.reshape(len(idx), cols, 1)).reshape(-1),
                what=f"short many rows lse {cols}")


def test_rows_special_values(orc):
    cols = 40000   # split across 3 workgroups
    x = inputs.normal((8, cols), seed=5, device=DEV).cpu()
    x[0, :] = -float("inf")                       # all -inf -> NaN row
    x[1, 12345] = float("inf")                    # +inf -> -inf / NaN
    x[2, 30000] = float("nan")                    # NaN -> NaN row
    x[3, :] = -float("inf"); x[3, 39999] = 2.5    # one finite entry -> 0 there
    x[4, :] = 3.0                                 # equal -> -log(cols)
    x[5, :20000] = -float("inf")                  # first chunks entirely -inf
    x[6, ::2] = -float("inf")
    x[7, 17] = 1e30
    y = _lsm(x.to(DEV))
    ref, _ = orc.log_softmax_rows(x.numpy())
    compare(y, ref, what="special")
    assert np.isnan(y[0]).all() and np.isnan(y[2]).all()
    assert y[3, 39999] == 0.0


def test_rows_mostly_empty_workgroup(orc):
    """Workgroups in which most lanes and whole waves hold no data: the (-inf, 0)
    identity must not turn into NaN (the failure the log_softmax page hit)."""
    for cols in (5, 70, 16385):
        x = inputs.normal((4, cols), seed=cols, device=DEV)
        ref, _ = orc.log_softmax_rows(x.cpu().numpy())
        y = _lsm(x)
        assert np.isfinite(y).all()
        compare(y, ref, what=f"cols={cols}")


def test_rows_workspace_contents_irrelevant(orc):
    x = inputs.normal((16, 50000), seed=77, device=DEV)
    nbytes = L.log_softmax_rows_workspace_bytes(16, 50000)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=DEV)
    ref, _ = orc.log_softmax_rows(x.cpu().numpy())
    compare(_lsm(x, ws), ref, what="dirty workspace")
    compare(_lsm(x, ws), ref, what="reused workspace")


def test_rows_large_workload(orc):
    """(4096, 393216) N(0, 1): 12 workgroups per row.  Every element against
    the oracle (blocks of 1024 rows), every row against properties that hold
    at any size, and run-to-run bit equality."""
    rows, cols = 4096, 393216
    x = inputs.make("rows_large", DEV)
    assert L.log_softmax_rows_plan(cols) == (12, 32768)
    y = L.log_softmax_rows(x)
    torch.cuda.synchronize()
    block = 1024
    for r0 in range(0, rows, block):
        ref, _ = orc.log_softmax_rows(x[r0:r0 + block].cpu().numpy())
        s = compare(y[r0:r0 + block].cpu().numpy(), ref, what=f"rows_large rows {r0}+")
        print("rows_large rows", r0, s)
        del ref
    # every row: logsumexp of y is 0 and y <= 0, evaluated in fp64 on the GPU
    lse = torch.logsumexp(y.double(), dim=1)
    assert lse.abs().max().item() < 1e-5
    assert (y <= 0).all().item()
    y2 = L.log_softmax_rows(x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


# ------------------------------------------------------------ partial/merge

@pytest.mark.parametrize("cols,chunk", [(393216 // 8, 49152 // 24), (4096, 4096), (4096, 2048),
                                        (4096, 1366), (50000, 2084), (4096, 64), (999, 7),
                                        (70000, 70000), (70000, 20000)])
def test_partials_and_merge(orc, cols, chunk):
    rows = 6
    x = inputs.normal((rows, cols), seed=cols + chunk, sigma=2.0, device=DEV)
    p = L.lse_rows_partial(x, chunk)
    lse = L.lse_rows_merge(p)
    torch.cuda.synchronize()
    xn = x.cpu().numpy()
    m_ref, s_ref = orc.lse_chunk_partials(xn, chunk)
    pc = p.cpu().numpy()
    assert np.array_equal(pc[..., 0], m_ref.astype(np.float32)), "chunk max must be exact"
    compare(pc[..., 1], s_ref, atol=0.0, rtol=1e-5, what="chunk sums")
    _, lse_ref = orc.log_softmax_rows(xn, want_y=False)
    compare(lse.cpu().numpy(), lse_ref, what="merged row lse")


def test_merge_of_oracle_pairs(orc):
    """lse_rows_merge on given pairs (including identities and +inf pairs)."""
    rng = np.random.default_rng(3)
    m = rng.normal(scale=10, size=(5, 40)).astype(np.float32)
    s = rng.uniform(1, 50, size=(5, 40)).astype(np.float32)
    m[1, :] = -np.inf; s[1, :] = 0          # all identity -> -inf
    m[2, 5:] = -np.inf; s[2, 5:] = 0        # mostly identity
    m[3, 7] = np.inf; s[3, 7] = 2           # +inf pair -> +inf
    s[4, 9] = np.nan                        # NaN -> NaN
    pairs = torch.from_numpy(np.stack([m, s], axis=-1)).to(DEV)
    got = L.lse_rows_merge(pairs).cpu().numpy()
    ref, _, _ = orc.lse_merge(m.astype(np.float64), s.astype(np.float64))
    compare(got, ref, what="merge")


def test_partials_special_values(orc):
    x = torch.tensor([[-np.inf, -np.inf, 1.0, 2.0, np.inf, np.inf, np.nan, 0.0, -np.inf, np.nan]],
                     dtype=torch.float32)
    p = L.lse_rows_partial(x.to(DEV), 2).cpu().numpy()[0]
    m_ref, s_ref = orc.lse_chunk_partials(x.numpy(), 2)
    assert p[0, 0] == -np.inf and p[0, 1] == 0.0
    assert p[1, 0] == 2.0 and abs(p[1, 1] - s_ref[0, 1]) < 1e-6
    assert p[2, 0] == np.inf and p[2, 1] == 2.0
    assert p[3, 0] == 0.0 and np.isnan(p[3, 1])
    assert p[4, 0] == -np.inf and np.isnan(p[4, 1])
    assert np.array_equal(p[:, 0], m_ref[0].astype(np.float32))


def test_rows_helping_path(orc):
    """With the test hook's poll limit at 0 no workgroup publishes its own pair:
    every pair is computed from x by the helping path (a workgroup that finds
    a sibling's slot empty).  Results must match the oracle, the workspace
    must count exactly rows x chunks helped pairs, and the output must be
    bit-identical to the default path's (a helper reproduces the owner's
    arithmetic), on full and partial chunks."""
    rows, cols = 64, 393216
    x = inputs.normal((rows, cols), seed=31, device=DEV)
    nbytes = L.log_softmax_rows_workspace_bytes(rows, cols)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    sample = [0, 5, 33, 63]
    ref, _ = orc.log_softmax_rows(x[sample].cpu().numpy())
    try:
        L.lse_testing_set_spin_limit(0)
        y = L.log_softmax_rows(x, ws=ws)
        torch.cuda.synchronize()
    finally:
        L.lse_testing_set_spin_limit(1 << 24)
    helped = int(ws[4:8].view(torch.int32).item())
    assert helped == rows * 12, helped      # every pair came from the helping path
    compare(y[sample].cpu().numpy(), ref, what="helping path")
    assert torch.logsumexp(y.double(), dim=1).abs().max().item() < 1e-5
    print("pairs computed by a sibling:", helped)
    y2 = L.log_softmax_rows(x, ws=ws)
    torch.cuda.synchronize()
    compare(y2[sample].cpu().numpy(), ref, what="default path after")
    assert torch.equal(y, y2)
    assert int(ws[4:8].view(torch.int32).item()) == 0


@pytest.mark.parametrize("rows,cols,softmax", [(16, 100003, False), (8, 262147, True),
                                                (24, 393216, True)])
def test_rows_helping_path_bit_identical(rows, cols, softmax):
    """Helping path against the default path, bit for bit: odd row lengths
    (the scalar path, a partial last chunk) and softmax."""
    x = inputs.normal((rows, cols), seed=cols % 97, device=DEV)
    fn = L.softmax_rows if softmax else L.log_softmax_rows
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(rows, cols), dtype=torch.uint8,
                     device=DEV)
    nchunks, _ = L.log_softmax_rows_plan(cols)
    try:
        L.lse_testing_set_spin_limit(0)
        y = fn(x, ws=ws)
        torch.cuda.synchronize()
    finally:
        L.lse_testing_set_spin_limit(1 << 24)
    assert int(ws[4:8].view(torch.int32).item()) == rows * nchunks
    y2 = fn(x, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_rows_more_workgroups_than_one_launch(orc):
    """(8400000, 64): one workgroup per row is more than a single dispatch can
    hold (8388607 workgroups of 512 lanes), so the rows run as two launches;
    the partial / merge pair with 2 chunks per row as well.  Sampled rows on
    both sides of the split against the oracle, every row by property."""
    rows, cols = 8_400_000, 64
    x = inputs.normal((rows, cols), seed=77, device=DEV)
    y = L.log_softmax_rows(x)
    p = L.lse_rows_partial(x, 32)
    lse = L.lse_rows_merge(p)
    torch.cuda.synchronize()
    sample = [0, 1, 4_194_303, 4_194_304, 8_388_606, 8_388_607, 8_388_608, rows - 1]
    ref, lref = orc.log_softmax_rows(x[sample].cpu().numpy())
    compare(y[sample].cpu().numpy(), ref, what="rows")
    compare(lse[sample].cpu().numpy(), lref, what="partial/merge")
    tail = slice(rows - 200_000, rows)
    assert torch.logsumexp(y[tail].double(), dim=1).abs().max().item() < 1e-5
    assert (lse[tail] - torch.logsumexp(x[tail], dim=1)).abs().max().item() < 1e-4


def test_rows_beyond_2g_elements(orc):
    """(6000, 393216): 2.36e9 elements (9.4 GB in, 9.4 GB out), past 32-bit
    element offsets; sampled rows against the oracle, every row by property."""
    rows, cols = 6000, 393216
    x = inputs.normal((rows, cols), seed=45, device=DEV)
    y = L.log_softmax_rows(x)
    torch.cuda.synchronize()
    sample = [0, 1, 2999, 5461, 5462, 5998, 5999]
    ref, _ = orc.log_softmax_rows(x[sample].cpu().numpy())
    compare(y[sample].cpu().numpy(), ref, what="rows > 2^31 elements")
    lse = torch.stack([torch.logsumexp(y[i:i + 500].double(), dim=1) for i in range(0, rows, 500)])
    assert lse.abs().max().item() < 1e-5
    del x, y
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- softmax
SOFTMAX_ATOL, SOFTMAX_RTOL = 1e-37, 1e-5


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 63), (7, 4096), (2, 16385), (4, 100001),
                                       (3, 393216)])
def test_softmax_rows(orc, rows, cols):
    x = inputs.normal((rows, cols), seed=rows * 13 + cols, sigma=3.0, device=DEV)
    y = L.softmax_rows(x)
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), orc.softmax_rows(x.cpu().numpy()), atol=SOFTMAX_ATOL,
            rtol=SOFTMAX_RTOL, what=f"softmax {rows}x{cols}")


def test_softmax_rows_small_workload_and_special(orc):
    x = inputs.make("rows_small", DEV)
    compare(L.softmax_rows(x).cpu().numpy(), orc.softmax_rows(x.cpu().numpy()),
            atol=SOFTMAX_ATOL, rtol=SOFTMAX_RTOL, what="softmax rows_small")
    s = inputs.normal((4, 40000), seed=9, device=DEV).cpu()
    s[0, :] = -float("inf")
    s[1, 7] = float("inf")
    s[2, 39000] = float("nan")
    s[3, :30000] = -float("inf")
    compare(L.softmax_rows(s.to(DEV)).cpu().numpy(), orc.softmax_rows(s.numpy()),
            atol=SOFTMAX_ATOL, rtol=SOFTMAX_RTOL, what="softmax special")


@pytest.mark.parametrize("rows,cols,xoff,yoff,softmax", [
    (40, 393215, 0, 0, False),     # odd row length: every row starts elsewhere
    (24, 393216, 1, 0, False),     # x one float past a 16-byte boundary, y aligned
    (24, 393216, 3, 3, True),      # both off by the same amount: 16-byte stores
    (16, 100002, 2, 1, False),     # x and y off by different amounts
    (64, 32767, 0, 0, True),       # one workgroup per row (no split), odd length
    (33, 5, 1, 2, False),          # rows shorter than a 16-byte vector
    (7, 3, 0, 0, False)])
def test_rows_head_tail(orc, rows, cols, xoff, yoff, softmax):
    """Rows that do not sit on 16-byte boundaries: the aligned body goes
    through the 128-bit register tile, the head and tail values beside it.
    Every element against the oracle, and the helping path bit-identical."""
    xb = inputs.normal((rows * cols + xoff,), seed=cols + 7 * xoff, device=DEV)
    x = xb[xoff:].view(rows, cols)
    yb = torch.full((rows * cols + yoff,), float("nan"), device=DEV)
    y = yb[yoff:].view(rows, cols)
    fn = L.softmax_rows if softmax else L.log_softmax_rows
    ws = torch.empty(max(1, L.log_softmax_rows_workspace_bytes(rows, cols)), dtype=torch.uint8,
                     device=DEV)
    fn(x, y, ws=ws)
    torch.cuda.synchronize()
    xc = x.cpu().numpy()
    if softmax:
        compare(y.cpu().numpy(), orc.softmax_rows(xc), atol=1e-37, rtol=1e-5, what="head/tail sm")
    else:
        compare(y.cpu().numpy(), orc.log_softmax_rows(xc)[0], what="head/tail")
    assert torch.isnan(yb[:yoff]).all()
    nchunks, _ = L.log_softmax_rows_plan(cols)
    if nchunks > 1:
        # y2 at y's offset: the same kernel and chunk partition as the first call
        y2 = torch.empty((rows * cols + yoff,), device=DEV)[yoff:].view(rows, cols)
        try:
            L.lse_testing_set_spin_limit(0)
            fn(x, y2, ws=ws)
            torch.cuda.synchronize()
        finally:
            L.lse_testing_set_spin_limit(1 << 24)
        assert int(ws[4:8].view(torch.int32).item()) == rows * nchunks
        diff = (y != y2).nonzero()
        assert diff.numel() == 0, (f"{diff.shape[0]} differ; first {diff[:6].tolist()}; "
                                   f"y {y[diff[:6, 0], diff[:6, 1]].tolist()} "
                                   f"y2 {y2[diff[:6, 0], diff[:6, 1]].tolist()}")


@pytest.mark.parametrize("cols,chunk,off", [(5003, 1001, 1), (4096, 1000, 2), (70001, 16383, 3)])
def test_partials_head_tail(orc, cols, chunk, off):
    """Chunks whose starts and lengths are not multiples of 4 floats."""
    xb = inputs.normal((6 * cols + off,), seed=chunk, device=DEV)
    x = xb[off:].view(6, cols)
    p = L.lse_rows_partial(x, chunk)
    lse = L.lse_rows_merge(p)
    torch.cuda.synchronize()
    m_ref, s_ref = orc.lse_chunk_partials(x.cpu().numpy(), chunk)
    pc = p.cpu().numpy()
    assert np.array_equal(pc[..., 0], m_ref.astype(np.float32))
    compare(pc[..., 1], s_ref, atol=0.0, rtol=1e-5, what="partial sums")
    compare(lse.cpu().numpy(), orc.log_softmax_rows(x.cpu().numpy())[1], what="merge")


def test_rows_head_tail_full_size(orc):
    """(4096, 393215) and the (4096, 393216) workload one float off a 16-byte
    boundary: sampled rows against the oracle, every row by property."""
    for cols, off in ((393215, 0), (393216, 1)):
        print(f"case: head/tail full size cols={cols} off={off}", flush=True)
        xb = inputs.normal((4096 * cols + off,), seed=41, device=DEV)
        x = xb[off:].view(4096, cols)
        y = L.log_softmax_rows(x)
        torch.cuda.synchronize()
        sample = [0, 1, 2, 3, 2047, 4095]
        compare(y[sample].cpu().numpy(), orc.log_softmax_rows(x[sample].cpu().numpy())[0],
                what=f"full size {cols} {off}")
        for r0 in range(0, 4096, 512):
            assert torch.logsumexp(y[r0:r0 + 512].double(), dim=1).abs().max().item() < 1e-5
        del xb, x, y


@pytest.mark.parametrize("rows,cols,softmax", [(64, 393216, False), (16, 100000, True),
                                               (8, 65540, False)])
def test_rows_reread_variant(orc, rows, cols, softmax):
    """The MALL re-read form of the split rows (test hook): every element
    against the oracle; the helping path against the default of the same form
    within the tolerance."""
    x = inputs.normal((rows, cols), seed=rows + cols, device=DEV)
    fn = L.softmax_rows if softmax else L.log_softmax_rows
    try:
        L.lse_testing_set_rows_reread(True)
        y = fn(x)
        torch.cuda.synchronize()
    finally:
        L.lse_testing_set_rows_reread(False)
    xc = x.cpu().numpy()
    if softmax:
        compare(y.cpu().numpy(), orc.softmax_rows(xc), atol=1e-37, rtol=1e-5, what="reread sm")
    else:
        compare(y.cpu().numpy(), orc.log_softmax_rows(xc)[0], what="reread")


@pytest.mark.parametrize("cols,off", [(50000003, 0), (40000000, 1)])
def test_rows_long_streams_within_tolerance(orc, cols, off):
    """Whole rows streamed by one workgroup (the axis entry points without a
    workspace over a contiguous last axis): each lane adds ~100K terms, most
    far below its running sum; the plain sum rounded them away (2.2 x the
    tolerance for the logsumexp of (2, 50000003) at sigma 3, 3.6 x for its
    log_softmax).  The logsumexp is checked against the oracle, log_softmax at
    sampled columns against x - LSE in fp64."""
    from log_softmax_reductions_amd import _lib
    lib = _lib.load()
    rows = 2
    buf = inputs.normal((rows * cols + off,), seed=cols, sigma=3.0, device="cuda")
    x = buf[off:].view(rows, cols)
    st = torch.cuda.current_stream().cuda_stream
    o = torch.empty(rows, device="cuda")
    y = torch.empty_like(x)
    _lib.check(lib.lse_reduce_axis(x.data_ptr(), o.data_ptr(), rows, cols, 1, st), "lse")
    _lib.check(lib.log_softmax_axis(x.data_ptr(), y.data_ptr(), rows, cols, 1, st), "lsm")
    torch.cuda.synchronize()
    xc = x.cpu().numpy()
    _, lse = orc.log_softmax_rows(xc, want_y=False)
    compare(o.cpu().numpy(), lse, what=f"long row lse ({rows},{cols})+{off}")
    idx = np.arange(0, cols, 997)
    ref = xc[:, idx].astype(np.float64) - lse[:, None]
    compare(y.cpu().numpy()[:, idx], ref, what=f"long row lsm ({rows},{cols})+{off}")


@pytest.mark.parametrize("rows,cols,off", [(8193, 8192, 0), (8195, 6144, 0), (8192, 12288, 0),
                                           (8194, 16384, 0), (8193, 8191, 0), (8192, 16383, 0),
                                           (8195, 6145, 0), (8192, 16384, 1), (8193, 8192, 3)])
@pytest.mark.parametrize("softmax", [False, True])
def test_rows_multi_row_workgroups(orc, rows, cols, off, softmax):
    """Rows of 6144-16384 columns, at least 8192 of them, share a workgroup (4
    or 2 rows, 64 values per lane): aligned, odd lengths (16-byte accesses at
    each row's phase, the last cols % 4 values in extra registers) and views
    at a 4- or 12-byte offset; a ragged last workgroup and special values in
    rows of one workgroup.  Sampled rows against the oracle, every row through
    the property that its outputs are a distribution, and the row logsumexp
    of sampled rows."""
    buf = inputs.normal((rows * cols + off,), seed=rows + cols + off, sigma=3.0, device=DEV)
    x = buf[off:].view(rows, cols)
    x[0, :] = -float("inf")
    x[1, 5] = float("inf")
    x[2, cols - 1] = float("nan")
    x[3, :] = -float("inf"); x[3, 17] = 2.0
    y = L.softmax_rows(x) if softmax else L.log_softmax_rows(x)
    torch.cuda.synchronize()
    idx = [0, 1, 2, 3, 4, 5, rows // 2, rows - 3, rows - 2, rows - 1]
    xs = x[idx].cpu().numpy()
    if softmax:
        compare(y[idx].cpu().numpy(), orc.softmax_rows(xs), rtol=1e-5, atol=1e-37,
                what=f"multi-row softmax {rows}x{cols}+{off}")
        tot = y[4:].double().sum(1)
    else:
        ref, _ = orc.log_softmax_rows(xs)
        compare(y[idx].cpu().numpy(), ref, what=f"multi-row log_softmax {rows}x{cols}+{off}")
        tot = y[4:].double().exp().sum(1)
    assert (tot - 1.0).abs().max().item() < 1e-4
    out = L.lse_reduce_axis(x, 1)
    torch.cuda.synchronize()
    compare(out[idx].cpu().numpy(), orc.lse_axis(xs.reshape(len(idx), cols, 1)).reshape(-1),
            what=f"multi-row logsumexp {rows}x{cols}+{off}")

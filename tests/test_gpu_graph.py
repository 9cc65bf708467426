"""Every entry point captured in a HIP graph (via torch.cuda.graph) must give,
on every replay, bit-for-bit the result of the same call made eagerly.  The
library enqueues only kernels (workspace clears included), so capture needs no
special mode.  Replays are interleaved with unrelated eager work and host
synchronisations, as a caller's loop would be."""
import pytest
import torch

import log_softmax_reductions_amd as L
from log_softmax_reductions_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _eager_noise():
    a = torch.randn(1 << 20, device=DEV)
    (a * 2).sum().item()


def _check_graph(run, outs, replays=4):
    """run() enqueues the library calls writing into `outs`."""
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o in outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # warm up on a side stream before capture
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"


def test_graph_axis0():
    x = inputs.normal((32, 64, 1024), seed=1, sigma=2.0, device=DEV)
    out = torch.empty((64, 1024), device=DEV)
    _check_graph(lambda: L.lse_reduce_axis0(x, out), [out])


def test_graph_rows_split_and_short():
    x1 = inputs.normal((16, 393216), seed=2, device=DEV)
    y1 = torch.empty_like(x1)
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(16, 393216), dtype=torch.uint8,
                     device=DEV)
    x2 = inputs.make("rows_small", DEV)
    y2 = torch.empty_like(x2)

    def run():
        L.log_softmax_rows(x1, y1, ws)
        L.log_softmax_rows(x2, y2)
    _check_graph(run, [y1, y2])


def test_graph_partial_merge():
    x = inputs.normal((8, 50000), seed=3, device=DEV)
    p = torch.empty((8, L.lse_rows_num_chunks(50000, 4096), 2), device=DEV)
    lse = torch.empty(8, device=DEV)

    def run():
        L.lse_rows_partial(x, 4096, p)
        L.lse_rows_merge(p, lse)
    _check_graph(run, [p, lse])


def test_graph_conv_chain():
    x, w, b, g, be = inputs.conv_chain_inputs(N=8, H=40, W=40, seed=5, device=DEV)
    out = torch.empty((8, 1, 38, 38), device=DEV)
    ws = torch.empty(L.fused_conv_gn_act_lse_workspace_bytes(8, 8, 40, 40, 64, 3, 16),
                     dtype=torch.uint8, device=DEV)
    _check_graph(lambda: L.fused_conv_gn_act_lse(x, w, b, g, be, 16, 1e-5, out, ws), [out])


def test_graph_axis_and_softmax():
    x = inputs.normal((16, 64, 500), seed=6, device=DEV)
    o1 = torch.empty((16, 500), device=DEV)
    o2 = torch.empty_like(x)
    x3 = inputs.normal((8, 100000), seed=7, device=DEV)
    o3 = torch.empty_like(x3)
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(8, 100000), dtype=torch.uint8, device=DEV)

    def run():
        L.lse_reduce_axis(x, 1, o1)
        L.log_softmax_axis(x, 1, o2)
        L.softmax_rows(x3, o3, ws)
    _check_graph(run, [o1, o2, o3])


def test_graph_strided_calls():
    big = inputs.normal((6, 40, 300), seed=8, device=DEV)
    x = big[:, 4:36, :256]                      # strided view: planes 300 apart, 256 wide
    o1 = torch.empty((6, 256), device=DEV)
    o2 = torch.empty((6, 32, 256), device=DEV)
    rows_big = inputs.normal((8, 60004), seed=9, device=DEV)
    xr = rows_big[:, :60000]                    # row pitch 60004
    yr = torch.empty((8, 60000), device=DEV)
    ws = torch.empty(L.log_softmax_rows_workspace_bytes(8, 60000), dtype=torch.uint8,
                     device=DEV)

    def run():
        L.lse_reduce_axis(x, 1, o1)
        L.log_softmax_axis(x, 1, o2)
        L.log_softmax_rows(xr, yr, ws)
    _check_graph(run, [o1, o2, yr])


def test_graph_split_axis_and_long_rows():
    """The split paths: 16 outputs over 200000 planes (column split, the
    binding's workspace allocated inside the capture), a row of 4.4M columns
    (three launches), split logsumexp rows, short rows in segments."""
    x = inputs.normal((200000, 16), seed=10, device=DEV)
    o1 = torch.empty(16, device=DEV)
    o2 = torch.empty_like(x)
    x2 = inputs.normal((1, 4400000), seed=11, device=DEV)
    y2 = torch.empty_like(x2)
    ws2 = torch.empty(L.log_softmax_rows_workspace_bytes(1, 4400000), dtype=torch.uint8,
                      device=DEV)
    x3 = inputs.normal((4, 40000), seed=12, device=DEV)
    o3 = torch.empty(4, device=DEV)
    x4 = inputs.normal((3000, 100), seed=13, device=DEV)
    y4 = torch.empty_like(x4)

    def run():
        L.lse_reduce_axis0(x, o1)
        L.log_softmax_axis(x, 0, o2)
        L.log_softmax_rows(x2, y2, ws2)
        L.lse_reduce_axis(x3, 1, o3)
        L.log_softmax_rows(x4, y4)
    _check_graph(run, [o1, o2, y2, o3, y4])


def test_graph_contiguous_blocks():
    """Contiguous blocks of short runs: chunk pairs then a merge (logsumexp),
    register-resident chunks that wait for each other after a clear kernel
    (log_softmax over 2200 chunk workgroups), a block per workgroup held in
    registers, workspaces passed in (no allocation inside the capture)."""
    x = inputs.normal((40, 4000, 49), seed=14, device=DEV)
    o = torch.empty((40, 49), device=DEV)
    wso = torch.empty(max(1, L.lse_axis_workspace_bytes(40, 4000, 49)), dtype=torch.uint8, device=DEV)
    x2 = inputs.normal((1100, 1000, 49), seed=15, device=DEV)
    y2 = torch.empty_like(x2)
    ws2 = torch.empty(L.lse_axis_workspace_bytes(1100, 1000, 49, True), dtype=torch.uint8,
                      device=DEV)
    x3 = inputs.normal((3000, 100, 49), seed=16, device=DEV)
    y3 = torch.empty_like(x3)

    def run():
        L.lse_reduce_axis(x, 1, o, ws=wso)
        L.log_softmax_axis(x2, 1, y2, ws=ws2)
        L.log_softmax_axis(x3, 1, y3)
    _check_graph(run, [o, y2, y3])


def test_concurrent_streams_match_sequential():
    """Calls on two streams at once, each with its own workspace, give the
    sequential results bit for bit: no state is shared between calls."""
    xa = inputs.normal((16, 200000), seed=10, device=DEV)
    xb = inputs.normal((16, 200000), seed=11, device=DEV)
    ca = inputs.conv_chain_inputs(N=8, H=60, W=60, seed=12, device=DEV)
    cb = inputs.conv_chain_inputs(N=8, H=60, W=60, seed=13, device=DEV)
    seq = [L.log_softmax_rows(xa), L.log_softmax_rows(xb),
           L.fused_conv_gn_act_lse(*ca, 16, 1e-5), L.fused_conv_gn_act_lse(*cb, 16, 1e-5)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = L.log_softmax_rows(xa)
            oa = L.fused_conv_gn_act_lse(*ca, 16, 1e-5)
        with torch.cuda.stream(s2):
            yb = L.log_softmax_rows(xb)
            ob = L.fused_conv_gn_act_lse(*cb, 16, 1e-5)
        torch.cuda.synchronize()
        for got, ref in zip((ya, yb, oa, ob), seq):
            assert torch.equal(got, ref)


def test_concurrent_streams_block_split():
    """Two streams each running the register-resident block split (chunks that
    wait for each other, workspaces from the binding) while the other holds
    part of the GPU: both results equal the sequential ones bit for bit."""
    xa = inputs.normal((1100, 1000, 49), seed=21, device=DEV)
    xb = inputs.normal((700, 701, 127), seed=22, device=DEV)
    seq = [L.log_softmax_axis(xa, 1), L.log_softmax_axis(xb, 1)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = L.log_softmax_axis(xa, 1)
        with torch.cuda.stream(s2):
            yb = L.log_softmax_axis(xb, 1)
        torch.cuda.synchronize()
        assert torch.equal(ya, seq[0]) and torch.equal(yb, seq[1])

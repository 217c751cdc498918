"""The calls inside a captured HIP graph: replays give the same bits as
eager calls, with other eager work (which overwrites the same outputs and
uses the same workspace) between the replays."""
import numpy as np
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_graph_replays_match_eager():
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    dev = G.torch_dev()
    x1 = G.to_dev(synth.glu_activation(0, K))
    x2 = G.to_dev(synth.glu_activation(1, K))
    t1 = synth.percentile_threshold(synth.glu_activation(0, K), 0.5)
    t2 = synth.percentile_threshold(synth.glu_activation(1, K), 0.8)
    idx = torch.zeros(K, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    idx2 = torch.zeros(K, dtype=torch.int32, device=dev)
    cnt2 = torch.zeros(1, dtype=torch.int32, device=dev)
    yf = torch.zeros(N, dtype=torch.float16, device=dev)
    ys = torch.zeros(N, dtype=torch.float16, device=dev)

    def step(x, t):
        sgemv.sgemv_run_fused(pm.desc, pm.blob, x, [t], yf, pm.workspace, idx, cnt)
        sgemv.sgemv_gather_indices(x, [t], idx2, cnt2)
        sgemv.sgemv_run(pm.desc, pm.blob, x, idx2, cnt2, ys, pm.workspace)

    def snap():
        torch.cuda.synchronize()
        return (yf.cpu().numpy().view(np.uint16).copy(), ys.cpu().numpy().view(np.uint16).copy(),
                idx.cpu().numpy().copy(), int(cnt.item()), idx2.cpu().numpy().copy(), int(cnt2.item()))

    step(x1, t1)
    ref = snap()
    step(x2, t2)
    other = snap()
    assert not np.array_equal(ref[0], other[0])

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(x1, t1)
    for rep in range(4):
        g.replay()
        got = snap()
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep}"
        step(x2, t2)               # eager work in between
        got = snap()
        for a, b in zip(got, other):
            assert np.array_equal(a, b), f"eager after replay {rep}"
    tiles = N // 256
    assert int(torch.count_nonzero(pm.workspace[:tiles * 256]).item()) == 0


def test_graph_replays_match_eager_many_rows_and_dense():
    """The same for 4 rows (the matrix-core kernel with its list workgroups,
    and over a given list), 2 rows over a given list, and the dense path."""
    from activation_sparse_bit_amd import sgemv
    K, N, M = 14336, 4096, 4
    pm = G.packed(0, N, K, 0.02)
    dev = G.torch_dev()
    X1 = np.stack([synth.glu_activation(m, K) for m in range(M)])
    X2 = np.stack([synth.glu_activation(10 + m, K) for m in range(M)])
    T1 = [synth.percentile_threshold(X1[m], 0.7) for m in range(M)]
    T2 = [synth.percentile_threshold(X2[m], 0.5) for m in range(M)]
    x1, x2 = G.to_dev(X1), G.to_dev(X2)
    idx = torch.zeros(K, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    yf = torch.zeros((M, N), dtype=torch.float32, device=dev)
    yl = torch.zeros((M, N), dtype=torch.float32, device=dev)
    y2 = torch.zeros((2, N), dtype=torch.float32, device=dev)
    yd = torch.zeros(N, dtype=torch.float16, device=dev)

    def step(x, t):
        sgemv.sgemv_run_fused(pm.desc, pm.blob, x, t, yf, pm.workspace, idx, cnt)
        sgemv.sgemv_run_batched(pm.desc, pm.blob, x, t, idx, cnt, yl, pm.workspace)
        sgemv.sgemv_run_batched(pm.desc, pm.blob, x[:2], t[:2], idx, cnt, y2, pm.workspace)
        sgemv.sgemv_run(pm.desc, pm.blob, x[0], None, None, yd, pm.workspace)

    def snap():   # the list up to its count (entries past it keep older lists' values)
        torch.cuda.synchronize()
        c = int(cnt.item())
        return (yf.cpu().numpy().view(np.uint32).copy(), yl.cpu().numpy().view(np.uint32).copy(),
                y2.cpu().numpy().view(np.uint32).copy(), yd.cpu().numpy().view(np.uint16).copy(),
                idx.cpu().numpy()[:c].copy(), c)

    step(x1, T1)
    ref = snap()
    step(x2, T2)
    other = snap()
    assert not np.array_equal(ref[0], other[0]) and not np.array_equal(ref[3], other[3])

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(x1, T1)
    names = ("fused", "given list, 4 rows", "given list, 2 rows", "dense", "list", "count")
    for rep in range(4):
        g.replay()
        got = snap()
        for nm, a, b in zip(names, got, ref):
            assert np.array_equal(a, b), f"replay {rep}: {nm} differs in {np.count_nonzero(np.asarray(a) != np.asarray(b))} entries"
        step(x2, T2)
        got = snap()
        for nm, a, b in zip(names, got, other):
            assert np.array_equal(a, b), f"eager after replay {rep}: {nm}"
    tiles = N // 256
    assert int(torch.count_nonzero(pm.workspace[:tiles * 256]).item()) == 0


def test_calls_on_a_side_stream_match_the_default_stream():
    """Every call enqueues on the stream it is given: the same calls on a
    second stream (default priority) give the same bits as on the current
    stream, with the work ordered by that stream alone."""
    from activation_sparse_bit_amd import sgemv
    K, N, M = 14336, 4096, 4
    pm = G.packed(0, N, K, 0.02)
    dev = G.torch_dev()
    X = np.stack([synth.glu_activation(20 + m, K) for m in range(M)])
    T = [synth.percentile_threshold(X[m], 0.6) for m in range(M)]

    def run(stream):
        with torch.cuda.stream(stream):
            xd = G.to_dev(X)
            idx = torch.zeros(K, dtype=torch.int32, device=dev)
            cnt = torch.zeros(1, dtype=torch.int32, device=dev)
            y1 = torch.zeros(N, dtype=torch.float32, device=dev)
            y4 = torch.zeros((M, N), dtype=torch.float32, device=dev)
            yl = torch.zeros((M, N), dtype=torch.float32, device=dev)
        sgemv.sgemv_run_fused(pm.desc, pm.blob, xd[0], T[:1], y1, pm.workspace, stream=stream)
        sgemv.sgemv_gather_indices(xd, T, idx, cnt, stream=stream)
        sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, T, y4, pm.workspace, stream=stream)
        sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, T, idx, cnt, yl, pm.workspace, stream=stream)
        stream.synchronize()
        return [a.cpu().numpy().view(np.uint32).copy() for a in (y1, y4, yl)] + [idx.cpu().numpy()[:int(cnt.item())]]

    torch.cuda.synchronize()
    ref = run(torch.cuda.current_stream())
    side = torch.cuda.Stream()
    got = run(side)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("M", [1, 4])
def test_graph_replays_groups_along_n(M):
    """Layout version 3 in a captured graph: one row (vector kernel) and four
    rows (matrix cores, with the list workgroups), replays bitwise equal to
    the eager call, with an eager call on other inputs between replays."""
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    q, s, z = synth.quantized_weights_ng(0, N, K, 0.02)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev(), ng=True)
    dev = G.torch_dev()
    X1 = np.stack([synth.glu_activation(m, K) for m in range(M)])
    X2 = np.stack([synth.glu_activation(10 + m, K) for m in range(M)])
    t1 = [synth.percentile_threshold(X1[m], 0.5) for m in range(M)]
    t2 = [synth.percentile_threshold(X2[m], 0.8) for m in range(M)]
    x1, x2 = (G.to_dev(X1), G.to_dev(X2)) if M > 1 else (G.to_dev(X1[0]), G.to_dev(X2[0]))
    idx = torch.zeros(K, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    y = torch.zeros((M, N) if M > 1 else (N,), dtype=torch.float32, device=dev)

    def step(x, t):
        sgemv.sgemv_run_fused(pm.desc, pm.blob, x, t, y, pm.workspace, idx, cnt)

    def snap():
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint32).copy(), idx.cpu().numpy().copy(), int(cnt.item())

    step(x1, t1)
    ref = snap()
    step(x2, t2)
    other = snap()
    assert not np.array_equal(ref[0], other[0])
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(x1, t1)
    for rep in range(4):
        g.replay()
        for a, b in zip(snap(), ref):
            assert np.array_equal(a, b), f"replay {rep}"
        step(x2, t2)
        for a, b in zip(snap(), other):
            assert np.array_equal(a, b), f"eager after replay {rep}"

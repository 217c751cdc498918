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

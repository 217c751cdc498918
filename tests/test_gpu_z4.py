"""Layout version 2 (fp16 scales, 4-bit integer zero-points) on every device
path: the kernels convert the compact metadata back to the same numbers, so
y must equal the version-1 result bit for bit (fp32 output), and both must
meet the oracle's bar."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _pair(j, N, K, sigma):
    from activation_sparse_bit_amd import sgemv
    q, s, z = G.weights(j, N, K, sigma)
    v1 = G.packed(j, N, K, sigma)
    v2 = sgemv.PackedMatrix(q, s, z, device=G.torch_dev(), z4=True)
    assert v2.desc.version == sgemv.SGEMV_LAYOUT_Z4 and v2.desc.m_bytes * 8 == v1.desc.m_bytes * 5
    return (q, s, z), v1, v2


def _fused(pm, X, ts):
    from activation_sparse_bit_amd import sgemv
    M = 1 if X.ndim == 1 else X.shape[0]
    K = X.shape[-1]
    y = torch.full((M, pm.N) if X.ndim > 1 else (pm.N,), float("nan"), dtype=torch.float32, device=G.torch_dev())
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_run_fused(pm.desc, pm.blob, G.to_dev(X), ts, y, pm.workspace, idx, cnt)
    torch.cuda.synchronize()
    c = int(cnt.item())
    return y.cpu().numpy(), idx.cpu().numpy()[:c]


@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_z4_fused_bitwise(M):
    K, N = 14336, 4096
    (q, s, z), v1, v2 = _pair(0, N, K, 0.02)
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.5 if M == 1 else 0.7) for m in range(M)]
    if M == 1:
        X, ts = X[0], ts[:1]
    y1, i1 = _fused(v1, X, ts)
    y2, i2 = _fused(v2, X, ts)
    assert np.array_equal(i1, i2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    rows = G.sample_rows(N, 256, seed=M)
    y_ref, B, U = G.oracle_rows(q, s, z, X, ts, rows)
    assert np.array_equal(i2, U)
    G.check_y(y2.reshape(-1, N)[:, rows], y_ref, B, f"z4 fused M={M}")


def test_z4_multi_round_grid_and_ragged_k():
    """The four-wavefront build (a grid of more than 256 workgroups) and a K
    that leaves the last segment partly empty."""
    for (K, N, p) in ((8192, 16384, 0.9), (5248, 2048, 0.5)):
        (q, s, z), v1, v2 = _pair(4, N, K, 0.02)
        x = synth.plain_activation(9, K)
        t = synth.percentile_threshold(x, p)
        y1, _ = _fused(v1, x, [t])
        y2, i2 = _fused(v2, x, [t])
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
        rows = G.sample_rows(N, 256, seed=K)
        y_ref, B, U = G.oracle_rows(q, s, z, x, t, rows)
        G.check_y(y2[rows][None, :], y_ref, B, f"z4 {K}->{N}")


def test_z4_dense_and_list_driven_bitwise():
    from activation_sparse_bit_amd import sgemv
    K, N = 4096, 4096
    (q, s, z), v1, v2 = _pair(1, N, K, 0.02)
    dev = G.torch_dev()
    for M in (1, 2, 3, 4, 16):
        X = np.stack([synth.plain_activation(30 + m, K) for m in range(M)])
        ts = [0.4 + 0.05 * m for m in range(M)]
        xd = G.to_dev(X if M > 1 else X[0])
        idx = torch.zeros(K, dtype=torch.int32, device=dev)
        cnt = torch.zeros(1, dtype=torch.int32, device=dev)
        sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
        outs = []
        for pm in (v1, v2):
            shape = (M, N) if M > 1 else (N,)
            yl = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
            yd = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
            if M == 1:
                sgemv.sgemv_run(pm.desc, pm.blob, xd, idx, cnt, yl, pm.workspace)
                sgemv.sgemv_run(pm.desc, pm.blob, xd, None, None, yd, pm.workspace)
            else:
                sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, idx, cnt, yl, pm.workspace)
                sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, None, None, None, yd, pm.workspace)
            torch.cuda.synchronize()
            outs.append((yl.cpu().numpy(), yd.cpu().numpy()))
        (l1, d1), (l2, d2) = outs
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), f"list path M={M}"
        assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32)), f"every column M={M}"
        y_ref, B, _ = oracle.gemv_masked(q, s, z, X, ts)
        G.check_y(l2.reshape(M, N), y_ref, B, f"z4 list M={M}")
        y_ref, B = oracle.gemv_dense(q, s, z, X)
        G.check_y(d2.reshape(M, N), y_ref, B, f"z4 dense M={M}")

"""Parity of one-row calls whose grid takes several rounds (more workgroups
than one per CU) with the fp64 oracle on MI355X, every output compared.
Such grids run the one-row kernel with 4-wavefront workgroups of 512
columns (up to 32 segments per half tile) or the 8-wavefront build limited to
128 registers (more segments).  The shapes pick each path with K ragged
against the segments, so that the last workgroup of every half tile has
wavefronts without a group."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (N, K, workgroup size in wavefronts): 56 half tiles x 10 segments of 512
# columns (the last 128 wide); 112 x 15 (the last 384 wide); 32 half tiles x
# 20 segments of 1024 columns (the last 640 wide)
SHAPES = [(14336, 4736, 4), (28672, 7552, 4), (8192, 20096, 8)]


def _waves(N, K):
    """The host's choice for one row, restated: 0 for a grid of one round,
    else the wavefronts per workgroup of the multi-round kernel."""
    tiles = N // 256
    if tiles * -(-K // 1024) <= 256:
        return 0
    return 4 if -(-K // 512) <= 32 else 8


@pytest.fixture(scope="module", params=SHAPES, ids=lambda s: f"{s[0]}x{s[1]}-W{s[2]}")
def problem(request):
    from activation_sparse_bit_amd import sgemv
    N, K, w = request.param
    assert _waves(N, K) == w
    q, s, z = synth.random_int4_problem(N + K, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev(), max_batch=1)
    return N, K, q, s, z, pm


def _call(pm, x, t, want_list=True, dtype=None):
    from activation_sparse_bit_amd import sgemv
    K, N = pm.K, pm.N
    xd = G.to_dev(np.asarray(x, dtype=np.float16).reshape(1, K))
    y = torch.full((1, N), float("nan"), dtype=dtype or torch.float16, device=G.torch_dev())
    idx = cnt = None
    if want_list:
        idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
        cnt = torch.full((1,), -7, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, [t], y, pm.workspace, idx, cnt)
    torch.cuda.synchronize()
    tiles = N // 256
    assert int(torch.count_nonzero(pm.workspace[:tiles * 256]).item()) == 0, "arrival counters not reset"
    yh = y.float().cpu().numpy()
    if not want_list:
        return yh, None, None
    return yh, idx.cpu().numpy(), int(cnt.item())


@pytest.mark.parametrize("p", [0.0, 0.5, 0.9, 0.995])
def test_multiround_fused_every_output(problem, p):
    N, K, q, s, z, pm = problem
    x = synth.plain_activation(7, K)
    t = synth.percentile_threshold(x, p)
    y, idx, c = _call(pm, x, t)
    U = oracle.active_indices(x, t)
    assert c == len(U) and np.array_equal(idx[:c], U) and np.all(idx[c:] == -7)
    y_ref, B, _ = oracle.gemv_masked(q, s, z, x, t)
    G.check_y(y, y_ref, B, f"multiround {N}x{K} p={p}")


def test_multiround_fp32_exactness_and_repeat(problem):
    """fp32 output at t = 0: products exact, fp32 accumulation only; the same
    call twice gives the same bits; without the list the same bits again."""
    N, K, q, s, z, pm = problem
    x = synth.glu_activation(3, K)
    y1, _, _ = _call(pm, x, 0.0, dtype=torch.float32)
    y2, _, _ = _call(pm, x, 0.0, dtype=torch.float32, want_list=False)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    y_ref, B, _ = oracle.gemv_masked(q, s, z, x, 0.0)
    rel = G.check_y(y1, y_ref, B, "multiround fp32 t=0")
    assert rel < 2e-6


def test_multiround_empty_and_single(problem):
    """No active column (y = +0 everywhere); one active column (y is that
    column times its activation)."""
    N, K, q, s, z, pm = problem
    x = synth.plain_activation(9, K)
    y, idx, c = _call(pm, x, float(np.abs(x.astype(np.float32)).max()) * 2)
    assert c == 0 and np.all(y == 0) and not np.any(np.signbit(y))
    x1 = np.zeros(K, dtype=np.float16)
    k = K - 77
    x1[k] = np.float16(-1.5)
    y, idx, c = _call(pm, x1, 0.5)
    assert c == 1 and idx[0] == k
    y_ref, B, _ = oracle.gemv_masked(q, s, z, x1, 0.5)
    G.check_y(y, y_ref, B, "multiround one column")


def test_multiround_dense_and_unmasked(problem):
    """Every column (sgemv_run without a list, rows unmasked) and the
    batched every-column call with a threshold for its one row."""
    from activation_sparse_bit_amd import sgemv
    N, K, q, s, z, pm = problem
    x = synth.plain_activation(11, K)
    xd = G.to_dev(x.reshape(1, K))
    y = torch.empty((1, N), dtype=torch.float32, device=G.torch_dev())
    sgemv.sgemv_run(pm.desc, pm.blob, xd[0], None, None, y[0], pm.workspace)
    torch.cuda.synchronize()
    y_ref, B = oracle.gemv_dense(q, s, z, x.reshape(1, K))
    rel = G.check_y(y.cpu().numpy(), y_ref, B, "multiround dense")
    assert rel < 2e-6
    t = synth.percentile_threshold(x, 0.6)
    sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, [t], None, None, y, pm.workspace)
    torch.cuda.synchronize()
    y_ref, B, _ = oracle.gemv_masked(q, s, z, x, t)
    G.check_y(y.cpu().numpy(), y_ref, B, "multiround dense, masked row")


def test_multiround_compact_metadata(problem):
    """Layout version 2 (4-bit zero-points): the same bits as version 1."""
    from activation_sparse_bit_amd import sgemv
    N, K, q, s, z, pm = problem
    pm2 = sgemv.PackedMatrix(q, s, z, device=G.torch_dev(), max_batch=1, z4=True)
    x = synth.glu_activation(5, K)
    t = synth.percentile_threshold(x, 0.5)
    y1, i1, c1 = _call(pm, x, t, dtype=torch.float32)
    y2, i2, c2 = _call(pm2, x, t, dtype=torch.float32)
    assert c1 == c2 and np.array_equal(i1, i2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))

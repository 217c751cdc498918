"""Layout version 3 (groups along N: one scale and one zero-point per input
column and 128 outputs) on every device path: one and two rows (vector
kernels) and 3..16 rows (matrix cores), fused (with and without the list),
over a gathered list, and every column.

The kernels fold each column's scale into its activation (s * x rounded
once to fp16, relative error at most 2^-11) and keep q - z exact, so with
fp32 output every element lies within 2^-11 * B (B = sum |w^| |x|) of the
exact product, plus fp32 accumulation: the tests assert 5.2e-4 * B beside
the acceptance bar (rel L2 1e-3, 2e-3 * B), and the list bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NG_BOUND = 5.2e-4   # 2^-11 (fp16 rounding of s * x) plus fp32 accumulation


def _matrix(j, N, K, sigma=0.02):
    from activation_sparse_bit_amd import sgemv
    q, s, z = synth.quantized_weights_ng(j, N, K, sigma)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev(), ng=True)
    assert pm.desc.version == sgemv.SGEMV_LAYOUT_NG
    return (q, s, z), pm


def _check(y, y_ref, B, what, f32):
    G.check_y(y, y_ref, B, what)
    if f32:
        err = np.abs(np.asarray(y, np.float64).reshape(y_ref.shape) - y_ref)
        worst = float((err / np.maximum(B, 1e-300)).max())
        assert np.all(err <= NG_BOUND * B + 1e-30), f"{what}: error/B up to {worst:.3e}"


def _fused(pm, X, ts, f32, with_list=True):
    from activation_sparse_bit_amd import sgemv
    dev = G.torch_dev()
    M = 1 if X.ndim == 1 else X.shape[0]
    K = X.shape[-1]
    shape = (M, pm.N) if X.ndim > 1 else (pm.N,)
    y = torch.full(shape, float("nan"), dtype=torch.float32 if f32 else torch.float16, device=dev)
    idx = torch.full((K,), -7, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    if with_list:
        sgemv.sgemv_run_fused(pm.desc, pm.blob, G.to_dev(X), ts, y, pm.workspace, idx, cnt)
    else:
        sgemv.sgemv_run_fused(pm.desc, pm.blob, G.to_dev(X), ts, y, pm.workspace)
    torch.cuda.synchronize()
    c = int(cnt.item())
    return y.float().cpu().numpy().reshape(M, pm.N), idx.cpu().numpy()[:c]


@pytest.mark.parametrize("f32", [True, False])
@pytest.mark.parametrize("M,p", [(1, 0.5), (1, 0.9), (1, 0.0), (2, 0.7)])
def test_ng_fused_full_size(M, p, f32):
    """The 14336 -> 4096 down projection, every output against the oracle."""
    K, N = 14336, 4096
    print(f"ng fused M={M} p={p} f32={f32}", flush=True)
    (q, s, z), pm = _matrix(0, N, K)
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], p) for m in range(M)]
    Xa = X[0] if M == 1 else X
    y, idx = _fused(pm, Xa, ts, f32)
    y_ref, B, U = oracle.gemv_masked(q, s, z, Xa, ts, along="n")
    assert np.array_equal(idx, U)
    _check(y, y_ref, B, f"ng fused M={M} p={p}", f32)
    y2, _ = _fused(pm, Xa, ts, True, with_list=False)
    if f32:
        assert np.array_equal(y2.view(np.uint32), y.view(np.uint32)), "with and without the list"


@pytest.mark.parametrize("K,N,p", [(2176, 1024, 0.5), (384, 512, 0.3), (2048, 2048, 0.5),
                                   (8192, 16384, 0.9), (28672, 1024, 0.5)])
@pytest.mark.parametrize("M", [1, 2])
def test_ng_shapes(K, N, p, M):
    """A K that leaves the last segment partly empty, tiny K, the small-grid
    (4-wavefront) build, a grid of several rounds, many segments."""
    print(f"ng shape K={K} N={N} p={p} M={M}", flush=True)
    (q, s, z), pm = _matrix(K % 7, N, K)
    X = np.stack([synth.plain_activation(20 + m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], p) for m in range(M)]
    Xa = X[0] if M == 1 else X
    y, idx = _fused(pm, Xa, ts, True)
    y_ref, B, U = oracle.gemv_masked(q, s, z, Xa, ts, along="n")
    assert np.array_equal(idx, U)
    _check(y, y_ref, B, f"ng K={K} N={N} M={M}", True)


@pytest.mark.parametrize("M", [1, 2])
def test_ng_list_and_dense_paths(M):
    """Over a gathered list (bit for bit the fused result) and every column."""
    from activation_sparse_bit_amd import sgemv
    K, N = 4096, 4096
    print(f"ng list/dense M={M}", flush=True)
    (q, s, z), pm = _matrix(1, N, K)
    dev = G.torch_dev()
    X = np.stack([synth.plain_activation(30 + m, K) for m in range(M)])
    ts = [0.4 + 0.05 * m for m in range(M)]
    Xa = X[0] if M == 1 else X
    xd = G.to_dev(Xa)
    idx = torch.zeros(K, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
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
    yl, yd = yl.cpu().numpy().reshape(M, N), yd.cpu().numpy().reshape(M, N)
    yf, _ = _fused(pm, Xa, ts, True)
    assert np.array_equal(yl.view(np.uint32), yf.view(np.uint32)), "list path and fused differ"
    y_ref, B, _ = oracle.gemv_masked(q, s, z, Xa, ts, along="n")
    _check(yl, y_ref, B, f"ng list M={M}", True)
    y_ref, B = oracle.gemv_dense(q, s, z, Xa, along="n")
    _check(yd, y_ref, B, f"ng dense M={M}", True)


@pytest.mark.parametrize("M", [3, 4, 8, 16])
def test_ng_many_rows(M):
    """3..16 rows on the matrix cores (k_fm): fused with the list, over the
    gathered list (bit for bit the fused result) and every column, at
    14336 -> 4096 with 70 % per row."""
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    print(f"ng many rows M={M}", flush=True)
    (q, s, z), pm = _matrix(0, N, K)
    dev = G.torch_dev()
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
    yf, idx = _fused(pm, X, ts, True)
    y_ref, B, U = oracle.gemv_masked(q, s, z, X, ts, along="n")
    assert np.array_equal(idx, U)
    _check(yf, y_ref, B, f"ng fused M={M}", True)
    xd = G.to_dev(X)
    li = torch.zeros(K, dtype=torch.int32, device=dev)
    lc = torch.zeros(1, dtype=torch.int32, device=dev)
    sgemv.sgemv_gather_indices(xd, ts, li, lc)
    yl = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, li, lc, yl, pm.workspace)
    yh = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, ts, yh, pm.workspace)
    torch.cuda.synchronize()
    yl = yl.cpu().numpy()
    assert np.array_equal(yl.view(np.uint32), yf.view(np.uint32)), "list path and fused differ"
    _check(yh.float().cpu().numpy(), y_ref, B, f"ng fused fp16 M={M}", False)
    if M in (3, 16):
        Xd = X[:, :2048].copy()
        (q2, s2, z2), pm2 = _matrix(5, 1024, 2048)
        yd = torch.full((M, 1024), float("nan"), dtype=torch.float32, device=dev)
        sgemv.sgemv_run_batched(pm2.desc, pm2.blob, G.to_dev(Xd), None, None, None, yd, pm2.workspace)
        torch.cuda.synchronize()
        y_ref, B = oracle.gemv_dense(q2, s2, z2, Xd, along="n")
        _check(yd.cpu().numpy(), y_ref, B, f"ng dense M={M}", True)

"""Parity of the fused threshold + compact + GEMV call (sgemv_run_fused)
with the fp64 oracle on MI355X: the optional list and count bit for bit,
y within the acceptance tolerance, across shapes whose K is not a multiple
of the 512-column segment, one and two rows, and the degenerate cases."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _fused(pm, X, ts, want_list=True, dtype=None, ldx=None, ldy=None):
    """Run the fused call on host rows X ([K] or [M][K]); returns y (float
    numpy, [M][N]), the list and the count (None when not asked for)."""
    from activation_sparse_bit_amd import sgemv
    X = np.atleast_2d(X)
    M, K = X.shape
    N = pm.N
    ldx = ldx or K
    ldy = ldy or N
    Xp = np.zeros((M, ldx), dtype=np.float16)
    Xp[:, :K] = X
    xd = G.to_dev(Xp)
    dtype = dtype or torch.float16
    y = torch.full((M, ldy), float("nan"), dtype=dtype, device=G.torch_dev())
    idx = cnt = None
    if want_list:
        idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
        cnt = torch.full((1,), -7, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, ts, y, pm.workspace, idx, cnt)
    torch.cuda.synchronize()
    tiles = N // 256
    assert int(torch.count_nonzero(pm.workspace[:tiles * 256]).item()) == 0, "arrival counters not reset"
    yh = y.float().cpu().numpy()[:, :N]
    if not want_list:
        return yh, None, None
    return yh, idx.cpu().numpy(), int(cnt.item())


def _check_list(idx, c, X, ts):
    U = oracle.active_indices(X, ts)
    assert c == len(U)
    assert np.array_equal(idx[:c], U)
    assert np.all(idx[c:] == -7)


@pytest.mark.parametrize("p", [0.0, 0.5, 0.7, 0.9, 0.999])
def test_fused_down_14336(p):
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    x = synth.glu_activation(0, K)
    t = synth.percentile_threshold(x, p)
    y, idx, c = _fused(pm, x, [t])
    _check_list(idx, c, x, t)
    y_ref, B, U = oracle.gemv_masked(q, s, z, x, t)
    G.check_y(y, y_ref, B, f"fused down p={p}")


@pytest.mark.parametrize("p", [0.0, 0.5, 0.9])
def test_fused_2048(p):
    K = N = 2048
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    x = synth.plain_activation(0, K)
    t = synth.percentile_threshold(x, p)
    y, _, _ = _fused(pm, x, [t], want_list=False)
    y_ref, B, _ = oracle.gemv_masked(q, s, z, x, t)
    G.check_y(y, y_ref, B, f"fused 2048 p={p}")


@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 1024), (4096, 14336)])
def test_fused_layer_8b(K, N):
    q, s, z = G.weights(1, N, K, 0.02)
    pm = G.packed(1, N, K, 0.02)
    x = synth.plain_activation(K // 1024, K)
    t = synth.percentile_threshold(x, 0.5)
    y, idx, c = _fused(pm, x, [t])
    _check_list(idx, c, x, t)
    y_ref, B, _ = oracle.gemv_masked(q, s, z, x, t)
    G.check_y(y, y_ref, B, f"fused layer {K}->{N}")


@pytest.mark.parametrize("K,N,glu", [(8192, 28672, False), (28672, 8192, True)])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_fused_mlp_70b_sampled(K, N, glu, p):
    q, s, z = G.weights(2, N, K, 0.015)
    pm = G.packed(2, N, K, 0.015)
    x = synth.glu_activation(0, K) if glu else synth.plain_activation(0, K)
    t = synth.percentile_threshold(x, p)
    y, idx, c = _fused(pm, x, [t])
    _check_list(idx, c, x, t)
    rows = G.sample_rows(N, 384)
    y_ref, B, _ = G.oracle_rows(q, s, z, x, t, rows)
    G.check_y(y[:, rows], y_ref, B, f"fused 70b {K}->{N} p={p}")


@pytest.mark.parametrize("K,N", [(128, 512), (384, 1536), (640, 512), (1152, 2560), (2176, 1024)])
def test_fused_ragged_segments(K, N):
    """K below, between and not a multiple of 512-column segments."""
    from activation_sparse_bit_amd import sgemv
    q, s, z = synth.random_int4_problem(K + N, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    x = synth.plain_activation(5, K)
    for p in (0.0, 0.3, 0.95):
        t = synth.percentile_threshold(x, p)
        y, idx, c = _fused(pm, x, [t], dtype=torch.float32)
        _check_list(idx, c, x, t)
        y_ref, B, _ = oracle.gemv_masked(q, s, z, x, t)
        G.check_y(y, y_ref, B, f"fused ragged {K}x{N} p={p}")


def test_fused_two_rows_union_and_strides():
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    X = np.stack([synth.glu_activation(m, K) for m in range(2)])
    ts = [synth.percentile_threshold(X[0], 0.7), synth.percentile_threshold(X[1], 0.8)]
    y, idx, c = _fused(pm, X, ts, ldx=K + 64, ldy=N + 8)
    _check_list(idx, c, X, ts)
    rows = G.sample_rows(N, 512, seed=2)
    y_ref, B, _ = G.oracle_rows(q, s, z, X, ts, rows)
    G.check_y(y[:, rows], y_ref, B, "fused M=2")


def test_fused_empty_and_full():
    K, N = 4096, 4096
    q, s, z = G.weights(1, N, K, 0.02)
    pm = G.packed(1, N, K, 0.02)
    x = np.zeros(K, dtype=np.float16)
    y, idx, c = _fused(pm, x, [0.5])
    assert c == 0 and np.all(idx == -7)
    assert np.all(y == 0) and not np.any(np.signbit(y))
    x = synth.plain_activation(1, K)
    y, idx, c = _fused(pm, x, [0.0], dtype=torch.float32)
    assert c == K and np.array_equal(idx, np.arange(K))
    y_ref, B = oracle.gemv_dense(q, s, z, x)
    rel = G.check_y(y, y_ref, B, "fused t=0")
    assert rel < 2e-6   # fp32 output: accumulation error only


def test_fused_special_values_list():
    """Signed zeros, subnormals, infinities and NaNs in x: the list follows
    the selection rule exactly (y is not checked: an infinite activation is
    active and makes y infinite)."""
    from activation_sparse_bit_amd import sgemv
    K, N = 1024, 512
    q, s, z = synth.random_int4_problem(11, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    rng = np.random.default_rng(5)
    bits = rng.standard_normal(K).astype(np.float16).view(np.uint16).copy()
    specials = [0x0000, 0x8000, 0x7E00, 0xFE00, 0x7C00, 0xFC00, 0x0001, 0x8001, 0x03FF, 0x7BFF]
    bits[rng.choice(K, len(specials) * 8, replace=False)] = np.repeat(specials, 8)
    x = bits.view(np.float16)
    for t in [0.0, 2.0 ** -24, 0.5, 65504.0, 1e30]:
        _, idx, c = _fused(pm, x, [t])
        _check_list(idx, c, x, t)


def test_fused_deterministic_and_scale_equivariant():
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    x = synth.glu_activation(0, K)
    t = synth.percentile_threshold(x, 0.5)
    outs = []
    for scale in (1.0, 1.0, 2.0):   # fp32 output: fp16 rounding of subnormal results is not scale-exact
        xs = (x.astype(np.float32) * scale).astype(np.float16)
        y, _, _ = _fused(pm, xs, [t * scale], want_list=False, dtype=torch.float32)
        outs.append(y)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))   # bitwise repeatable
    assert np.array_equal(outs[2], 2 * outs[0])                               # exact doubling


def test_fused_agrees_with_gather_and_run():
    """Same inputs through the two-launch path: the same list, and the same
    output bits (the run over the list compacts the same columns of every
    group in the same order, so its arithmetic is the fused call's)."""
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    x = synth.glu_activation(1, K)
    t = synth.percentile_threshold(x, 0.6)
    yf, idx_f, c_f = _fused(pm, x, [t], dtype=torch.float32)
    xd = G.to_dev(x)
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    y = torch.empty(N, dtype=torch.float32, device=G.torch_dev())
    sgemv.sgemv_gather_indices(xd, [t], idx, cnt)
    sgemv.sgemv_run(pm.desc, pm.blob, xd, idx, cnt, y, pm.workspace)
    torch.cuda.synchronize()
    assert int(cnt.item()) == c_f and np.array_equal(idx.cpu().numpy(), idx_f)
    ys = y.cpu().numpy()
    assert np.array_equal(yf[0].view(np.uint32), ys.view(np.uint32))


# ---------------------------------------------------------------------------
# 3 to 16 rows (matrix-core kernel)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M", [3, 4, 5, 8, 13, 16])
def test_fused_batched_rows(M):
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
    y, idx, c = _fused(pm, X, ts)
    _check_list(idx, c, X, ts)
    rows = G.sample_rows(N, 384, seed=M)
    y_ref, B, _ = G.oracle_rows(q, s, z, X, ts, rows)
    G.check_y(y[:, rows], y_ref, B, f"fused M={M}")


@pytest.mark.parametrize("K,N", [(128, 512), (640, 512), (1152, 1536), (2176, 1024)])
def test_fused_batched_ragged(K, N):
    """K below and not a multiple of the 1024-column segment; every row has
    its own threshold; fp32 output."""
    from activation_sparse_bit_amd import sgemv
    q, s, z = synth.random_int4_problem(K + 2 * N, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    M = 7
    X = np.stack([synth.plain_activation(10 + m, K) for m in range(M)])
    ts = [0.2 * m for m in range(M)]
    y, idx, c = _fused(pm, X, ts, dtype=torch.float32, ldx=K + 8, ldy=N + 24)
    _check_list(idx, c, X, ts)
    y_ref, B, _ = oracle.gemv_masked(q, s, z, X, ts)
    G.check_y(y, y_ref, B, f"fused M=7 {K}x{N}")


@pytest.mark.parametrize("M,K,p", [(16, 65536, 0.9), (5, 40960, 0.6), (3, 65536, 0.999)])
def test_fused_batched_long_rows(M, K, p):
    """Long rows: the list is built by the most list workgroups (8 ranges of
    up to 8192 columns, joined by the last to finish) while the matrix-core
    workgroups compute; list bit-exact, every output within the bar."""
    from activation_sparse_bit_amd import sgemv
    N = 512
    q, s, z = synth.random_int4_problem(K + M, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    X = np.stack([synth.glu_activation(30 + m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], p) for m in range(M)]
    y, idx, c = _fused(pm, X, ts)
    _check_list(idx, c, X, ts)
    y_ref, B, _ = oracle.gemv_masked(q, s, z, X, ts)
    G.check_y(y, y_ref, B, f"fused M={M} K={K} p={p}")


def test_fused_batched_dense_fp32_and_empty():
    K, N = 4096, 4096
    q, s, z = G.weights(1, N, K, 0.02)
    pm = G.packed(1, N, K, 0.02)
    M = 16
    X = np.stack([synth.plain_activation(20 + m, K) for m in range(M)])
    y, idx, c = _fused(pm, X, [0.0] * M, dtype=torch.float32)
    assert c == K and np.array_equal(idx, np.arange(K))
    rows = G.sample_rows(N, 512, seed=3)
    y_ref, B = oracle.gemv_dense(q[rows], s[rows], z[rows], X)
    rel = G.check_y(y[:, rows], y_ref, B, "fused M=16 t=0")
    assert rel < 2e-6          # products exact, fp32 accumulation only
    Z = np.zeros((5, K), dtype=np.float16)
    y, idx, c = _fused(pm, Z, [0.5] * 5)
    assert c == 0 and np.all(y == 0) and not np.any(np.signbit(y))


def test_fused_batched_deterministic_and_scale_equivariant():
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    M = 8
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
    outs = []
    for scale in (1.0, 1.0, 2.0):   # fp32 output: fp16 rounding of subnormal results is not scale-exact
        Xs = (X.astype(np.float32) * scale).astype(np.float16)
        y, _, _ = _fused(pm, Xs, [t * scale for t in ts], want_list=False, dtype=torch.float32)
        outs.append(y)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))   # bitwise repeatable
    assert np.array_equal(outs[2], 2 * outs[0])                               # exact doubling


@pytest.mark.parametrize("M", [2, 8])
def test_fused_batched_agrees_with_run_batched(M):
    """Same rows through gather + run_batched: same list, and the same output
    bits (the run over the union list builds the fused call's union)."""
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
    yf, idx_f, c_f = _fused(pm, X, ts, dtype=torch.float32)
    xd = G.to_dev(X)
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    Y = torch.empty((M, N), dtype=torch.float32, device=G.torch_dev())
    sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
    sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, idx, cnt, Y, pm.workspace)
    torch.cuda.synchronize()
    assert int(cnt.item()) == c_f and np.array_equal(idx.cpu().numpy(), idx_f)
    ys = Y.cpu().numpy()
    assert np.array_equal(yf.view(np.uint32), ys.view(np.uint32))

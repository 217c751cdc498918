"""Parity of the HIP path with the fp64 oracle (MI355X).

Index lists are compared bit for bit; outputs within per-row relative L2
1e-3 and per-element 2e-3 * sum|w^||xe| of the oracle.  Every call goes
through the C ABI (ctypes binding)."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gather(x_np, ts, K=None):
    from activation_sparse_bit_amd import sgemv
    x = G.to_dev(x_np)
    K = x_np.shape[-1] if K is None else K
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.full((1,), -7, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_gather_indices(x, ts, idx, cnt, K=K)
    torch.cuda.synchronize()
    c = int(cnt.item())
    return idx.cpu().numpy(), c


# ---------------------------------------------------------------------------
# index gathering
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K", [128, 2048, 4096, 8192, 14336, 28672, 65536])
@pytest.mark.parametrize("p", [0.0, 0.5, 0.7, 0.9, 0.999])
def test_gather_single(K, p):
    x = synth.glu_activation(K % 97, K)
    t = synth.percentile_threshold(x, p)
    idx, c = _gather(x, [t])
    U = oracle.active_indices(x, t)
    assert c == len(U)
    assert np.array_equal(idx[:c], U)
    assert np.all(idx[c:] == -7)   # untouched beyond count


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
def test_gather_batched_union(M):
    K = 14336
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
    idx, c = _gather(X, ts)
    U = oracle.active_indices(X, ts)
    assert c == len(U) and np.array_equal(idx[:c], U)


def test_gather_strided_rows():
    K, ldx, M = 2048, 2048 + 64, 3
    X = np.zeros((M, ldx), dtype=np.float16)
    X[:, :K] = np.stack([synth.plain_activation(m, K) for m in range(M)])
    X[:, K:] = np.float16(100.0)     # padding beyond K must be ignored
    ts = [1.0, 1.5, 2.0]
    from activation_sparse_bit_amd import sgemv
    x = G.to_dev(X)
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_gather_indices(x, ts, idx, cnt, K=K)
    torch.cuda.synchronize()
    U = oracle.active_indices(X[:, :K], ts)
    c = int(cnt.item())
    assert c == len(U) and np.array_equal(idx.cpu().numpy()[:c], U)


def test_gather_special_values():
    rng = np.random.default_rng(5)
    K = 1024
    bits = rng.standard_normal(K).astype(np.float16).view(np.uint16).copy()
    specials = [0x0000, 0x8000, 0x7E00, 0xFE00, 0x7C00, 0xFC00, 0x0001, 0x8001, 0x03FF, 0x7BFF]
    bits[rng.choice(K, len(specials) * 8, replace=False)] = np.repeat(specials, 8)
    x = bits.view(np.float16)
    mags = sorted(set(np.abs(x[np.isfinite(x)].astype(np.float32)).tolist()))
    for t in [0.0, 2.0 ** -24, mags[len(mags) // 2], 65504.0, 1e30, 0.9995, float(np.float32(1 / 3))]:
        idx, c = _gather(x, [t])
        U = oracle.active_indices(x, t)
        assert c == len(U) and np.array_equal(idx[:c], U), t


def test_gather_empty_and_full():
    K = 4096
    x = np.zeros(K, dtype=np.float16)
    idx, c = _gather(x, [0.5])
    assert c == 0 and np.all(idx == -7)
    idx, c = _gather(x, [0.0])
    assert c == K and np.array_equal(idx, np.arange(K))


# ---------------------------------------------------------------------------
# sparse GEMV, one row
# ---------------------------------------------------------------------------
def _run_single(j, N, K, sigma, x, t, dtype=None, dense=False):
    from activation_sparse_bit_amd import sgemv
    pm = G.packed(j, N, K, sigma)
    xd = G.to_dev(x)
    dtype = dtype or torch.float16
    y = torch.full((N,), float("nan"), dtype=dtype, device=G.torch_dev())
    if dense:
        sgemv.sgemv_run(pm.desc, pm.blob, xd, None, None, y, pm.workspace)
        torch.cuda.synchronize()
        return y.float().cpu().numpy(), None
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_gather_indices(xd, [t], idx, cnt)
    sgemv.sgemv_run(pm.desc, pm.blob, xd, idx, cnt, y, pm.workspace)
    torch.cuda.synchronize()
    ws_nonzero = int(torch.count_nonzero(pm.workspace[:(N // 256) * 256]).item())
    assert ws_nonzero == 0, "arrival counters not reset"
    return y.float().cpu().numpy(), int(cnt.item())


@pytest.mark.parametrize("p", [0.0, 0.5, 0.7, 0.9])
def test_run_single_2048(p):
    K = N = 2048
    q, s, z = G.weights(0, N, K, 0.02)
    x = synth.plain_activation(0, K)
    t = synth.percentile_threshold(x, p)
    y, c = _run_single(0, N, K, 0.02, x, t)
    y_ref, B, U = oracle.gemv_masked(q, s, z, x, t)
    assert c == len(U)
    G.check_y(y, y_ref, B, f"2048x2048 p={p}")


@pytest.mark.parametrize("p", [0.0, 0.5, 0.7, 0.9])
def test_run_down_14336(p):
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    x = synth.glu_activation(0, K)
    t = synth.percentile_threshold(x, p)
    y, c = _run_single(0, N, K, 0.02, x, t)
    y_ref, B, U = oracle.gemv_masked(q, s, z, x, t)
    assert c == len(U)
    G.check_y(y, y_ref, B, f"down p={p}")


@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096)])
def test_run_layer_8b(K, N):
    q, s, z = G.weights(1, N, K, 0.02)
    x = synth.plain_activation(K // 1024, K)
    t = synth.percentile_threshold(x, 0.5)
    y, c = _run_single(1, N, K, 0.02, x, t)
    y_ref, B, U = oracle.gemv_masked(q, s, z, x, t)
    G.check_y(y, y_ref, B, f"layer {K}->{N}")


@pytest.mark.parametrize("K,N,glu", [(8192, 28672, False), (28672, 8192, True)])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_run_mlp_70b_sampled(K, N, glu, p):
    q, s, z = G.weights(2, N, K, 0.015)
    x = synth.glu_activation(0, K) if glu else synth.plain_activation(0, K)
    t = synth.percentile_threshold(x, p)
    y, c = _run_single(2, N, K, 0.015, x, t)
    rows = G.sample_rows(N, 384)
    y_ref, B, U = G.oracle_rows(q, s, z, x, t, rows)
    assert c == len(U)
    G.check_y(y[rows][None, :], y_ref, B, f"70b {K}->{N} p={p}")


@pytest.mark.parametrize("K,N,glu", [(8192, 28672, False), (28672, 8192, True)])
def test_run_mlp_70b_dense_sampled(K, N, glu):
    """Every column (no list, no threshold) at the full 70B shapes, the
    multi-round grids of the dense GEMV: sampled rows within the bar, and
    with fp32 output only fp32 accumulation error."""
    q, s, z = G.weights(2, N, K, 0.015)
    x = synth.glu_activation(0, K) if glu else synth.plain_activation(0, K)
    rows = G.sample_rows(N, 384)
    y_ref, B = oracle.gemv_dense(q[rows], s[rows], z[rows], x)
    y, _ = _run_single(2, N, K, 0.015, x, 0.0, dense=True)
    G.check_y(y[rows][None, :], y_ref, B, f"70b dense {K}->{N}")
    y32, _ = _run_single(2, N, K, 0.015, x, 0.0, dtype=torch.float32, dense=True)
    rel = G.check_y(y32[rows][None, :], y_ref, B, f"70b dense fp32 {K}->{N}")
    assert rel < 2e-6


@pytest.mark.parametrize("K,N", [(128, 512), (384, 1536), (1152, 512), (2176, 2560)])
def test_run_ragged_shapes(K, N):
    """K not a multiple of the 1024- (or 512-) column workgroup segment, tiny K, several tiles."""
    q, s, z = synth.random_int4_problem(K + N, N, K)
    from activation_sparse_bit_amd import sgemv
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    x = synth.plain_activation(3, K)
    for p in (0.0, 0.3, 0.95):
        t = synth.percentile_threshold(x, p)
        xd = G.to_dev(x)
        idx = torch.zeros(K, dtype=torch.int32, device=G.torch_dev())
        cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
        y = torch.full((N,), float("nan"), dtype=torch.float32, device=G.torch_dev())
        sgemv.sgemv_gather_indices(xd, [t], idx, cnt)
        sgemv.sgemv_run(pm.desc, pm.blob, xd, idx, cnt, y, pm.workspace)
        torch.cuda.synchronize()
        y_ref, B, U = oracle.gemv_masked(q, s, z, x, t)
        G.check_y(y.cpu().numpy(), y_ref, B, f"ragged {K}x{N} p={p}")


def test_run_dense_equals_oracle():
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    x = synth.glu_activation(0, K)
    y, _ = _run_single(0, N, K, 0.02, x, 0.0, dense=True)
    y_ref, B = oracle.gemv_dense(q, s, z, x)
    G.check_y(y, y_ref, B, "dense")


def test_run_fp32_output_and_t0_equals_dense():
    K, N = 4096, 4096
    q, s, z = G.weights(1, N, K, 0.02)
    x = synth.plain_activation(1, K)
    y32, c = _run_single(1, N, K, 0.02, x, 0.0, dtype=torch.float32)
    yd, _ = _run_single(1, N, K, 0.02, x, 0.0, dtype=torch.float32, dense=True)
    assert c == K
    # the dense call runs the fused kernels (another summation order): the two
    # agree to fp32 reassociation
    assert np.max(np.abs(y32 - yd)) <= 4e-6 * max(1.0, float(np.max(np.abs(y32))))
    y_ref, B = oracle.gemv_dense(q, s, z, x)
    rel = G.check_y(y32, y_ref, B, "fp32")
    assert rel < 2e-6                  # no fp16 rounding: fp32 accumulation error only


def test_run_count_zero_gives_plus_zero():
    K, N = 4096, 4096
    x = np.zeros(K, dtype=np.float16)
    y, c = _run_single(1, N, K, 0.02, x, 1.0)
    assert c == 0
    assert np.all(y == 0) and not np.any(np.signbit(y))


def test_run_deterministic_and_scale_equivariant():
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    x = synth.glu_activation(0, K)
    t = synth.percentile_threshold(x, 0.7)
    outs = []
    for scale in (1.0, 1.0, 2.0):
        xs = (x.astype(np.float32) * scale).astype(np.float16)
        xd = G.to_dev(xs)
        idx = torch.zeros(K, dtype=torch.int32, device=G.torch_dev())
        cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
        # fp32 output: fp16 rounding of subnormal results is not scale-exact
        y = torch.empty(N, dtype=torch.float32, device=G.torch_dev())
        sgemv.sgemv_gather_indices(xd, [t * scale], idx, cnt)
        sgemv.sgemv_run(pm.desc, pm.blob, xd, idx, cnt, y, pm.workspace)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))   # bitwise repeatable
    assert np.array_equal(outs[2], 2 * outs[0])                               # exact doubling


def test_run_user_index_list():
    """An arbitrary ascending list (not from the gather) and a count below the
    list length: only the first count entries are used."""
    from activation_sparse_bit_amd import sgemv
    K, N = 4096, 4096
    q, s, z = G.weights(1, N, K, 0.02)
    pm = G.packed(1, N, K, 0.02)
    rng = np.random.default_rng(9)
    lst = np.sort(rng.choice(K, 1500, replace=False)).astype(np.int32)
    full = np.full(K, K + 5, dtype=np.int32)      # junk beyond count
    full[:1500] = lst
    x = synth.plain_activation(2, K)
    xd = G.to_dev(x)
    idx = G.to_dev(full)
    for c in (1500, 1001, 1, 0):
        cnt = G.to_dev(np.array([c], dtype=np.int32))
        y = torch.full((N,), float("nan"), dtype=torch.float32, device=G.torch_dev())
        sgemv.sgemv_run(pm.desc, pm.blob, xd, idx, cnt, y, pm.workspace)
        torch.cuda.synchronize()
        y_ref, B = oracle.gemv_listed(q, s, z, x, lst[:c])
        G.check_y(y.cpu().numpy(), y_ref, B, f"user list c={c}")


# ---------------------------------------------------------------------------
# batched
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
def test_run_batched(M):
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    X = np.stack([synth.glu_activation(m, K) for m in range(M)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
    xd = G.to_dev(X)
    idx = torch.zeros(K, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device=G.torch_dev())
    sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
    sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, idx, cnt, y, pm.workspace)
    torch.cuda.synchronize()
    rows = G.sample_rows(N, 512, seed=M)
    y_ref, B, U = G.oracle_rows(q, s, z, X, ts, rows)
    assert int(cnt.item()) == len(U)
    G.check_y(y.float().cpu().numpy()[:, rows], y_ref, B, f"batched M={M}")


def test_run_batched_unmasked_and_strides():
    from activation_sparse_bit_amd import sgemv
    K, N, M = 4096, 4096, 3
    q, s, z = G.weights(1, N, K, 0.02)
    pm = G.packed(1, N, K, 0.02)
    ldx, ldy = K + 8, N + 16
    X = np.zeros((M, ldx), dtype=np.float16)
    X[:, :K] = np.stack([synth.plain_activation(m, K) for m in range(M)])
    ts = [0.6, 1.0, 1.4]
    xd = G.to_dev(X)
    idx = torch.zeros(K, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_gather_indices(xd, ts, idx, cnt, K=K)
    y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device=G.torch_dev())
    sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, None, idx, cnt, y, pm.workspace)
    torch.cuda.synchronize()
    U = oracle.active_indices(X[:, :K], ts)
    y_ref, B = oracle.gemv_listed(q, s, z, X[:, :K], U)     # rows unmasked over the union
    yy = y.cpu().numpy()
    G.check_y(yy[:, :N], y_ref, B, "batched unmasked")
    assert np.all(np.isnan(yy[:, N:]))                        # padding untouched


@pytest.mark.gpu
@pytest.mark.parametrize("M", [2, 3, 16])
def test_run_batched_every_column(M):
    """run_batched with no list: every column, rows unmasked (no thresholds)
    or each masked by its own threshold; a ragged K over several segments."""
    from activation_sparse_bit_amd import sgemv
    K, N = 5248, 2048
    q, s, z = G.weights(2, N, K, 0.02)
    pm = G.packed(2, N, K, 0.02)
    X = np.stack([synth.plain_activation(40 + m, K) for m in range(M)])
    ts = [0.3 + 0.1 * m for m in range(M)]
    xd = G.to_dev(X)
    rows = G.sample_rows(N, 400, seed=M)
    for thr in (None, ts):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=G.torch_dev())
        sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, thr, None, None, y, pm.workspace)
        torch.cuda.synchronize()
        if thr is None:
            y_ref, B = oracle.gemv_dense(q[rows], s[rows], z[rows], X)
        else:
            y_ref, B, _ = oracle.gemv_masked(q[rows], s[rows], z[rows], X, ts)
        G.check_y(y.cpu().numpy()[:, rows], y_ref, B, f"every column M={M} masked={thr is not None}")


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 2, 5])
def test_run_batched_given_list_edges(M):
    """Rows over a given list (the list builds of the fused kernels: one or
    two rows on the vector units, 3+ on the matrix cores): an empty list, a
    hand-made list touching the first and last groups with junk beyond its
    count, a ragged K, and a count above K (clamped)."""
    from activation_sparse_bit_amd import sgemv
    K, N = 1152, 1024
    q, s, z = synth.random_int4_problem(77, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    X = np.stack([synth.plain_activation(60 + m, K) for m in range(M)])
    ts = [0.3 + 0.2 * m for m in range(M)]
    xd = G.to_dev(X)
    dev = G.torch_dev()
    lists = [np.zeros(0, dtype=np.int32),
             np.array([0, 1, 127, 128, 300, 640, 641, 1023, 1024, 1151], dtype=np.int32),
             np.arange(0, K, 3, dtype=np.int32)]
    for L in lists:
        buf = np.full(K, 5000, dtype=np.int32)          # junk beyond the count
        buf[:len(L)] = L
        idx = torch.from_numpy(buf).to(dev)
        cnt = torch.tensor([len(L)], dtype=torch.int32, device=dev)
        for thr in (ts, None):
            y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
            sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, thr, idx, cnt, y, pm.workspace)
            torch.cuda.synchronize()
            yy = y.cpu().numpy()
            if len(L) == 0:
                assert np.all(yy == 0) and not np.any(np.signbit(yy))
                continue
            if thr is None:
                y_ref, B = oracle.gemv_listed(q, s, z, X, L)
            else:
                Xm = np.where(oracle.active_mask(X, ts), X, np.float16(0))
                y_ref, B = oracle.gemv_listed(q, s, z, Xm, L)
            G.check_y(yy, y_ref, B, f"given list len={len(L)} masked={thr is not None}")
    # a count above K is clamped to K: every column
    idx = torch.arange(K, dtype=torch.int32, device=dev)
    cnt = torch.tensor([K + 100], dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, None, idx, cnt, y, pm.workspace)
    torch.cuda.synchronize()
    y_ref, B = oracle.gemv_dense(q, s, z, X)
    G.check_y(y.cpu().numpy(), y_ref, B, "given list count > K")


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("K,keep", [(28672, 0.95), (65536, 0.6), (65536, 0.002)])
def test_run_batched_given_list_long(K, keep, M):
    """Rows over a long given list: the window searched for each group spans
    several rounds of loads when the count is above 16384, and a near-empty
    list leaves most groups with no entry."""
    from activation_sparse_bit_amd import sgemv
    N = 512
    q, s, z = synth.random_int4_problem(int(K * keep) + 5, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    X = np.stack([synth.plain_activation(90 + m, K) for m in range(M)])
    rng = np.random.default_rng(K)
    L = np.flatnonzero(rng.random(K) < keep).astype(np.int32)
    dev = G.torch_dev()
    buf = np.full(K, -3, dtype=np.int32)
    buf[:len(L)] = L
    idx = torch.from_numpy(buf).to(dev)
    cnt = torch.tensor([len(L)], dtype=torch.int32, device=dev)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    sgemv.sgemv_run_batched(pm.desc, pm.blob, G.to_dev(X), None, idx, cnt, y, pm.workspace)
    torch.cuda.synchronize()
    y_ref, B = oracle.gemv_listed(q, s, z, X, L)
    G.check_y(y.cpu().numpy(), y_ref, B, f"long given list K={K} count={len(L)}")

"""The fused call without a workspace (sgemv_run_fused_static, the library's
fixed device array as scratch) against the call with one (sgemv_run_fused):
two calls in a row on different matrices, the second smaller, each giving
the same list, the same count and the same output bits, within the
acceptance bar of the fp64 oracle.  Also: sizes beyond the array are refused
before any HIP call."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

torch = pytest.importorskip("torch")


def _both(pm, X, ts, dtype):
    """The same call through both entry points; returns (y_ws, idx_ws, c_ws,
    y_static, idx_static, c_static) as host arrays."""
    from activation_sparse_bit_amd import sgemv
    dev = G.torch_dev()
    M, K = X.shape
    xd = G.to_dev(X)
    out = []
    for static in (False, True):
        y = torch.full((M, pm.N), float("nan"), dtype=dtype, device=dev)
        idx = torch.full((K,), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((1,), -7, dtype=torch.int32, device=dev)
        xa, ya = (xd, y) if M > 1 else (xd[0], y[0])
        if static:
            sgemv.sgemv_run_fused_static(pm.desc, pm.blob, xa, ts, ya, idx, cnt)
        else:
            sgemv.sgemv_run_fused(pm.desc, pm.blob, xa, ts, ya, pm.workspace, idx, cnt)
        torch.cuda.synchronize()
        out += [y.cpu().numpy(), idx.cpu().numpy(), int(cnt.item())]
    return out


def _check(pm, q, s, z, X, ts, dtype, what, rows=None):
    yw, iw, cw, ys, is_, cs = _both(pm, X, ts, dtype)
    U = oracle.active_indices(X, ts)
    assert cw == cs == len(U), what
    assert np.array_equal(is_[:cs], U) and np.array_equal(is_, iw), what
    bits = np.uint32 if dtype == torch.float32 else np.uint16
    assert np.array_equal(ys.view(bits), yw.view(bits)), f"{what}: static and workspace outputs differ"
    r = np.arange(pm.N) if rows is None else rows
    y_ref, B, _ = G.oracle_rows(q, s, z, X, ts, r)
    G.check_y(ys.astype(np.float64)[:, r], y_ref, B, what)


@pytest.mark.gpu
def test_static_scratch_two_calls_second_smaller():
    """Eight rows on the 14336 -> 4096 down projection (the many-row kernel,
    its list workgroups and segment sums), then one row on a 2048 x 2048
    matrix (the one-row kernel): both equal the workspace call bit for bit."""
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    X = np.stack([synth.glu_activation(m, K) for m in range(8)])
    ts = [synth.percentile_threshold(X[m], 0.7) for m in range(8)]
    print("static scratch: 8 rows, 14336 -> 4096", flush=True)
    _check(pm, q, s, z, X, ts, torch.float16, "static M=8 down", rows=G.sample_rows(N, 256, seed=8))

    K2 = N2 = 2048
    q2, s2, z2 = G.weights(0, N2, K2, 0.02)
    pm2 = G.packed(0, N2, K2, 0.02)
    x2 = synth.plain_activation(0, K2)[None, :]
    t2 = [synth.percentile_threshold(x2[0], 0.5)]
    print("static scratch: 1 row, 2048 x 2048", flush=True)
    _check(pm2, q2, s2, z2, x2, t2, torch.float32, "static M=1 2048")


@pytest.mark.gpu
def test_static_scratch_one_and_two_rows_down():
    """One and two rows on the down projection (one round of workgroups,
    14 or 28 segments per half tile), after the calls above or alone."""
    K, N = 14336, 4096
    q, s, z = G.weights(0, N, K, 0.02)
    pm = G.packed(0, N, K, 0.02)
    for M, p in ((1, 0.5), (2, 0.7), (1, 0.9)):
        X = np.stack([synth.glu_activation(10 + m, K) for m in range(M)])
        ts = [synth.percentile_threshold(X[m], p) for m in range(M)]
        print(f"static scratch: {M} row(s), p={p}", flush=True)
        _check(pm, q, s, z, X, ts, torch.float16, f"static M={M} p={p}", rows=G.sample_rows(N, 256, seed=M))


def test_static_scratch_refuses_sizes_beyond_the_array():
    """No GPU needed: the size checks come before any HIP call."""
    from activation_sparse_bit_amd import sgemv
    L = sgemv.lib()
    FAKE = 1 << 20
    t = np.array([0.5] * 16, dtype=np.float32)
    # N = 1024 half tiles + one tile: more arrival counters than the array holds
    N, K = 1024 * 256 + 512, 128
    q = np.zeros((512, 128), dtype=np.uint8)
    s_ = np.full((512, 1), 0x3C00, dtype=np.uint16)
    z_ = np.zeros((512, 1), dtype=np.uint16)
    d, _ = sgemv.sgemv_pack_layout(q, s_, z_)
    d.N = N
    d.w_bytes = N * K // 2
    d.m_off = 256 + (d.w_bytes + 255) // 256 * 256
    d.m_bytes = (K // 128) * N * 4
    d.total_bytes = d.m_off + (d.m_bytes + 255) // 256 * 256
    r = L.sgemv_run_fused_static(ctypes.byref(d), FAKE, FAKE, 1, K, t.ctypes.data, None, None, FAKE, N, 0, None)
    assert r == sgemv.SGEMV_ESIZE
    # partial sums of 16 rows on a 57344 x 8192 matrix (224 half tiles x 8
    # segments x 16 KiB = 28 MiB) exceed the array's 15.5 MiB
    N, K = 57344, 8192
    d.N, d.K = N, K
    d.w_bytes = N * K // 2
    d.m_off = 256 + (d.w_bytes + 255) // 256 * 256
    d.m_bytes = (K // 128) * N * 4
    d.total_bytes = d.m_off + (d.m_bytes + 255) // 256 * 256
    r = L.sgemv_run_fused_static(ctypes.byref(d), FAKE, FAKE, 16, K, t.ctypes.data, None, None, FAKE, N, 0, None)
    assert r == sgemv.SGEMV_ESIZE
    # the same matrix with two rows fits the array; argument checks still apply
    r = L.sgemv_run_fused_static(ctypes.byref(d), FAKE, FAKE, 2, K, None, None, None, FAKE, N, 0, None)
    assert r == sgemv.SGEMV_EINVAL      # thresholds are required


@pytest.mark.gpu
def test_static_scratch_groups_along_n():
    """Layout version 3 through both entry points: four rows (matrix cores)
    then one row (vector kernel), bit for bit the workspace call, within the
    bar of the groups-along-N oracle."""
    from activation_sparse_bit_amd import sgemv
    K, N = 4096, 4096
    q, s, z = synth.quantized_weights_ng(1, N, K, 0.02)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev(), ng=True)
    for M, p in ((4, 0.7), (1, 0.5)):
        X = np.stack([synth.plain_activation(50 + m, K) for m in range(M)])
        ts = [synth.percentile_threshold(X[m], p) for m in range(M)]
        print(f"static scratch: groups along N, {M} rows", flush=True)
        yw, iw, cw, ys, is_, cs = _both(pm, X, ts, torch.float32)
        U = oracle.active_indices(X, ts)
        assert cw == cs == len(U) and np.array_equal(is_[:cs], U) and np.array_equal(is_, iw)
        assert np.array_equal(ys.view(np.uint32), yw.view(np.uint32)), "static and workspace outputs differ"
        y_ref, B, _ = oracle.gemv_masked(q, s, z, X, ts, along="n")
        G.check_y(ys.astype(np.float64), y_ref, B, f"static ng M={M}")

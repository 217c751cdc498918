"""Parity on activations whose active entries are mostly or entirely
subnormal fp16 numbers (|x| < 2^-14), on every device path.

The selection rule keeps |x| >= t, so with t = 0 or t = 2^-24 every nonzero
subnormal entry is active and takes part in the product.  Each path (one and
two rows on the vector units, 3..16 rows on the matrix cores; the fused call,
a run over the gathered list and the every-column run) must then agree with
the fp64 oracle within the acceptance bar: per-row relative L2 <= 1e-3 and
every element within 2e-3 * sum |w^| |xe|.  When nearly all of a row's active
entries are subnormal, that bound is set by the subnormal terms themselves,
so a path that flushed them to zero, or rounded their products coarsely,
fails it.

Weights use scales near 1 so that y stays well inside the normal fp16 range
(the fp16 output rounding is then far below the bar)."""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SUB_MAX = 0x03FF   # largest subnormal fp16 magnitude code


def _weights(seed, N, K):
    """q and z uniform over the code space, fp16 scales in [0.5, 2)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16)
    s = rng.uniform(0.5, 2.0, size=(N, K // 128)).astype(np.float16)
    return q, s.view(np.uint16), z.view(np.uint16)


def _subnormal_rows(seed, M, K, normal_frac):
    """fp16 rows: about 5 % exact zeros (both signs), a fraction `normal_frac`
    of small normal numbers (2^-14 .. 2^-12), the rest subnormal with a
    uniform magnitude code 1..1023 and a random sign."""
    rng = np.random.default_rng(seed)
    mag = rng.integers(1, SUB_MAX + 1, size=(M, K)).astype(np.uint16)
    u = rng.random((M, K))
    normal = u < normal_frac
    # small normals: exponent field 1 or 2, any mantissa
    mag[normal] = (rng.integers(1, 3, size=int(normal.sum())) << 10 |
                   rng.integers(0, 1024, size=int(normal.sum()))).astype(np.uint16)
    mag[u > 0.95] = 0
    sign = (rng.integers(0, 2, size=(M, K)) << 15).astype(np.uint16)
    return (mag | sign).view(np.float16)


def _share_subnormal(X, ts):
    """Fraction of the active, nonzero entries that are subnormal."""
    act = oracle.active_mask(X, ts) & (X != 0)
    sub = act & (np.abs(X.astype(np.float32)) < np.float32(2.0 ** -14))
    return float(sub.sum()) / max(1, int(act.sum()))


def _call(entry, pm, X, ts, dtype):
    from activation_sparse_bit_amd import sgemv
    dev = G.torch_dev()
    M, K = X.shape
    xd = G.to_dev(X)
    y = torch.full((M, pm.N), float("nan"), dtype=dtype, device=dev)
    idx = torch.full((K,), -7, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    if entry == "fused":
        sgemv.sgemv_run_fused(pm.desc, pm.blob, xd if M > 1 else xd[0], ts, y if M > 1 else y[0],
                              pm.workspace, idx, cnt)
    elif entry == "list":
        sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
        if M == 1:
            sgemv.sgemv_run(pm.desc, pm.blob, xd[0], idx, cnt, y[0], pm.workspace)
        else:
            sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, idx, cnt, y, pm.workspace)
    elif entry == "dense":
        # every column; rows masked by their thresholds (one row: unmasked,
        # which is the same set for t = 0)
        if M == 1:
            sgemv.sgemv_run(pm.desc, pm.blob, xd[0], None, None, y[0], pm.workspace)
        else:
            sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, None, None, y, pm.workspace)
    else:
        raise KeyError(entry)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("entry", ["fused", "list", "dense"])
@pytest.mark.parametrize("t", [0.0, 2.0 ** -24])
@pytest.mark.parametrize("normal_frac", [0.0, 0.1])
@pytest.mark.parametrize("f32", [True, False])
def test_subnormal_activations(M, entry, t, normal_frac, f32):
    from activation_sparse_bit_amd import sgemv
    if entry == "dense" and M == 1 and t > 0:
        pytest.skip("the one-row every-column call takes no threshold")
    K, N = 2176, 1024           # ragged against the 512- and 1024-column segments
    print(f"subnormal M={M} entry={entry} t={t} normal_frac={normal_frac} f32={f32}", flush=True)
    q, s, z = _weights(77, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    X = _subnormal_rows(100 + M, M, K, normal_frac)
    ts = [t] * M
    assert _share_subnormal(X, ts) > (0.99 if normal_frac == 0 else 0.85)
    y = _call(entry, pm, X, ts, torch.float32 if f32 else torch.float16)
    y_ref, B, _ = oracle.gemv_masked(q, s, z, X, ts)
    assert np.all(B > 0)
    rel = G.check_y(y, y_ref, B, f"subnormal M={M} {entry} t={t} normal_frac={normal_frac} f32={f32}")
    if f32:
        # fp32 output: the products (q - z) x are exact in fp32 for subnormal x
        # too, so the only error left is fp32 accumulation
        assert rel < 2e-6, rel


@pytest.mark.parametrize("M", [1, 2, 8])
def test_subnormal_activations_down_14336(M):
    """The down-projection shape (one full round of workgroups) with every
    active entry subnormal, fp32 output, sampled rows."""
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    q, s, z = _weights(78, N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=G.torch_dev())
    X = _subnormal_rows(200 + M, M, K, 0.0)
    ts = [2.0 ** -24] * M
    y = _call("fused", pm, X, ts, torch.float32)
    rows = G.sample_rows(N, 384, seed=M)
    y_ref, B, _ = G.oracle_rows(q, s, z, X, ts, rows)
    rel = G.check_y(y[:, rows], y_ref, B, f"subnormal down M={M}")
    assert rel < 2e-6, rel

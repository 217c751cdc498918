"""Seeded random combinations through the C ABI on MI355X: every entry point
(fused with and without the list, gather + run, a given list with and
without thresholds, every column), every layout version, fp16 and fp32
outputs, 1..16 rows, K from one group to 72 groups (ragged against every
segment size), N from one tile to eight, sparsity from dense to empty.
Lists and counts are compared bit for bit with the oracle, y on sampled
output rows within the acceptance tolerance, and the arrival counters must
be back at zero after every call."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ENTRIES = ("fused_list", "fused", "split", "given_list", "every_column")
CASES = 80
CASES_NG = 40      # groups along N (layout version 3), seeds of their own


def _case(i):
    rng = np.random.default_rng(9000 + i)
    N = int(rng.choice([512, 1024, 1536, 2048, 2560, 4096]))
    K = 128 * int(rng.integers(1, 73))
    M = int(rng.choice([1, 1, 1, 2, 2, 3, 4, 5, 7, 8, 11, 16]))
    p = float(rng.choice([0.0, 0.25, 0.5, 0.7, 0.9, 0.97, 1.0]))
    return dict(seed=9000 + i, N=N, K=K, M=M, p=p, z4=bool(rng.integers(2)),
                f32=bool(rng.integers(2)), gauss=bool(rng.integers(2)),
                entry=ENTRIES[i % len(ENTRIES)], masked=bool(rng.integers(2)), ng=False)


def _case_ng(i):
    c = _case(500 + i)
    c["ng"], c["z4"] = True, False
    return c


def _thresholds(X, p):
    if p >= 1.0:   # above every magnitude: nothing is active
        return [float(np.abs(X.astype(np.float32)).max()) * 2.0 + 1.0] * X.shape[0]
    return [synth.percentile_threshold(X[m], p) for m in range(X.shape[0])]


@pytest.mark.parametrize("i", range(CASES))
def test_random_combination(i):
    _run(_case(i))


@pytest.mark.parametrize("i", range(CASES_NG))
def test_random_combination_groups_along_n(i):
    _run(_case_ng(i))


def _run(c):
    from activation_sparse_bit_amd import sgemv
    print("case", c, flush=True)
    N, K, M, dev = c["N"], c["K"], c["M"], G.torch_dev()
    if c["ng"]:
        q, s, z = (synth.quantized_weights_ng(c["seed"] % 7, N, K, 0.02) if c["gauss"]
                   else synth.random_int4_problem_ng(c["seed"], N, K))
    elif c["gauss"]:
        q, s, z = synth.quantized_weights(c["seed"] % 7, N, K, 0.02)
    else:
        q, s, z = synth.random_int4_problem(c["seed"], N, K)
    pm = sgemv.PackedMatrix(q, s, z, device=dev, z4=c["z4"], ng=c["ng"])
    X = np.stack([synth.glu_activation(c["seed"] + m, K) for m in range(M)])
    ts = _thresholds(X, c["p"])
    xd = G.to_dev(X)
    ydt = torch.float32 if c["f32"] else torch.float16
    y = torch.full((M, N), float("nan"), dtype=ydt, device=dev)
    idx = torch.full((K,), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=dev)
    U = oracle.active_indices(X, ts)
    rows = G.sample_rows(N, 256, seed=c["seed"])
    entry = c["entry"]
    listed = None
    if entry in ("fused_list", "fused"):
        want = entry == "fused_list"
        sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, ts, y, pm.workspace,
                              idx if want else None, cnt if want else None)
        thr = ts
    elif entry == "split":
        sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
        if M == 1:
            sgemv.sgemv_run(pm.desc, pm.blob, xd[0], idx, cnt, y[0], pm.workspace)
            thr = None      # one row over its own list: masking changes nothing
        else:
            sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, idx, cnt, y, pm.workspace)
            thr = ts
    elif entry == "given_list":
        rng = np.random.default_rng(c["seed"] + 1)
        keep = rng.random(K) < rng.choice([0.02, 0.3, 0.8, 1.0])
        listed = np.flatnonzero(keep).astype(np.int32)
        buf = np.full(K, K + 999, dtype=np.int32)   # junk past the count
        buf[:len(listed)] = listed
        idx = torch.from_numpy(buf).to(dev)
        cnt = torch.tensor([len(listed)], dtype=torch.int32, device=dev)
        thr = ts if c["masked"] else None
        sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, thr, idx, cnt, y, pm.workspace)
    else:   # every column
        thr = ts if c["masked"] else None
        sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, thr, None, None, y, pm.workspace)
    torch.cuda.synchronize()
    tiles = N // 256
    assert int(torch.count_nonzero(pm.workspace[:tiles * 256]).item()) == 0, "arrival counters not reset"

    if entry in ("fused_list", "split"):
        assert int(cnt.item()) == len(U)
        ii = idx.cpu().numpy()
        assert np.array_equal(ii[:len(U)], U)
        assert np.all(ii[len(U):] == -7)

    # groups along N: the oracle on every row (a row's group is n // 128),
    # then the sample; groups along K: the oracle on the sampled rows only
    along = "n" if c["ng"] else "k"
    qs, ss, zs = (q, s, z) if c["ng"] else (q[rows], s[rows], z[rows])
    if entry == "given_list":
        Xe = X if thr is None else np.where(oracle.active_mask(X, thr), X, np.float16(0))
        y_ref, B = oracle.gemv_listed(qs, ss, zs, Xe, listed, along)
    elif entry == "every_column" and thr is None:
        y_ref, B = oracle.gemv_dense(qs, ss, zs, X, along)
    elif thr is None:    # one row over the list of its own active columns
        y_ref, B = oracle.gemv_listed(qs, ss, zs, X, U, along)
    else:
        y_ref, B, _ = oracle.gemv_masked(qs, ss, zs, X, thr, along)
    if c["ng"]:
        y_ref, B = y_ref[:, rows], B[:, rows]
    G.check_y(y.float().cpu().numpy()[:, rows], y_ref, B, str(c))

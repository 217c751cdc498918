"""The hand-off of partial sums between workgroups (device-scope stores, an
arrival counter, device-scope loads by the last workgroup): calls with two
different inputs alternate twenty times through every kernel that splits
the list, and every result must equal, bit for bit, the first result for
the same input.  A stale partial sum from the other input would show."""
import numpy as np
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _alternate(call, inputs, reps=20):
    first = {}
    for r in range(reps):
        for i, inp in enumerate(inputs):
            y = call(inp)
            torch.cuda.synchronize()
            got = y.cpu().numpy().copy()
            if i not in first:
                first[i] = got
            else:
                assert np.array_equal(got.view(np.uint32), first[i].view(np.uint32)), f"input {i}, repetition {r}"
    assert not np.array_equal(first[0], first[1])


@pytest.mark.parametrize("path", ["run", "batched2", "batched4", "fused1", "fused4list", "fused16", "dense"])
def test_alternating_inputs_bitwise(path):
    from activation_sparse_bit_amd import sgemv
    K, N = 14336, 4096
    pm = G.packed(0, N, K, 0.02)
    dev = G.torch_dev()
    M = {"run": 1, "batched2": 2, "batched4": 4, "fused1": 1, "fused4list": 4, "fused16": 16, "dense": 1}[path]
    inputs = []
    for j in range(2):
        X = np.stack([synth.glu_activation(7 * j + m, K) for m in range(M)])
        ts = [synth.percentile_threshold(X[m], 0.5 + 0.2 * j) for m in range(M)]
        inputs.append((G.to_dev(X), ts))
    idx = torch.zeros(K, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def call(inp):
        xd, ts = inp
        if path == "run":
            sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
            sgemv.sgemv_run(pm.desc, pm.blob, xd[0], idx, cnt, y[0], pm.workspace)
        elif path in ("batched2", "batched4"):
            sgemv.sgemv_gather_indices(xd, ts, idx, cnt)
            sgemv.sgemv_run_batched(pm.desc, pm.blob, xd, ts, idx, cnt, y, pm.workspace)
        elif path == "fused4list":
            sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, ts, y, pm.workspace, idx, cnt)
        elif path == "dense":
            sgemv.sgemv_run(pm.desc, pm.blob, xd[0], None, None, y[0], pm.workspace)
        else:
            sgemv.sgemv_run_fused(pm.desc, pm.blob, xd, ts, y, pm.workspace)
        return y

    _alternate(call, inputs)
    tiles = N // 256
    assert int(torch.count_nonzero(pm.workspace[:tiles * 256]).item()) == 0

"""The Python binding checks every buffer before its address crosses the C
ABI: a wrong dtype, a short buffer, a non-contiguous row, a workspace too
small for the call's row count or a host tensor raise ValueError before any
library call is made (on the CPU, a call that reached the library would fail
with SgemvError instead)."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def packed():
    from activation_sparse_bit_amd import sgemv
    K, N = 2048, 1024
    q, s, z = synth.random_int4_problem(3, N, K)
    desc, blob = sgemv.sgemv_pack_layout(q, s, z)
    return sgemv, desc, torch.from_numpy(blob)


def _bufs(desc, M=1, ws_rows=1):
    from activation_sparse_bit_amd import sgemv
    x = torch.zeros((M, desc.K), dtype=torch.float16)
    y = torch.zeros((M, desc.N), dtype=torch.float16)
    idx = torch.zeros(desc.K, dtype=torch.int32)
    cnt = torch.zeros(1, dtype=torch.int32)
    ws = torch.zeros(max(sgemv.sgemv_workspace_bytes(desc, ws_rows), 256), dtype=torch.uint8)
    return x, y, idx, cnt, ws


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_host_tensors_are_refused(packed):
    sgemv, desc, blob = packed
    x, y, idx, cnt, ws = _bufs(desc)
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0], idx, cnt, y[0], ws), "GPU tensor")
    _raises(lambda: sgemv.sgemv_run_fused(desc, blob, x[0], [0.5], y[0], ws, idx, cnt), "GPU tensor")
    _raises(lambda: sgemv.sgemv_gather_indices(x, [0.5], idx, cnt), "GPU tensor")


def test_wrong_dtypes(packed):
    sgemv, desc, blob = packed
    x, y, idx, cnt, ws = _bufs(desc)
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0].float(), idx, cnt, y[0], ws), "x: dtype float32")
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0], idx.long(), cnt, y[0], ws), "idx: dtype int64")
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0], idx, cnt, y[0].double(), ws), "y: dtype float64")
    _raises(lambda: sgemv.sgemv_run(desc, blob.view(torch.int8), x[0], idx, cnt, y[0], ws), "packed: dtype int8")
    _raises(lambda: sgemv.sgemv_gather_indices(x.float(), [0.5], idx, cnt), "x: dtype")


def test_short_buffers(packed):
    sgemv, desc, blob = packed
    x, y, idx, cnt, ws = _bufs(desc)
    _raises(lambda: sgemv.sgemv_run(desc, blob[:-1], x[0], idx, cnt, y[0], ws), "packed")
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0, :-8], idx, cnt, y[0], ws), "x:")
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0], idx[:-1], cnt, y[0], ws), "idx:")
    _raises(lambda: sgemv.sgemv_run(desc, blob, x[0], idx, cnt, y[0, :-8], ws), "y:")
    _raises(lambda: sgemv.sgemv_gather_indices(x, [0.5], idx[:100], cnt), "idx:")
    _raises(lambda: sgemv.sgemv_gather_indices(x, [0.5], idx, cnt[:0]), "count:")


def test_workspace_too_small_for_the_row_count(packed):
    """A workspace sized for one row, used for three: the kernels would write
    the partial sums of three rows past its end."""
    sgemv, desc, blob = packed
    x, y, idx, cnt, ws = _bufs(desc, M=3, ws_rows=1)
    assert sgemv.sgemv_workspace_bytes(desc, 3) > ws.numel()
    _raises(lambda: sgemv.sgemv_run_fused(desc, blob, x, [0.5] * 3, y, ws, idx, cnt), "workspace")
    _raises(lambda: sgemv.sgemv_run_batched(desc, blob, x, [0.5] * 3, idx, cnt, y, ws), "workspace")


def test_rows_and_strides(packed):
    sgemv, desc, blob = packed
    x, y, idx, cnt, ws = _bufs(desc, M=2, ws_rows=2)
    xt = torch.zeros((desc.K, 2), dtype=torch.float16).t()   # columns not contiguous
    _raises(lambda: sgemv.sgemv_run_fused(desc, blob, xt, [0.5] * 2, y, ws), "contiguous")
    _raises(lambda: sgemv.sgemv_run_fused(desc, blob, x, [0.5] * 2, y[:1], ws), r"y: shape")
    _raises(lambda: sgemv.sgemv_run_fused(desc, blob, x, [0.5] * 2, y, ws, idx, None), "both or neither")


def test_checks_come_before_the_library():
    """A call with correct host tensors fails at the device check, not in the
    library: the message names the buffer."""
    from activation_sparse_bit_amd import sgemv
    K, N = 128, 512
    q, s, z = synth.random_int4_problem(4, N, K)
    desc, blob = sgemv.sgemv_pack_layout(q, s, z)
    x = torch.from_numpy(np.zeros(K, dtype=np.float16))
    y = torch.zeros(N, dtype=torch.float16)
    with pytest.raises(ValueError, match="packed: must be a GPU tensor"):
        sgemv.sgemv_run(desc, torch.from_numpy(blob), x, None, None, y, None)

"""A Llama-3-8B-shaped decode layer through the fused call with projections
that share their input packed together (q/k/v as one 4096 -> 6144 matrix,
gate/up as one 4096 -> 28672 matrix): every projection's slice of the
output is checked against the fp64 oracle of that projection alone, and the
list against the oracle's list for the shared input."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _projections(names):
    wl = synth.workload("layer-8b")
    P = {p.name: p for p in wl.projections}
    out = []
    for n in names:
        p = P[n]
        q, s, z = G.weights(p.weight_seed, p.N, p.K, p.sigma)
        out.append((n, q, s, z))
    return out, wl.inputs[P[names[0]].input_name]


@pytest.mark.parametrize("names,rows", [(("q", "k", "v"), None), (("gate", "up"), 384)])
def test_fused_projections_match_each_projection(names, rows):
    from activation_sparse_bit_amd import sgemv
    parts, (kind, index, K) = _projections(names)
    fp = sgemv.FusedProjections(parts, device=G.torch_dev(), max_batch=1)
    x = synth.activation(kind, index, K)
    t = synth.percentile_threshold(x, 0.5)
    xd = G.to_dev(x)
    y = torch.full((fp.N,), float("nan"), dtype=torch.float16, device=G.torch_dev())
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_run_fused(fp.matrix.desc, fp.matrix.blob, xd, [t], y, fp.matrix.workspace, idx, cnt)
    torch.cuda.synchronize()
    U = oracle.active_indices(x, t)
    c = int(cnt.item())
    assert c == len(U) and np.array_equal(idx.cpu().numpy()[:c], U)
    ys = fp.split(y.float().cpu().numpy())
    for name, q, s, z in parts:
        sel = np.arange(q.shape[0]) if rows is None else G.sample_rows(q.shape[0], rows)
        y_ref, B, _ = G.oracle_rows(q, s, z, x, t, sel)
        G.check_y(ys[name][sel][None, :], y_ref, B, f"fused {name}")



def test_fused_projections_groups_along_n():
    """q/k/v quantized with groups along N (layout version 3), packed as
    parts: every projection's slice against its own oracle."""
    from activation_sparse_bit_amd import sgemv
    wl = synth.workload("layer-8b")
    P = {p.name: p for p in wl.projections}
    parts = []
    for n in ("q", "k", "v"):
        p = P[n]
        parts.append((n, *synth.quantized_weights_ng(p.weight_seed, p.N, p.K, p.sigma)))
    kind, index, K = wl.inputs["x_attn"]
    fp = sgemv.FusedProjections(parts, device=G.torch_dev(), max_batch=1, ng=True)
    assert fp.matrix.desc.version == sgemv.SGEMV_LAYOUT_NG
    x = synth.activation(kind, index, K)
    t = synth.percentile_threshold(x, 0.5)
    y = torch.full((fp.N,), float("nan"), dtype=torch.float32, device=G.torch_dev())
    idx = torch.full((K,), -7, dtype=torch.int32, device=G.torch_dev())
    cnt = torch.zeros(1, dtype=torch.int32, device=G.torch_dev())
    sgemv.sgemv_run_fused(fp.matrix.desc, fp.matrix.blob, G.to_dev(x), [t], y, fp.matrix.workspace, idx, cnt)
    torch.cuda.synchronize()
    U = oracle.active_indices(x, t)
    c = int(cnt.item())
    assert c == len(U) and np.array_equal(idx.cpu().numpy()[:c], U)
    ys = fp.split(y.cpu().numpy())
    for name, q, s, z in parts:
        y_ref, B, _ = oracle.gemv_masked(q, s, z, x, t, along="n")
        G.check_y(ys[name][None, :], y_ref, B, f"fused {name} (groups along N)")

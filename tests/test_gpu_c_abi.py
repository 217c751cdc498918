"""The device calls from a plain C program (gcc, the HIP runtime API, no
Python and no PyTorch in the process that calls the library): one fused
launch with the list, the gather then the GEMV over its list, and the dense
GEMV, on the down-projection shape at 50 % sparsity and on a ragged small
matrix.  The list and its count must equal the oracle's bit for bit, the
two sparse outputs must agree bit for bit with each other, and every output
on sampled rows must be within the acceptance tolerance of the fp64 oracle.
The program is built by build() next to the library."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "activation_sparse_bit_amd", "lib", "c_abi_device")


@pytest.mark.parametrize("N,K,p,seed", [(4096, 14336, 0.5, 31), (1536, 128 * 37, 0.7, 32)])
def test_c_program_device_calls(tmp_path, N, K, p, seed):
    print("case", dict(N=N, K=K, p=p, seed=seed), flush=True)
    assert os.path.exists(EXE), "c_abi_device is missing: run build() first"
    q, s, z = synth.quantized_weights(seed % 7, N, K, 0.02)
    x = synth.glu_activation(seed, K)
    t = float(np.float32(synth.percentile_threshold(x, p)))   # the library takes fp32
    q.tofile(tmp_path / "q.bin")
    np.ascontiguousarray(s).view(np.uint16).tofile(tmp_path / "s.bin")
    np.ascontiguousarray(z).view(np.uint16).tofile(tmp_path / "z.bin")
    np.ascontiguousarray(x).view(np.uint16).tofile(tmp_path / "x.bin")
    np.array([t], dtype=np.float32).tofile(tmp_path / "t.bin")

    r = subprocess.run([EXE, str(tmp_path), str(N), str(K)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)

    U = oracle.active_indices(x, t)
    cnt = int(np.fromfile(tmp_path / "count.bin", dtype=np.int32)[0])
    lst = np.fromfile(tmp_path / "list.bin", dtype=np.int32)
    assert cnt == len(U) and np.array_equal(lst, U)

    y1, y2, y3 = (np.fromfile(tmp_path / f"y{i}.bin", dtype=np.float32) for i in (1, 2, 3))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "fused and two-launch outputs differ"
    rows = G.sample_rows(N, 256, seed=seed)
    y_ref, B, _ = oracle.gemv_masked(q[rows], s[rows], z[rows], x, t)
    G.check_y(y1[rows][None], y_ref, B, "fused")
    G.check_y(y2[rows][None], y_ref, B, "gather + run")
    y_ref, B = oracle.gemv_dense(q[rows], s[rows], z[rows], x)
    G.check_y(y3[rows][None], y_ref, B, "every column")

"""Input generator checks (CPU): quantizer error bound, code ranges, seeds,
thresholds that realise the requested sparsity."""
import numpy as np

import synth
from tests.oracle_pins import f16_table


def test_quantizer_bounds():
    W = synth.normal_f32(1, (64, 1024), 0.02)
    W[3, :128] = 0.0                      # a zero group
    W[5, 128:256] = 0.01                  # a constant positive group
    q, s, z = synth.quantize_int4_g128(W)
    F = f16_table()
    assert q.dtype == np.uint8 and q.max() <= 15
    zf = F[z]
    assert np.all(zf == np.rint(zf)) and zf.min() >= 0 and zf.max() <= 15
    sf = F[s]
    assert np.all(sf > 0)
    g = np.arange(1024) // 128
    What = sf[:, g] * (q.astype(np.float64) - zf[:, g])
    err = np.abs(W.astype(np.float64) - What)
    assert np.all(err <= sf[:, g] * (0.5 + 2 ** -9) + 1e-12)
    assert np.all(What[3, :128] == 0.0)


def test_quantizer_ng_bounds():
    """Groups along the outputs: every weight within half a step of its
    reconstruction s[n // 128, k] * (q - z[n // 128, k])."""
    W = synth.normal_f32(2, (512, 256), 0.02)
    W[:128, 7] = 0.0                      # a zero group
    W[128:256, 9] = 0.01                  # a constant positive group
    q, s, z = synth.quantize_int4_ng128(W)
    F = f16_table()
    assert q.shape == (512, 256) and s.shape == (4, 256) and z.shape == (4, 256)
    assert q.dtype == np.uint8 and q.max() <= 15
    zf, sf = F[z], F[s]
    assert np.all(zf == np.rint(zf)) and zf.min() >= 0 and zf.max() <= 15 and np.all(sf > 0)
    b = np.arange(512) // 128
    What = sf[b, :] * (q.astype(np.float64) - zf[b, :])
    err = np.abs(W.astype(np.float64) - What)
    # half a step, except at a clipped code (0 or 15), where the rounding of
    # the zero-point can add up to another half step
    clipped = (q == 0) | (q == 15)
    assert np.all(err[~clipped] <= (sf[b, :] * (0.5 + 2 ** -9))[~clipped] + 1e-12)
    assert np.all(err[clipped] <= (sf[b, :] * (1.0 + 2 ** -9))[clipped] + 1e-12)
    assert np.all(What[:128, 7] == 0.0)
    # a group's step follows its own column and output block only
    W2 = W.copy()
    W2[256:384, 11] *= 4
    q2, s2, z2 = synth.quantize_int4_ng128(W2)
    changed = np.argwhere(s2 != s)
    assert len(changed) == 1 and tuple(changed[0]) == (2, 11)


def test_seeds_reproducible():
    a = synth.glu_activation(0, 2048)
    b = synth.glu_activation(0, 2048)
    assert a.dtype == np.float16 and np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert not np.array_equal(synth.glu_activation(1, 2048), a)


def test_percentile_threshold_sparsity():
    x = synth.glu_activation(0, 14336)
    for p in (0.5, 0.7, 0.9):
        t = synth.percentile_threshold(x, p)
        kept = np.count_nonzero(np.abs(x.astype(np.float32)) >= np.float32(t))
        realised = 1 - kept / x.size
        assert realised <= p + 1e-12 and realised >= p - 0.01
    assert synth.percentile_threshold(x, 0.0) == 0.0


def test_workloads():
    for name in ("single-2048", "down-14336", "layer-8b", "mlp-70b", "batched-14336"):
        wl = synth.workload(name)
        for p in wl.projections:
            assert p.K % 128 == 0 and p.N % 512 == 0
            assert p.input_name in wl.inputs

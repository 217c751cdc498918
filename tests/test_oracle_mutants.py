"""The pins catch plausible mistakes planted in a copy of the oracle (CPU).

Each case edits one line of the oracle's source text, loads the edited copy
as a fresh module and runs every pin against it; at least one pin must
fail.  The real oracle is never modified.
"""
import os
import types

import pytest

from tests import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("gemv.py", "mag >= T[:, None]", "mag > T[:, None]", "strict threshold"),
    ("gemv.py", "act = act.any(axis=0)", "act = act.all(axis=0)", "intersection instead of union"),
    ("gemv.py", "        g = k // GROUP\n", "        g = (k // GROUP) % sT.shape[0] if k < 128 else (k - 1) // GROUP\n", "off-by-one group index"),
    ("gemv.py", "w = sT[g] * (qT[pos[k]].astype(np.float64) - zT[g])",
     "w = sT[g] * (zT[g] - qT[pos[k]].astype(np.float64))", "sign of q - z"),
    ("gemv.py", "w = sT[g] * (qT[pos[k]].astype(np.float64) - zT[g])",
     "w = sT[g] * qT[pos[k]].astype(np.float64) - zT[g]", "zero-point not scaled"),
    ("gemv.py", "XE = np.where(act[:, U], X[:, U].astype(np.float64), 0.0)",
     "XE = X[:, U].astype(np.float64)", "batched rows not masked"),
    ("gemv.py", "B[m] += np.abs(w) * abs(xv)", "B[m] += w * abs(xv)", "error scale signed"),
    ("gemv.py", "s = _f16_bits_to_f64(s_bits)[:, g]", "s = _f16_bits_to_f64(z_bits)[:, g]", "scale/zero swapped in dequantize"),
    ("gemv.py", "with np.errstate(invalid=\"ignore\"):\n        act = mag >= T[:, None]",
     "with np.errstate(invalid=\"ignore\"):\n        act = ~(mag < T[:, None])", "NaN treated as active"),
    ("layout.py", "byte = qt[:, :, 0::2] | (qt[:, :, 1::2] << 4)",
     "byte = (qt[:, :, 0::2] << 4) | qt[:, :, 1::2]", "nibble order"),
    ("layout.py", "qt = q.reshape(T, tile_n, K).transpose(0, 2, 1)",
     "qt = q.reshape(tile_n, T, K).transpose(1, 2, 0)", "tile rows interleaved"),
    ("layout.py", "pair[..., 0] = s_bits", "pair[..., 0] = z_bits", "metadata order"),
    ("layout.py", "struct.pack(\"<iiii\", N, K, GROUP, tile_n)", "struct.pack(\"<iiii\", K, N, GROUP, tile_n)", "header N/K"),
    ("layout.py", "run[:, :, 2 * tile_n:] = zt[:, :, 0::2] | (zt[:, :, 1::2] << 4)",
     "run[:, :, 2 * tile_n:] = (zt[:, :, 0::2] << 4) | zt[:, :, 1::2]", "compact zero-point nibble order"),
    ("layout.py", "zt = zc.reshape(T, tile_n, Gk).transpose(0, 2, 1)",
     "zt = zc.reshape(T, Gk, tile_n)", "compact zero-points not transposed to [t][g][i]"),
    ("gemv.py", "        blk = np.arange(N) // GROUP\n", "        blk = np.arange(N) % (N // GROUP)\n",
     "groups along N: output blocks interleaved"),
    ("gemv.py", "w = sC[k][blk] * (qT[pos[k]].astype(np.float64) - zC[k][blk])",
     "w = sC[k][blk] * (qT[pos[k]].astype(np.float64) - zC[k][blk[::-1]])", "groups along N: zero-point of another block"),
    ("gemv.py", "        s = _f16_bits_to_f64(s_bits)[blk][:, cols]\n", "        s = _f16_bits_to_f64(s_bits)[:, cols][blk % 1]\n",
     "groups along N: one block's scale for every output in dequantize"),
    ("layout.py", "pair[..., 0] = s_bits.reshape(H, 2, K).transpose(0, 2, 1)",
     "pair[..., 0] = s_bits.reshape(2, H, K).transpose(1, 2, 0)", "groups along N: groups paired across halves"),
    ("layout.py", "pair[..., 1] = z_bits.reshape(H, 2, K).transpose(0, 2, 1)",
     "pair[..., 1] = s_bits.reshape(H, 2, K).transpose(0, 2, 1)", "groups along N: scale written as zero-point"),
]


def _load_mutant(fname, old, new):
    impl = types.SimpleNamespace()
    for mod in ("gemv.py", "layout.py"):
        with open(os.path.join(ROOT, "oracle", mod)) as f:
            src = f.read()
        if mod == fname:
            assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
            src = src.replace(old, new, 1)
        ns = {"__name__": "oracle_mutant_" + mod[:-3]}
        exec(compile(src, f"<mutant {mod}>", "exec"), ns)
        for k, v in ns.items():
            if callable(v) and not k.startswith("__"):
                setattr(impl, k, v)
    return impl


@pytest.mark.parametrize("fname,old,new,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_pins_catch_mutant(fname, old, new, what):
    impl = _load_mutant(fname, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(impl)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake: {what}"


def test_unmutated_copy_passes():
    impl = _load_mutant("gemv.py", "GROUP = 128", "GROUP = 128")
    for pin in P.ALL_PINS:
        pin(impl)

"""fp64 CPU oracle for the dynamically sparse int4 GEMV.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library (no
kernels, headers, helpers, tables or constant generators); both sides receive
the same seeded arrays from ``synth`` and nothing else.

What it computes comes from "Enabling Dynamic Sparsity in Quantized LLM
Inference" (Abstract): at decode time the activation vector is dynamically
sparse, only the weight columns that match the surviving activation indices
are used, and the weights are stored group-wise quantized.  The method only
changes how fast that result is reached, so the oracle is the plain
definition written out in float64:

  active(m,k) = float32(|x[m,k]|) >= t[m]          (NaN is never active)
  U           = ascending { k : active(m,k) for some m }
  w^(n,k)     = s[n,k//128] * (q[n,k] - z[n,k//128])
  xe(m,k)     = x[m,k] if active(m,k) else 0
  y[m,n]      = sum over k in U, ascending, of w^(n,k) * xe(m,k)
  B[m,n]      = sum over k of |w^(n,k)| * |xe(m,k)|   (error scale)

and the packed weight layout is the byte formula in ``oracle.layout``.

Pins: every function here is checked against values fixed independently of
it (brute force on tiny inputs, exact rational arithmetic, closed forms and
invariants) by the CPU tests; see tests/test_oracle_*.py.
"""
from .gemv import (GROUP, active_mask, active_indices, dequantize_columns,
                   gemv_listed, gemv_masked, gemv_dense)
from .layout import pack_spec, unpack_spec, header_fields, read_header

__all__ = ["GROUP", "active_mask", "active_indices", "dequantize_columns",
           "gemv_listed", "gemv_masked", "gemv_dense",
           "pack_spec", "unpack_spec", "header_fields", "read_header"]

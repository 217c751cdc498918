"""fp64 definition of thresholding, index selection and the sparse GEMV.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Enabling Dynamic Sparsity in Quantized LLM Inference", Abstract.
The page states the problem (dynamically sparse activations select weight
columns of a group-wise low-bit quantized matrix during decode; the active
indices are gathered at run time) but not the thresholding rule, the
quantization format or any constant.  The readings taken here:

* activation selection is magnitude thresholding with a calibrated scalar
  per input row, as in training-free activation sparsity ("Training-Free
  Activation Sparsity in Large Language Models", listed among the works the
  page builds on): entry k of row m is active iff float32(|x[m,k]|) >= t[m];
  ties are kept, NaN is never active, -0 is active when t == 0;
* weights are asymmetric int4 with one fp16 scale s and one fp16 zero-point
  z per output row and group of 128 consecutive inputs, dequantized as
  s*(q - z) ("GPTQ", also on that list);
* layout version 3 reads the groups the other way ("groups along N", so
  that a column's scale and zero-point are read only when the column is
  active, and metadata bytes fall with the sparsity, as the page's call for a
  layout consistent with activation sparsity suggests): one scale s and one
  zero-point z per input column k and block of 128 consecutive outputs,
  dequantized as s[n//128, k]*(q[n, k] - z[n//128, k]); every function takes
  ``along="n"`` for that format (s and z then have shape [N/128][K]);
* a batch of rows is served over the union of the rows' active indices,
  every row using its own masked activations ("Polar Sparsity: High
  Throughput Batched LLM Inferencing with Scalable Contextual Sparsity",
  same list).

Every function is plain NumPy in float64, one weight column at a time in
ascending column order, with no blocking or reordering.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def _f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _rows(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("activations must be float16")
    return x.reshape(1, -1) if x.ndim == 1 else x


def active_mask(x, t) -> np.ndarray:
    """Boolean mask of active entries.

    ``x`` is fp16 [K] or [M][K]; ``t`` is one threshold or one per row.  The
    thresholds cross the library boundary as fp32, so they are rounded to
    fp32 first; |x| of an fp16 value is exact in fp32.  A NaN compares false
    and is therefore never active.
    """
    X = _rows(x)
    T = np.asarray(t, dtype=np.float64).reshape(-1).astype(np.float32)
    if T.size == 1 and X.shape[0] > 1:
        T = np.repeat(T, X.shape[0])
    if T.size != X.shape[0]:
        raise ValueError("one threshold per row")
    mag = np.abs(X.astype(np.float32))
    with np.errstate(invalid="ignore"):
        act = mag >= T[:, None]
    return act.reshape(np.asarray(x).shape)


def active_indices(x, t) -> np.ndarray:
    """Ascending int32 list of the indices active in at least one row."""
    act = active_mask(x, t)
    if act.ndim == 2:
        act = act.any(axis=0)
    return np.flatnonzero(act).astype(np.int32)


def dequantize_columns(q, s_bits, z_bits, cols, along="k") -> np.ndarray:
    """w^[:, cols] in float64: s[n, k//128] * (q[n, k] - z[n, k//128]), or
    with ``along="n"`` s[n//128, k] * (q[n, k] - z[n//128, k])."""
    cols = np.asarray(cols, dtype=np.int64)
    if along == "n":
        blk = np.arange(np.asarray(q).shape[0]) // GROUP
        s = _f16_bits_to_f64(s_bits)[blk][:, cols]
        z = _f16_bits_to_f64(z_bits)[blk][:, cols]
        return s * (np.asarray(q)[:, cols].astype(np.float64) - z)
    g = cols // GROUP
    s = _f16_bits_to_f64(s_bits)[:, g]
    z = _f16_bits_to_f64(z_bits)[:, g]
    return s * (np.asarray(q)[:, cols].astype(np.float64) - z)


def _sum_columns(q, s_bits, z_bits, XE, cols, along="k"):
    """y[m,n] = sum_j w^(n, cols[j]) * XE[m, j] and the error scale
    B[m,n] = sum_j |w^(n, cols[j])| * |XE[m, j]|, one column at a time in the
    order given (groups along K, or along N with ``along="n"``)."""
    q = np.asarray(q)
    N = q.shape[0]
    M = XE.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    B = np.zeros((M, N), dtype=np.float64)
    if len(cols) == 0:
        return y, B
    # Column-major copies so that one weight column is one contiguous row
    # (a transposition only; no arithmetic is reordered).
    qT = np.ascontiguousarray(q[:, np.unique(cols)].T)
    pos = {int(k): i for i, k in enumerate(np.unique(cols))}
    if along == "n":
        # scale and zero-point of column k for every output n: block n // 128
        blk = np.arange(N) // GROUP
        sC = np.ascontiguousarray(_f16_bits_to_f64(s_bits).T)   # [K][N/128]
        zC = np.ascontiguousarray(_f16_bits_to_f64(z_bits).T)
    else:
        sT = np.ascontiguousarray(_f16_bits_to_f64(s_bits).T)
        zT = np.ascontiguousarray(_f16_bits_to_f64(z_bits).T)
    for j, k in enumerate(cols):
        k = int(k)
        if along == "n":
            w = sC[k][blk] * (qT[pos[k]].astype(np.float64) - zC[k][blk])
        else:
            g = k // GROUP
            w = sT[g] * (qT[pos[k]].astype(np.float64) - zT[g])
        for m in range(M):
            xv = XE[m, j]
            if xv != 0.0:
                y[m] += w * xv
                B[m] += np.abs(w) * abs(xv)
    return y, B


def gemv_listed(q, s_bits, z_bits, x, idx, along="k"):
    """The product over a given index list, activations used unmasked.

    y[m,n] = sum over listed k (in list order) of w^(n,k) * x[m,k].
    Returns (y, B) as float64 [M][N] (M = 1 for a vector ``x``).
    """
    X = _rows(x)
    idx = np.asarray(idx, dtype=np.int64)
    XE = X[:, idx].astype(np.float64)
    return _sum_columns(q, s_bits, z_bits, XE, idx, along)


def gemv_masked(q, s_bits, z_bits, x, t, along="k"):
    """The thresholded product: columns of the union U, each row masked by
    its own threshold.  Returns (y, B, U)."""
    X = _rows(x)
    act = active_mask(X, t)
    U = np.flatnonzero(act.any(axis=0))
    XE = np.where(act[:, U], X[:, U].astype(np.float64), 0.0)
    y, B = _sum_columns(q, s_bits, z_bits, XE, U, along)
    return y, B, U.astype(np.int32)


def gemv_dense(q, s_bits, z_bits, x, along="k"):
    """Every column, no thresholding: the dense dequantized GEMV."""
    X = _rows(x)
    K = X.shape[1]
    return gemv_listed(q, s_bits, z_bits, X, np.arange(K), along)

"""Pins of the fp64 oracle: checks against values fixed independently of it.

Each ``pin_*`` takes an oracle implementation (the ``oracle`` package, or a
copy of it with a planted mistake) and raises AssertionError when the
implementation disagrees with:

* brute force on tiny inputs (pure-Python loops, fp16 decoded with
  ``struct`` rather than NumPy),
* exact rational arithmetic (``fractions.Fraction``) on inputs chosen so
  that every float64 sum is exact,
* closed forms (q == z gives zero, one-hot activations, constant groups),
* invariants (doubling x and t doubles y, batched row m equals the single
  row, the listed product over the selected indices equals the masked one,
  t = 0 equals the dense product, a full dense matrix product),
* hand-derived golden fixtures under tests/golden/.
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# fp16 decode table built with struct, independent of numpy's float16
_F16 = None


def f16_table() -> np.ndarray:
    global _F16
    if _F16 is None:
        _F16 = np.array([struct.unpack("<e", struct.pack("<H", b))[0]
                         for b in range(65536)], dtype=np.float64)
    return _F16


def f16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def f32_round(t: float) -> float:
    return struct.unpack("<f", struct.pack("<f", t))[0]


def bits_to_f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


# --------------------------------------------------------------------------
# index selection
# --------------------------------------------------------------------------
def brute_force_indices(rows_bits, ts):
    """Pure-Python selection: k is selected iff some row m has
    |x[m][k]| >= fp32(t[m]); NaN never is."""
    K = len(rows_bits[0])
    out = []
    for k in range(K):
        hit = False
        for m, row in enumerate(rows_bits):
            v = f16_value(row[k])
            if v != v:        # NaN
                continue
            if abs(v) >= f32_round(ts[m]):
                hit = True
        if hit:
            out.append(k)
    return out


def _special_rows(seed, M, K):
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16).copy()
    specials = [0x0000, 0x8000, 0x7E00, 0xFE00, 0x7C00, 0xFC00, 0x0001, 0x8001,
                0x03FF, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF]
    for m in range(M):
        pos = rng.choice(K, size=len(specials), replace=False)
        rows[m, pos] = specials
    return rows


def pin_select_bruteforce(impl):
    for seed in range(6):
        for M in (1, 3):
            K = 128 if seed % 2 == 0 else 256
            rows = _special_rows(seed, M, K)
            rng = np.random.default_rng(100 + seed)
            # thresholds: zero, an existing magnitude (a tie), random, above max
            cand = [0.0, abs(f16_value(rows[0, 5])), float(rng.uniform(0, 2)), 1e6,
                    f16_value(0x0001)]
            for t0 in cand:
                ts = [t0] + [float(rng.choice(cand)) for _ in range(M - 1)]
                got = impl.active_indices(bits_to_f16(rows if M > 1 else rows[0]),
                                          ts if M > 1 else ts[0])
                exp = brute_force_indices(rows.tolist(), ts)
                assert list(np.asarray(got)) == exp, (seed, M, ts)
                assert np.asarray(got).dtype == np.int32


def pin_select_golden(impl):
    with open(os.path.join(GOLDEN, "select_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        rows = np.array(c["rows"], dtype=np.uint16)
        x = bits_to_f16(rows if len(rows) > 1 else rows[0])
        t = c["t"] if len(rows) > 1 else c["t"][0]
        got = list(np.asarray(impl.active_indices(x, t)))
        assert got == c["expect"], (c, got)


# --------------------------------------------------------------------------
# GEMV
# --------------------------------------------------------------------------
def _exact_problem(seed, N=6, K=256, M=2):
    """Power-of-two scales, integer zero points, activations with magnitudes
    in [2^-6, 2^3): every product is exact and every float64 sum of at most
    K such terms is exact, in any order."""
    rng = np.random.default_rng(seed)
    Gk = K // 128
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    expo = rng.integers(-8, -2, size=(N, Gk))
    s = (2.0 ** expo).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, Gk)).astype(np.float16).view(np.uint16)
    e = rng.integers(15 - 6, 15 + 3, size=(M, K))          # biased exponent
    mant = rng.integers(0, 1024, size=(M, K))
    sign = rng.integers(0, 2, size=(M, K))
    xb = ((sign << 15) | (e << 10) | mant).astype(np.uint16)
    # thresholds: the magnitude of an existing entry (ties are kept)
    ts = [abs(f16_value(xb[m, rng.integers(0, K)])) for m in range(M)]
    return q, s, z, xb, ts


def _exact_masked(q, s, z, xb, ts):
    N, K = q.shape
    M = xb.shape[0]
    act = [[abs(f16_value(xb[m, k])) >= f32_round(ts[m]) for k in range(K)] for m in range(M)]
    y = [[Fraction(0)] * N for _ in range(M)]
    B = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            g = k // 128
            w = Fraction(f16_value(s[n, g])) * (int(q[n, k]) - Fraction(f16_value(z[n, g])))
            for m in range(M):
                if act[m][k]:
                    xv = Fraction(f16_value(xb[m, k]))
                    y[m][n] += w * xv
                    B[m][n] += abs(w) * abs(xv)
    return y, B


def pin_gemv_exact_rational(impl):
    for seed in range(3):
        q, s, z, xb, ts = _exact_problem(seed)
        y_ex, B_ex = _exact_masked(q, s, z, xb, ts)
        y, B, U = impl.gemv_masked(q, s, z, bits_to_f16(xb), ts)
        for m in range(len(ts)):
            for n in range(q.shape[0]):
                assert y[m, n] == float(y_ex[m][n]), (seed, m, n, y[m, n], float(y_ex[m][n]))
                assert B[m, n] == float(B_ex[m][n]), (seed, m, n)
        # single row, listed form over that row's own selection
        for m in range(len(ts)):
            idx = impl.active_indices(bits_to_f16(xb[m]), ts[m])
            y1, B1 = impl.gemv_listed(q, s, z, bits_to_f16(xb[m]), idx)
            y_ex1, _ = _exact_masked(q, s, z, xb[m:m + 1], ts[m:m + 1])
            for n in range(q.shape[0]):
                assert y1[0, n] == float(y_ex1[0][n])


def pin_gemv_q_equals_z(impl):
    rng = np.random.default_rng(7)
    N, K = 8, 256
    z_int = rng.integers(0, 16, size=(N, K // 128))
    q = np.repeat(z_int, 128, axis=1).astype(np.uint8)
    s = (rng.uniform(0.001, 0.1, size=(N, K // 128))).astype(np.float16).view(np.uint16)
    z = z_int.astype(np.float16).view(np.uint16)
    x = rng.standard_normal(K).astype(np.float16)
    y, B, U = impl.gemv_masked(q, s, z, x, 0.0)
    assert np.all(y == 0.0) and np.all(B == 0.0)
    assert len(U) == K


def pin_gemv_one_hot(impl):
    rng = np.random.default_rng(11)
    N, K = 16, 384
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.001, 0.1, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    for k0 in (0, 127, 128, 200, 383):
        cbits = 0x4A80  # 13.0
        x = np.zeros(K, dtype=np.uint16)
        x[k0] = cbits
        y, B, U = impl.gemv_masked(q, s, z, bits_to_f16(x), 0.5)
        assert list(U) == [k0]
        g = k0 // 128
        for n in range(N):
            w = f16_value(s[n, g]) * (int(q[n, k0]) - f16_value(z[n, g]))
            assert y[0, n] == w * 13.0
            assert B[0, n] == abs(w) * 13.0


def pin_gemv_constant_group(impl):
    rng = np.random.default_rng(12)
    N, K = 8, 512
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    a = rng.integers(0, 16, size=N)
    g0 = 2
    q[:, g0 * 128:(g0 + 1) * 128] = a[:, None]
    s = rng.uniform(0.001, 0.1, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    x = np.zeros(K, dtype=np.float16)
    x[g0 * 128:(g0 + 1) * 128] = np.float16(0.75)
    y, B, U = impl.gemv_masked(q, s, z, x, 0.5)
    for n in range(N):
        exp = f16_value(s[n, g0]) * (int(a[n]) - f16_value(z[n, g0])) * 0.75 * 128
        assert abs(y[0, n] - exp) <= 1e-15 * abs(exp), (n, y[0, n], exp)


def pin_gemv_scale_equivariance(impl):
    rng = np.random.default_rng(13)
    N, K = 32, 1024
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.001, 0.1, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    x = rng.standard_normal(K).astype(np.float16)
    t = 0.7
    y1, B1, U1 = impl.gemv_masked(q, s, z, x, t)
    y2, B2, U2 = impl.gemv_masked(q, s, z, (x.astype(np.float32) * 2).astype(np.float16), 2 * t)
    assert np.array_equal(U1, U2)
    assert np.array_equal(y2, 2 * y1) and np.array_equal(B2, 2 * B1)


def pin_gemv_matches_matrix_product(impl):
    """Masked and dense products against a full dequantized matrix product,
    the matrix decoded with the struct-built fp16 table."""
    F = f16_table()
    rng = np.random.default_rng(14)
    N, K, M = 48, 640, 3
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.001, 0.1, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    xb = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    ts = [0.3, 0.9, 1.6]
    Wd = F[s][:, np.arange(K) // 128] * (q.astype(np.float64) - F[z][:, np.arange(K) // 128])
    X = F[xb]
    act = np.abs(X) >= np.array([f32_round(t) for t in ts])[:, None]
    XE = np.where(act, X, 0.0)
    y, B, U = impl.gemv_masked(q, s, z, bits_to_f16(xb), ts)
    ref = XE @ Wd.T
    refB = np.abs(XE) @ np.abs(Wd).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(refB).max())
    assert np.allclose(B, refB, rtol=1e-12)
    assert list(U) == list(np.flatnonzero(act.any(axis=0)))
    yd, Bd = impl.gemv_dense(q, s, z, bits_to_f16(xb[0]))
    assert np.allclose(yd[0], Wd @ X[0], rtol=1e-12, atol=1e-12 * refB.max())
    # t = 0 selects every column: equals the dense product exactly
    y0, B0, U0 = impl.gemv_masked(q, s, z, bits_to_f16(xb[0]), 0.0)
    assert len(U0) == K and np.array_equal(y0, yd)


def pin_batched_rows(impl):
    rng = np.random.default_rng(15)
    N, K, M = 24, 512, 5
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.001, 0.1, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    ts = [0.2, 0.5, 1.0, 1.5, 2.5]
    y, B, U = impl.gemv_masked(q, s, z, X, ts)
    for m in range(M):
        ym, Bm, Um = impl.gemv_masked(q, s, z, X[m], ts[m])
        assert np.allclose(y[m], ym[0], rtol=1e-13, atol=1e-13 * Bm.max())
        assert set(Um.tolist()) <= set(U.tolist())


def pin_dequantize(impl):
    F = f16_table()
    rng = np.random.default_rng(16)
    N, K = 10, 384
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.001, 0.1, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    cols = np.array([0, 5, 127, 128, 255, 256, 383])
    got = impl.dequantize_columns(q, s, z, cols)
    for j, k in enumerate(cols):
        for n in range(N):
            assert got[n, j] == F[s[n, k // 128]] * (int(q[n, k]) - F[z[n, k // 128]])


# --------------------------------------------------------------------------
# packed layout
# --------------------------------------------------------------------------
def pin_layout_closed_form(impl):
    for (N, K, Tn) in ((64, 128, 64), (256, 256, 128), (512, 384, 512), (1024, 128, 1024)):
        n = np.arange(N)[:, None]
        k = np.arange(K)[None, :]
        q = ((n + 3 * k) % 16).astype(np.uint8)
        Gk = K // 128
        g = np.arange(Gk)[None, :]
        s = ((0x3000 + 7 * n + 13 * g) & 0x7BFF).astype(np.uint16)
        z = (((n + g) % 16)).astype(np.float16).view(np.uint16)
        blob = np.asarray(impl.pack_spec(q, s, z, Tn))
        w_off = 256
        m_off = w_off + ((N * K // 2 + 255) // 256) * 256
        T = N // Tn
        for t in range(T):
            for kk in (0, 1, K // 2, K - 1):
                base = w_off + (t * K + kk) * (Tn // 2)
                for j in range(Tn // 2):
                    exp = ((t * Tn + 2 * j + 3 * kk) % 16) | (((t * Tn + 2 * j + 1 + 3 * kk) % 16) << 4)
                    assert blob[base + j] == exp, (N, K, Tn, t, kk, j)
            for gg in range(Gk):
                for i in (0, 1, Tn - 1):
                    off = m_off + ((t * Gk + gg) * Tn + i) * 4
                    nn = t * Tn + i
                    sb = int(blob[off]) | int(blob[off + 1]) << 8
                    zb = int(blob[off + 2]) | int(blob[off + 3]) << 8
                    assert sb == ((0x3000 + 7 * nn + 13 * gg) & 0x7BFF)
                    assert f16_value(zb) == (nn + gg) % 16


def pin_layout_roundtrip(impl):
    rng = np.random.default_rng(17)
    for Tn in (64, 128, 256, 512, 1024):
        N, K = 1024, 256
        q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        s = rng.integers(0, 0x7C00, size=(N, K // 128)).astype(np.uint16)
        z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
        blob = impl.pack_spec(q, s, z, Tn)
        q2, s2, z2, h = impl.unpack_spec(blob)
        assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(z, z2)
        assert h["tile_n"] == Tn and h["N"] == N and h["K"] == K


def pin_layout_golden(impl):
    with open(os.path.join(GOLDEN, "layout_tiny.json")) as f:
        gd = json.load(f)
    N, K, Tn = gd["N"], gd["K"], gd["tile_n"]
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    q = ((n + 3 * k) % 16).astype(np.uint8)
    s = (0x3C00 + np.arange(N)[:, None]).astype(np.uint16)
    z = (0x4000 + np.arange(N)[:, None]).astype(np.uint16)
    blob = np.asarray(impl.pack_spec(q, s, z, Tn))
    h = impl.read_header(blob)
    for key, v in gd["header"].items():
        assert h[key] == v, key
    assert bytes(blob[:4]) == b"SGV1" and h["version"] == 1
    assert len(blob) == gd["header"]["total_bytes"]

    def hexat(off, nbytes):
        return bytes(blob[off:off + nbytes]).hex()

    assert hexat(256, 32) == gd["weight_bytes_at_w_off"].replace(" ", "")
    assert hexat(256 + 32, 32) == gd["weight_bytes_at_w_off_plus_32"].replace(" ", "")
    assert hexat(4352, 16) == gd["metadata_bytes_at_m_off"].replace(" ", "")


def pin_layout_z4_closed_form(impl):
    """Version 2: same weight bytes as version 1; per (tile, group) the fp16
    scales, then the integer zero-points two per byte (even row low)."""
    for (N, K, Tn) in ((64, 128, 64), (256, 384, 128), (1024, 256, 512)):
        n = np.arange(N)[:, None]
        k = np.arange(K)[None, :]
        q = ((n + 3 * k) % 16).astype(np.uint8)
        Gk = K // 128
        g = np.arange(Gk)[None, :]
        s = ((0x3000 + 7 * n + 13 * g) & 0x7BFF).astype(np.uint16)
        z = (((n + 5 * g) % 16)).astype(np.float16).view(np.uint16)
        b2 = np.asarray(impl.pack_spec(q, s, z, Tn, 2))
        b1 = np.asarray(impl.pack_spec(q, s, z, Tn))
        h = impl.read_header(b2)
        m_off = 256 + ((N * K // 2 + 255) // 256) * 256
        assert h["version"] == 2 and h["m_off"] == m_off and h["m_bytes"] == Gk * N * 5 // 2
        assert h["total_bytes"] == m_off + (Gk * N * 5 // 2 + 255) // 256 * 256 == len(b2)
        assert np.array_equal(b2[256:m_off], b1[256:m_off])
        run = 5 * Tn // 2
        for t in range(N // Tn):
            for gg in range(Gk):
                base = m_off + (t * Gk + gg) * run
                for i in (0, 1, Tn // 2, Tn - 1):
                    nn = t * Tn + i
                    assert int(b2[base + 2 * i]) | int(b2[base + 2 * i + 1]) << 8 == ((0x3000 + 7 * nn + 13 * gg) & 0x7BFF)
                for j in (0, 1, Tn // 4, Tn // 2 - 1):
                    nn = t * Tn + 2 * j
                    assert b2[base + 2 * Tn + j] == ((nn + 5 * gg) % 16) | (((nn + 1 + 5 * gg) % 16) << 4)


def pin_layout_z4_roundtrip(impl):
    rng = np.random.default_rng(29)
    for Tn in (64, 256, 1024):
        N, K = 1024, 384
        q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        s = rng.integers(0, 0x7C00, size=(N, K // 128)).astype(np.uint16)
        z = rng.integers(0, 16, size=(N, K // 128)).astype(np.float16).view(np.uint16)
        q2, s2, z2, h = impl.unpack_spec(impl.pack_spec(q, s, z, Tn, 2))
        assert h["version"] == 2
        assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(z, z2)
    bad = np.full((N, K // 128), np.float16(7.5).view(np.uint16), dtype=np.uint16)
    try:
        impl.pack_spec(q, s, bad, 512, 2)
    except ValueError:
        return
    raise AssertionError("a zero-point that is not an integer 0..15 was packed in 4 bits")


# --------------------------------------------------------------------------
# groups along N (layout version 3)
# --------------------------------------------------------------------------
def _ng_problem(seed, N, K, exact=False):
    """Codes, and scale/zero-point bit patterns per (group of 128 outputs,
    column): [N/128][K].  ``exact``: power-of-two scales, so every product
    with an fp16 activation of small exponent range is exact."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    if exact:
        s = (2.0 ** rng.integers(-8, -2, size=(N // 128, K))).astype(np.float16).view(np.uint16)
    else:
        s = rng.uniform(0.001, 0.1, size=(N // 128, K)).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 16, size=(N // 128, K)).astype(np.float16).view(np.uint16)
    return q, s, z


def pin_ng_transpose_duality(impl):
    """Groups along N of W are groups along K of W transposed: the matrix
    that version 3 dequantizes from (q, s, z) is the transpose of what the
    groups-along-K product dequantizes from (q^T, s^T, z^T), and for any u, x
    u . (W x) = (W^T u) . x.  Shapes are not square, so a transposed lookup
    cannot pass."""
    for (N, K, seed) in ((384, 256, 31), (256, 640, 32)):
        q, s, z = _ng_problem(seed, N, K, exact=True)
        W3 = impl.dequantize_columns(q, s, z, np.arange(K), along="n")
        W1 = impl.dequantize_columns(np.ascontiguousarray(q.T), np.ascontiguousarray(s.T),
                                     np.ascontiguousarray(z.T), np.arange(N))
        assert W3.shape == (N, K) and np.array_equal(W3, W1.T)
        rng = np.random.default_rng(seed + 100)
        # small integers: every sum below is exact in float64
        x = rng.integers(-3, 4, size=K).astype(np.float16)
        u = rng.integers(-3, 4, size=N).astype(np.float16)
        y3, _ = impl.gemv_dense(q, s, z, x, along="n")
        y1, _ = impl.gemv_dense(np.ascontiguousarray(q.T), np.ascontiguousarray(s.T),
                                np.ascontiguousarray(z.T), u)
        lhs = float(np.dot(u.astype(np.float64), y3[0]))
        rhs = float(np.dot(y1[0], x.astype(np.float64)))
        assert lhs == rhs, (N, K, lhs, rhs)


def pin_ng_exact_rational(impl):
    """Brute force with exact rationals on a tiny problem (struct-decoded
    fp16, pure-Python loops)."""
    for seed in range(2):
        N, K, M = 256, 256, 2
        q, s, z = _ng_problem(40 + seed, N, K, exact=True)
        _, _, _, xb, ts = _exact_problem(60 + seed, N=6, K=K, M=M)
        y, B, U = impl.gemv_masked(q, s, z, bits_to_f16(xb), ts, along="n")
        act = [[abs(f16_value(xb[m, k])) >= f32_round(ts[m]) for k in range(K)] for m in range(M)]
        assert list(U) == [k for k in range(K) if any(act[m][k] for m in range(M))]
        for n in range(0, N, 37):
            b = n // 128
            for m in range(M):
                acc, accB = Fraction(0), Fraction(0)
                for k in range(K):
                    if act[m][k]:
                        w = Fraction(f16_value(s[b, k])) * (int(q[n, k]) - Fraction(f16_value(z[b, k])))
                        xv = Fraction(f16_value(xb[m, k]))
                        acc += w * xv
                        accB += abs(w) * abs(xv)
                assert y[m, n] == float(acc) and B[m, n] == float(accB), (seed, m, n)


def pin_ng_constant_metadata(impl):
    """One scale and one zero-point for the whole matrix: groups along N and
    along K describe the same weights, and the two products agree bit for bit
    (same columns, same order)."""
    rng = np.random.default_rng(33)
    N, K = 256, 384
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s0 = np.float16(0.0372).view(np.uint16)
    z0 = np.float16(6.0).view(np.uint16)
    x = rng.standard_normal((2, K)).astype(np.float16)
    y1, B1, U1 = impl.gemv_masked(q, np.full((N, K // 128), s0, np.uint16),
                                  np.full((N, K // 128), z0, np.uint16), x, [0.4, 1.1])
    y3, B3, U3 = impl.gemv_masked(q, np.full((N // 128, K), s0, np.uint16),
                                  np.full((N // 128, K), z0, np.uint16), x, [0.4, 1.1], along="n")
    assert np.array_equal(U1, U3) and np.array_equal(y1, y3) and np.array_equal(B1, B3)


def pin_layout_ng_closed_form(impl):
    """Version 3: the weight bytes of version 1; per 256 outputs and column,
    8 bytes: s, z of the even group, then s, z of the odd one."""
    for (N, K, Tn) in ((256, 128, 256), (512, 384, 512), (1024, 256, 1024)):
        n = np.arange(N)[:, None]
        k = np.arange(K)[None, :]
        q = ((n + 3 * k) % 16).astype(np.uint8)
        b = np.arange(N // 128)[:, None]
        s = ((0x3000 + 7 * b + 13 * k) & 0x7BFF).astype(np.uint16)
        z = ((b + 5 * k) % 16).astype(np.float16).view(np.uint16)
        b3 = np.asarray(impl.pack_spec(q, s, z, Tn, 3))
        b1 = np.asarray(impl.pack_spec(q, np.zeros((N, K // 128), np.uint16),
                                       np.zeros((N, K // 128), np.uint16), Tn))
        h = impl.read_header(b3)
        m_off = 256 + ((N * K // 2 + 255) // 256) * 256
        assert h["version"] == 3 and h["m_off"] == m_off and h["m_bytes"] == (N // 128) * K * 4
        assert h["total_bytes"] == m_off + ((N // 128) * K * 4 + 255) // 256 * 256 == len(b3)
        assert np.array_equal(b3[256:m_off], b1[256:m_off])
        for hh in range(N // 256):
            for kk in (0, 1, K // 2, K - 1):
                base = m_off + (hh * K + kk) * 8
                for e in (0, 1):
                    bb = 2 * hh + e
                    sb = int(b3[base + 4 * e]) | int(b3[base + 4 * e + 1]) << 8
                    zb = int(b3[base + 4 * e + 2]) | int(b3[base + 4 * e + 3]) << 8
                    assert sb == ((0x3000 + 7 * bb + 13 * kk) & 0x7BFF), (N, K, hh, kk, e)
                    assert f16_value(zb) == (bb + 5 * kk) % 16
    try:
        impl.pack_spec(q[:128], s[:1], z[:1], 128, 3)
    except ValueError:
        return
    raise AssertionError("groups along N were packed with tiles narrower than 256 outputs")


def pin_layout_ng_roundtrip(impl):
    rng = np.random.default_rng(34)
    for Tn in (256, 512, 1024):
        N, K = 1024, 384
        q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        s = rng.integers(0, 0x7C00, size=(N // 128, K)).astype(np.uint16)
        z = rng.integers(0, 16, size=(N // 128, K)).astype(np.float16).view(np.uint16)
        q2, s2, z2, h = impl.unpack_spec(impl.pack_spec(q, s, z, Tn, 3))
        assert h["version"] == 3
        assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(z, z2)


ALL_PINS = [pin_select_bruteforce, pin_select_golden, pin_gemv_exact_rational,
            pin_gemv_q_equals_z, pin_gemv_one_hot, pin_gemv_constant_group,
            pin_gemv_scale_equivariance, pin_gemv_matches_matrix_product,
            pin_batched_rows, pin_dequantize, pin_layout_closed_form,
            pin_layout_roundtrip, pin_layout_golden, pin_layout_z4_closed_form,
            pin_layout_z4_roundtrip, pin_ng_transpose_duality, pin_ng_exact_rational,
            pin_ng_constant_metadata, pin_layout_ng_closed_form, pin_layout_ng_roundtrip]

"""The C ABI without a GPU: the library loads, exports every declared symbol,
the host packer matches the layout specification byte for byte, and every
argument check fires before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
from activation_sparse_bit_amd import sgemv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "sgemv.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sgemv_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    L = sgemv.lib()
    names = declared_functions()
    assert set(names) == set(sgemv.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("N,K,tile", [(512, 128, 512), (1024, 384, 512), (512, 256, 64),
                                      (2048, 256, 1024), (256, 512, 256), (4096, 1024, 512)])
def test_packer_matches_spec(N, K, tile):
    q, s, z = synth.random_int4_problem(N * 7 + K, N, K)
    d, blob = sgemv.sgemv_pack_layout(q, s, z, tile)
    ref = oracle.pack_spec(q, s, z, tile)
    assert blob.shape == ref.shape and np.array_equal(blob, ref)
    h = oracle.header_fields(N, K, tile)
    for k, v in h.items():
        assert getattr(d, k) == v, k
    d2 = sgemv.sgemv_desc_from_header(blob)
    assert d2.as_dict() == d.as_dict()


@pytest.mark.parametrize("N,K,tile", [(512, 128, 512), (1024, 384, 512), (512, 256, 64),
                                      (2048, 256, 1024), (4096, 1024, 512)])
def test_packer_z4_matches_spec(N, K, tile):
    """Layout version 2 (4-bit zero-points) byte for byte against the spec,
    and its weight region equal to version 1's."""
    q, s, z = synth.random_int4_problem(N * 5 + K, N, K)
    d, blob = sgemv.sgemv_pack_layout_z4(q, s, z, tile)
    ref = oracle.pack_spec(q, s, z, tile, 2)
    assert blob.shape == ref.shape and np.array_equal(blob, ref)
    for k, v in oracle.header_fields(N, K, tile, 2).items():
        assert getattr(d, k) == v, k
    assert d.version == sgemv.SGEMV_LAYOUT_Z4
    d1, blob1 = sgemv.sgemv_pack_layout(q, s, z, tile)
    assert d1.version == sgemv.SGEMV_LAYOUT_PAIRS
    assert np.array_equal(blob[d.w_off:d.m_off], blob1[d1.w_off:d1.m_off])
    d2 = sgemv.sgemv_desc_from_header(blob)
    assert d2.as_dict() == d.as_dict()
    # a negative zero zero-point is the integer 0
    z0 = z.copy(); z0[0, 0] = 0x8000
    _, b0 = sgemv.sgemv_pack_layout_z4(q, s, z0, tile)
    assert b0[d.m_off + 2 * tile] & 0x0F == 0


@pytest.mark.parametrize("N,K,tile", [(512, 128, 512), (1024, 384, 512), (256, 256, 256),
                                      (2048, 256, 1024), (4096, 1024, 512)])
def test_packer_ng_matches_spec(N, K, tile):
    """Layout version 3 (groups along N) byte for byte against the spec, its
    weight region equal to version 1's, and tiles below 256 outputs refused."""
    q, s, z = synth.random_int4_problem_ng(N * 3 + K, N, K)
    d, blob = sgemv.sgemv_pack_layout_ng(q, s, z, tile)
    ref = oracle.pack_spec(q, s, z, tile, 3)
    assert blob.shape == ref.shape and np.array_equal(blob, ref)
    for k, v in oracle.header_fields(N, K, tile, 3).items():
        assert getattr(d, k) == v, k
    assert d.version == sgemv.SGEMV_LAYOUT_NG
    q1, s1, z1 = synth.random_int4_problem(1, N, K)
    d1, blob1 = sgemv.sgemv_pack_layout(q, s1, z1, tile)
    assert np.array_equal(blob[d.w_off:d.m_off], blob1[d1.w_off:d1.m_off])
    assert sgemv.sgemv_desc_from_header(blob).as_dict() == d.as_dict()
    with pytest.raises(sgemv.SgemvError, match="size"):
        sgemv.sgemv_pack_layout_ng(q, s, z, 128)
    bad = z.copy(); bad[0, 5] = np.float16(2.5).view(np.uint16)
    with pytest.raises(sgemv.SgemvError):
        sgemv.sgemv_pack_layout_ng(q, s, bad, tile)


@pytest.mark.parametrize("version", [1, 2, 3])
@pytest.mark.parametrize("rows,tile", [((512, 1024, 512), 512), ((1024,), 512), ((256, 64, 128), 64)])
def test_packer_parts_matches_spec(rows, tile, version):
    """Projections packed as parts: byte for byte the layout specification
    of the row-concatenated matrix."""
    K = 384
    if version == 3 and tile < 256:
        pytest.skip("groups along N need tiles of at least 256 outputs")
    gen = synth.random_int4_problem_ng if version == 3 else synth.random_int4_problem
    parts = [gen(31 * i + n, n, K) for i, n in enumerate(rows)]
    d, blob = sgemv.sgemv_pack_layout_parts(parts, tile_n=tile, version=version)
    q = np.concatenate([p[0] for p in parts])
    s = np.concatenate([p[1] for p in parts])
    z = np.concatenate([p[2] for p in parts])
    ref = oracle.pack_spec(q, s, z, tile, version)
    assert blob.shape == ref.shape and np.array_equal(blob, ref)
    assert d.N == sum(rows) and d.version == version


def test_packer_parts_validation():
    L = sgemv.lib()
    E = sgemv
    K = 256
    q, s, z = synth.random_int4_problem(1, 512, K)
    qa = (ctypes.c_void_p * 1)(q.ctypes.data)
    sa = (ctypes.c_void_p * 1)(s.ctypes.data)
    za = (ctypes.c_void_p * 1)(z.ctypes.data)
    d = sgemv.Desc()
    n_ok = np.array([512], dtype=np.int32)
    n_bad = np.array([384], dtype=np.int32)       # not whole 512-row tiles
    f = L.sgemv_pack_layout_parts
    assert f(0, qa, sa, za, n_ok.ctypes.data, K, 128, 512, 1, None, 0, ctypes.byref(d)) == E.SGEMV_EINVAL
    assert f(1, qa, sa, za, None, K, 128, 512, 1, None, 0, ctypes.byref(d)) == E.SGEMV_EINVAL
    assert f(1, qa, sa, za, n_ok.ctypes.data, K, 128, 512, 4, None, 0, ctypes.byref(d)) == E.SGEMV_EINVAL
    assert f(1, qa, sa, za, n_bad.ctypes.data, K, 128, 512, 1, None, 0, ctypes.byref(d)) == E.SGEMV_ESIZE
    assert f(1, qa, sa, za, n_ok.ctypes.data, K, 128, 512, 1, None, 0, ctypes.byref(d)) == E.SGEMV_OK
    blob = np.empty(d.total_bytes, dtype=np.uint8)
    assert f(1, qa, sa, za, n_ok.ctypes.data, K, 128, 512, 1, blob.ctypes.data, blob.nbytes - 1,
             ctypes.byref(d)) == E.SGEMV_ESIZE
    assert f(1, None, sa, za, n_ok.ctypes.data, K, 128, 512, 1, blob.ctypes.data, blob.nbytes,
             ctypes.byref(d)) == E.SGEMV_EINVAL
    q2 = q.copy(); q2[3, 7] = 16
    qb = (ctypes.c_void_p * 1)(q2.ctypes.data)
    assert f(1, qb, sa, za, n_ok.ctypes.data, K, 128, 512, 1, blob.ctypes.data, blob.nbytes,
             ctypes.byref(d)) == E.SGEMV_EINVAL


def test_packer_quantized_weights():
    q, s, z = synth.quantized_weights(3, 1024, 2048, 0.02)
    d, blob = sgemv.sgemv_pack_layout(q, s, z)
    assert np.array_equal(blob, oracle.pack_spec(q, s, z, 512))


def _pack_raw(q, s, z, N, K, group=128, tile=512, cap=None):
    L = sgemv.lib()
    d = sgemv.Desc()
    if cap is None:
        cap = oracle.header_fields(N, K, tile)["total_bytes"] if K % 128 == 0 and N % tile == 0 else 0
    out = np.zeros(max(cap, 1), dtype=np.uint8)
    return L.sgemv_pack_layout(q.ctypes.data if q is not None else None,
                               s.ctypes.data if s is not None else None,
                               z.ctypes.data if z is not None else None,
                               N, K, group, tile, out.ctypes.data, cap, ctypes.byref(d))


def test_packer_errors():
    N, K = 512, 256
    q, s, z = synth.random_int4_problem(1, N, K)
    assert _pack_raw(q, s, z, N, K) == sgemv.SGEMV_OK
    assert _pack_raw(None, s, z, N, K) == sgemv.SGEMV_EINVAL
    assert _pack_raw(q, s, z, N, K, group=64) == sgemv.SGEMV_EINVAL
    assert _pack_raw(q, s, z, N, 200) == sgemv.SGEMV_ESIZE
    assert _pack_raw(q, s, z, N, K, tile=384) == sgemv.SGEMV_ESIZE
    assert _pack_raw(q, s, z, N, K, tile=2048) == sgemv.SGEMV_ESIZE
    assert _pack_raw(q, s, z, 300, K, tile=64) == sgemv.SGEMV_ESIZE
    assert _pack_raw(q, s, z, N, K, cap=1000) == sgemv.SGEMV_ESIZE
    bad = q.copy(); bad[5, 7] = 16
    assert _pack_raw(bad, s, z, N, K) == sgemv.SGEMV_EINVAL
    badz = z.copy(); badz[1, 1] = np.float16(2.5).view(np.uint16)
    assert _pack_raw(q, s, badz, N, K) == sgemv.SGEMV_EINVAL
    badz[1, 1] = np.float16(16.0).view(np.uint16)
    assert _pack_raw(q, s, badz, N, K) == sgemv.SGEMV_EINVAL
    badz[1, 1] = np.float16(-1.0).view(np.uint16)
    assert _pack_raw(q, s, badz, N, K) == sgemv.SGEMV_EINVAL
    bads = s.copy(); bads[0, 0] = 0x7C00
    assert _pack_raw(q, bads, z, N, K) == sgemv.SGEMV_EINVAL
    # every integer zero-point 0..15, including -0, is accepted
    okz = np.tile(np.arange(16, dtype=np.float16).view(np.uint16), (N * (K // 128)) // 16 + 1)[:N * (K // 128)].reshape(N, K // 128).copy()
    okz[0, 0] = 0x8000
    assert _pack_raw(q, s, okz, N, K) == sgemv.SGEMV_OK


def test_desc_from_header_rejects():
    q, s, z = synth.random_int4_problem(2, 512, 128)
    d, blob = sgemv.sgemv_pack_layout(q, s, z)
    for off, val in ((0, 0x58), (4, 2), (24, 0x10)):
        b = blob.copy(); b[off] = val
        with pytest.raises(sgemv.SgemvError):
            sgemv.sgemv_desc_from_header(b)


def _desc(N=4096, K=14336, tile=512):
    d = sgemv.Desc()
    L = sgemv.lib()
    assert L.sgemv_pack_layout(None, None, None, N, K, 128, tile, None, 0, ctypes.byref(d)) == 0
    return d


FAKE = 1 << 20  # a well-aligned address that is never dereferenced: every call below fails validation


def test_gather_validation():
    L = sgemv.lib()
    t = np.array([0.5] * 16, dtype=np.float32)
    tp = t.ctypes.data
    E = sgemv
    assert L.sgemv_gather_indices(None, 1, 2048, 2048, tp, FAKE, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_gather_indices(FAKE, 1, 2048, 2048, None, FAKE, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_gather_indices(FAKE, 0, 2048, 2048, tp, FAKE, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_gather_indices(FAKE, 17, 2048, 2048, tp, FAKE, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_gather_indices(FAKE, 1, 2000, 2048, tp, FAKE, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_gather_indices(FAKE, 1, 131072, 131072, tp, FAKE, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_gather_indices(FAKE, 2, 2048, 2000, tp, FAKE, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_gather_indices(FAKE, 2, 2048, 2052, tp, FAKE, FAKE, None) == E.SGEMV_EALIGN
    assert L.sgemv_gather_indices(FAKE + 2, 1, 2048, 2048, tp, FAKE, FAKE, None) == E.SGEMV_EALIGN
    for bad in (np.nan, -0.25, np.inf):
        tb = np.array([bad], dtype=np.float32)
        assert L.sgemv_gather_indices(FAKE, 1, 2048, 2048, tb.ctypes.data, FAKE, FAKE, None) == E.SGEMV_EINVAL


def test_run_validation():
    L = sgemv.lib()
    E = sgemv
    d = _desc()
    pd = ctypes.byref(d)
    assert L.sgemv_run(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, None, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE, None, FAKE, 0, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, None) == E.SGEMV_EINVAL
    assert L.sgemv_run(pd, FAKE + 16, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EALIGN
    assert L.sgemv_run(pd, FAKE, FAKE + 2, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EALIGN
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 0, FAKE, None) == E.SGEMV_EALIGN
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE + 2, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EALIGN   # idx: 4 bytes
    assert L.sgemv_run(pd, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE + 64, None) == E.SGEMV_EALIGN
    # a description the kernels do not run, and inconsistent ones
    d2 = _desc(N=4096, K=14336, tile=256)
    assert L.sgemv_run(ctypes.byref(d2), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EUNSUPPORTED
    d3 = _desc(); d3.m_off += 256
    assert L.sgemv_run(ctypes.byref(d3), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EINVAL
    d4 = _desc(); d4.group = 64
    assert L.sgemv_run(ctypes.byref(d4), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E.SGEMV_EINVAL


def test_run_batched_validation():
    L = sgemv.lib()
    E = sgemv
    d = _desc()
    pd = ctypes.byref(d)
    t = np.array([0.5] * 16, dtype=np.float32)
    tp = t.ctypes.data
    K, N = d.K, d.N
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 0, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 17, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 4, K - 8, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 4, K, tp, FAKE, FAKE, FAKE, N - 8, 0, FAKE, None) == E.SGEMV_ESIZE
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 4, K + 4, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EALIGN
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 4, K, tp, FAKE, FAKE, FAKE, N + 4, 0, FAKE, None) == E.SGEMV_EALIGN
    tb = np.array([0.5, np.nan, 0.5, 0.5], dtype=np.float32)
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 4, K, tb.ctypes.data, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL
    tb = np.array([0.5, 0.5, -1.0, 0.5], dtype=np.float32)
    assert L.sgemv_run_batched(pd, FAKE, FAKE, 4, K, tb.ctypes.data, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL


def test_run_fused_validation():
    L = sgemv.lib()
    E = sgemv
    d = _desc()
    pd = ctypes.byref(d)
    t = np.array([0.5, 0.5, 0.5], dtype=np.float32)
    tp = t.ctypes.data
    K, N = d.K, d.N
    f = L.sgemv_run_fused
    assert f(None, FAKE, FAKE, 1, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL
    assert f(pd, None, FAKE, 1, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL
    assert f(pd, FAKE, None, 1, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL
    assert f(pd, FAKE, FAKE, 1, K, None, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL
    assert f(pd, FAKE, FAKE, 1, K, tp, FAKE, FAKE, None, N, 0, FAKE, None) == E.SGEMV_EINVAL
    assert f(pd, FAKE, FAKE, 1, K, tp, FAKE, None, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL  # idx without count
    assert f(pd, FAKE, FAKE, 1, K, tp, None, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL  # count without idx
    assert f(pd, FAKE, FAKE, 1, K, tp, FAKE, FAKE, FAKE, N, 2, FAKE, None) == E.SGEMV_EINVAL
    assert f(pd, FAKE, FAKE, 1, K, tp, None, None, FAKE, N, 0, None, None) == E.SGEMV_EINVAL  # no workspace
    assert f(pd, FAKE, FAKE, 0, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_ESIZE
    assert f(pd, FAKE, FAKE, 17, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_ESIZE
    assert f(pd, FAKE, FAKE, 2, K - 8, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_ESIZE
    assert f(pd, FAKE, FAKE, 2, K + 4, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EALIGN
    assert f(pd, FAKE, FAKE, 1, K, tp, FAKE, FAKE, FAKE + 4, N, 0, FAKE, None) == E.SGEMV_EALIGN
    assert f(pd, FAKE, FAKE, 1, K, tp, FAKE + 2, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EALIGN
    assert f(pd, FAKE, FAKE, 1, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE + 64, None) == E.SGEMV_EALIGN
    tb = np.array([np.inf], dtype=np.float32)
    assert f(pd, FAKE, FAKE, 1, K, tb.ctypes.data, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EINVAL
    d2 = _desc(N=4096, K=14336, tile=256)
    assert f(ctypes.byref(d2), FAKE, FAKE, 1, K, tp, FAKE, FAKE, FAKE, N, 0, FAKE, None) == E.SGEMV_EUNSUPPORTED


def test_workspace_bytes():
    d = _desc()
    w1 = sgemv.sgemv_workspace_bytes(d, 1)
    w16 = sgemv.sgemv_workspace_bytes(d, 16)
    assert w1 > 0 and w16 >= w1
    for m in range(1, 17):
        assert sgemv.sgemv_workspace_bytes(d, m) >= sgemv.sgemv_workspace_bytes(d, max(1, m - 1))
    assert sgemv.sgemv_workspace_bytes(d, 0) == 0
    assert sgemv.sgemv_workspace_bytes(d, 17) == 0
    bad = _desc(); bad.K = 100
    assert sgemv.sgemv_workspace_bytes(bad, 1) == 0


def test_strerror():
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(sgemv.strerror(st), str) and sgemv.strerror(st)


def test_fused_projections_rejects_bad_parts():
    """Packing checks of the projection helper fire before any device work."""
    q, s, z = synth.random_int4_problem(3, 512, 256)
    q2, s2, z2 = synth.random_int4_problem(4, 256, 256)
    with pytest.raises(ValueError):      # N not a multiple of the tile
        sgemv.FusedProjections([("a", q, s, z), ("b", q2, s2, z2)], device="cpu")
    q3, s3, z3 = synth.random_int4_problem(5, 512, 384)
    with pytest.raises(ValueError):      # different K
        sgemv.FusedProjections([("a", q, s, z), ("b", q3, s3, z3)], device="cpu")
    with pytest.raises(ValueError):      # duplicate names
        sgemv.FusedProjections([("a", q, s, z), ("a", q, s, z)], device="cpu")


def test_partials_beyond_32bit_offsets_rejected():
    """A call whose partial sums would not fit 32-bit offsets (largest N, K
    and M) is refused before any launch; a smaller M on the same matrix
    passes validation up to the launch (not made here: no GPU)."""
    L = sgemv.lib()
    E = sgemv
    d = sgemv.Desc()
    N, K = sgemv.SGEMV_MAX_N, sgemv.SGEMV_MAX_K
    assert L.sgemv_pack_layout(None, None, None, N, K, 128, 512, None, 0, ctypes.byref(d)) == E.SGEMV_OK
    assert sgemv.sgemv_workspace_bytes(d, 16) > (1 << 32)
    t = np.zeros(16, dtype=np.float32)
    st = L.sgemv_run_fused(ctypes.byref(d), FAKE, FAKE, 16, K, t.ctypes.data, None, None, FAKE, N, 0,
                           FAKE, None)
    assert st == E.SGEMV_ESIZE


def test_plain_c_program_against_the_abi(tmp_path):
    """The header and library from plain C (gcc, no Python, no GPU): size
    queries, packing of both layout versions, the header round trip,
    workspace sizes and argument checks of the device calls; the blobs it
    writes equal the oracle's layout specification byte for byte."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    libdir = os.path.dirname(sgemv.LIB_PATH)
    exe = tmp_path / "c_abi_host"
    src = os.path.join(os.path.dirname(__file__), "c_abi_host.c")
    inc = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
    subprocess.run([gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-I", inc, src, "-L", libdir, "-lsgemv",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr
    N, K = 1024, 384
    q = np.fromfile(tmp_path / "q.bin", dtype=np.uint8).reshape(N, K)
    s = np.fromfile(tmp_path / "s.bin", dtype=np.uint16).reshape(N, K // 128)
    z = np.fromfile(tmp_path / "z.bin", dtype=np.uint16).reshape(N, K // 128)
    for v in (1, 2):
        blob = np.fromfile(tmp_path / f"blob{v}.bin", dtype=np.uint8)
        assert np.array_equal(blob, np.asarray(oracle.pack_spec(q, s, z, 512, v)))

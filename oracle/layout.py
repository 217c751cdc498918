"""Byte formula of the packed int4 weight layout (the specification).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Enabling Dynamic Sparsity in Quantized LLM Inference" (Abstract) calls for
a quantization layout that is consistent with activation sparsity and
improves GPU memory locality, but does not give the pattern.  This layout is
our own reading of that requirement: the output dimension is cut into tiles
of ``tile_n`` rows, and for every tile and every input index k the
``tile_n`` 4-bit codes of that column are one contiguous run of tile_n/2
bytes, so a single active input index costs exactly one contiguous read per
tile and an inactive one costs nothing.  Scales and zero-points live in a
separate region, one contiguous run of tile_n (scale, zero) pairs per tile
and group.

Blob = header (256 bytes) | weight region | metadata region, little-endian:

  header  0: b"SGV1"           4: u32 version = 1
          8: i32 N            12: i32 K        16: i32 group = 128
         20: i32 tile_n       24: u64 w_off    32: u64 w_bytes
         40: u64 m_off        48: u64 m_bytes  56: u64 total_bytes
         64..255: zero
  w_off = 256, w_bytes = N*K/2,   m_off = w_off + roundup(w_bytes, 256),
  m_bytes = (K/128)*N*4,          total = m_off + roundup(m_bytes, 256)

  weight byte  w_off + (t*K + k)*(tile_n/2) + j
               = q[t*tile_n + 2j][k] | q[t*tile_n + 2j + 1][k] << 4
  metadata     m_off + ((t*(K/128) + g)*tile_n + i)*4 : fp16 bits of
               s[t*tile_n + i][g], then fp16 bits of z[t*tile_n + i][g]

for tiles t < N/tile_n, columns k < K, bytes j < tile_n/2, groups g < K/128
and rows i < tile_n.  Padding bytes are zero.

Version 2 (compact metadata) differs only in the metadata region.  The
zero-points of this format are integers 0..15, so each one needs 4 bits: per
(tile, group) the run holds the tile_n fp16 scales, then tile_n/2 bytes of
zero-points, two per byte, even row in the low nibble:

  m_bytes = (K/128)*N*5/2
  scale        m_off + (t*(K/128) + g)*(5*tile_n/2) + 2i : fp16 bits of
               s[t*tile_n + i][g]
  zero-points  m_off + (t*(K/128) + g)*(5*tile_n/2) + 2*tile_n + j
               = z[t*tile_n + 2j][g] | z[t*tile_n + 2j + 1][g] << 4

It stores the same numbers in 2.5 instead of 4 bytes per row and group, so
the metadata read per touched group shrinks by 37.5 %; the page's call for a
layout that serves sparse reads applies to this region as much as to the
weights.

Version 3 (groups along N) stores a different quantization: one scale and
one zero-point per input column k and group of 128 consecutive outputs, so
s_bits and z_bits are [N/128][K].  The weight region is the same as in
version 1; the metadata region holds, per 256 outputs (groups b = 2h and
2h + 1) and column k, 8 contiguous bytes: s, z of group 2h, then s, z of
group 2h + 1.  A column's metadata is then read only with the column, so
metadata bytes fall with the sparsity.  tile_n must be at least 256:

  m_bytes = (N/128)*K*4
  metadata     m_off + ((h*K + k)*2 + e)*4 : fp16 bits of s[2h + e][k], then
               fp16 bits of z[2h + e][k]    (h < N/256, e in {0, 1})
"""
from __future__ import annotations

import struct

import numpy as np

GROUP = 128
HEADER_BYTES = 256
MAGIC = b"SGV1"
VERSION = 1
VERSION_Z4 = 2
VERSION_NG = 3


def _roundup(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def header_fields(N: int, K: int, tile_n: int, version: int = VERSION) -> dict:
    w_off = HEADER_BYTES
    w_bytes = N * K // 2
    m_off = w_off + _roundup(w_bytes, 256)
    m_bytes = (K // GROUP) * N * 5 // 2 if version == VERSION_Z4 else (K // GROUP) * N * 4
    total = m_off + _roundup(m_bytes, 256)
    return dict(N=N, K=K, group=GROUP, tile_n=tile_n, w_off=w_off,
                w_bytes=w_bytes, m_off=m_off, m_bytes=m_bytes, total_bytes=total)


def _check(q, s_bits, z_bits, tile_n, version=VERSION):
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if K % GROUP or K <= 0 or N <= 0:
        raise ValueError("K must be a positive multiple of 128")
    if tile_n < 64 or tile_n > 1024 or tile_n & (tile_n - 1) or N % tile_n:
        raise ValueError("tile_n must be a power of two in [64, 1024] dividing N")
    if version == VERSION_NG and tile_n < 256:
        raise ValueError("groups along N need tile_n >= 256")
    if q.max(initial=0) > 15:
        raise ValueError("codes must be 4-bit")
    s_bits = np.asarray(s_bits, dtype=np.uint16)
    z_bits = np.asarray(z_bits, dtype=np.uint16)
    shape = (N // GROUP, K) if version == VERSION_NG else (N, K // GROUP)
    if s_bits.shape != shape or z_bits.shape != shape:
        raise ValueError("scale/zero shape must be [N/128][K]" if version == VERSION_NG
                         else "scale/zero shape must be [N][K/128]")
    return q, s_bits, z_bits, N, K


def zero_codes(z_bits) -> np.ndarray:
    """Integer values 0..15 of fp16 zero-point bit patterns (raises on any
    other value)."""
    zf = np.asarray(z_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if not np.all(np.isfinite(zf)) or np.any(zf != np.rint(zf)) or np.any(zf < 0) or np.any(zf > 15):
        raise ValueError("zero-points must be integers 0..15")
    return np.abs(zf).astype(np.uint8)


def pack_spec(q, s_bits, z_bits, tile_n: int, version: int = VERSION) -> np.ndarray:
    """Return the blob (uint8 array) for codes ``q`` [N][K] and fp16 bit
    patterns ``s_bits``, ``z_bits`` [N][K/128]; version 1 (scale/zero pairs)
    or 2 (scales, then 4-bit zero-points); version 3 takes them as
    [N/128][K] (groups along N)."""
    if version not in (VERSION, VERSION_Z4, VERSION_NG):
        raise ValueError("unknown layout version")
    q, s_bits, z_bits, N, K = _check(q, s_bits, z_bits, tile_n, version)
    h = header_fields(N, K, tile_n, version)
    blob = np.zeros(h["total_bytes"], dtype=np.uint8)
    head = (MAGIC + struct.pack("<I", version)
            + struct.pack("<iiii", N, K, GROUP, tile_n)
            + struct.pack("<QQQQQ", h["w_off"], h["w_bytes"], h["m_off"],
                          h["m_bytes"], h["total_bytes"]))
    blob[:len(head)] = np.frombuffer(head, dtype=np.uint8)

    T = N // tile_n
    # q[t*tile_n + i][k] viewed as [t][k][i]
    qt = q.reshape(T, tile_n, K).transpose(0, 2, 1)
    byte = qt[:, :, 0::2] | (qt[:, :, 1::2] << 4)          # [t][k][j]
    blob[h["w_off"]:h["w_off"] + h["w_bytes"]] = byte.reshape(-1)

    Gk = K // GROUP
    if version == VERSION_NG:
        H = N // 256
        pair = np.empty((H, K, 2, 2), dtype=np.uint16)             # [h][k][e][s|z]
        pair[..., 0] = s_bits.reshape(H, 2, K).transpose(0, 2, 1)
        pair[..., 1] = z_bits.reshape(H, 2, K).transpose(0, 2, 1)
        blob[h["m_off"]:h["m_off"] + h["m_bytes"]] = \
            pair.astype("<u2").reshape(-1).view(np.uint8)
        return blob
    if version == VERSION:
        pair = np.empty((T, Gk, tile_n, 2), dtype=np.uint16)     # [t][g][i][s|z]
        pair[..., 0] = s_bits.reshape(T, tile_n, Gk).transpose(0, 2, 1)
        pair[..., 1] = z_bits.reshape(T, tile_n, Gk).transpose(0, 2, 1)
        blob[h["m_off"]:h["m_off"] + h["m_bytes"]] = \
            pair.astype("<u2").reshape(-1).view(np.uint8)
        return blob
    zc = zero_codes(z_bits)
    run = np.empty((T, Gk, 5 * tile_n // 2), dtype=np.uint8)   # [t][g][scales | zero bytes]
    st = s_bits.reshape(T, tile_n, Gk).transpose(0, 2, 1)       # [t][g][i]
    run[:, :, :2 * tile_n] = np.ascontiguousarray(st).astype("<u2").view(np.uint8).reshape(T, Gk, 2 * tile_n)
    zt = zc.reshape(T, tile_n, Gk).transpose(0, 2, 1)           # [t][g][i]
    run[:, :, 2 * tile_n:] = zt[:, :, 0::2] | (zt[:, :, 1::2] << 4)
    blob[h["m_off"]:h["m_off"] + h["m_bytes"]] = run.reshape(-1)
    return blob


def read_header(blob) -> dict:
    b = bytes(np.asarray(blob, dtype=np.uint8)[:64])
    if b[:4] != MAGIC:
        raise ValueError("bad magic")
    version, = struct.unpack_from("<I", b, 4)
    N, K, G, tile_n = struct.unpack_from("<iiii", b, 8)
    w_off, w_bytes, m_off, m_bytes, total = struct.unpack_from("<QQQQQ", b, 24)
    return dict(version=version, N=N, K=K, group=G, tile_n=tile_n, w_off=w_off,
                w_bytes=w_bytes, m_off=m_off, m_bytes=m_bytes, total_bytes=total)


def unpack_spec(blob):
    """Inverse of ``pack_spec``: returns (q, s_bits, z_bits, header)."""
    blob = np.asarray(blob, dtype=np.uint8)
    h = read_header(blob)
    N, K, tile_n = h["N"], h["K"], h["tile_n"]
    T, Gk = N // tile_n, K // GROUP
    byte = blob[h["w_off"]:h["w_off"] + h["w_bytes"]].reshape(T, K, tile_n // 2)
    qt = np.empty((T, K, tile_n), dtype=np.uint8)
    qt[:, :, 0::2] = byte & 0x0F
    qt[:, :, 1::2] = byte >> 4
    q = qt.transpose(0, 2, 1).reshape(N, K)
    md = blob[h["m_off"]:h["m_off"] + h["m_bytes"]]
    if h["version"] == VERSION_NG:
        H = N // 256
        pair = md.view("<u2").reshape(H, K, 2, 2)
        s_bits = pair[..., 0].transpose(0, 2, 1).reshape(N // GROUP, K).astype(np.uint16)
        z_bits = pair[..., 1].transpose(0, 2, 1).reshape(N // GROUP, K).astype(np.uint16)
        return np.ascontiguousarray(q), s_bits, z_bits, h
    if h["version"] == VERSION:
        pair = md.view("<u2").reshape(T, Gk, tile_n, 2)
        s_bits = pair[..., 0].transpose(0, 2, 1).reshape(N, Gk).astype(np.uint16)
        z_bits = pair[..., 1].transpose(0, 2, 1).reshape(N, Gk).astype(np.uint16)
        return np.ascontiguousarray(q), s_bits, z_bits, h
    run = md.reshape(T, Gk, 5 * tile_n // 2)
    s_bits = np.ascontiguousarray(run[:, :, :2 * tile_n]).view("<u2").transpose(0, 2, 1).reshape(N, Gk)
    zb = run[:, :, 2 * tile_n:]
    zt = np.empty((T, Gk, tile_n), dtype=np.uint8)
    zt[:, :, 0::2] = zb & 0x0F
    zt[:, :, 1::2] = zb >> 4
    z_bits = zt.transpose(0, 2, 1).reshape(N, Gk).astype(np.float16).view(np.uint16)
    return np.ascontiguousarray(q), s_bits.astype(np.uint16), np.ascontiguousarray(z_bits), h

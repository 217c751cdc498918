"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and turns them into the arrays the sparse
GEMV consumes: fp16 activations, fp32 weights quantized to asymmetric int4
with one fp16 scale and one fp16 zero-point per group of 128 inputs, and the
magnitude thresholds that give a requested sparsity.  It holds none of the
GEMV's own arithmetic (no thresholding, no dequantization, no dot products):
both the fp64 oracle and the HIP library receive exactly the arrays built
here and nothing else.

Shapes and distributions follow the workloads described for decode-time
dynamic activation sparsity ("Enabling Dynamic Sparsity in Quantized LLM
Inference", Abstract): Llama-3-shaped projections with group-wise int4
weights, activations ~N(0,1) or silu(g)*u as produced by a gated feed-forward
block ("GLU Variants Improve Transformer", cited on the same page).  Trained
weights and real activations are not available, so Gaussian draws stand in.

Seed scheme (``numpy.random.default_rng``):
  weights of projection j : 1000 + j
  gate draw g of row m    : 2000 + m
  up draw u of row m      : 3000 + m
  plain activation input i: 4000 + i
Every draw is fp32, then rounded to fp16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GROUP = 128

SEED_W = 1000
SEED_G = 2000
SEED_U = 3000
SEED_X = 4000


# --------------------------------------------------------------------------
# raw draws
# --------------------------------------------------------------------------
def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def normal_f16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    return normal_f32(seed, shape, sigma).astype(np.float16)


def silu_times_up(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Gated feed-forward activation silu(g)*u, computed in fp32 from fp16
    draws and rounded once to fp16 (the input of a down projection)."""
    gf = g.astype(np.float32)
    uf = u.astype(np.float32)
    with np.errstate(over="ignore"):
        a = gf / (np.float32(1.0) + np.exp(-gf)) * uf
    return a.astype(np.float16)


def glu_activation(row: int, K: int) -> np.ndarray:
    return silu_times_up(normal_f16(SEED_G + row, (K,)), normal_f16(SEED_U + row, (K,)))


def plain_activation(i: int, K: int) -> np.ndarray:
    return normal_f16(SEED_X + i, (K,))


# --------------------------------------------------------------------------
# thresholds
# --------------------------------------------------------------------------
def percentile_threshold(x: np.ndarray, p: float) -> float:
    """Magnitude threshold that zeroes (about) the fraction ``p`` of ``x``.

    Sort float32(|x|) ascending and take the element at position floor(p*K);
    p == 0 gives t = 0 (every finite entry kept).  Entries equal to t are
    kept, so fp16 ties can make the realised sparsity slightly below p.  The
    value is returned as a float that is exactly representable in fp32.
    """
    x = np.asarray(x).reshape(-1)
    if p <= 0.0:
        return 0.0
    a = np.sort(np.abs(x.astype(np.float32)))
    pos = min(int(math.floor(p * a.size)), a.size - 1)
    return float(a[pos])


# --------------------------------------------------------------------------
# asymmetric int4 group quantizer (offline; produces q, s, z)
# --------------------------------------------------------------------------
def quantize_int4_g128(W: np.ndarray, group: int = GROUP, chunk_rows: int = 1024):
    """Asymmetric min-max int4 quantization per (output row, group of inputs).

    For every row n and group g of ``group`` consecutive inputs:
      lo = min(0, min w), hi = max(0, max w), s = (hi - lo)/15 (1 if 0),
      s16 = fp16(s) (round to nearest even), z = clamp(rint(-lo/s16), 0, 15),
      q = clamp(rint(w/s16) + z, 0, 15).
    The reconstruction s16*(q - z) is what every consumer uses; it is the
    GPTQ-style asymmetric format ("GPTQ", cited by "Enabling Dynamic Sparsity
    in Quantized LLM Inference").  z is an integer code stored as fp16.

    Returns q (uint8 [N][K], values 0..15), s and z (uint16 fp16 bit
    patterns, [N][K/group]).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    Gk = K // group
    q = np.empty((N, K), dtype=np.uint8)
    s_bits = np.empty((N, Gk), dtype=np.uint16)
    z_bits = np.empty((N, Gk), dtype=np.uint16)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        w = W[r0:r1].astype(np.float64).reshape(r1 - r0, Gk, group)
        lo = np.minimum(w.min(axis=2), 0.0)
        hi = np.maximum(w.max(axis=2), 0.0)
        s = (hi - lo) / 15.0
        s = np.where(s == 0.0, 1.0, s)
        s16 = s.astype(np.float16)
        s16 = np.where(s16 == 0, np.float16(2.0 ** -24), s16)  # never a zero scale
        s64 = s16.astype(np.float64)
        z = np.clip(np.rint(-lo / s64), 0, 15)
        qq = np.clip(np.rint(w / s64[:, :, None]) + z[:, :, None], 0, 15)
        q[r0:r1] = qq.reshape(r1 - r0, K).astype(np.uint8)
        s_bits[r0:r1] = s16.view(np.uint16)
        z_bits[r0:r1] = z.astype(np.float16).view(np.uint16)
    return q, s_bits, z_bits


def quantize_int4_ng128(W: np.ndarray, group: int = GROUP):
    """The same asymmetric min-max int4 quantizer with its groups along the
    outputs: one (s, z) per input column k and block of ``group`` consecutive
    outputs (the format of layout version 3).  It is the groups-along-inputs
    quantizer applied to W transposed.

    Returns q (uint8 [N][K]), s and z (uint16 fp16 bit patterns,
    [N/group][K]).
    """
    W = np.asarray(W, dtype=np.float32)
    if W.shape[0] % group:
        raise ValueError("N must be a multiple of the group size")
    qT, sT, zT = quantize_int4_g128(np.ascontiguousarray(W.T), group)
    return np.ascontiguousarray(qT.T), np.ascontiguousarray(sT.T), np.ascontiguousarray(zT.T)


def quantized_weights(j: int, N: int, K: int, sigma: float):
    """Weights of projection ``j`` ~ N(0, sigma^2), quantized to int4 g128."""
    return quantize_int4_g128(normal_f32(SEED_W + j, (N, K), sigma))


def quantized_weights_ng(j: int, N: int, K: int, sigma: float):
    """The same draw as ``quantized_weights``, quantized with groups of 128
    outputs per input column (layout version 3)."""
    return quantize_int4_ng128(normal_f32(SEED_W + j, (N, K), sigma))


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------
@dataclass
class Projection:
    name: str
    K: int
    N: int
    sigma: float
    weight_seed: int          # index j of the weight draw
    input_name: str           # which activation vector feeds it


@dataclass
class Workload:
    name: str
    projections: list
    inputs: dict = field(default_factory=dict)  # name -> (kind, index, K)
    sparsities: tuple = (0.5,)
    batch: tuple = (1,)


def workload(name: str) -> Workload:
    """The synthetic workloads, by name.

    single-2048     : K=2048 -> N=2048, W~N(0,0.02), x~N(0,1), p=0.5
    down-14336      : Llama-3-8B down projection K=14336 -> N=4096,
                      x = silu(g)*u, p in {0.5, 0.7, 0.9}
    layer-8b        : the seven projections of a Llama-3-8B decode layer at
                      p=0.5; q/k/v share one input, gate/up share one, o and
                      down have their own (four N(0,1) inputs)
    mlp-70b         : Llama-3-70B MLP, gate/up 8192 -> 28672 and down
                      28672 -> 8192, W~N(0,0.015); gate/up input N(0,1),
                      down input silu(g)*u; p in {0.5, 0.9}
    batched-14336   : M in {1,2,4,8,16} rows of silu(g_m)*u_m, each
                      thresholded at p=0.7, against one 14336 -> 4096 matrix
    """
    if name == "single-2048":
        return Workload(name, [Projection("w", 2048, 2048, 0.02, 0, "x0")],
                        {"x0": ("plain", 0, 2048)}, (0.5,), (1,))
    if name == "down-14336":
        return Workload(name, [Projection("down", 14336, 4096, 0.02, 0, "a0")],
                        {"a0": ("glu", 0, 14336)}, (0.5, 0.7, 0.9), (1,))
    if name == "layer-8b":
        P = [Projection("q", 4096, 4096, 0.02, 0, "x_attn"),
             Projection("k", 4096, 1024, 0.02, 1, "x_attn"),
             Projection("v", 4096, 1024, 0.02, 2, "x_attn"),
             Projection("o", 4096, 4096, 0.02, 3, "x_o"),
             Projection("gate", 4096, 14336, 0.02, 4, "x_mlp"),
             Projection("up", 4096, 14336, 0.02, 5, "x_mlp"),
             Projection("down", 14336, 4096, 0.02, 6, "x_down")]
        I = {"x_attn": ("plain", 0, 4096), "x_o": ("plain", 1, 4096),
             "x_mlp": ("plain", 2, 4096), "x_down": ("plain", 3, 14336)}
        return Workload(name, P, I, (0.5,), (1,))
    if name == "mlp-70b":
        P = [Projection("gate", 8192, 28672, 0.015, 0, "x_mlp"),
             Projection("up", 8192, 28672, 0.015, 1, "x_mlp"),
             Projection("down", 28672, 8192, 0.015, 2, "a_down")]
        I = {"x_mlp": ("plain", 0, 8192), "a_down": ("glu", 0, 28672)}
        return Workload(name, P, I, (0.5, 0.9), (1,))
    if name == "batched-14336":
        return Workload(name, [Projection("down", 14336, 4096, 0.02, 0, "a")],
                        {"a": ("glu-rows", 0, 14336)}, (0.7,), (1, 2, 4, 8, 16))
    raise KeyError(name)


def activation(kind: str, index: int, K: int, rows: int = 1) -> np.ndarray:
    """fp16 activations; 'glu-rows' returns [rows][K], the others [K]."""
    if kind == "plain":
        return plain_activation(index, K)
    if kind == "glu":
        return glu_activation(index, K)
    if kind == "glu-rows":
        return np.stack([glu_activation(index + m, K) for m in range(rows)])
    raise KeyError(kind)


# --------------------------------------------------------------------------
# small helpers for tests: special fp16 values by bit pattern
# --------------------------------------------------------------------------
def f16_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


def random_int4_problem(seed: int, N: int, K: int, group: int = GROUP):
    """Random q/s/z directly in the stored format (no float weights): q and
    z uniform in 0..15, s = fp16 of a positive value.  Used where a test
    wants the whole code space exercised rather than Gaussian weights."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, K // group)).astype(np.float16)
    s = (rng.uniform(0.5, 2.0, size=(N, K // group)) * 0.01).astype(np.float16)
    return q, s.view(np.uint16), z.view(np.uint16)


def random_int4_problem_ng(seed: int, N: int, K: int, group: int = GROUP):
    """As ``random_int4_problem``, with the scales and zero-points of the
    groups-along-outputs format ([N/group][K])."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N // group, K)).astype(np.float16)
    s = (rng.uniform(0.5, 2.0, size=(N // group, K)) * 0.01).astype(np.float16)
    return q, s.view(np.uint16), z.view(np.uint16)

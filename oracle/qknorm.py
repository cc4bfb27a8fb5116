"""Layerwise QK-Norm, written out in float64 (test infrastructure only).

Source: "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for
Query-Key Normalization" (arXiv 2608.09160v1), arXiv HTML page.

Layerwise QK-Norm normalizes each token's whole projected Q vector with one
RMS factor, and separately its whole projected K vector with another (the
paper's introduction contrasts this with headwise QK-Norm, one factor per
head). For one vector x of full width H (RMS-Norm, Eq. 1, read as stated in
the package docstring):

    y_j = x_j * gamma_j / sqrt( (sum_i x_i**2) / H + eps )

Phase A of the paper observes that the denominator needs only the sum of
squares, which splits over contiguous column shards: each shard contributes
its own sum, and the global sum is the sum of the shard sums. Phase B and the
final scaling multiply the shard by gamma and then by the global factor.

Each step below is one function so that a reader can check it against those
passages by eye. There is no blocking, fusion or reordering: every reduction
is a plain ``numpy.sum`` over float64 values.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits
from .fp8 import f64_to_fp8_bits, fp8_bits_to_f64


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def decode_input(a, dtype):
    """Exact float64 value of an input array.

    ``dtype == "bf16"``: ``a`` holds bf16 bit patterns (uint16).
    ``dtype == "f32"``:  ``a`` holds float32 values.
    ``dtype == "fp8"``:  ``a`` holds FP8 E4M3 (E4M3FN) bit patterns (uint8).
    """
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        return fp8_bits_to_f64(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode_gamma(a, dtype):
    """Exact float64 value of gamma: bf16 bit patterns for bf16 and FP8 rows
    (FP8 E4M3 is the activation format; the scale stays in bf16), float32
    values for float32 rows."""
    return decode_input(a, "bf16" if dtype == "fp8" else dtype)


def eps_as_passed(eps):
    """The kernel receives eps as float32; the oracle uses that exact value."""
    return float(np.float32(eps))


# --------------------------------------------------------------------------
# Phase A: per-shard partial sums of squares, then their combination
# --------------------------------------------------------------------------
def shard_sum_of_squares(x, shards):
    """partial[s, t] = sum over the columns j of shard s of x[t, j]**2.

    ``x`` is float64 [T, h]; shard s covers the contiguous columns
    [s*h/S, (s+1)*h/S). Returns float64 [S, T]. (Phase A: the local squared
    sum of a hidden-dimension shard.)
    """
    x = np.asarray(x, dtype=np.float64)
    T, h = x.shape
    if shards < 1 or h % shards:
        raise ValueError(f"width {h} is not divisible into {shards} shards")
    w = h // shards
    out = np.empty((shards, T), dtype=np.float64)
    for s in range(shards):
        out[s] = np.sum(x[:, s * w:(s + 1) * w] ** 2, axis=1)
    return out


def combine_partials(partials):
    """Global sum of squares per token: the sum of the partials over axis 0.

    (Phase A: aggregating the shard sums recovers the global squared sum.)
    """
    return np.sum(np.asarray(partials, dtype=np.float64), axis=0)


# --------------------------------------------------------------------------
# the RMS factor and the scaling (Eq. 1; Phase B and the final scaling)
# --------------------------------------------------------------------------
def rms_denominator(ss, h_full, eps):
    """sqrt(ss / H + eps): the denominator of Eq. 1 for each token."""
    return np.sqrt(np.asarray(ss, dtype=np.float64) / float(h_full) + eps)


def scale_rows(x, gamma, denom):
    """y[t, j] = x[t, j] * gamma[j] / denom[t]."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    return x * gamma[None, :] / np.asarray(denom, dtype=np.float64)[:, None]


def layerwise_rmsnorm(x, gamma, eps, shards=1):
    """RMS-Norm of every row of x over its full width, via S shard partials.

    Returns (y [T, h], partials [S, T]), both float64.
    """
    x = np.asarray(x, dtype=np.float64)
    partials = shard_sum_of_squares(x, shards)
    ss = combine_partials(partials)
    denom = rms_denominator(ss, x.shape[1], eps)
    return scale_rows(x, gamma, denom), partials


def apply_with_stats(x, gamma, planes, h_full, eps):
    """Normalize a local slice x with sums of squares supplied from outside.

    ``planes`` is [P, T]: P partial (or already combined, P = 1) sums of
    squares per token, which are added to form the global sum; ``h_full`` is
    the full vector width H that Eq. 1 divides by (not the local width).
    """
    ss = combine_partials(planes)
    denom = rms_denominator(ss, h_full, eps)
    return scale_rows(x, gamma, denom)


def headwise_rmsnorm(x, gamma, eps, head_dim, gamma_head_stride):
    """Headwise QK-Norm: every head (head_dim contiguous columns) of every row
    is its own vector for Eq. 1, with H = head_dim and its own factor.

    The paper's introduction defines the headwise granularity as one
    independent normalization factor per attention head. gamma element
    (head, j) is gamma[head * gamma_head_stride + j]: stride 0 shares one
    [head_dim] vector across heads, stride head_dim gives every column its
    own scale.
    """
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    T, h = x.shape
    if head_dim < 1 or h % head_dim:
        raise ValueError(f"width {h} is not a whole number of heads of {head_dim}")
    y = np.empty_like(x)
    for head in range(h // head_dim):
        cols = slice(head * head_dim, (head + 1) * head_dim)
        g0 = head * gamma_head_stride
        y[:, cols], _ = layerwise_rmsnorm(x[:, cols], gamma[g0:g0 + head_dim], eps, 1)
    return y


# --------------------------------------------------------------------------
# the calls of the library, on the same inputs the library receives
# --------------------------------------------------------------------------
class QKResult:
    """Oracle outputs for one call.

    ``yq``/``yk``: float64 results. ``yq_bits``/``yk_bits``: the result in the
    I/O format, rounded once from float64 (bf16 bits for bf16 I/O, E4M3 bits for
    FP8 I/O; None for float32). ``pq``/``pk``:
    float64 shard partials [S, T] (fused only, else None).
    """

    def __init__(self, yq, yk, dtype, pq=None, pk=None):
        self.yq = yq
        self.yk = yk
        self.pq = pq
        self.pk = pk
        if dtype == "bf16":
            self.yq_bits = f64_to_bf16_bits(yq)
            self.yk_bits = f64_to_bf16_bits(yk)
        elif dtype == "fp8":
            self.yq_bits = f64_to_fp8_bits(yq)
            self.yk_bits = f64_to_fp8_bits(yk)
        else:
            self.yq_bits = None
            self.yk_bits = None


def qknorm_fused(xq, xk, gamma_q, gamma_k, dtype, eps, shards):
    """Layerwise QK-Norm of Q rows and, separately, K rows.

    Each of Q [T, hq] and K [T, hk] is split into ``shards`` equal column
    shards; H is the whole local width (hq for Q, hk for K).
    """
    e = eps_as_passed(eps)
    yq, pq = layerwise_rmsnorm(decode_input(xq, dtype), decode_gamma(gamma_q, dtype), e, shards)
    yk, pk = layerwise_rmsnorm(decode_input(xk, dtype), decode_gamma(gamma_k, dtype), e, shards)
    return QKResult(yq, yk, dtype, pq, pk)


def qknorm_partial_stats(xq, xk, dtype, shards):
    """Shard partial sums of squares, float64 [S, 2, T] (index 0 = Q, 1 = K)."""
    pq = shard_sum_of_squares(decode_input(xq, dtype), shards)
    pk = shard_sum_of_squares(decode_input(xk, dtype), shards)
    return np.stack([pq, pk], axis=1)


def qknorm_apply_with_stats(xq, xk, gamma_q, gamma_k, dtype, eps, stats, hq_full, hk_full):
    """Normalize local Q/K slices with given statistics.

    ``stats`` is float32 [P, 2, T]: P planes of sums of squares (index 0 = Q,
    1 = K) that are added to form each token's global sum; they are read as
    the exact float64 values of those float32 numbers.
    """
    e = eps_as_passed(eps)
    st = np.asarray(stats, dtype=np.float32).astype(np.float64)
    yq = apply_with_stats(decode_input(xq, dtype), decode_gamma(gamma_q, dtype), st[:, 0, :], hq_full, e)
    yk = apply_with_stats(decode_input(xk, dtype), decode_gamma(gamma_k, dtype), st[:, 1, :], hk_full, e)
    return QKResult(yq, yk, dtype)


def qknorm_headwise(xq, xk, gamma_q, gamma_k, dtype, eps, head_dim, gamma_head_stride):
    """Headwise QK-Norm of Q rows and, separately, K rows (heads of head_dim)."""
    e = eps_as_passed(eps)
    yq = headwise_rmsnorm(decode_input(xq, dtype), decode_gamma(gamma_q, dtype), e, head_dim, gamma_head_stride)
    yk = headwise_rmsnorm(decode_input(xk, dtype), decode_gamma(gamma_k, dtype), e, head_dim, gamma_head_stride)
    return QKResult(yq, yk, dtype)

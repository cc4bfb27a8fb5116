"""Seeded synthetic inputs for the QK-Norm workloads.

This module only draws random numbers and lays them out; it holds none of the
normalization arithmetic. Both the HIP path (tests, bench) and the CPU oracle
(tests) consume the arrays it returns, so the two sides see the same bits.

Every draw uses ``numpy.random.Generator(PCG64(SeedSequence([cfg_id, stream])))``
in float64, then one conversion to the I/O type (float32 by numpy's cast;
bf16 by round-to-nearest-even of that float32 pattern).

Streams: 0 = x (Q and K columns), 1 = gamma_q, 2 = gamma_k, 3 = per-token
scale or outlier mask, 4.. = peer slices, 7 = V-column fill.

The workloads are the synthetic stand-ins for the paper's evaluation: the
paper serves real models on a real request set, but QK-Norm acts on each token
independently, so a request mix only changes the token count T, which the
workloads sweep. Widths follow the GQA shapes the paper's models use (heads of
128 columns).
"""

from dataclasses import dataclass, field, replace

import numpy as np

STREAM_X, STREAM_GQ, STREAM_GK, STREAM_AUX, STREAM_PEER0, STREAM_V = 0, 1, 2, 3, 4, 7


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration.

    Layout ``packed``: one row-major buffer [T, hq + hk + hv]; Q at column 0,
    K at column hq, V (never touched by the library) at column hq + hk.
    Layout ``separate``: Q [T, hq] and K [T, hk] as two contiguous arrays.
    """

    key: str
    title: str
    cfg_id: int
    T: int
    hq: int
    hk: int
    hv: int
    dtype: str                 # "bf16", "f32" or "fp8" (FP8 E4M3 rows, bf16 gamma)
    packed: bool
    shards: tuple              # shard counts S exercised by the fused call
    x_dist: str = "normal"     # normal | normal_token_scale | normal_outliers
    gamma_dist: str = "normal_1_0.1"   # normal_1_0.1 | uniform_0.5_1.5
    eps: float = 1e-6
    hq_full: int = 0           # apply_with_stats divisor (0: same as hq)
    hk_full: int = 0
    peers: int = 0             # number of peer slices drawn (rank-slice workload)
    outlier_p: float = 0.001
    outlier_mult: float = 50.0
    head_dim: int = 0          # > 0: headwise QK-Norm over heads of this width

    @property
    def ld(self):
        return self.hq + self.hk + self.hv

    def with_T(self, T):
        return replace(self, T=T)


TINY = Workload("tiny", "Tiny: fp32, separate Q/K [16,256], S=2", 1, 16, 256, 256, 0, "f32", False,
              (2,), gamma_dist="uniform_0.5_1.5")
SMALL_DENSE = Workload("small_dense", "Small dense: bf16 packed [512, 3*2048], per-token LogNormal scale", 2, 512,
              2048, 2048, 2048, "bf16", True, (1, 4), x_dist="normal_token_scale")
DECODE = tuple(
    Workload(f"decode_t{T}", f"Decode-shaped: T={T}, bf16 packed [T, 12288]", 30 + i, T, 4096, 4096,
             4096, "bf16", True, (1, 2, 4, 8))
    for i, T in enumerate((1, 8, 64, 256)))
GQA_PREFILL = Workload("gqa_prefill", "GQA prefill: T=8192, bf16 packed [8192, 7168], 0.1% outliers x50, S=1", 4,
              8192, 5120, 1024, 1024, "bf16", True, (1,), x_dist="normal_outliers")
RANK_SLICE = Workload("rank_slice", "Rank slice: T=16384, local 1280/256 of 5120/1024, bf16 packed [16384, 1792]",
              5, 16384, 1280, 256, 256, "bf16", True, (1,), hq_full=5120, hk_full=1024, peers=3)

# The GQA prefill inputs normalized headwise: 40 Q heads and 8 K heads of 128,
# one shared [128] gamma per tensor (the first 128 entries of the drawn gamma).
GQA_PREFILL_HEADWISE = replace(GQA_PREFILL, key="gqa_prefill_headwise",
                               title="GQA prefill, headwise: T=8192, 40+8 heads of 128, bf16 packed [8192, 7168]",
                               head_dim=128)

# The same shapes with FP8 E4M3 activations (bf16 gamma), the paper's second
# precision in Fig. 2(b).
GQA_PREFILL_FP8 = replace(GQA_PREFILL, key="gqa_prefill_fp8",
                          title="GQA prefill, FP8 E4M3: T=8192, fp8 packed [8192, 7168], bf16 gamma, S=1",
                          dtype="fp8")
RANK_SLICE_FP8 = replace(RANK_SLICE, key="rank_slice_fp8",
                         title="Rank slice, FP8 E4M3: T=16384, local 1280/256 of 5120/1024, fp8 packed [16384, 1792]",
                         dtype="fp8")

# Prefill row widths (hq, hk, hv) besides the GQA prefill one, in packed
# rows: grouped-query shapes from 1024/256 to 16384/2048 and one multi-head
# shape (5120/5120). The planner's launch differs across them (1 to 12 waves
# per token, 2 to 6 chunks per lane, several tokens per block at the
# narrowest).
PREFILL_WIDTHS = ((1024, 256, 256), (2048, 512, 512), (3072, 1024, 1024), (4096, 1024, 1024),
                  (5120, 1024, 1024), (6144, 1024, 1024), (8192, 1024, 1024), (12288, 1024, 1024),
                  (16384, 2048, 2048), (5120, 5120, 5120))


def prefill_width(dtype, hq, hk, hv, T=8192):
    """A packed prefill workload of the given widths and row type."""
    return Workload(f"prefill_{dtype}_{hq}_{hk}", f"prefill {dtype} packed [{T}, {hq + hk + hv}]", 6, T, hq, hk, hv,
                    dtype, True, (1,))


WORKLOADS = {w.key: w for w in (TINY, SMALL_DENSE, *DECODE, GQA_PREFILL, RANK_SLICE, GQA_PREFILL_HEADWISE,
                                GQA_PREFILL_FP8, RANK_SLICE_FP8)}


def _rng(cfg_id, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, stream])))


def to_bf16_bits(a):
    """float64 -> float32 -> bf16 bit patterns (round to nearest even). Finite data only."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def to_fp8_bits(a):
    """float64 -> float32 -> FP8 E4M3 (E4M3FN) bit patterns, nearest even, via
    torch's float8_e4m3fn cast. Data must stay within +-448."""
    import torch
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    if np.abs(f).max(initial=0.0) > 448:
        raise ValueError("FP8 E4M3 inputs must lie within +-448")
    return torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def to_io(a, dtype):
    """Convert float64 draws to the I/O representation (bf16 bits, float32 or FP8 bits)."""
    if dtype == "bf16":
        return to_bf16_bits(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "fp8":
        return to_fp8_bits(a)
    raise ValueError(dtype)


def gamma_dtype(dtype):
    """gamma is bf16 for FP8 rows, the row type otherwise."""
    return "bf16" if dtype == "fp8" else dtype


def _gamma(dist, rng, n):
    if dist == "normal_1_0.1":
        return rng.normal(1.0, 0.1, n)
    if dist == "uniform_0.5_1.5":
        return rng.uniform(0.5, 1.5, n)
    raise ValueError(dist)


@dataclass
class Inputs:
    """Arrays in the I/O representation (bf16 bit patterns as uint16, or float32).

    ``q``/``k`` are views into ``qkv`` for the packed layout. ``peer_q``/``peer_k``
    are [P, T, h] peer slices (rank-slice workload only).
    """

    workload: Workload
    q: np.ndarray
    k: np.ndarray
    gamma_q: np.ndarray
    gamma_k: np.ndarray
    qkv: np.ndarray = None
    peer_q: np.ndarray = None
    peer_k: np.ndarray = None
    meta: dict = field(default_factory=dict)


def make_inputs(w: Workload) -> Inputs:
    """Draw the inputs of workload ``w`` (deterministic in ``w.cfg_id`` and shapes)."""
    T, hq, hk = w.T, w.hq, w.hk
    x = _rng(w.cfg_id, STREAM_X).standard_normal((T, hq + hk))
    meta = {}
    if w.x_dist == "normal_token_scale":
        x *= _rng(w.cfg_id, STREAM_AUX).lognormal(0.0, 1.0, (T, 1))
    elif w.x_dist == "normal_outliers":
        mask = _rng(w.cfg_id, STREAM_AUX).random((T, hq + hk)) < w.outlier_p
        x[mask] *= w.outlier_mult
        meta["n_outliers"] = int(mask.sum())
    elif w.x_dist != "normal":
        raise ValueError(w.x_dist)
    gq = to_io(_gamma(w.gamma_dist, _rng(w.cfg_id, STREAM_GQ), hq), gamma_dtype(w.dtype))
    gk = to_io(_gamma(w.gamma_dist, _rng(w.cfg_id, STREAM_GK), hk), gamma_dtype(w.dtype))

    if w.packed:
        v = _rng(w.cfg_id, STREAM_V).standard_normal((T, w.hv))
        qkv = to_io(np.concatenate([x, v], axis=1), w.dtype)
        q, k = qkv[:, :hq], qkv[:, hq:hq + hk]
    else:
        qkv = None
        xio = to_io(x, w.dtype)
        q, k = np.ascontiguousarray(xio[:, :hq]), np.ascontiguousarray(xio[:, hq:])

    peer_q = peer_k = None
    if w.peers:
        pq, pk = [], []
        for p in range(w.peers):
            xp = to_io(_rng(w.cfg_id, STREAM_PEER0 + p).standard_normal((T, hq + hk)), w.dtype)
            pq.append(xp[:, :hq])
            pk.append(xp[:, hq:])
        peer_q, peer_k = np.stack(pq), np.stack(pk)
    return Inputs(w, q, k, gq, gk, qkv, peer_q, peer_k, meta)


def make_custom(T, hq, hk, hv=0, dtype="bf16", seed=1000, scale=1.0, gamma_dist="normal_1_0.1"):
    """Inputs for edge cases: N(0, scale^2) x, packed if hv > 0 else separate arrays."""
    w = Workload(f"custom_{seed}", "custom", seed, T, hq, hk, hv, dtype, hv > 0, (1,),
                 gamma_dist=gamma_dist)
    inp = make_inputs(w)
    if scale != 1.0:
        # rescale the draw itself (not the rounded data), then re-round
        x = _rng(seed, STREAM_X).standard_normal((T, hq + hk)) * scale
        xio = to_io(x, dtype)
        if inp.qkv is not None:
            inp.qkv[:, :hq + hk] = xio
        else:
            inp.q[...] = xio[:, :hq]
            inp.k[...] = xio[:, hq:]
    return inp

"""Shared helpers for the GPU parity tests: host<->device copies of bf16 bit
patterns, guard-banded device buffers, and the two acceptance criteria
(float32 I/O: elementwise relative error <= 1e-5 against the float64 oracle;
bf16 I/O: within one bf16 step of the oracle's once-rounded result)."""

import numpy as np
import torch

DEV = "cuda:0"
F32_REL_TOL = 1e-5
BF16_ULP_TOL = 1
GUARD = 4096  # bytes of canary before and after every device buffer


def np_to_torch(a):
    """numpy uint16 (bf16 bits), uint8 (FP8 E4M3 bits) or float32 -> CPU torch
    tensor of the I/O dtype."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a.copy()).view(torch.float8_e4m3fn)
    if a.dtype == np.float32:
        return torch.from_numpy(a.copy())
    raise TypeError(a.dtype)


def torch_to_np(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    raise TypeError(t.dtype)


class Guarded:
    """A device matrix [rows, cols] inside a larger allocation whose guard
    bands (and any columns the caller marks) hold random canary bits."""

    def __init__(self, host, seed=0, offset_elems=0):
        host = np.ascontiguousarray(host)
        self.dtype = host.dtype
        esz = host.dtype.itemsize
        ge = GUARD // esz
        self.n = host.size
        self.offset = ge + offset_elems
        rng = np.random.default_rng(seed)
        total = self.offset + self.n + ge
        canary = rng.integers(0, 1 << (8 * esz), total, dtype=np.uint64).astype(
            {1: np.uint8, 2: np.uint16, 4: np.uint32}[esz])
        if esz == 4:
            canary = canary.view(np.float32)
            # keep canaries finite so that equality checks are plain
            canary = np.where(np.isfinite(canary), canary, np.float32(1.5))
        canary[self.offset:self.offset + self.n] = host.reshape(-1)
        self.initial = canary.copy()
        self.buf = np_to_torch(canary).to(DEV)
        self.shape = host.shape

    def view(self):
        return self.buf[self.offset:self.offset + self.n].view(self.shape)

    def host(self):
        return torch_to_np(self.view())

    def guards_intact(self):
        now = torch_to_np(self.buf)
        a = now[:self.offset].view(np.uint8) if now.dtype != np.uint8 else now[:self.offset]
        b = self.initial[:self.offset].view(np.uint8)
        c = now[self.offset + self.n:].view(np.uint8)
        d = self.initial[self.offset + self.n:].view(np.uint8)
        return np.array_equal(a, b) and np.array_equal(c, d)


def bf16_order(bits):
    """Monotone integer for bf16 patterns: adjacent values differ by 1, +0 == -0."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_bf16(got_bits, want_bits, what=""):
    """|order(got) - order(want)| <= 1 everywhere; NaN exactly where the oracle has NaN.

    Returns (exact-match fraction, max step difference)."""
    got_bits = np.asarray(got_bits, np.uint16)
    want_bits = np.asarray(want_bits, np.uint16)
    assert got_bits.shape == want_bits.shape, (got_bits.shape, want_bits.shape)
    gnan = ((got_bits & 0x7F80) == 0x7F80) & ((got_bits & 0x7F) != 0)
    wnan = ((want_bits & 0x7F80) == 0x7F80) & ((want_bits & 0x7F) != 0)
    assert np.array_equal(gnan, wnan), f"{what}: NaN positions differ ({gnan.sum()} vs {wnan.sum()})"
    ok = ~wnan
    d = np.abs(bf16_order(got_bits[ok]) - bf16_order(want_bits[ok]))
    dmax = int(d.max()) if d.size else 0
    if dmax > BF16_ULP_TOL:
        idx = np.argwhere(np.abs(bf16_order(got_bits) - bf16_order(want_bits)) > BF16_ULP_TOL)[:5]
        raise AssertionError(f"{what}: {int((d > BF16_ULP_TOL).sum())} elements beyond 1 bf16 ulp, "
                             f"max {dmax}; first at {idx.tolist()}")
    exact = float((d == 0).mean()) if d.size else 1.0
    return exact, dmax


def check_f32(got, want64, what=""):
    """Elementwise |got - want| <= 1e-5 |want| (want == 0 -> got == 0); NaN where the oracle has NaN."""
    got = np.asarray(got, np.float32).astype(np.float64)
    want64 = np.asarray(want64, np.float64)
    assert got.shape == want64.shape
    assert np.array_equal(np.isnan(got), np.isnan(want64)), f"{what}: NaN positions differ"
    ok = ~np.isnan(want64)
    err = np.abs(got[ok] - want64[ok])
    bound = F32_REL_TOL * np.abs(want64[ok])
    bad = err > bound
    if bad.any():
        rel = err[bad] / np.maximum(np.abs(want64[ok][bad]), 1e-300)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond rel {F32_REL_TOL}, max rel {rel.max():.3g}")
    rel = err / np.maximum(np.abs(want64[ok]), 1e-300)
    return float(rel.max()) if rel.size else 0.0


def fig2b_errors(got64, gold64):
    """Max abs, mean abs and RMS error against the float64 gold (the paper's
    Fig. 2(b) statistics), as diagnostics."""
    d = np.abs(np.asarray(got64, np.float64) - np.asarray(gold64, np.float64))
    d = d[np.isfinite(d)]
    return float(d.max()), float(d.mean()), float(np.sqrt(np.mean(d * d)))


def fp8_order(bits):
    """Monotone integer for FP8 E4M3 patterns: adjacent values differ by 1, +0 == -0."""
    b = bits.astype(np.int64)
    mag = b & 0x7F
    return np.where(b & 0x80, -mag, mag)


def check_fp8(got_bits, want_bits, what=""):
    """|order(got) - order(want)| <= 1 everywhere; NaN (0x7F/0xFF) exactly where
    the oracle has NaN. Returns (exact-match fraction, max step difference)."""
    got_bits = np.asarray(got_bits, np.uint8)
    want_bits = np.asarray(want_bits, np.uint8)
    assert got_bits.shape == want_bits.shape
    gnan = (got_bits & 0x7F) == 0x7F
    wnan = (want_bits & 0x7F) == 0x7F
    assert np.array_equal(gnan, wnan), f"{what}: NaN positions differ ({gnan.sum()} vs {wnan.sum()})"
    ok = ~wnan
    d = np.abs(fp8_order(got_bits[ok]) - fp8_order(want_bits[ok]))
    dmax = int(d.max()) if d.size else 0
    if dmax > 1:
        raise AssertionError(f"{what}: {int((d > 1).sum())} elements beyond 1 FP8 step, max {dmax}")
    return (float((d == 0).mean()) if d.size else 1.0), dmax

"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant below is a plausible slip in writing the oracle (a dropped term,
eps in the wrong place, a wrong divisor, a shifted shard, a transposed gamma,
double rounding, ...). The test swaps one oracle function for the broken copy,
on the CPU only, runs every pin, and requires at least one to fail. This is
what shows that the pins pin the oracle rather than restate it.
"""

import numpy as np
import pytest

from oracle import bf16 as obf16
from oracle import qknorm as oq
from oracle_pins import ALL_PINS

_orig_shard = oq.shard_sum_of_squares
_orig_fp8 = oq.f64_to_fp8_bits
_orig_round = obf16.f64_to_bf16_bits


def _shards(fn):
    def f(x, shards):
        x = np.asarray(x, dtype=np.float64)
        T, h = x.shape
        if shards < 1 or h % shards:
            raise ValueError("bad shards")
        w = h // shards
        out = np.empty((shards, T))
        for s in range(shards):
            out[s] = fn(x, s, w, shards)
        return out
    return f


def _round_truncate(v):
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _round_via_f32(v):
    return _orig_round(np.asarray(v, np.float64).astype(np.float32).astype(np.float64))


def _round_ties_away(v):
    v = np.asarray(v, np.float64)
    b = _orig_round(v)
    lo = obf16.bf16_bits_to_f64(b)
    # where v sits exactly on a midpoint and was sent toward zero, step away from zero
    nxt = obf16.bf16_bits_to_f64((b.astype(np.uint32) + 1).astype(np.uint16))
    prv = obf16.bf16_bits_to_f64((b.astype(np.uint32) - 1).astype(np.uint16))
    tie_down = (np.abs(v) > np.abs(lo)) & (np.abs(v) - np.abs(lo) == np.abs(nxt) - np.abs(v))
    tie_up = (np.abs(v) < np.abs(lo)) & (np.abs(lo) - np.abs(v) == np.abs(v) - np.abs(prv))
    b = np.where(tie_down, b + 1, b).astype(np.uint16)
    del tie_up
    return b


def _fused_gamma_swapped(xq, xk, gamma_q, gamma_k, dtype, eps, shards):
    e = oq.eps_as_passed(eps)
    gq = oq.decode_input(gamma_q, dtype)
    gk = oq.decode_input(gamma_k, dtype)
    n = min(len(gq), len(gk))
    gq2, gk2 = gq.copy(), gk.copy()
    gq2[:n], gk2[:n] = gk[:n], gq[:n]
    yq, pq = oq.layerwise_rmsnorm(oq.decode_input(xq, dtype), gq2, e, shards)
    yk, pk = oq.layerwise_rmsnorm(oq.decode_input(xk, dtype), gk2, e, shards)
    return oq.QKResult(yq, yk, dtype, pq, pk)


def _fused_joint(xq, xk, gamma_q, gamma_k, dtype, eps, shards):
    e = oq.eps_as_passed(eps)
    xq64, xk64 = oq.decode_input(xq, dtype), oq.decode_input(xk, dtype)
    x = np.concatenate([xq64, xk64], axis=1)
    g = np.concatenate([oq.decode_input(gamma_q, dtype), oq.decode_input(gamma_k, dtype)])
    y, p = oq.layerwise_rmsnorm(x, g, e, 1)
    hq = xq64.shape[1]
    pq = oq.shard_sum_of_squares(xq64, shards)
    pk = oq.shard_sum_of_squares(xk64, shards)
    return oq.QKResult(y[:, :hq], y[:, hq:], dtype, pq, pk)


def _headwise_as_layerwise(x, gamma, eps, head_dim, gamma_head_stride):
    g = np.asarray(gamma, np.float64)
    h = np.asarray(x).shape[1]
    full = np.concatenate([g[i * gamma_head_stride:i * gamma_head_stride + head_dim] for i in range(h // head_dim)])
    return oq.layerwise_rmsnorm(x, full, eps)[0]


def _headwise_stride(forced):
    def f(x, gamma, eps, head_dim, gamma_head_stride):
        g = np.asarray(gamma, np.float64)
        stride = head_dim if forced == "full" else 0
        return _orig_headwise(x, g, eps, head_dim, stride)
    return f


def _headwise_shifted(x, gamma, eps, head_dim, gamma_head_stride):
    x = np.asarray(x, np.float64)
    y = np.empty_like(x)
    h = x.shape[1]
    g = np.asarray(gamma, np.float64)
    for head in range(h // head_dim):
        lo = max(head * head_dim - 1, 0)
        cols = slice(lo, lo + head_dim)
        g0 = head * gamma_head_stride
        yh = oq.layerwise_rmsnorm(x[:, cols], g[g0:g0 + head_dim], eps)[0]
        y[:, head * head_dim:(head + 1) * head_dim] = yh
    return y


_orig_headwise = oq.headwise_rmsnorm

MUTANTS = {
    "eps_dropped": ("rms_denominator", lambda ss, h, eps: np.sqrt(np.asarray(ss) / float(h))),
    "eps_outside_sqrt": ("rms_denominator", lambda ss, h, eps: np.sqrt(np.asarray(ss) / float(h)) + eps),
    "eps_added_to_sum": ("rms_denominator", lambda ss, h, eps: np.sqrt((np.asarray(ss) + eps) / float(h))),
    "sum_not_mean": ("rms_denominator", lambda ss, h, eps: np.sqrt(np.asarray(ss) + eps)),
    "mean_square_not_rms": ("rms_denominator", lambda ss, h, eps: np.asarray(ss) / float(h) + eps),
    "divide_by_h_minus_1": ("rms_denominator", lambda ss, h, eps: np.sqrt(np.asarray(ss) / max(float(h) - 1, 1.0) + eps)),
    "gamma_reversed": ("scale_rows", lambda x, g, d: np.asarray(x) * np.asarray(g)[::-1][None, :] / np.asarray(d)[:, None]),
    "gamma_dropped": ("scale_rows", lambda x, g, d: np.asarray(x) / np.asarray(d)[:, None]),
    "multiply_by_denominator": ("scale_rows", lambda x, g, d: np.asarray(x) * np.asarray(g)[None, :] * np.asarray(d)[:, None]),
    "sign_lost": ("scale_rows", lambda x, g, d: np.abs(np.asarray(x)) * np.asarray(g)[None, :] / np.asarray(d)[:, None]),
    "abs_not_square": ("shard_sum_of_squares", _shards(lambda x, s, w, S: np.sum(np.abs(x[:, s * w:(s + 1) * w]), axis=1))),
    "shard_drops_last_column": ("shard_sum_of_squares", _shards(lambda x, s, w, S: np.sum(x[:, s * w:(s + 1) * w - 1] ** 2, axis=1))),
    "shard_one_column_late": ("shard_sum_of_squares", _shards(lambda x, s, w, S: np.sum(x[:, s * w + 1:(s + 1) * w + 1] ** 2, axis=1))),
    "shards_reversed": ("shard_sum_of_squares", _shards(lambda x, s, w, S: np.sum(x[:, (S - 1 - s) * w:(S - s) * w] ** 2, axis=1))),
    "combine_mean": ("combine_partials", lambda p: np.mean(np.asarray(p, np.float64), axis=0)),
    "combine_first_only": ("combine_partials", lambda p: np.asarray(p, np.float64)[0]),
    "combine_in_float32": ("combine_partials", lambda p: np.sum(np.asarray(p, np.float32), axis=0, dtype=np.float32).astype(np.float64)),
    "apply_local_width": ("apply_with_stats", lambda x, g, planes, h_full, eps: oq.scale_rows(x, g, oq.rms_denominator(oq.combine_partials(planes), np.asarray(x).shape[1], eps))),
    "eps_not_float32": ("eps_as_passed", lambda eps: float(eps)),
    "round_truncate": ("f64_to_bf16_bits", _round_truncate),
    "round_via_float32": ("f64_to_bf16_bits", _round_via_f32),
    "round_ties_away": ("f64_to_bf16_bits", _round_ties_away),
    "decode_bf16_shift15": ("bf16_bits_to_f64", lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)),
    "q_k_gamma_swapped": ("qknorm_fused", _fused_gamma_swapped),
    "q_k_normalized_jointly": ("qknorm_fused", _fused_joint),
    "fp8_gamma_read_as_fp8": ("decode_gamma", lambda a, dtype: oq.decode_input(a, dtype)),
    "fp8_output_not_saturated": ("f64_to_fp8_bits", lambda v: np.where(np.abs(np.asarray(v)) > 464, np.uint8(0x7F), _orig_fp8(v)).astype(np.uint8)),
    "headwise_one_factor_per_row": ("headwise_rmsnorm", _headwise_as_layerwise),
    "headwise_gamma_always_shared": ("headwise_rmsnorm", _headwise_stride("shared")),
    "headwise_gamma_always_per_column": ("headwise_rmsnorm", _headwise_stride("full")),
    "headwise_heads_shifted_by_one_column": ("headwise_rmsnorm", _headwise_shifted),
}


def _run_pins():
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # an exception is a failed pin as well
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oq, attr, fn)
    failed = _run_pins()
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []

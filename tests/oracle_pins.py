"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, an invariant, a library special case, exact rational brute
force or a hand-worked example. ``test_oracle_pins.py`` runs them against the
oracle; ``test_oracle_mutants.py`` runs them against deliberately broken
copies of the oracle to show that each plausible mistake fails at least one.

Formula (the paper's Eq. 1, whose body is missing from the page text, read as
y_j = x_j * gamma_j / sqrt(sum x^2 / H + eps)); Phase A splits the sum of
squares over column shards. Source: "SwiftQK: Fast and Communication-
Efficient Tensor Parallelism for Query-Key Normalization", arXiv HTML page.
"""

import json
import math
import os
from decimal import Decimal
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import bf16 as obf16
from oracle import qknorm as oq

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def _close(a, b, rel=1e-14, abs_=0.0):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    ok = np.abs(a - b) <= rel * np.abs(b) + abs_
    assert ok.all(), f"max diff {np.max(np.abs(a - b))}: {a[~ok][:4]} vs {b[~ok][:4]}"


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- golden
def pin_golden_worked_examples():
    """Hand-worked examples (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        x = np.array([ex["x"]], dtype=np.float64)
        g = np.array(ex["gamma"], dtype=np.float64)
        want = np.array([[float(Decimal(v)) for v in ex["y"]]])
        if ex["op"] == "fused":
            y, p = oq.layerwise_rmsnorm(x, g, float(ex["eps"]), ex["shards"])
            assert np.array_equal(p[:, 0], np.array(ex["partials"], dtype=np.float64)), ex["name"]
        else:
            planes = np.array(ex["stats"], dtype=np.float64)[:, None]
            y = oq.apply_with_stats(x, g, planes, ex["h_full"], float(ex["eps"]))
        _close(y, want, rel=4e-16)


def pin_golden_bf16_rounding():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["bf16_rounding"]["cases"]:
        v = Decimal(c["value"])
        f64 = float(v)
        if c.get("exact_in_f64"):
            assert Decimal(f64) == v, "tie cases must be exact in float64"
        got = int(oq.f64_to_bf16_bits(np.array([f64]))[0])
        assert got == int(c["bits"], 16), (c, hex(got))
    # the rounding the top-level result uses must be the same single rounding
    r = oq.QKResult(np.array([[0.4, 1.0 + 2.0 ** -8 + 2.0 ** -40]]), np.zeros((1, 1)), "bf16")
    assert list(r.yq_bits[0]) == [0x3ECD, 0x3F81]


def pin_golden_headwise():
    """Hand-worked headwise examples: one factor per head, gamma shared across
    heads (stride 0) or read per column (stride head_dim); and the same row
    under one layerwise factor, which differs."""
    with open(GOLDEN) as f:
        data = json.load(f)["headwise_examples"]
    for c in data["cases"]:
        x = np.array([c["x"]], dtype=np.float64)
        want = np.array([[float(Decimal(v)) for v in c["y"]]])
        y = oq.headwise_rmsnorm(x, np.array(c["gamma"], dtype=np.float64), float(c["eps"]), c["head_dim"],
                                c["gamma_head_stride"])
        _close(y, want, rel=4e-16)
        # and through the top-level call (Q and K are independent)
        r = oq.qknorm_headwise(np.asarray(x, np.float32), np.asarray(x[:, :c["head_dim"]], np.float32),
                               np.asarray(c["gamma"], np.float32), np.asarray(c["gamma"], np.float32), "f32",
                               np.float32(c["eps"]), c["head_dim"], c["gamma_head_stride"])
        _close(r.yq, want, rel=4e-16)
    lc = data["layerwise_contrast"]
    y, _ = oq.layerwise_rmsnorm(np.array([lc["x"]], dtype=np.float64), np.array(lc["gamma"], dtype=np.float64),
                                float(lc["eps"]))
    _close(y, np.array([[float(Decimal(v)) for v in lc["y"]]]), rel=4e-16)


def pin_golden_fp8_rounding():
    """Hand-derived E4M3 roundings: nearest, ties to even (normal and
    subnormal), the smallest subnormal, saturation at +-448, signed zero."""
    with open(GOLDEN) as f:
        cases = json.load(f)["fp8_e4m3_rounding"]["cases"]
    for c in cases:
        v = Decimal(c["value"])
        f64 = float(v)
        if c.get("exact_in_f64"):
            assert Decimal(f64) == v, "tie cases must be exact in float64"
        got = int(oq.f64_to_fp8_bits(np.array([f64]))[0])
        assert got == int(c["bits"], 16), (c, hex(got))


# ---------------------------------------------------------------- closed forms
def pin_constant_vector():
    """x_j = c for all j gives y_j = c / sqrt(c^2 + eps) * gamma_j."""
    rng = _rng(1)
    for h in (1, 3, 64, 1000):
        for c in (3.0, -2.5, 1e-3, 7e3):
            for eps in (0.0, 1e-6, 0.25):
                g = rng.uniform(0.5, 1.5, h)
                x = np.full((2, h), c)
                y, _ = oq.layerwise_rmsnorm(x, g, eps)
                want = c / math.sqrt(c * c + eps) * g
                _close(y, np.vstack([want, want]), rel=1e-14)


def pin_one_hot():
    """x = a e_k gives y_k = a gamma_k / sqrt(a^2/H + eps), zero elsewhere."""
    rng = _rng(2)
    for h in (2, 5, 128):
        for eps in (0.0, 1e-6, 3.0):
            k = int(rng.integers(h))
            a = -3.75
            g = rng.uniform(0.5, 1.5, h)
            x = np.zeros((1, h))
            x[0, k] = a
            y, _ = oq.layerwise_rmsnorm(x, g, eps)
            want = np.zeros((1, h))
            want[0, k] = a * g[k] / math.sqrt(a * a / h + eps)
            _close(y, want, rel=1e-15)
            if eps == 0.0:
                _close(y[0, k], -math.sqrt(h) * g[k], rel=1e-15)


def pin_width_one():
    """H = 1 gives y = x gamma / sqrt(x^2 + eps)."""
    for xv in (-4.0, 0.5, 3.0):
        for eps in (0.0, 1e-6, 2.0):
            y, _ = oq.layerwise_rmsnorm(np.array([[xv]]), np.array([1.7]), eps)
            _close(y[0, 0], xv * 1.7 / math.sqrt(xv * xv + eps), rel=1e-15)


# ---------------------------------------------------------------- invariants
def pin_scale_invariance_eps0():
    """With eps = 0, scaling x by 2^k leaves y bit-for-bit unchanged."""
    rng = _rng(3)
    x = rng.standard_normal((5, 96))
    g = rng.normal(1, 0.1, 96)
    y0, _ = oq.layerwise_rmsnorm(x, g, 0.0)
    for k in (-20, -3, 1, 7, 20):
        y, _ = oq.layerwise_rmsnorm(x * 2.0 ** k, g, 0.0)
        assert np.array_equal(y, y0), k
    # with eps = 1e-6 and unit-scale data the change stays within eps-size effects
    y1, _ = oq.layerwise_rmsnorm(x * 3.0, g, 1e-6)
    y2, _ = oq.layerwise_rmsnorm(x, g, 1e-6)
    _close(y1, y2, rel=2e-6)


def pin_oddness():
    rng = _rng(4)
    x = rng.standard_normal((4, 40))
    g = rng.normal(1, 0.1, 40)
    for s in (1, 2, 4, 8):
        a, _ = oq.layerwise_rmsnorm(x, g, 1e-6, s)
        b, _ = oq.layerwise_rmsnorm(-x, g, 1e-6, s)
        assert np.array_equal(a, -b)


def pin_unit_rms():
    """mean_j (y_j / gamma_j)^2 = m / (m + eps), m = mean square of x."""
    rng = _rng(5)
    x = rng.standard_normal((6, 300)) * rng.lognormal(0, 1, (6, 1))
    g = rng.uniform(0.5, 1.5, 300)
    for eps in (0.0, 1e-6, 0.5):
        y, _ = oq.layerwise_rmsnorm(x, g, eps)
        m = np.mean(x * x, axis=1)
        _close(np.mean((y / g) ** 2, axis=1), m / (m + eps), rel=1e-13)


# ---------------------------------------------------------------- library special case
def pin_torch_rms_norm_fp64():
    """S = 1 equals torch.nn.functional.rms_norm over the last dim, in fp64 on the CPU."""
    rng = _rng(6)
    for h, eps in ((256, 1e-6), (1000, 1e-6), (37, 0.3)):
        x = rng.standard_normal((9, h)) * rng.lognormal(0, 1, (9, 1))
        g = rng.normal(1, 0.1, h)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), [h], torch.from_numpy(g), eps).numpy()
        for s in (1, next(d for d in (4, 2, 1) if h % d == 0)):
            y, _ = oq.layerwise_rmsnorm(x, g, eps, s)
            _close(y, ref, rel=1e-14)


# ---------------------------------------------------------------- brute force
def _exact_y_squared(xrow, grow, eps, h_full=None):
    """Exact rational y_j^2 = x_j^2 g_j^2 / (sum x^2 / H + eps)."""
    xs = [Fraction(float(v)) for v in xrow]
    gs = [Fraction(float(v)) for v in grow]
    H = h_full if h_full is not None else len(xs)
    ms = sum(v * v for v in xs) / H + Fraction(eps)
    return [(xv * xv * gv * gv) / ms for xv, gv in zip(xs, gs)]


def pin_brute_force_rational():
    """Tiny rows: y^2 against exact rationals (sum, mean, eps), and signs."""
    rng = _rng(7)
    for h in (1, 2, 3, 4, 6, 8):
        for s in [d for d in range(1, h + 1) if h % d == 0]:
            x = rng.standard_normal((3, h))
            g = rng.normal(1, 0.3, h)
            eps = float(rng.choice([0.0, 1e-6, 0.7]))
            y, p = oq.layerwise_rmsnorm(x, g, eps, s)
            for t in range(3):
                ex = _exact_y_squared(x[t], g, eps)
                _close(y[t] ** 2, np.array([float(v) for v in ex]), rel=1e-14)
                assert np.array_equal(np.sign(y[t]), np.sign(x[t] * g))
                w = h // s
                for si in range(s):
                    exact = sum(Fraction(float(v)) ** 2 for v in x[t, si * w:(si + 1) * w])
                    _close(p[si, t], float(exact), rel=1e-15)


def pin_partials_exact_on_integers():
    """Integer inputs: every shard sum and the combined sum are exact."""
    rng = _rng(8)
    for h, shards in ((64, (1, 2, 4, 8, 16)), (96, (1, 3, 6, 32)), (4096, (1, 2, 4, 8))):
        x = rng.integers(-16, 17, (4, h)).astype(np.float64)
        full = [sum(int(v) ** 2 for v in row) for row in x]
        for s in shards:
            p = oq.shard_sum_of_squares(x, s)
            w = h // s
            for t in range(4):
                for si in range(s):
                    assert p[si, t] == sum(int(v) ** 2 for v in x[t, si * w:(si + 1) * w])
                assert oq.combine_partials(p)[t] == full[t]


def pin_decomposition_random():
    """Phase A: the sum of shard partials equals the full sum of squares."""
    rng = _rng(9)
    x = rng.standard_normal((7, 4096))
    full = np.array([math.fsum(v * v for v in row) for row in x])
    for s in (1, 2, 4, 8, 64):
        _close(oq.combine_partials(oq.shard_sum_of_squares(x, s)), full, rel=1e-14)
        y_s, _ = oq.layerwise_rmsnorm(x, np.ones(4096), 1e-6, s)
        y_1, _ = oq.layerwise_rmsnorm(x, np.ones(4096), 1e-6, 1)
        _close(y_s, y_1, rel=1e-14)


# ---------------------------------------------------------------- apply with external statistics
def pin_apply_local_slice():
    """A shard scaled with the full-row sum and the full width H equals that
    shard of the full-row result (Phase B and the final scaling)."""
    rng = _rng(10)
    H, S = 512, 4
    x = rng.standard_normal((5, H))
    g = rng.normal(1, 0.1, H)
    y_full, _ = oq.layerwise_rmsnorm(x, g, 1e-6)
    exact_ss = np.array([float(sum(Fraction(float(v)) ** 2 for v in row)) for row in x])
    w = H // S
    for s in range(S):
        sl = slice(s * w, (s + 1) * w)
        y = oq.apply_with_stats(x[:, sl], g[sl], exact_ss[None, :], H, 1e-6)
        _close(y, y_full[:, sl], rel=1e-14)
        # planes split the same sum in any way
        planes = np.stack([exact_ss * 0.25, exact_ss * 0.5, exact_ss * 0.25])
        _close(oq.apply_with_stats(x[:, sl], g[sl], planes, H, 1e-6), y_full[:, sl], rel=1e-14)


def pin_top_level_calls():
    """The library-shaped calls: Q and K each normalized over their own width
    with their own gamma, no mixing; bf16 bits are the single rounding of y;
    eps is the float32 value the kernel would receive."""
    rng = _rng(11)
    T, hq, hk = 6, 48, 16
    xq = rng.standard_normal((T, hq)).astype(np.float32)
    xk = (rng.standard_normal((T, hk)) * 3).astype(np.float32)
    gq = np.full(hq, 2.0, np.float32)
    gk = np.full(hk, 0.5, np.float32)
    eps = 0.1    # not a float32 number: the kernel receives float32(0.1)
    r = oq.qknorm_fused(xq, xk, gq, gk, "f32", eps, 2)
    e32 = float(np.float32(eps))
    for x, g, y in ((xq, 2.0, r.yq), (xk, 0.5, r.yk)):
        x64 = x.astype(np.float64)
        d = np.sqrt(np.mean(x64 * x64, axis=1) + e32)
        _close(y, x64 * g / d[:, None], rel=1e-15)
    # changing K changes nothing in Q
    r2 = oq.qknorm_fused(xq, xk * 7, gq, gk, "f32", eps, 2)
    assert np.array_equal(r.yq, r2.yq)
    # bf16: bits are the rounding of the float64 result
    bq = obf16.f64_to_bf16_bits(xq.astype(np.float64))
    bk = obf16.f64_to_bf16_bits(xk.astype(np.float64))
    gb = obf16.f64_to_bf16_bits(np.full(hq, 1.25))
    gkb = obf16.f64_to_bf16_bits(np.full(hk, 0.75))
    rb = oq.qknorm_fused(bq, bk, gb, gkb, "bf16", 1e-6, 4)
    assert np.array_equal(rb.yq_bits, obf16.f64_to_bf16_bits(rb.yq))
    xqb = obf16.bf16_bits_to_f64(bq)
    dq = np.sqrt(np.mean(xqb * xqb, axis=1) + float(np.float32(1e-6)))
    _close(rb.yq, xqb * 1.25 / dq[:, None], rel=1e-15)
    # partial_stats and apply_with_stats agree with fused
    ps = oq.qknorm_partial_stats(bq, bk, "bf16", 4)
    assert ps.shape == (4, 2, T)
    assert np.array_equal(ps[:, 0, :], rb.pq) and np.array_equal(ps[:, 1, :], rb.pk)
    ra = oq.qknorm_apply_with_stats(bq, bk, gb, gkb, "bf16", 1e-6, ps.astype(np.float32), hq, hk)
    # float32 statistics differ from float64 ones by < 2^-24 relative
    _close(ra.yq, rb.yq, rel=1e-7)
    _close(ra.yk, rb.yk, rel=1e-7)


def pin_nonfinite_and_zero_rows():
    """IEEE behaviour of the formula on degenerate rows."""
    g = np.array([1.0, 2.0, 3.0, 4.0])
    y, _ = oq.layerwise_rmsnorm(np.zeros((1, 4)), g, 1e-6)
    assert np.array_equal(y, np.zeros((1, 4)))
    with np.errstate(invalid="ignore", divide="ignore"):
        y, _ = oq.layerwise_rmsnorm(np.zeros((1, 4)), g, 0.0)
        assert np.isnan(y).all()
        y, _ = oq.layerwise_rmsnorm(np.array([[1.0, np.nan, 2.0, 3.0]]), g, 1e-6)
        assert np.isnan(y).all()
        y, _ = oq.layerwise_rmsnorm(np.array([[1.0, np.inf, 2.0, 3.0]]), g, 1e-6)
        assert y[0, 0] == 0 and np.isnan(y[0, 1]) and y[0, 2] == 0 and y[0, 3] == 0


# ---------------------------------------------------------------- headwise QK-Norm
def pin_headwise_one_head_is_layerwise():
    """A single head spanning the row is layerwise RMS-Norm."""
    rng = _rng(12)
    x = rng.standard_normal((5, 96))
    g = rng.normal(1, 0.1, 96)
    for stride in (0, 96):
        _close(oq.headwise_rmsnorm(x, g, 1e-6, 96, stride), oq.layerwise_rmsnorm(x, g, 1e-6)[0], rel=1e-15)


def pin_headwise_torch_rms_norm_fp64():
    """[T, heads, head_dim] RMS-Norm over the last dim (torch, fp64): a shared
    [head_dim] weight is stride 0; a per-column weight is stride head_dim."""
    rng = _rng(13)
    T, nh, hd = 7, 6, 40
    x = rng.standard_normal((T, nh * hd)) * rng.lognormal(0, 1, (T, 1))
    xt = torch.from_numpy(x).view(T, nh, hd)
    g_shared = rng.normal(1, 0.2, hd)
    ref = torch.nn.functional.rms_norm(xt, [hd], torch.from_numpy(g_shared), 1e-6).reshape(T, -1).numpy()
    _close(oq.headwise_rmsnorm(x, g_shared, 1e-6, hd, 0), ref, rel=1e-14)
    g_full = rng.normal(1, 0.2, nh * hd)
    ref = (torch.nn.functional.rms_norm(xt, [hd], None, 1e-6).reshape(T, -1) * torch.from_numpy(g_full)).numpy()
    _close(oq.headwise_rmsnorm(x, g_full, 1e-6, hd, hd), ref, rel=1e-14)


def pin_headwise_constant_heads():
    """Head h constant c_h: y = c_h / sqrt(c_h^2 + eps) * gamma, per head."""
    hd, cs = 16, (3.0, -0.5, 7.0, 1e-3)
    x = np.concatenate([np.full((2, hd), c) for c in cs], axis=1)
    g = np.linspace(0.5, 1.5, hd)
    y = oq.headwise_rmsnorm(x, g, 0.25, hd, 0)
    for i, c in enumerate(cs):
        _close(y[:, i * hd:(i + 1) * hd], np.tile(c / math.sqrt(c * c + 0.25) * g, (2, 1)), rel=1e-14)


def pin_headwise_heads_independent():
    """Changing one head changes no other head's result (bit for bit)."""
    rng = _rng(14)
    x = rng.standard_normal((3, 8 * 32))
    g = rng.normal(1, 0.1, 32)
    y0 = oq.headwise_rmsnorm(x, g, 1e-6, 32, 0)
    x2 = x.copy()
    x2[:, 96:128] *= 17.0
    y1 = oq.headwise_rmsnorm(x2, g, 1e-6, 32, 0)
    assert np.array_equal(np.delete(y0, np.s_[96:128], axis=1), np.delete(y1, np.s_[96:128], axis=1))
    assert not np.array_equal(y0[:, 96:128], y1[:, 96:128])


def pin_headwise_top_level():
    """Q and K with different head counts, each head over head_dim; bf16 bits rounded once."""
    rng = _rng(15)
    T, hd = 4, 32
    xq = obf16.f64_to_bf16_bits(rng.standard_normal((T, 5 * hd)))
    xk = obf16.f64_to_bf16_bits(rng.standard_normal((T, 2 * hd)))
    gq = obf16.f64_to_bf16_bits(rng.normal(1, 0.1, hd))
    gk = obf16.f64_to_bf16_bits(rng.normal(1, 0.1, hd))
    r = oq.qknorm_headwise(xq, xk, gq, gk, "bf16", 1e-6, hd, 0)
    e = float(np.float32(1e-6))
    for x, g, y in ((xq, gq, r.yq), (xk, gk, r.yk)):
        xd = obf16.bf16_bits_to_f64(x).reshape(T, -1, hd)
        d = np.sqrt(np.mean(xd * xd, axis=2, keepdims=True) + e)
        _close(y, (xd * obf16.bf16_bits_to_f64(g) / d).reshape(T, -1), rel=1e-15)
    assert np.array_equal(r.yq_bits, obf16.f64_to_bf16_bits(r.yq))


def pin_fp8_top_level():
    """FP8 E4M3 rows with bf16 gamma: the result is Eq. 1 on the exact decoded
    values, rounded once to E4M3 with saturation; sums of squares are exact
    on small integers."""
    from oracle import fp8 as ofp8
    rng = _rng(16)
    T, hq, hk = 5, 64, 32
    xq = ofp8.f64_to_fp8_bits(rng.standard_normal((T, hq)) * 3)
    xk = ofp8.f64_to_fp8_bits(rng.integers(-8, 9, (T, hk)).astype(np.float64))
    gq = obf16.f64_to_bf16_bits(rng.normal(1, 0.1, hq))
    gk = obf16.f64_to_bf16_bits(np.full(hk, 300.0))          # drives some outputs past 448
    r = oq.qknorm_fused(xq, xk, gq, gk, "fp8", 1e-6, 2)
    e = float(np.float32(1e-6))
    xqd = ofp8.fp8_bits_to_f64(xq)
    dq = np.sqrt(np.mean(xqd * xqd, axis=1) + e)
    _close(r.yq, xqd * obf16.bf16_bits_to_f64(gq) / dq[:, None], rel=1e-15)
    assert np.array_equal(r.yq_bits, ofp8.f64_to_fp8_bits(r.yq))
    xkd = ofp8.fp8_bits_to_f64(xk)
    assert np.array_equal(r.pk.sum(axis=0), (xkd * xkd).sum(axis=1))  # integers: exact
    big = np.abs(r.yk) > 464
    assert big.any() and np.all((r.yk_bits[big] & 0x7F) == 0x7E)     # saturated to +-448


ALL_PINS = [
    pin_golden_worked_examples,
    pin_golden_bf16_rounding,
    pin_golden_headwise,
    pin_golden_fp8_rounding,
    pin_constant_vector,
    pin_one_hot,
    pin_width_one,
    pin_scale_invariance_eps0,
    pin_oddness,
    pin_unit_rms,
    pin_torch_rms_norm_fp64,
    pin_brute_force_rational,
    pin_partials_exact_on_integers,
    pin_decomposition_random,
    pin_apply_local_slice,
    pin_top_level_calls,
    pin_nonfinite_and_zero_rows,
    pin_headwise_one_head_is_layerwise,
    pin_headwise_torch_rms_norm_fp64,
    pin_headwise_constant_heads,
    pin_headwise_heads_independent,
    pin_headwise_top_level,
    pin_fp8_top_level,
]

assert oracle.qknorm_fused is oq.qknorm_fused

"""The seeded input generators: deterministic, right shapes and layouts,
right value distributions (CPU only)."""

import numpy as np

from layerwise_qk_norm_qknorm_amd import inputs as I
from oracle.bf16 import bf16_bits_to_f64


def test_deterministic_and_seeded_by_config():
    a = I.make_inputs(I.SMALL_DENSE.with_T(8))
    b = I.make_inputs(I.SMALL_DENSE.with_T(8))
    assert np.array_equal(a.qkv, b.qkv) and np.array_equal(a.gamma_q, b.gamma_q)
    other = I.make_inputs(I.DECODE[2].with_T(8))
    assert not np.array_equal(a.qkv[:, :64], other.qkv[:, :64])


def test_layouts():
    tiny = I.make_inputs(I.TINY)
    assert tiny.qkv is None and tiny.q.dtype == np.float32 and tiny.q.shape == (16, 256)
    assert tiny.q.flags.c_contiguous and tiny.k.flags.c_contiguous
    prefill = I.make_inputs(I.GQA_PREFILL.with_T(4))
    assert prefill.qkv.shape == (4, 7168) and prefill.qkv.dtype == np.uint16
    assert prefill.q.base is prefill.qkv or prefill.q.base is prefill.qkv.base
    assert prefill.q.shape == (4, 5120) and prefill.k.shape == (4, 1024)
    assert np.shares_memory(prefill.k, prefill.qkv)
    rank = I.make_inputs(I.RANK_SLICE.with_T(8))
    assert rank.peer_q.shape == (3, 8, 1280) and rank.peer_k.shape == (3, 8, 256)


def test_distributions():
    tiny = I.make_inputs(I.TINY)
    assert 0.5 <= tiny.gamma_q.min() and tiny.gamma_q.max() <= 1.5
    prefill = I.make_inputs(I.GQA_PREFILL.with_T(512))
    x = bf16_bits_to_f64(prefill.qkv[:, :6144])
    n = prefill.meta["n_outliers"]
    assert abs(n - 0.001 * x.size) < 5 * np.sqrt(0.001 * x.size)
    assert np.abs(x).max() > 50            # outliers x50
    g = bf16_bits_to_f64(prefill.gamma_q)
    assert abs(g.mean() - 1) < 0.02 and abs(g.std() - 0.1) < 0.02
    dense = I.make_inputs(I.SMALL_DENSE)
    rms = np.sqrt(np.mean(bf16_bits_to_f64(dense.qkv[:, :4096]) ** 2, axis=1))
    assert rms.max() / rms.min() > 20      # per-token LogNormal(0,1) scale


def test_bf16_input_rounding_is_nearest():
    v = np.array([1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, -2.5, 0.1])
    b = I.to_bf16_bits(v)
    assert list(b) == [0x3F80, 0x3F81, 0xC020, 0x3DCD]


def test_fp8_inputs():
    w = I.GQA_PREFILL_FP8.with_T(64)
    inp = I.make_inputs(w)
    assert inp.qkv.dtype == np.uint8 and inp.gamma_q.dtype == np.uint16      # FP8 rows, bf16 gamma
    from oracle.fp8 import fp8_bits_to_f64
    x = fp8_bits_to_f64(inp.qkv[:, :6144])
    assert np.isfinite(x).all() and np.abs(x).max() <= 448
    assert np.array_equal(I.to_fp8_bits(np.array([1.0, -2.5, 448.0, 1.0625])), np.array([0x38, 0xC2, 0x7E, 0x38]))

"""The seeded input generators: deterministic, right shapes and layouts,
right value distributions (CPU only)."""

import numpy as np

from layerwise_qk_norm_qknorm_amd import inputs as I
from oracle.bf16 import bf16_bits_to_f64


def test_deterministic_and_seeded_by_config():
    a = I.make_inputs(I.C2.with_T(8))
    b = I.make_inputs(I.C2.with_T(8))
    assert np.array_equal(a.qkv, b.qkv) and np.array_equal(a.gamma_q, b.gamma_q)
    c = I.make_inputs(I.C3[2].with_T(8))
    assert not np.array_equal(a.qkv[:, :64], c.qkv[:, :64])


def test_layouts():
    c1 = I.make_inputs(I.C1)
    assert c1.qkv is None and c1.q.dtype == np.float32 and c1.q.shape == (16, 256)
    assert c1.q.flags.c_contiguous and c1.k.flags.c_contiguous
    c4 = I.make_inputs(I.C4.with_T(4))
    assert c4.qkv.shape == (4, 7168) and c4.qkv.dtype == np.uint16
    assert c4.q.base is c4.qkv or c4.q.base is c4.qkv.base
    assert c4.q.shape == (4, 5120) and c4.k.shape == (4, 1024)
    assert np.shares_memory(c4.k, c4.qkv)
    c5 = I.make_inputs(I.C5.with_T(8))
    assert c5.peer_q.shape == (3, 8, 1280) and c5.peer_k.shape == (3, 8, 256)


def test_distributions():
    c1 = I.make_inputs(I.C1)
    assert 0.5 <= c1.gamma_q.min() and c1.gamma_q.max() <= 1.5
    c4 = I.make_inputs(I.C4.with_T(512))
    x = bf16_bits_to_f64(c4.qkv[:, :6144])
    n = c4.meta["n_outliers"]
    assert abs(n - 0.001 * x.size) < 5 * np.sqrt(0.001 * x.size)
    assert np.abs(x).max() > 50            # outliers x50
    g = bf16_bits_to_f64(c4.gamma_q)
    assert abs(g.mean() - 1) < 0.02 and abs(g.std() - 0.1) < 0.02
    c2 = I.make_inputs(I.C2)
    rms = np.sqrt(np.mean(bf16_bits_to_f64(c2.qkv[:, :4096]) ** 2, axis=1))
    assert rms.max() / rms.min() > 20      # per-token LogNormal(0,1) scale


def test_bf16_input_rounding_is_nearest():
    v = np.array([1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, -2.5, 0.1])
    b = I.to_bf16_bits(v)
    assert list(b) == [0x3F80, 0x3F81, 0xC020, 0x3DCD]

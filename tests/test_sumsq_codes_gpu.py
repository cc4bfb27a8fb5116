"""The in-lane sums of squares (Phase A) on every input value a row can hold.

Rows of one repeated value have an exactly representable sum of squares
(bf16: 8 squares of an 8-bit significand; FP8 E4M3: 16 squares of a 4-bit
one), so qknorm_partial_stats must return the oracle's float64 sum rounded to
float32 bit for bit, for every bf16 pattern whose square is a normal float32
(|x| from 2^-60 to 2^60) and for every one of the 256 E4M3 codes (NaN codes
give NaN). This pins the decoding and the squaring of each value inside the
dot-product sums, including subnormal E4M3 inputs and negative zero."""

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from gpu_helpers import DEV, np_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _run(q_bits, k_bits, dtype, shards):
    """Packed rows [T, hq + hk] through partial_stats; returns the planes."""
    host = np.concatenate([q_bits, k_bits], axis=1)
    x = np_to_torch(host).to(DEV)
    hq = q_bits.shape[1]
    part = qk.qknorm_partial_stats(x[:, :hq], x[:, hq:], shards)
    torch.cuda.synchronize()
    return part.cpu().numpy()


def _expect(q_bits, k_bits, dtype, shards):
    return oracle.qknorm_partial_stats(q_bits, k_bits, dtype, shards).astype(np.float32)


@pytest.mark.parametrize("shards", [1, 2])
def test_every_bf16_value_with_a_normal_square(shards):
    bits = np.arange(1 << 16, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    keep = (exp >= 127 - 60) & (exp <= 127 + 60)
    vals = bits[keep].astype(np.uint16)            # both signs, every significand
    T = vals.shape[0]
    print(f"[case] bf16 rows of one repeated value: {T} values, S={shards}", flush=True)
    q = np.repeat(vals[:, None], 16, axis=1)        # 8 per shard at S = 2
    k = np.repeat(vals[::-1, None], 16, axis=1)
    got, want = _run(q, k, "bf16", shards), _expect(q, k, "bf16", shards)
    assert np.all(np.isfinite(want))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_every_fp8_code():
    codes = np.arange(256, dtype=np.uint8)
    q = np.repeat(codes[:, None], 16, axis=1)
    k = np.repeat(codes[::-1, None], 32, axis=1)
    print("[case] FP8 rows of one repeated code: all 256 codes", flush=True)
    got, want = _run(q, k, "fp8", 1), _expect(q, k, "fp8", 1)
    nan = np.isnan(want)
    assert nan.sum() == 4                           # 0x7F and 0xFF, in Q and in K
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))

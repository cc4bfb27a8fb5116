"""GPU parity of qknorm_headwise (one RMS factor per attention head) against
the float64 oracle, element by element; same acceptance as the layerwise
calls (fp32: rel 1e-5; bf16: within one bf16 step of the once-rounded
oracle result), plus untouched V columns and guard bands."""

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, Guarded, check_bf16, check_f32, np_to_torch

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _run(T, hq, hk, hv, dtype, head_dim, stride, seed, offset=0, ld_pad=0, in_place=False, inp=None, eps=1e-6):
    inp = inp or I.make_custom(T, hq, hk, hv, dtype, seed=seed)
    _log(f"[case] headwise T={T} hq={hq} hk={hk} hv={hv} {dtype} head_dim={head_dim} stride={stride} "
         f"offset={offset} ld_pad={ld_pad} in_place={in_place} plan: "
         f"{qk.describe_headwise_plan(hq, hk, T, head_dim, dtype, stride, ld=hq + hk + hv + ld_pad)}")
    ld = hq + hk + hv + ld_pad
    host = np.zeros((T, ld), dtype=inp.q.dtype)
    host[:, :hq] = inp.q
    host[:, hq:hq + hk] = inp.k
    if hv + ld_pad:
        rng = np.random.default_rng(seed)
        host[:, hq + hk:] = rng.integers(0, 1 << 14, (T, hv + ld_pad)).astype(host.dtype)
    src = Guarded(host, seed=seed, offset_elems=offset)
    dst = src if in_place else Guarded(host, seed=seed + 1, offset_elems=offset)
    dst_init = dst.host().copy()
    x, y = src.view(), dst.view()
    if stride == 0:   # one [head_dim] vector shared by all heads
        gq_h, gk_h = inp.gamma_q[:head_dim].copy(), inp.gamma_k[:head_dim].copy()
    else:
        gq_h, gk_h = inp.gamma_q, inp.gamma_k
    gq, gk = np_to_torch(gq_h).to(DEV), np_to_torch(gk_h).to(DEV)
    qk.qknorm_headwise(x[:, :hq], x[:, hq:hq + hk], gq, gk, eps, head_dim, stride, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    out = dst.host()
    ref = oracle.qknorm_headwise(inp.q, inp.k, gq_h, gk_h, dtype, eps, head_dim, stride)
    if dtype == "bf16":
        eq, _ = check_bf16(out[:, :hq], ref.yq_bits, "headwise Q")
        ek, _ = check_bf16(out[:, hq:hq + hk], ref.yk_bits, "headwise K")
        _log(f"[parity] headwise: exact bf16 match Q {eq:.5f} K {ek:.5f}")
    else:
        rq = check_f32(out[:, :hq], ref.yq, "headwise Q")
        rk = check_f32(out[:, hq:hq + hk], ref.yk, "headwise K")
        _log(f"[parity] headwise: max rel err Q {rq:.3g} K {rk:.3g}")
    assert np.array_equal(out[:, hq + hk:].view(np.uint8), dst_init[:, hq + hk:].view(np.uint8))
    assert src.guards_intact() and dst.guards_intact()
    if not in_place:
        assert np.array_equal(src.host().view(np.uint8), host.view(np.uint8))
    return out


@pytest.mark.parametrize("stride", [0, 128])
def test_gqa_prefill_headwise_full_size(stride):
    w = I.GQA_PREFILL
    inp = I.make_inputs(w)
    _run(w.T, w.hq, w.hk, w.hv, "bf16", 128, stride, seed=0, inp=inp)


@pytest.mark.parametrize("T", [1, 8, 64, 256])
def test_decode_headwise(T):
    _run(T, 4096, 4096, 4096, "bf16", 128, 0, seed=100 + T)


def test_fp32_and_other_head_sizes():
    _run(16, 256, 256, 0, "f32", 64, 0, seed=201)
    _run(33, 72 * 8, 72 * 2, 16, "f32", 72, 72, seed=202)
    _run(40, 64 * 32, 64 * 4, 64 * 4, "bf16", 64, 0, seed=203)
    _run(9, 256 * 16, 256 * 2, 0, "bf16", 256, 256, seed=204)


def test_elementwise_path_headwise():
    _run(50, 36 * 6, 36 * 2, 8, "bf16", 36, 0, seed=301)             # 36 bf16: not whole 16-byte chunks
    _run(21, 128 * 4, 128, 128, "bf16", 128, 0, seed=302, offset=1)  # misaligned base
    _run(17, 96 * 3, 96, 0, "f32", 96, 96, seed=303, ld_pad=1)      # odd row stride


def test_in_place_headwise_equals_out_of_place():
    inp = I.make_custom(77, 1024, 256, 256, "bf16", seed=401)
    a = _run(77, 1024, 256, 256, "bf16", 128, 0, seed=401, inp=inp)
    b = _run(77, 1024, 256, 256, "bf16", 128, 0, seed=401, inp=inp, in_place=True)
    assert np.array_equal(a[:, :1280], b[:, :1280])


def test_widest_heads_and_most_heads():
    _run(4, 4096 * 2, 4096, 0, "bf16", 4096, 0, seed=501)    # 512 chunks per head
    _run(3, 8 * 200, 8 * 56, 0, "bf16", 8, 8, seed=502)      # 256 heads of one chunk


def test_tiny_heads():
    """Heads of 1, 2 and 4 elements, each normalized on its own (a one-element
    head gives gamma * x / sqrt(x^2 + eps), about gamma * sign(x)): the
    element-wise path with one lane per head, shared and per-column gamma,
    and (1029 tokens) several tokens per wave."""
    _run(37, 64, 32, 8, "bf16", 1, 0, seed=601)
    _run(37, 64, 32, 8, "bf16", 1, 1, seed=602)
    _run(19, 128, 64, 0, "f32", 2, 0, seed=603)
    _run(1029, 96, 32, 0, "bf16", 4, 4, seed=604)
    _run(7, 200, 56, 0, "f32", 1, 1, seed=605)


@pytest.mark.parametrize("head_dim,hq,hk", [(96, 3072, 768), (80, 5120, 1280), (96, 3072, 3072), (128, 12288, 1024),
                                            (64, 4096, 1024), (128, 16384, 2048)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_head_layouts(dtype, head_dim, hq, hk):
    """Prefill launches (T = 1024, the same layouts as at T = 8192): per-head
    lane groups for 80- and 96-wide heads, token-wide layouts of up to 16
    waves for 64- and 128-wide heads."""
    _run(1024, hq, hk, hk, dtype, head_dim, 0, seed=300 + head_dim + hq // 64)

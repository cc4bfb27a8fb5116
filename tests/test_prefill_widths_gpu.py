"""GPU parity over the prefill row widths (1024/256 to 16384/2048, and
5120/5120) in bf16, FP8 and fp32 rows, in the launches `bench.py --shapes`
times at T = 8192 (1 to 12 waves per token, 2 to 6 chunks per lane, several
tokens per block at the narrowest; 128 sampled tokens against the oracle) and
at T = 1024 (the mid-size bf16 layouts; every element), with the usual
acceptance, plus V columns and guard bands untouched; and the headwise call
over the same widths in 128-wide heads with one shared gamma per tensor (the
token-wide layouts, and the per-head layout of the narrowest FP8 rows)."""

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, Guarded, check_bf16, check_f32, check_fp8, np_to_torch

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1024, 8192])
@pytest.mark.parametrize("hq,hk,hv", I.PREFILL_WIDTHS)
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_prefill_width(dtype, hq, hk, hv, T):
    w = I.prefill_width(dtype, hq, hk, hv, T)
    plan = qk.describe_plan(0, hq, hk, T, dtype, 1, ld=w.ld)
    print(f"[case] fused prefill {dtype} T={T} {hq}/{hk}/{hv} plan: {plan}", flush=True)
    inp = I.make_inputs(w)
    src = Guarded(inp.qkv, seed=11)
    canvas = np.random.default_rng(12).integers(0, 0x7F, inp.qkv.shape).astype(inp.qkv.dtype)
    dst = Guarded(canvas, seed=13)
    x, y = src.view(), dst.view()
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    qk.qknorm_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, 1, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    out = dst.host()
    assert src.guards_intact() and dst.guards_intact()
    assert np.array_equal(src.host(), inp.qkv)
    assert np.array_equal(out[:, hq + hk:].view(np.uint8), canvas[:, hq + hk:].view(np.uint8))
    rows = np.arange(T) if T <= 1024 else np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(hq + hk).choice(T, 126, replace=False)]))
    ref = oracle.qknorm_fused(inp.q[rows], inp.k[rows], inp.gamma_q, inp.gamma_k, dtype, w.eps, 1)
    got_q, got_k = out[rows, :hq], out[rows, hq:hq + hk]
    if dtype == "bf16":
        check_bf16(got_q, ref.yq_bits, "Q")
        check_bf16(got_k, ref.yk_bits, "K")
    elif dtype == "fp8":
        check_fp8(got_q, ref.yq_bits, "Q")
        check_fp8(got_k, ref.yk_bits, "K")
    else:
        check_f32(got_q, ref.yq, "Q")
        check_f32(got_k, ref.yk, "K")


@pytest.mark.parametrize("T", [1024, 8192])
@pytest.mark.parametrize("hq,hk,hv", I.PREFILL_WIDTHS)
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_prefill_width_headwise(dtype, hq, hk, hv, T):
    head_dim = 128
    w = I.prefill_width(dtype, hq, hk, hv, T)
    plan = qk.describe_headwise_plan(hq, hk, T, head_dim, dtype, 0, ld=w.ld)
    print(f"[case] headwise prefill {dtype} T={T} {hq}/{hk}/{hv} plan: {plan}", flush=True)
    inp = I.make_inputs(w)
    src = Guarded(inp.qkv, seed=21)
    canvas = np.random.default_rng(22).integers(0, 0x7F, inp.qkv.shape).astype(inp.qkv.dtype)
    dst = Guarded(canvas, seed=23)
    x, y = src.view(), dst.view()
    gq = np_to_torch(inp.gamma_q[:head_dim].copy()).to(DEV)
    gk = np_to_torch(inp.gamma_k[:head_dim].copy()).to(DEV)
    qk.qknorm_headwise(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, head_dim, 0, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    out = dst.host()
    assert src.guards_intact() and dst.guards_intact()
    assert np.array_equal(src.host(), inp.qkv)
    assert np.array_equal(out[:, hq + hk:].view(np.uint8), canvas[:, hq + hk:].view(np.uint8))
    rows = np.arange(T) if T <= 1024 else np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(hq + hk + 1).choice(T, 126, replace=False)]))
    ref = oracle.qknorm_headwise(inp.q[rows], inp.k[rows], inp.gamma_q[:head_dim], inp.gamma_k[:head_dim], dtype,
                                 w.eps, head_dim, 0)
    got_q, got_k = out[rows, :hq], out[rows, hq:hq + hk]
    if dtype == "bf16":
        check_bf16(got_q, ref.yq_bits, "Q")
        check_bf16(got_k, ref.yk_bits, "K")
    elif dtype == "fp8":
        check_fp8(got_q, ref.yq_bits, "Q")
        check_fp8(got_k, ref.yk_bits, "K")
    else:
        check_f32(got_q, ref.yq, "Q")
        check_f32(got_k, ref.yk, "K")

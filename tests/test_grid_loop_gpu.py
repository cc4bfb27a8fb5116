"""Blocks that loop over several token groups: with QKNORM_MAX_GRID capping
the grid far below the number of token groups, every block runs its token
loop many times (the LDS double buffer alternating, tokens past the end on
the last pass). Results must equal, bit for bit, the same calls with one
token group per block, for each layout: several waves per token, one-wave
tokens four to a block, several tokens per wave, the split path and both
headwise kernels."""

import os

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, check_bf16, np_to_torch, torch_to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    os.environ.pop("QKNORM_MAX_GRID", None)
    torch.cuda.synchronize()


def _run(cap, fn):
    if cap:
        os.environ["QKNORM_MAX_GRID"] = str(cap)
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        os.environ.pop("QKNORM_MAX_GRID", None)
    return [torch_to_np(o) for o in out]


@pytest.mark.parametrize("T,hq,hk,dtype,shards", [
    (1031, 5120, 1024, "bf16", 1),     # 4 waves per token, LDS exchange
    (1029, 1280, 256, "bf16", 1),      # one-wave tokens, four to a block
    (1500, 640, 128, "bf16", 1),       # 32 lanes per token, 8 tokens per block
    (999, 2048, 512, "fp8", 4),        # FP8, four shards in one wave (few tokens: one slot)
    (777, 1024, 256, "f32", 2),        # fp32, two shards over two waves
])
def test_looping_blocks_equal_one_group_per_block(T, hq, hk, dtype, shards):
    inp = I.make_custom(T, hq, hk, 0, dtype, seed=T + hq)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)

    def calls():
        fq, fk = torch.empty_like(xq), torch.empty_like(xk)
        qk.qknorm_fused(xq, xk, gq, gk, 1e-6, shards, fq, fk)
        part = qk.qknorm_partial_stats(xq, xk, shards)
        aq, ak = torch.empty_like(xq), torch.empty_like(xk)
        qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, hq, hk, aq, ak)
        return fq, fk, part, aq, ak

    plan = qk.describe_plan(0, hq, hk, T, dtype, shards)
    tpb = int(plan.split("tokens/block=")[1].split()[0])
    cap = 7                                   # far fewer blocks than token groups
    assert -(-T // tpb) > 20 * cap
    print(f"[case] grid loop T={T} {dtype} S={shards} plan: {plan}; cap {cap}", flush=True)
    base = _run(0, calls)
    looped = _run(cap, calls)
    for a, b in zip(base, looped):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    if dtype == "bf16":
        ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, dtype, 1e-6, shards)
        check_bf16(looped[0], ref.yq_bits, "looped Q")


@pytest.mark.parametrize("head_dim", [128, 72])    # token-wide and per-head kernels
def test_looping_blocks_headwise(head_dim):
    T, hq, hk = 1201, 16 * head_dim, 4 * head_dim
    inp = I.make_custom(T, hq, hk, 0, "bf16", seed=77 + head_dim)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q[:head_dim].copy()).to(DEV), np_to_torch(inp.gamma_k[:head_dim].copy()).to(DEV)

    def calls():
        oq, ok = torch.empty_like(xq), torch.empty_like(xk)
        qk.qknorm_headwise(xq, xk, gq, gk, 1e-6, head_dim, 0, oq, ok)
        return oq, ok

    base = _run(0, calls)
    looped = _run(5, calls)
    for a, b in zip(base, looped):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))

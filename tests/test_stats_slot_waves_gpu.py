"""partial_stats in the slot-wave form (one shard of packed rows, tokens of
32 or 64 lanes, 2 to 4 chunks per lane: a chunk per thread in row order, the
chunk sums exchanged in LDS, XCD-ordered runs of blocks). Its sums must be
the fused kernel's, bit for bit: fused(S = 1) == partial_stats + apply for
every shape below, and the partial sums match the float64 oracle (Phase A
of the SwiftQK paper) within 1e-5. Shapes cover both token widths, 2, 3 and
4 slots, an idle slot, every row type and token counts that leave a partial
block and a partial run of blocks; the same widths in separate Q and K
arrays take the general kernel and must agree the same way."""

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, np_to_torch, torch_to_np

pytestmark = pytest.mark.gpu

CASES = [
    # T, hq, hk, dtype, packed rows (separate Q and K arrays take the general kernel)
    (16384 + 37, 1280, 256, "bf16", True),   # the rank slice's widths; 37 tokens past the last run of 1024
    (1025, 1280, 256, "fp8", True),          # two tokens per block, the last block's second token absent
    (4097, 512, 256, "f32", True),           # fp32 rows, 64 lanes x 3
    (3000, 768, 256, "bf16", True),          # 32 lanes x 4
    (2500, 1536, 512, "bf16", True),         # 64 lanes x 4
    (2049, 768, 256, "fp8", True),           # 32 lanes x 2
    (1999, 1280, 248, "bf16", True),         # 191 chunks over 64 lanes x 3: one idle slot
    (1025, 1280, 256, "fp8", False),
    (3000, 768, 256, "bf16", False),
    (1999, 1280, 248, "bf16", False),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _operands(inp, packed):
    """Device Q and K views: one packed buffer [T, hq + hk + 64] or two arrays."""
    T, hq, hk = inp.q.shape[0], inp.q.shape[1], inp.k.shape[1]
    if not packed:
        return np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    host = np.zeros((T, hq + hk + 64), inp.q.dtype)
    host[:, :hq] = inp.q
    host[:, hq:hq + hk] = inp.k
    x = np_to_torch(host).to(DEV)
    return x[:, :hq], x[:, hq:hq + hk]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_slot_wave_partials_equal_the_fused_sums(case):
    T, hq, hk, dtype, packed = case
    plan = qk.describe_plan(1, hq, hk, T, dtype, 1, ld=hq + hk + 64)   # the packed layout
    print(f"[case] slot waves {case} packed-rows plan: {plan}", flush=True)
    assert "form=slot-waves" in plan
    inp = I.make_custom(T, hq, hk, 0, dtype, seed=T + hq + hk)
    xq, xk = _operands(inp, packed)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    fq, fk = torch.empty(xq.shape, dtype=xq.dtype, device=DEV), torch.empty(xk.shape, dtype=xk.dtype, device=DEV)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 1, fq, fk)
    part = qk.qknorm_partial_stats(xq, xk, 1)
    aq, ak = torch.empty_like(fq), torch.empty_like(fk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, hq, hk, aq, ak)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_np(fq).view(np.uint8), torch_to_np(aq).view(np.uint8))
    assert np.array_equal(torch_to_np(fk).view(np.uint8), torch_to_np(ak).view(np.uint8))
    ref = oracle.qknorm_partial_stats(inp.q, inp.k, dtype, 1)
    got = part.cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    assert np.all(np.abs(got - ref) <= 1e-5 * ref)

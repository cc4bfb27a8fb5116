"""The grid-loop cases shared by tests/test_grid_loop_gpu.py and its child
process: each runs the library calls of one shape and returns the outputs
as host arrays."""

import torch

import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, np_to_torch, torch_to_np

ROW_CASES = [
    (1031, 5120, 1024, "bf16", 1),     # 4 waves per token, LDS exchange
    (1029, 1280, 256, "bf16", 1),      # one-wave tokens, four to a block
    (1500, 640, 128, "bf16", 1),       # 32 lanes per token, 8 tokens per block
    (999, 2048, 512, "fp8", 4),        # FP8, four shards in one wave (few tokens: one slot)
    (777, 1024, 256, "f32", 2),        # fp32, two shards over two waves
    (1501, 1280, 256, "fp8", 1),       # FP8 32-lane tokens; partial_stats in the slot-wave form
]
HEAD_CASES = [128, 72]                 # token-wide and per-head kernels


def row_inputs(T, hq, hk, dtype):
    return I.make_custom(T, hq, hk, 0, dtype, seed=T + hq)


def run_row_case(T, hq, hk, dtype, shards):
    inp = row_inputs(T, hq, hk, dtype)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    fq, fk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, shards, fq, fk)
    part = qk.qknorm_partial_stats(xq, xk, shards)
    aq, ak = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, hq, hk, aq, ak)
    torch.cuda.synchronize()
    return [torch_to_np(o) for o in (fq, fk, part, aq, ak)]


def head_inputs(head_dim):
    T, hq, hk = 1201, 16 * head_dim, 4 * head_dim
    return I.make_custom(T, hq, hk, 0, "bf16", seed=77 + head_dim)


def run_head_case(head_dim):
    inp = head_inputs(head_dim)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq = np_to_torch(inp.gamma_q[:head_dim].copy()).to(DEV)
    gk = np_to_torch(inp.gamma_k[:head_dim].copy()).to(DEV)
    oq, ok = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_headwise(xq, xk, gq, gk, 1e-6, head_dim, 0, oq, ok)
    torch.cuda.synchronize()
    return [torch_to_np(o) for o in (oq, ok)]

"""Randomized parity sweep (fixed seed, so every run checks the same cases):
shapes, dtypes, shard counts, token counts, row strides, base offsets, in
place or out of place, for the fused call, the split path and the headwise
call, each against the float64 oracle with the usual acceptance, plus V
columns and guard bands untouched. The planner picks a different layout for
many of these shapes (lane groups from 4 to 1024 threads, 1 to 16 slots,
several tokens per wave, the element-wise path)."""

import os

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, Guarded, check_bf16, check_f32, check_fp8, np_to_torch

pytestmark = pytest.mark.gpu

# 120 cases by default; QKNORM_RANDOM_CASES=n runs the first n (cases past the
# 120th also draw 16, 32 and 64 shards), for occasional longer sweeps.
N_CASES = int(os.environ.get("QKNORM_RANDOM_CASES", "120"))
VW = {"bf16": 8, "f32": 4, "fp8": 16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = ["bf16", "f32", "fp8"][rng.integers(0, 3)]
    op = ["fused", "split", "headwise"][rng.integers(0, 3)]
    vw = VW[dtype]
    if op == "headwise":
        head_dim = int(rng.choice([8, 16, 32, 64, 72, 96, 128, 256]))
        hq, hk = head_dim * int(rng.integers(1, 20)), head_dim * int(rng.integers(1, 8))
        shards = 1
    else:
        shards = int(rng.choice([1, 1, 2, 3, 4, 8] if i < 120 else [1, 2, 4, 8, 16, 32, 64]))
        chunky = rng.random() < 0.7          # whole 16-byte chunks per shard, usually
        q_s = int(rng.integers(1, 700)) * (vw if chunky else 1)
        k_s = int(rng.integers(1, 200)) * (vw if chunky else 1)
        if shards >= 16:  # narrower shards, so that most of these rows fit a block
            q_s, k_s = max(1, q_s // (shards // 4)), max(1, k_s // (shards // 4))
        hq, hk, head_dim = q_s * shards, k_s * shards, 0
    T = int(rng.choice([1, 2, 7, 64, 100, 513, 1024, 1031, 2000, 3001]))
    while T * (hq + hk) > 3_000_000:
        T = max(1, T // 2)
    hv = int(rng.choice([0, 0, vw, 3 * vw, 1]))
    ld_pad = int(rng.choice([0, 0, 0, 1, vw]))
    offset = int(rng.choice([0, 0, 0, 1, 3]))
    in_place = bool(rng.random() < 0.25)
    return dict(dtype=dtype, op=op, shards=shards, hq=hq, hk=hk, head_dim=head_dim, T=T, hv=hv, ld_pad=ld_pad,
                offset=offset, in_place=in_place, seed=7000 + i)


# Launches of several thousand tokens, where the planner's loop, residency and
# register rules take effect (FP8 blocks over 2-4 token groups with gamma in
# registers, FP8 headwise blocks over 2 groups, GQA-shaped bf16 launches at
# 5 blocks per CU): 16 seeded cases of the GQA-like and rank-slice widths and
# random ones, at token counts that leave the last block's loop short.
N_LARGE = 16
LARGE_WIDTHS = ((5120, 1024), (4096, 1024), (2048, 512), (1280, 256), (3072, 1024))


def _large_case(i):
    rng = np.random.default_rng(9000 + i)
    dtype = ["bf16", "fp8", "fp8", "f32"][rng.integers(0, 4)]
    op = ["fused", "split", "headwise"][rng.integers(0, 3)]
    vw = VW[dtype]
    hq, hk = LARGE_WIDTHS[int(rng.integers(0, len(LARGE_WIDTHS)))]
    if rng.random() < 0.25:
        hq, hk = int(rng.integers(8, 400)) * vw, int(rng.integers(2, 100)) * vw
        hq, hk = hq - hq % 128 or 128, hk - hk % 128 or 128
    T = int(rng.choice([4097, 5000, 6144, 6500, 8191]))
    if i == 0:  # the GQA prefill shape at a ragged token count: the residency cap
        dtype, op, hq, hk, T = "bf16", "fused", 5120, 1024, 6500
    return dict(dtype=dtype, op=op, shards=1, hq=hq, hk=hk, head_dim=128 if op == "headwise" else 0, T=T,
                hv=int(rng.choice([0, 128])), ld_pad=0, offset=int(rng.choice([0, 0, 3])),
                in_place=bool(rng.random() < 0.25), seed=9000 + i)


def large_cases():
    return [_large_case(i) for i in range(N_LARGE)]


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_token_case(i):
    c = _large_case(i)
    if c["op"] == "headwise":
        plan = qk.describe_headwise_plan(c["hq"], c["hk"], c["T"], 128, c["dtype"], 0, ld=c["hq"] + c["hk"] + c["hv"])
    else:
        plan = qk.describe_plan(0 if c["op"] == "fused" else 2, c["hq"], c["hk"], c["T"], c["dtype"], 1,
                                ld=c["hq"] + c["hk"] + c["hv"])
    print(f"[case] large {i}: {c} plan: {plan}", flush=True)
    _run(c, f"large {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    _run(_case(i), str(i))


def _run(c, i):
    dtype, op, S, hq, hk, T = c["dtype"], c["op"], c["shards"], c["hq"], c["hk"], c["T"]
    inp = I.make_custom(T, hq, hk, 0, dtype, seed=c["seed"])
    ld = hq + hk + c["hv"] + c["ld_pad"]
    host = np.zeros((T, ld), dtype=inp.q.dtype)
    host[:, :hq] = inp.q
    host[:, hq:hq + hk] = inp.k
    rng = np.random.default_rng(c["seed"] + 1)
    if ld > hq + hk:
        fill = rng.integers(0, 0x7F, (T, ld - hq - hk)) if dtype != "f32" else rng.standard_normal((T, ld - hq - hk))
        host[:, hq + hk:] = fill.astype(host.dtype)
    src = Guarded(host, seed=c["seed"], offset_elems=c["offset"])
    dst = src if c["in_place"] else Guarded(host, seed=c["seed"] + 2, offset_elems=c["offset"])
    before = dst.host().copy()
    x, y = src.view(), dst.view()
    xq, xk, yq, yk = x[:, :hq], x[:, hq:hq + hk], y[:, :hq], y[:, hq:hq + hk]
    print(f"[case] {i}: {c}", flush=True)
    try:
        ref = _call_and_oracle(c, inp, xq, xk, yq, yk)
    except qk.QKNormError as e:       # a row wider than the kernels hold: refused, nothing written
        assert e.status == 2, e
        torch.cuda.synchronize()
        assert np.array_equal(dst.host().view(np.uint8), before.view(np.uint8))
        return
    torch.cuda.synchronize()
    out = dst.host()
    if dtype == "bf16":
        check_bf16(out[:, :hq], ref.yq_bits, f"case {i} Q")
        check_bf16(out[:, hq:hq + hk], ref.yk_bits, f"case {i} K")
    elif dtype == "fp8":
        check_fp8(out[:, :hq], ref.yq_bits, f"case {i} Q")
        check_fp8(out[:, hq:hq + hk], ref.yk_bits, f"case {i} K")
    else:
        check_f32(out[:, :hq], ref.yq, f"case {i} Q")
        check_f32(out[:, hq:hq + hk], ref.yk, f"case {i} K")
    assert np.array_equal(out[:, hq + hk:].view(np.uint8), before[:, hq + hk:].view(np.uint8))
    assert src.guards_intact() and dst.guards_intact()
    if not c["in_place"]:
        assert np.array_equal(src.host().view(np.uint8), host.view(np.uint8))


def _call_and_oracle(c, inp, xq, xk, yq, yk):
    dtype, op, S, hq, hk = c["dtype"], c["op"], c["shards"], c["hq"], c["hk"]
    if op == "headwise":
        hd = c["head_dim"]
        gq_h, gk_h = inp.gamma_q[:hd].copy(), inp.gamma_k[:hd].copy()
        qk.qknorm_headwise(xq, xk, np_to_torch(gq_h).to(DEV), np_to_torch(gk_h).to(DEV), 1e-6, hd, 0, yq, yk)
        ref = oracle.qknorm_headwise(inp.q, inp.k, gq_h, gk_h, dtype, 1e-6, hd, 0)
    else:
        gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
        if op == "fused":
            qk.qknorm_fused(xq, xk, gq, gk, 1e-6, S, yq, yk)
        else:
            part = qk.qknorm_partial_stats(xq, xk, S)
            qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, hq, hk, yq, yk)
        ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, dtype, 1e-6, S)
    return ref

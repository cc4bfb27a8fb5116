"""Blocks that loop over several token groups: with QKNORM_MAX_GRID capping
the grid far below the number of token groups, every block runs its token
loop many times (the LDS double buffer alternating, tokens past the end on
the last pass). Results must equal, bit for bit, the same calls with one
token group per block, for each layout: several waves per token, one-wave
tokens four to a block, several tokens per wave, the split path and both
headwise kernels.

The library reads the cap once per process, so the capped calls run in one
child process (tests/grid_cap_child.py) started with the variable set; this
process makes the uncapped calls and compares."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from gpu_helpers import check_bf16
from grid_cases import HEAD_CASES, ROW_CASES, row_inputs, run_head_case, run_row_case

pytestmark = pytest.mark.gpu

CAP = 7   # far fewer blocks than token groups
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def capped(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert "QKNORM_MAX_GRID" not in os.environ, "the uncapped calls need the variable unset"
    qk.load_library()
    out = str(tmp_path_factory.mktemp("gridcap") / "capped.npz")
    env = dict(os.environ, QKNORM_MAX_GRID=str(CAP))
    print(f"[case] grid loop: child process with QKNORM_MAX_GRID={CAP}", flush=True)
    res = subprocess.run([sys.executable, "-u", os.path.join(HERE, "grid_cap_child.py"), out], env=env,
                         capture_output=True, text=True, timeout=300)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0, f"child process failed ({res.returncode})"
    with np.load(out) as d:
        return {k: d[k] for k in d.files}


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "_".join(map(str, c)))
def test_looping_blocks_equal_one_group_per_block(case, capped):
    T, hq, hk, dtype, shards = case
    plan = qk.describe_plan(0, hq, hk, T, dtype, shards)
    tpb = int(plan.split("tokens/block=")[1].split()[0])
    assert -(-T // tpb) > 20 * CAP
    print(f"[case] grid loop T={T} {dtype} S={shards} plan: {plan}; cap {CAP}", flush=True)
    base = run_row_case(*case)
    for n, a in enumerate(base):
        assert np.array_equal(a.view(np.uint8), capped[f"rows_{'_'.join(map(str, case))}_{n}"])
    if dtype == "bf16":
        inp = row_inputs(T, hq, hk, dtype)
        ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, dtype, 1e-6, shards)
        looped_q = capped[f"rows_{'_'.join(map(str, case))}_0"].view(np.uint16).reshape(T, hq)
        check_bf16(looped_q, ref.yq_bits, "looped Q")


@pytest.mark.parametrize("head_dim", HEAD_CASES)
def test_looping_blocks_headwise(head_dim, capped):
    print(f"[case] grid loop headwise head_dim={head_dim}; cap {CAP}", flush=True)
    base = run_head_case(head_dim)
    for n, a in enumerate(base):
        assert np.array_equal(a.view(np.uint8), capped[f"heads_{head_dim}_{n}"])

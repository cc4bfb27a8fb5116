"""Child process of tests/test_grid_loop_gpu.py: runs the grid-loop cases
with QKNORM_MAX_GRID already set in its environment (the library reads the
cap once per process) and writes every output's bytes to an .npz file.

    QKNORM_MAX_GRID=7 python tests/grid_cap_child.py OUT.npz
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import numpy as np  # noqa: E402
import torch  # noqa: E402

from grid_cases import HEAD_CASES, ROW_CASES, run_head_case, run_row_case  # noqa: E402


def main(out):
    res = {}
    for case in ROW_CASES:
        print(f"[child] cap {os.environ.get('QKNORM_MAX_GRID')} rows {case}", flush=True)
        for n, a in enumerate(run_row_case(*case)):
            res[f"rows_{'_'.join(map(str, case))}_{n}"] = a.view(np.uint8)
    for head_dim in HEAD_CASES:
        print(f"[child] cap {os.environ.get('QKNORM_MAX_GRID')} heads {head_dim}", flush=True)
        for n, a in enumerate(run_head_case(head_dim)):
            res[f"heads_{head_dim}_{n}"] = a.view(np.uint8)
    torch.cuda.synchronize()
    np.savez(out, **res)
    print("[child] done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])

"""The streaming ceiling kernels (libstreamceil.so, the benchmark's plain
copy and read of the bytes a call moves): the copy writes exactly the
selected leading bytes of every row, unchanged, for every launch shape the
benchmark sweeps (including the XCD-ordered runs and the non-temporal
loads), and leaves the rest of the rows alone; bad arguments are refused
before any launch."""

import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ceil():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    return bench, bench.CeilingLib()


@pytest.mark.parametrize("rows,row_bytes,ld", [(1000, 3072, 3584), (333, 12288, 14336), (1, 4096, 4096)])
def test_copy_moves_exactly_the_row_prefixes(ceil, rows, row_bytes, ld):
    bench, lib = ceil
    x = torch.randint(0, 255, (rows, ld), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for per, block, xk, ntl in bench.CEIL_CONFIGS:
        print(f"[case] copy rows={rows} row_bytes={row_bytes} per={per} block={block} xcd_run={xk} nt_loads={ntl}",
              flush=True)
        y = torch.full_like(x, 7)
        lib.stream(x.data_ptr(), ld, y.data_ptr(), ld, rows, row_bytes, per, block, xk, ntl, sink.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(y[:, :row_bytes], x[:, :row_bytes])
        assert bool((y[:, row_bytes:] == 7).all())


def test_read_writes_nothing_and_bad_arguments_are_refused(ceil):
    bench, lib = ceil
    x = torch.ones(64, 1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    lib.stream(x.data_ptr(), 1024, None, 0, 64, 1024, 1, 512, 16, 1, sink.data_ptr(), st)
    torch.cuda.synchronize()
    assert bool((x == 1).all())
    with pytest.raises(RuntimeError):
        lib.stream(x.data_ptr(), 1024, None, 0, 64, 1024, 1, 512, 3, 0, sink.data_ptr(), st)   # xcd_run
    with pytest.raises(RuntimeError):
        lib.stream(x.data_ptr(), 1024, None, 0, 64, 1024, 1, 512, 0, 2, sink.data_ptr(), st)   # nt_loads
    with pytest.raises(RuntimeError):
        lib.stream(x.data_ptr(), 1024, None, 0, 64, 1000, 1, 512, 0, 0, sink.data_ptr(), st)   # row_bytes % 16

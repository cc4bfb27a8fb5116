"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (stand-in device
addresses are only compared, never dereferenced)."""

import ctypes
import os
import re
import subprocess

import pytest

import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd.binding import (EXPORTS, OP_APPLY_WITH_STATS, OP_FUSED,
                                                  OP_PARTIAL_STATS, Operand)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qknorm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qk.library_path()),
                                reason="libqknorm.so not built (run __graft_entry__.build())")

INVALID, UNSUPPORTED = 1, 2
BF16, F32 = 1, 0


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qknorm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_calls():
    assert declared_functions() == sorted(EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = qk.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qk.library_path()], capture_output=True,
                         text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_block_clocks_only_in_the_timing_build():
    """The block-clock hook exists only in the timing-only twin that
    bench.py --timeline loads; the library the boundary ships has none, and
    both export the same calls otherwise."""
    from layerwise_qk_norm_qknorm_amd import build_lib
    if not os.path.exists(build_lib.CLOCKS_LIB):
        pytest.skip("libqknorm_clocks.so not built")

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
        return {l.split()[-1] for l in out.splitlines() if " T " in l}

    product, timing = exported(qk.library_path()), exported(build_lib.CLOCKS_LIB)
    assert "qknorm_set_block_clocks" not in product
    assert timing - product == {"qknorm_set_block_clocks"}
    for name in declared_functions():
        assert name in timing, name


def test_abi_version():
    assert qk.abi_version() == 3


# stand-in addresses: packed rows, outputs elsewhere
BASE, YOFF, GQ, GK, STATS = 1 << 32, 1 << 44, 1 << 46, (1 << 46) + (1 << 30), 1 << 48


def ops(hq=256, hk=128, ld=None, esz=2, y_same=False, off=0):
    ld = ld if ld is not None else hq + hk
    q = Operand(BASE + off, ld, (BASE if y_same else BASE + YOFF) + off, ld, GQ, hq)
    k = Operand(BASE + off + hq * esz, ld, (BASE if y_same else BASE + YOFF) + off + hq * esz, ld, GK, hk)
    return q, k


def fused(q, k, T=16, dtype=BF16, eps=1e-6, shards=1):
    lib = qk.load_library()
    return lib.qknorm_fused(ctypes.byref(q) if q else None, ctypes.byref(k) if k else None, T, dtype,
                            eps, shards, None)


def partial(q, k, T=16, dtype=BF16, shards=1, buf=STATS):
    lib = qk.load_library()
    return lib.qknorm_partial_stats(ctypes.byref(q), ctypes.byref(k), T, dtype, shards, buf, None)


def apply(q, k, T=16, dtype=BF16, eps=1e-6, buf=STATS, planes=1, hqf=256, hkf=128):
    lib = qk.load_library()
    return lib.qknorm_apply_with_stats(ctypes.byref(q), ctypes.byref(k), T, dtype, eps, buf, planes, hqf,
                                       hkf, None)


def last_error():
    return qk.load_library().qknorm_last_error().decode()


def test_noop_when_T_is_zero():
    q, k = ops()
    q.x = k.x = 0  # pointers are not needed for T == 0
    assert fused(q, k, T=0) == 0 and last_error() == ""
    assert partial(q, k, T=0, buf=0) == 0
    assert apply(q, k, T=0, buf=0) == 0


@pytest.mark.parametrize("case", [
    "null_q", "bad_dtype", "neg_T", "shards0", "shards_big", "shards_indivisible", "eps_neg", "eps_nan",
    "eps_inf", "h0", "ld_small", "ldy_small", "null_x", "null_y", "null_gamma", "yq_overlaps_yk",
    "yq_overlaps_xk", "partial_inplace_shift", "gamma_in_output", "huge_T", "x_misaligned", "y_misaligned",
    "gamma_misaligned",
])
def test_fused_rejects(case):
    q, k = ops()
    kw = {}
    if case == "null_q":
        assert fused(None, k) == INVALID
        return
    if case == "bad_dtype":
        kw["dtype"] = 7
    elif case == "neg_T":
        kw["T"] = -1
    elif case == "shards0":
        kw["shards"] = 0
    elif case == "shards_big":
        kw["shards"] = 65
    elif case == "shards_indivisible":
        kw["shards"] = 3
    elif case == "eps_neg":
        kw["eps"] = -1e-6
    elif case == "eps_nan":
        kw["eps"] = float("nan")
    elif case == "eps_inf":
        kw["eps"] = float("inf")
    elif case == "h0":
        k.h = 0
    elif case == "ld_small":
        q.ld_x = 100
    elif case == "ldy_small":
        k.ld_y = 64
    elif case == "null_x":
        q.x = 0
    elif case == "null_y":
        k.y = 0
    elif case == "null_gamma":
        q.gamma = 0
    elif case == "yq_overlaps_yk":
        k.y = q.y + 100 * 2
    elif case == "yq_overlaps_xk":
        q.y = k.x
        q.ld_y = q.ld_x
    elif case == "partial_inplace_shift":
        q.y = q.x + 2
    elif case == "gamma_in_output":
        q.gamma = q.y + 10 * (q.ld_y * 2)
    elif case == "huge_T":
        kw["T"] = 1 << 62
    elif case == "x_misaligned":          # a bf16 pointer at an odd address
        q.x = q.x + 1
    elif case == "y_misaligned":
        k.y = k.y + 1
    elif case == "gamma_misaligned":
        k.gamma = k.gamma + 1
    assert fused(q, k, **kw) == INVALID, case
    assert last_error().startswith("qknorm_fused:"), last_error()


def test_accepts_packed_in_place_and_out_of_place():
    for y_same in (True, False):
        q, k = ops(hq=5120, hk=1024, ld=7168, y_same=y_same)
        buf = ctypes.create_string_buffer(256)
        lib = qk.load_library()
        assert lib.qknorm_describe_plan(OP_FUSED, ctypes.byref(q), ctypes.byref(k), 8192, BF16, 1, buf, 256) == 0


def test_partial_and_apply_reject():
    q, k = ops()
    assert partial(q, k, buf=0) == INVALID
    assert partial(q, k, buf=q.x) == INVALID                  # partials over the input
    assert apply(q, k, planes=0) == INVALID
    assert apply(q, k, planes=65) == INVALID
    assert apply(q, k, hqf=255) == INVALID                    # full width below local width
    assert apply(q, k, hkf=(1 << 24) + 1) == INVALID
    assert apply(q, k, buf=0) == INVALID
    assert apply(q, k, buf=q.y) == INVALID                    # stats over the output
    assert apply(q, k, eps=-1.0) == INVALID
    assert partial(q, k, buf=STATS + 2) == INVALID            # float32 partials must be 4-byte aligned
    assert apply(q, k, buf=STATS + 1) == INVALID


def test_describe_plans_of_the_workloads():
    # GQA prefill: 768 chunks per token over 256 lanes, 3 each, one token per block
    d = qk.describe_plan(OP_FUSED, 5120, 1024, 8192, "bf16", 1, ld=7168)
    assert "path=16B" in d and "slots=3" in d and "waves/token=4" in d and "tokens/block=1" in d
    # rank slice: 192 chunks over one wave, 3 each, four tokens per block
    d = qk.describe_plan(OP_FUSED, 1280, 256, 16384, "bf16", 1, ld=1792)
    assert "path=16B" in d and "slots=3" in d and "waves/token=1" in d and "tokens/block=4" in d
    # its partial_stats: the same lanes and slots in the slot-wave form (one
    # wave per slot, a chunk per thread, a token per block, runs of 128 tokens
    # per XCD); FP8 rows: two 32-lane tokens per block, runs of 64 blocks
    d = qk.describe_plan(OP_PARTIAL_STATS, 1280, 256, 16384, "bf16", 1, ld=1792)
    assert "lanes/shard=64" in d and "slots=3" in d and "form=slot-waves" in d and "tokens/block=1" in d
    assert "threads/block=192" in d and "xcd_run=128" in d
    d = qk.describe_plan(OP_PARTIAL_STATS, 1280, 256, 16384, "fp8", 1, ld=1792)
    assert "lanes/shard=32" in d and "slots=3" in d and "form=slot-waves" in d and "tokens/block=2" in d
    assert "xcd_run=64" in d
    # a single decode token is spread over 8 waves, two chunks per lane
    d = qk.describe_plan(OP_FUSED, 4096, 4096, 1, "bf16", 1, ld=12288)
    assert "slots=2" in d and "waves/token=8" in d
    d = qk.describe_plan(OP_APPLY_WITH_STATS, 1280, 256, 16384, "bf16", 1, ld=1792)
    assert "apply_with_stats" in d
    d = qk.describe_plan(OP_FUSED, 256, 256, 16, "f32", 2, ld=256)
    assert "f32" in d and "shards=2" in d
    d = qk.describe_plan(OP_FUSED, 512, 128, 16, "bf16", 1, ld=704, aligned=False)
    assert "elementwise" in d
    for T in (1, 8, 64, 256):
        for S in (1, 2, 4, 8):
            qk.describe_plan(OP_FUSED, 4096, 4096, T, "bf16", S, ld=12288)


def test_widest_rows_and_beyond():
    assert "slots=8" in qk.describe_plan(OP_FUSED, 57344, 8192, 4, "bf16", 1, ld=65536)
    with pytest.raises(qk.QKNormError) as e:
        qk.describe_plan(OP_FUSED, 65536, 8, 4, "bf16", 1, ld=65544)
    assert e.value.status == UNSUPPORTED


@pytest.mark.parametrize("dtype,aligned,max_chunks", [
    ("bf16", True, 8192), ("f32", True, 8192), ("fp8", True, 4096),
    ("bf16", False, 4096), ("f32", False, 6144), ("fp8", False, 2048)])
def test_row_width_limit_per_path(dtype, aligned, max_chunks):
    """Q + K chunks per shard: the widest row that plans, and one chunk more
    that is refused as unsupported, with every kernel's slots in registers."""
    vw = {"bf16": 8, "f32": 4, "fp8": 16}[dtype]
    hk = 4 * vw
    pad = 0 if aligned else 1                      # odd row stride: element-wise path
    hq = (max_chunks - 4) * vw
    d = qk.describe_plan(OP_FUSED, hq, hk, 100, dtype, 1, ld=hq + hk + pad)
    assert ("path=16B" if aligned else "elementwise") in d
    with pytest.raises(qk.QKNormError) as e:
        qk.describe_plan(OP_FUSED, hq + vw, hk, 100, dtype, 1, ld=hq + vw + hk + pad)
    assert e.value.status == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qk.qknorm_fused(x[:, :32], x[:, 32:], g, g, 1e-6, 1)


class FakeDevice:
    """A CPU tensor posing as device memory of GPU `index` for the binding's
    checks. Its data pointer is NULL, so anything that got past the binding
    would be refused by the library's own argument check, never launched."""

    def __init__(self, t, index=0):
        self.t, self.index = t, index

    shape = property(lambda self: self.t.shape)
    dtype = property(lambda self: self.t.dtype)
    is_cuda = True

    def stride(self, *a):
        return self.t.stride(*a)

    def dim(self):
        return self.t.dim()

    def is_contiguous(self):
        return self.t.is_contiguous()

    def data_ptr(self):
        return 0

    def get_device(self):
        return self.index

    def __getitem__(self, idx):
        return FakeDevice(self.t[idx], self.index)


def _fake_case(dtype="bf16"):
    import torch
    td = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    x = FakeDevice(torch.zeros(4, 96, dtype=td))
    g = FakeDevice(torch.ones(64, dtype=td))
    return x, g, td


@pytest.mark.parametrize("bad", ["gamma_cpu", "gamma_other_gpu", "out_cpu", "out_other_gpu"])
def test_binding_refuses_host_or_foreign_operands(bad):
    import torch
    x, g, td = _fake_case()
    q, k = x[:, :64], x[:, 64:]
    gk = FakeDevice(torch.ones(32, dtype=td))
    oq = FakeDevice(torch.zeros(4, 64, dtype=td))
    gq = g
    if bad == "gamma_cpu":
        gq = torch.ones(64, dtype=td)
    elif bad == "gamma_other_gpu":
        gq = FakeDevice(torch.ones(64, dtype=td), index=1)
    elif bad == "out_cpu":
        oq = torch.zeros(4, 64, dtype=td)
    else:
        oq = FakeDevice(torch.zeros(4, 64, dtype=td), index=1)
    with pytest.raises(ValueError):
        qk.qknorm_fused(q, k, gq, gk, 1e-6, 1, oq, None)
    with pytest.raises(ValueError):
        qk.qknorm_apply_with_stats(q, k, gq, gk, 1e-6, FakeDevice(torch.zeros(1, 2, 4)), 64, 32, oq, None)


def test_binding_refuses_host_statistics():
    import torch
    x, g, td = _fake_case()
    q, k = x[:, :64], x[:, 64:]
    gk = FakeDevice(torch.ones(32, dtype=td))
    with pytest.raises(ValueError, match="partials"):
        qk.qknorm_partial_stats(q, k, 1, torch.zeros(1, 2, 4))
    with pytest.raises(ValueError, match="partials"):
        qk.qknorm_partial_stats(q, k, 1, FakeDevice(torch.zeros(1, 2, 4), index=1))
    with pytest.raises(ValueError, match="stats"):
        qk.qknorm_apply_with_stats(q, k, g, gk, 1e-6, torch.zeros(1, 2, 4), 64, 32)
    with pytest.raises(ValueError, match="stats"):
        qk.qknorm_apply_with_stats(q, k, g, gk, 1e-6, FakeDevice(torch.zeros(2, 2, 4), index=1), 64, 32)


@pytest.mark.parametrize("where", ["q", "k"])
def test_binding_refuses_host_headwise_gamma(where):
    import torch
    x, _, td = _fake_case()
    q, k = x[:, :64], x[:, 64:]
    good = FakeDevice(torch.ones(32, dtype=td))
    host = torch.ones(32, dtype=td)
    gq, gk = (host, good) if where == "q" else (good, host)
    with pytest.raises(ValueError, match="gamma"):
        qk.qknorm_headwise(q, k, gq, gk, 1e-6, 32, 0)


def test_binding_fake_device_reaches_library_check():
    """The fake operands pass the binding when they are all on one GPU; the
    library then refuses the NULL pointers itself (nothing is launched)."""
    import torch
    x, g, td = _fake_case()
    gk = FakeDevice(torch.ones(32, dtype=td))
    with pytest.raises(qk.QKNormError) as e:
        qk.qknorm_fused(x[:, :64], x[:, 64:], g, gk, 1e-6, 1, stream=0)
    assert e.value.status == INVALID


def headwise(q, k, T=16, dtype=BF16, eps=1e-6, head_dim=64, stride=0):
    lib = qk.load_library()
    return lib.qknorm_headwise(ctypes.byref(q), ctypes.byref(k), T, dtype, eps, head_dim, stride, None)


def test_headwise_rejects():
    q, k = ops(hq=256, hk=128)
    assert headwise(q, k, T=0) == 0
    assert headwise(q, k, head_dim=0) == INVALID
    assert headwise(q, k, head_dim=96) == INVALID          # 256 % 96 != 0
    assert headwise(q, k, stride=-1) == INVALID
    assert headwise(q, k, eps=float("nan")) == INVALID
    assert headwise(q, k, T=-3) == INVALID
    assert headwise(q, k, dtype=5) == INVALID
    q2, k2 = ops(hq=256, hk=128)
    k2.y = q2.y + 64 * 2                                    # K output over Q output
    assert headwise(q2, k2) == INVALID
    q3, k3 = ops(hq=256, hk=128)
    q3.gamma = q3.y                                         # gamma inside an output
    assert headwise(q3, k3) == INVALID
    q4, k4 = ops(hq=256, hk=128)
    k4.x = k4.x + 1                                         # a bf16 input at an odd address
    assert headwise(q4, k4) == INVALID
    assert last_error().startswith("qknorm_headwise:")


def test_headwise_plans():
    # heads of 16 chunks: token-wide layout, 768 chunks over 512 lanes (8 waves, 2 slots), a 16-lane
    # group per head
    d = qk.describe_headwise_plan(5120, 1024, 8192, 128, ld=7168)
    assert "heads=(40,8)" in d and "layout=token-wide" in d and "lanes/head=16" in d and "slots=2" in d
    assert "threads/token=512" in d
    # heads of 18 fp32 chunks (not a power of two): one lane group per head
    d = qk.describe_headwise_plan(576, 144, 33, 72, "f32")
    assert "layout=per-head" in d
    d = qk.describe_headwise_plan(4096, 4096, 1, 128, ld=12288)
    assert "slots=1" in d                                   # one token: one chunk per lane
    d = qk.describe_headwise_plan(36 * 4, 36 * 2, 100, 36)
    assert "elementwise" in d                               # 36 bf16 is not whole 16-byte chunks
    with pytest.raises(qk.QKNormError) as e:
        qk.describe_headwise_plan(8192, 8192, 4, 8192)      # a head wider than a lane group holds
    assert e.value.status == UNSUPPORTED
    with pytest.raises(qk.QKNormError) as e:
        qk.describe_headwise_plan(257 * 8, 8, 4, 8)         # more heads than a block holds
    assert e.value.status == UNSUPPORTED


def test_fp8_plans_and_checks():
    # FP8 rows: 16 elements per 16-byte chunk; GQA prefill is 384 chunks per token
    d = qk.describe_plan(OP_FUSED, 5120, 1024, 8192, "fp8", 1, ld=7168)
    assert "fp8_e4m3" in d and "chunks=(320,64)" in d and "slots=3" in d and "path=16B" in d
    d = qk.describe_plan(OP_FUSED, 5120, 1024, 8192, "fp8", 1, ld=7176)
    assert "elementwise" in d                              # row stride not a multiple of 16
    d = qk.describe_headwise_plan(5120, 1024, 8192, 128, "fp8", ld=7168)
    assert "chunks/head=8" in d and "layout=token-wide" in d
    q, k = ops(hq=256, hk=128, esz=1)
    buf = ctypes.create_string_buffer(256)
    lib = qk.load_library()
    assert lib.qknorm_describe_plan(OP_FUSED, ctypes.byref(q), ctypes.byref(k), 16, 2, 1, buf, 256) == 0
    q.y = q.x + 1                                          # partial in-place shift by one FP8 element
    assert fused(q, k, dtype=2) == INVALID


def test_error_message_is_per_thread():
    """Each thread reads the message of its own last call (the library keeps one
    per thread): two threads fail differently, many times, interleaved."""
    import threading
    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, kind, n=200):
        q, k = ops()
        msgs = set()
        barrier.wait()
        for _ in range(n):
            if kind == "shards":
                rc = fused(q, k, shards=0)
            else:
                rc = fused(q, k, eps=-1.0)
            assert rc == INVALID
            msgs.add(last_error())
        seen[name] = msgs

    ts = [threading.Thread(target=worker, args=("a", "shards")), threading.Thread(target=worker, args=("b", "eps"))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert len(seen["a"]) == 1 and len(seen["b"]) == 1
    (ma,), (mb,) = seen["a"], seen["b"]
    assert ma != mb and "shard" in ma.lower() and "eps" in mb.lower()
    # a successful call clears this thread's message
    q, k = ops()
    q.x = k.x = 0
    assert fused(q, k, T=0) == 0 and last_error() == ""


def test_prepared_calls_refuse_host_tensors():
    """The prepared calls run the binding's checks once, when prepared: a
    host tensor is refused there, before any library call."""
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qk.prepare_fused(x[:, :32], x[:, 32:], g, g, 1e-6, 1)
    with pytest.raises(ValueError):
        qk.prepare_partial_stats(x[:, :32], x[:, 32:], 1, torch.zeros(1, 2, 4))
    with pytest.raises(ValueError):
        qk.prepare_apply_with_stats(x[:, :32], x[:, 32:], g, g, 1e-6, torch.zeros(1, 2, 4), 32, 32)


def test_prepared_fused_reaches_the_library_check():
    """A prepared call whose tensors pass the binding's checks (device
    stand-ins with NULL data) is refused by the library when called, with
    nothing launched."""
    x, g, _ = _fake_case()
    call = qk.prepare_fused(x[:, :32], x[:, 32:64], g[:32], g[32:64], 1e-6, 1)
    with pytest.raises(qk.QKNormError) as e:
        call(stream=0)
    assert e.value.status == INVALID

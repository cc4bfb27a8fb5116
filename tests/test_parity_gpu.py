"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle,
element by element, on the seeded synthetic workloads and on edge cases.

Acceptance (written here, applied to every element):
  * float32 I/O: |gpu - oracle| <= 1e-5 |oracle|;
  * bf16 I/O:    the GPU bf16 result is the oracle's once-rounded bf16 result
                 or one of its two neighbours.
Plus bitwise properties: V columns and guard bands untouched, in place ==
out of place, run-to-run determinism, fused == partial_stats + apply.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import (DEV, Guarded, check_bf16, check_f32, check_fp8, fig2b_errors, np_to_torch,
                         torch_to_np)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    _log(f"[gpu] {torch.cuda.get_device_name(0)} lib={qk.library_path()}")
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------------------- runners
def _canvas(like, seed):
    """Random canary bits of the shape and type of `like`."""
    rng = np.random.default_rng(seed)
    if like.dtype == np.uint16:
        return rng.integers(0, 1 << 16, like.shape, dtype=np.uint32).astype(np.uint16)
    return rng.standard_normal(like.shape).astype(np.float32)


class Packed:
    """Device copy of a workload's inputs in its own layout, plus an output
    buffer of the same layout full of canary bits."""

    def __init__(self, inp, seed=1, out_of_place=True):
        w = inp.workload
        self.w = w
        self.inp = inp
        if w.packed:
            self.src = Guarded(inp.qkv, seed=seed)
            self.dst = Guarded(_canvas(inp.qkv, seed + 100), seed=seed + 3) if out_of_place else None
            x = self.src.view()
            self.q, self.k = x[:, :w.hq], x[:, w.hq:w.hq + w.hk]
            if out_of_place:
                y = self.dst.view()
                self.oq, self.ok = y[:, :w.hq], y[:, w.hq:w.hq + w.hk]
            else:
                self.oq, self.ok = self.q, self.k
        else:
            self.srcq, self.srck = Guarded(inp.q, seed=seed), Guarded(inp.k, seed=seed + 1)
            self.q, self.k = self.srcq.view(), self.srck.view()
            if out_of_place:
                self.dstq = Guarded(np.zeros_like(inp.q), seed=seed + 2)
                self.dstk = Guarded(np.zeros_like(inp.k), seed=seed + 3)
                self.oq, self.ok = self.dstq.view(), self.dstk.view()
            else:
                self.oq, self.ok = self.q, self.k
        self.gq = np_to_torch(inp.gamma_q).to(DEV)
        self.gk = np_to_torch(inp.gamma_k).to(DEV)

    def fused(self, shards):
        qk.qknorm_fused(self.q, self.k, self.gq, self.gk, self.w.eps, shards, self.oq, self.ok)
        torch.cuda.synchronize()
        return torch_to_np(self.oq), torch_to_np(self.ok)

    def untouched_outside_qk(self):
        """V columns of the output (packed) and every guard band are unchanged."""
        w = self.w
        if w.packed:
            ok = self.src.guards_intact()
            if hasattr(self, "dst") and self.dst is not None:
                ok = ok and self.dst.guards_intact()
                init = self.dst.initial[self.dst.offset:self.dst.offset + self.dst.n].reshape(self.dst.shape)
                now = self.dst.host()
                ok = ok and np.array_equal(now[:, w.hq + w.hk:].view(np.uint8), init[:, w.hq + w.hk:].view(np.uint8))
            # the input V columns too
            now_in = self.src.host()
            ok = ok and np.array_equal(now_in[:, w.hq + w.hk:], self.inp.qkv[:, w.hq + w.hk:])
            return ok
        bufs = [self.srcq, self.srck] + ([self.dstq, self.dstk] if hasattr(self, "dstq") else [])
        return all(b.guards_intact() for b in bufs)


def _compare(w, got_q, got_k, ref, what):
    if w.dtype == "bf16":
        eq, _ = check_bf16(got_q, ref.yq_bits, what + " Q")
        ek, _ = check_bf16(got_k, ref.yk_bits, what + " K")
        gq = oracle.bf16_bits_to_f64(got_q)
        e = fig2b_errors(gq, ref.yq)
        _log(f"[parity] {what}: exact bf16 match Q {eq:.5f} K {ek:.5f}; vs fp64 gold Q max/mean/rms "
             f"{e[0]:.3g}/{e[1]:.3g}/{e[2]:.3g}")
        return min(eq, ek)
    rq = check_f32(got_q, ref.yq, what + " Q")
    rk = check_f32(got_k, ref.yk, what + " K")
    _log(f"[parity] {what}: max rel err Q {rq:.3g} K {rk:.3g}")
    return None


def _run_fused_case(w, shards, out_of_place=True):
    _log(f"[case] fused {w.key} T={w.T} hq={w.hq} hk={w.hk} {w.dtype} S={shards} "
         f"plan: {qk.describe_plan(0, w.hq, w.hk, w.T, w.dtype, shards, ld=w.ld if w.packed else w.hq)}")
    inp = I.make_inputs(w)
    dev = Packed(inp, out_of_place=out_of_place)
    got_q, got_k = dev.fused(shards)
    ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, w.dtype, w.eps, shards)
    _compare(w, got_q, got_k, ref, f"{w.key} S={shards}")
    assert dev.untouched_outside_qk(), "write outside the Q/K columns"
    return dev, ref


# ----------------------------------------------------------------------- the five workloads
def test_tiny_fp32():
    _run_fused_case(I.TINY, 2)


@pytest.mark.parametrize("shards", [1, 4])
def test_small_dense(shards):
    _run_fused_case(I.SMALL_DENSE, shards)


@pytest.mark.parametrize("shards", [1, 2, 4, 8])
@pytest.mark.parametrize("idx", range(4))
def test_decode(idx, shards):
    _run_fused_case(I.DECODE[idx], shards)


def test_gqa_prefill_full_size():
    """The bench's workload and launch configuration (out of place, S=1), every element."""
    dev, ref = _run_fused_case(I.GQA_PREFILL, 1)
    assert dev.inp.meta["n_outliers"] > 40000


def _oracle_planes(inp):
    """Statistic planes [1 + P, 2, T] float32: this slice's sums of squares and
    the peers' (oracle values rounded to float32), as a rank would receive them."""
    planes = [oracle.qknorm_partial_stats(inp.q, inp.k, "bf16", 1)[0]]
    for p in range(inp.peer_q.shape[0]):
        planes.append(oracle.qknorm_partial_stats(inp.peer_q[p], inp.peer_k[p], "bf16", 1)[0])
    return np.stack(planes).astype(np.float32)


def test_rank_slice_partial_and_apply():
    w = I.RANK_SLICE
    _log(f"[case] rank_slice partial_stats + apply_with_stats T={w.T} local {w.hq}/{w.hk} full {w.hq_full}/{w.hk_full}")
    inp = I.make_inputs(w)
    dev = Packed(inp)
    part = qk.qknorm_partial_stats(dev.q, dev.k, 1)
    torch.cuda.synchronize()
    got_p = part.cpu().numpy()
    ref_p = oracle.qknorm_partial_stats(inp.q, inp.k, "bf16", 1)
    rel = np.abs(got_p.astype(np.float64) - ref_p) / ref_p
    _log(f"[parity] rank_slice partial_stats max rel err {rel.max():.3g}")
    assert rel.max() <= 1e-5

    planes = _oracle_planes(inp)
    stats = torch.from_numpy(planes).to(DEV)
    qk.qknorm_apply_with_stats(dev.q, dev.k, dev.gq, dev.gk, w.eps, stats, w.hq_full, w.hk_full,
                               dev.oq, dev.ok)
    torch.cuda.synchronize()
    ref = oracle.qknorm_apply_with_stats(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "bf16", w.eps, planes,
                                         w.hq_full, w.hk_full)
    _compare(w, torch_to_np(dev.oq), torch_to_np(dev.ok), ref, "rank_slice apply 4 planes")
    assert dev.untouched_outside_qk()


# ----------------------------------------------------------------------- bitwise properties
@pytest.mark.parametrize("key,shards", [("tiny", 2), ("small_dense", 4), ("decode_t64", 8), ("decode_t1", 2), ("decode_t256", 4)])
def test_fused_equals_partial_stats_plus_apply_bitwise(key, shards):
    _log(f"[case] fused == split {key} S={shards}")
    _check_fused_equals_split(I.make_inputs(I.WORKLOADS[key]), shards)


# Layouts where fused and split once disagreed: 2 chunks per lane (decode
# rows, S = 1), where the fused kernel summed squares by fused multiply-adds
# and partial_stats by dot products, and mid-size bf16 launches (1024 to 4096
# tokens), where partial_stats took another lane layout than the fused call.
# The GQA prefill draws (0.1% of elements x50) mix large and small squares in
# one chunk, which is where the two ways of adding them differ.
@pytest.mark.parametrize("key,T,shards", [("decode_t256", 256, 1), ("gqa_prefill", 2048, 1),
                                          ("gqa_prefill", 1536, 2), ("gqa_prefill", 4096, 1)])
def test_fused_equals_split_where_layouts_once_differed(key, T, shards):
    w = I.WORKLOADS[key].with_T(T)
    _log(f"[case] fused == split {key} T={T} S={shards} "
         f"plan: {qk.describe_plan(0, w.hq, w.hk, w.T, w.dtype, shards, ld=w.ld)}")
    _check_fused_equals_split(I.make_inputs(w), shards)


@pytest.mark.parametrize("dtype,shards", [("bf16", 64), ("bf16", 32), ("bf16", 16), ("f32", 64)])
def test_many_shards_fused_equals_partial_stats_plus_apply_bitwise(dtype, shards):
    """Narrow shards (4 to 16 lanes each) put 16 to 64 lane groups of one
    token through the cross-wave exchange, the most it takes; partial_stats
    picks each shard's sum out of the same exchange."""
    inp = I.make_custom(13, 4096, 1024, 512, dtype, seed=60 + shards)
    w = inp.workload
    _log(f"[case] fused == split custom {dtype} S={shards} "
         f"plan: {qk.describe_plan(0, w.hq, w.hk, w.T, dtype, shards, ld=w.ld)}")
    fq, fk = _check_fused_equals_split(inp, shards)
    _compare(w, fq, fk, oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, dtype, w.eps, shards),
             f"custom S={shards}")


def _check_fused_equals_split(inp, shards):
    """Fused == partial_stats + apply (S planes) == partial_stats + float32
    combine in rank order + apply (one plane), bit for bit; the partials
    against the oracle."""
    w = inp.workload
    a = Packed(inp, seed=5)
    fq, fk = a.fused(shards)
    b = Packed(inp, seed=6)
    part = qk.qknorm_partial_stats(b.q, b.k, shards)
    qk.qknorm_apply_with_stats(b.q, b.k, b.gq, b.gk, w.eps, part, w.hq, w.hk, b.oq, b.ok)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_np(b.oq).view(np.uint8), fq.view(np.uint8))
    assert np.array_equal(torch_to_np(b.ok).view(np.uint8), fk.view(np.uint8))
    # and the partials against the oracle
    ref = oracle.qknorm_partial_stats(inp.q, inp.k, w.dtype, shards)
    got = part.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-5 * ref)
    # host combine: the planes summed in rank order in float32, handed over as one plane
    p32 = part.cpu().numpy()
    comb = p32[0].copy()
    for s_ in range(1, shards):
        comb = (comb + p32[s_]).astype(np.float32)
    c = Packed(inp, seed=7)
    qk.qknorm_apply_with_stats(c.q, c.k, c.gq, c.gk, w.eps, torch.from_numpy(comb[None]).to(DEV), w.hq, w.hk,
                               c.oq, c.ok)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_np(c.oq).view(np.uint8), fq.view(np.uint8))
    assert np.array_equal(torch_to_np(c.ok).view(np.uint8), fk.view(np.uint8))
    return fq, fk


@pytest.mark.parametrize("key", ["small_dense", "decode_t8", "tiny"])
def test_in_place_equals_out_of_place(key):
    w = I.WORKLOADS[key]
    inp = I.make_inputs(w)
    s = w.shards[-1]
    a = Packed(inp, out_of_place=True)
    oq, ok = a.fused(s)
    b = Packed(inp, out_of_place=False)
    iq, ik = b.fused(s)
    assert np.array_equal(oq.view(np.uint8), iq.view(np.uint8))
    assert np.array_equal(ok.view(np.uint8), ik.view(np.uint8))
    assert b.untouched_outside_qk()


def test_run_to_run_deterministic():
    w = I.GQA_PREFILL.with_T(2048)
    inp = I.make_inputs(w)
    a = Packed(inp)
    r1 = a.fused(1)
    r2 = a.fused(1)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_partials_exact_on_integer_inputs():
    """Integer-valued bf16 inputs in [-16, 16]: every float32 partial is exact,
    so it must equal the integer sum bit for bit."""
    rng = np.random.default_rng(21)
    for (T, hq, hk, S) in ((37, 4096, 1024, 8), (300, 1280, 256, 1), (5, 2048, 2048, 4)):
        xi = rng.integers(-16, 17, (T, hq + hk)).astype(np.float64)
        w = I.Workload("int", "int", 0, T, hq, hk, 0, "bf16", False, (S,))
        inp = I.Inputs(w, I.to_bf16_bits(xi[:, :hq]), I.to_bf16_bits(xi[:, hq:]),
                       I.to_bf16_bits(np.ones(hq)), I.to_bf16_bits(np.ones(hk)))
        dev = Packed(inp)
        part = qk.qknorm_partial_stats(dev.q, dev.k, S).cpu().numpy()
        wq, wk = hq // S, hk // S
        for s in range(S):
            assert np.array_equal(part[s, 0], (xi[:, s * wq:(s + 1) * wq] ** 2).sum(1).astype(np.float32))
            assert np.array_equal(part[s, 1], (xi[:, hq + s * wk:hq + (s + 1) * wk] ** 2).sum(1).astype(np.float32))


# ----------------------------------------------------------------------- edge cases
def _custom_case(T, hq, hk, hv, dtype, S, seed, scale=1.0, offset=0, ld_pad=0, eps=1e-6):
    inp = I.make_custom(T, hq, hk, hv, dtype, seed=seed, scale=scale)
    w = inp.workload
    _log(f"[case] custom T={T} hq={hq} hk={hk} hv={hv} {dtype} S={S} offset={offset} ld_pad={ld_pad}")
    ld = hq + hk + hv + ld_pad
    host = np.zeros((T, ld), dtype=inp.q.dtype)
    host[:, :hq] = inp.q
    host[:, hq:hq + hk] = inp.k
    rng = np.random.default_rng(seed)
    if hv + ld_pad:
        host[:, hq + hk:] = rng.integers(0, 1 << 14, (T, hv + ld_pad)).astype(host.dtype)
    src = Guarded(host, seed=seed, offset_elems=offset)
    dst = Guarded(host, seed=seed + 1, offset_elems=offset)
    dst_init = dst.host().copy()
    x, y = src.view(), dst.view()
    gq = np_to_torch(inp.gamma_q).to(DEV)
    gk = np_to_torch(inp.gamma_k).to(DEV)
    qk.qknorm_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, eps, S, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    out = dst.host()
    ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, dtype, eps, S)
    _compare(w, out[:, :hq], out[:, hq:hq + hk], ref, f"custom {hq}/{hk} S={S}")
    assert np.array_equal(out[:, hq + hk:].view(np.uint8), dst_init[:, hq + hk:].view(np.uint8))
    assert src.guards_intact() and dst.guards_intact()
    assert np.array_equal(src.host(), host)
    return out, ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_widths(dtype):
    # chunk counts that do not fill a lane group or a slot: ragged tails
    _custom_case(77, 264, 40, 24, dtype, 1, seed=31)
    _custom_case(130, 8 * 37, 8 * 5, 0, dtype, 1, seed=32)
    _custom_case(19, 1032, 520, 8, dtype, 2, seed=33)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_elementwise_path(dtype):
    # misaligned base, odd row stride, shard widths not a multiple of a chunk
    _custom_case(45, 512, 128, 64, dtype, 1, seed=41, offset=1)
    _custom_case(33, 500, 100, 0, dtype, 1, seed=42, ld_pad=3)
    _custom_case(29, 60, 12, 4, dtype, 3, seed=43)
    _custom_case(17, 4100, 1030, 2, dtype, 2, seed=44, offset=3, ld_pad=1)


@pytest.mark.parametrize("T,hq,hk,hv,dtype,offset", [
    (1500, 128, 64, 64, "bf16", 0),     # 24 chunks: 8 lanes per token, 8 tokens per wave
    (2000, 64, 32, 0, "f32", 0),        # 24 fp32 chunks: 8 lanes per token
    (1100, 40, 24, 8, "bf16", 0),       # 8 chunks: 4 lanes per token, 16 per wave, ragged slots
    (4097, 640, 128, 128, "bf16", 0),   # 96 chunks: 32 lanes per token, ragged last block
    (1025, 128, 64, 0, "bf16", 1),      # element-wise path, several tokens per wave
])
def test_several_tokens_per_wave(T, hq, hk, hv, dtype, offset):
    """Rows of fewer than 64 lanes' chunks: several tokens share a wave, each
    reduced over its own lane group; token counts that leave the last block
    partly empty."""
    ld = hq + hk + hv
    plan = qk.describe_plan(0, hq, hk, T, dtype, 1, ld=ld, aligned=offset == 0)
    tok_threads = int(plan.split("threads/token=")[1].split()[0])
    assert tok_threads < 64, plan
    _log(f"[plan] {plan}")
    _custom_case(T, hq, hk, hv, dtype, 1, seed=T + hq, offset=offset)


def test_several_tokens_per_wave_fused_equals_split_bitwise():
    inp = I.make_custom(3000, 256, 128, 0, "bf16", seed=61)
    assert "threads/token=16" in qk.describe_plan(0, 256, 128, 3000, "bf16", 1, ld=256)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    fq, fk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 1, fq, fk)
    part = qk.qknorm_partial_stats(xq, xk, 1)
    aq, ak = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, 256, 128, aq, ak)
    torch.cuda.synchronize()
    ref_p = oracle.qknorm_partial_stats(inp.q, inp.k, "bf16", 1)
    got_p = part.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_p - ref_p) <= 1e-5 * ref_p)
    assert torch.equal(fq.view(torch.int16), aq.view(torch.int16))
    assert torch.equal(fk.view(torch.int16), ak.view(torch.int16))


def test_elementwise_path_is_bitwise_identical_to_vector_path():
    """Same data through the 16-byte path and (shifted by one element) the
    element-wise path: the reduction order is the same, so are the bits."""
    a, _ = _custom_case(64, 1280, 256, 256, "bf16", 1, seed=45)
    b, _ = _custom_case(64, 1280, 256, 256, "bf16", 1, seed=45, offset=1)
    assert np.array_equal(a[:, :1536], b[:, :1536])


def test_many_shards_and_widest_rows():
    _custom_case(9, 4096, 1024, 0, "bf16", 64, seed=51)
    _custom_case(6, 57344, 8192, 0, "bf16", 1, seed=52)       # 8192 chunks: the widest bf16 row
    _custom_case(5, 28672, 4096, 0, "f32", 1, seed=53)        # the widest fp32 row
    _custom_case(3, 49152, 16384, 0, "bf16", 8, seed=54)


def test_row_offsets_beyond_4_gib():
    """Packed bf16 rows [262147, 8192] (4.3 GB): rows past the first 4 GiB need
    64-bit offsets. Inputs are drawn on the device from a seeded generator;
    sampled rows are copied back and checked against the oracle one by one,
    for the fused call and for partial_stats + apply_with_stats."""
    T, hq, hk, ld = 262147, 4096, 1024, 8192
    assert (T - 1) * ld * 2 > 1 << 32
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20260)
    x = torch.randn((T, ld), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(20261)
    gq_bits = I.to_bf16_bits(rng.normal(1.0, 0.1, hq))
    gk_bits = I.to_bf16_bits(rng.normal(1.0, 0.1, hk))
    gq, gk = np_to_torch(gq_bits).to(DEV), np_to_torch(gk_bits).to(DEV)
    y = torch.zeros_like(x)
    _log(f"[case] 4 GiB rows T={T} ld={ld} plan: {qk.describe_plan(0, hq, hk, T, 'bf16', 1, ld=ld)}")
    qk.qknorm_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, 1e-6, 1, y[:, :hq], y[:, hq:hq + hk])
    part = qk.qknorm_partial_stats(x[:, :hq], x[:, hq:hq + hk], 1)
    y2 = torch.zeros_like(x)
    qk.qknorm_apply_with_stats(x[:, :hq], x[:, hq:hq + hk], gq, gk, 1e-6, part, hq, hk, y2[:, :hq], y2[:, hq:hq + hk])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, T // 2, 262143, 262144, T - 2, T - 1],
                                     rng.integers(0, T, 25)]))
    idx = torch.from_numpy(rows).to(DEV)
    xs = torch_to_np(x.index_select(0, idx))
    ys = torch_to_np(y.index_select(0, idx))
    ys2 = torch_to_np(y2.index_select(0, idx))
    ps = part.index_select(2, idx).cpu().numpy().astype(np.float64)
    del x, y, y2
    torch.cuda.empty_cache()
    ref = oracle.qknorm_fused(xs[:, :hq], xs[:, hq:hq + hk], gq_bits, gk_bits, "bf16", 1e-6, 1)
    check_bf16(ys[:, :hq], ref.yq_bits, "4 GiB Q")
    check_bf16(ys[:, hq:hq + hk], ref.yk_bits, "4 GiB K")
    assert not ys[:, hq + hk:].any(), "V columns were written"
    assert np.array_equal(ys, ys2), "split path differs from fused"
    ref_p = oracle.qknorm_partial_stats(xs[:, :hq], xs[:, hq:hq + hk], "bf16", 1)
    assert np.all(np.abs(ps - ref_p) <= 1e-5 * ref_p)
    _log(f"[parity] 4 GiB rows: {len(rows)} sampled rows match")


@pytest.mark.parametrize("dtype,n_planes", [("bf16", 64), ("f32", 64), ("bf16", 1), ("f32", 7)])
def test_apply_with_many_planes(dtype, n_planes):
    """apply_with_stats with up to the maximum number of statistic planes (one
    per rank of a 64-way split): the planes are added in order in fp32 and
    divided by the full widths; the oracle adds them in fp64."""
    T, hq, hk = 300, 256, 64
    inp = I.make_custom(T, hq, hk, 0, dtype, seed=90 + n_planes)
    rng = np.random.default_rng(91 + n_planes)
    local = oracle.qknorm_partial_stats(inp.q, inp.k, dtype, 1)[0]
    # peers: sums of squares of the same scale as the local slice
    planes = np.concatenate([local[None], local[None] * rng.uniform(0.5, 1.5, (n_planes - 1, 2, T))])
    planes = planes.astype(np.float32)
    hq_full, hk_full = hq * n_planes, hk * n_planes
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    yq, yk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, torch.from_numpy(planes).to(DEV), hq_full, hk_full, yq, yk)
    torch.cuda.synchronize()
    ref = oracle.qknorm_apply_with_stats(inp.q, inp.k, inp.gamma_q, inp.gamma_k, dtype, 1e-6, planes,
                                         hq_full, hk_full)
    _compare(inp.workload, torch_to_np(yq), torch_to_np(yk), ref, f"apply {n_planes} planes")


@pytest.mark.parametrize("ranks", [2, 4])
def test_tensor_parallel_emulation_on_one_gpu(ranks):
    """The sharded path of the paper's Phase A / Phase B, each rank's share as
    its own calls: every rank runs partial_stats on its column slice, the
    planes are exchanged (here: stacked in rank order), and every rank runs
    apply_with_stats with all planes and the full widths. The slices together
    must equal the full-row oracle, and the split must match fused(S = ranks),
    whose per-shard sums are what the ranks would exchange."""
    T, hq, hk = 700, 5120, 1024
    inp = I.make_custom(T, hq, hk, 0, "bf16", seed=3000 + ranks)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    wq, wk = hq // ranks, hk // ranks
    planes = torch.cat([qk.qknorm_partial_stats(xq[:, r * wq:(r + 1) * wq], xk[:, r * wk:(r + 1) * wk], 1)
                        for r in range(ranks)])                       # [ranks, 2, T], rank order
    yq, yk = torch.empty_like(xq), torch.empty_like(xk)
    for r in range(ranks):
        qk.qknorm_apply_with_stats(xq[:, r * wq:(r + 1) * wq], xk[:, r * wk:(r + 1) * wk], gq[r * wq:(r + 1) * wq],
                                   gk[r * wk:(r + 1) * wk], 1e-6, planes, hq, hk,
                                   yq[:, r * wq:(r + 1) * wq], yk[:, r * wk:(r + 1) * wk])
    fq, fk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, ranks, fq, fk)
    torch.cuda.synchronize()
    ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "bf16", 1e-6, 1)
    check_bf16(torch_to_np(yq), ref.yq_bits, f"{ranks} ranks Q")
    check_bf16(torch_to_np(yk), ref.yk_bits, f"{ranks} ranks K")
    # the ranks' planes are the fused kernel's per-shard sums up to summation order
    ref_p = oracle.qknorm_partial_stats(inp.q, inp.k, "bf16", ranks)
    got_p = planes.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_p - ref_p) <= 1e-5 * ref_p)
    # fused(S = ranks) computes the same factors with its own float32
    # summation order, so every output is the ranks' bf16 value or one of its
    # two neighbours, and a differing factor rounds differently only next to a
    # bf16 rounding boundary (a few elements in 10^4)
    for name, fused, split, want in (("Q", fq, yq, ref.yq_bits), ("K", fk, yk, ref.yk_bits)):
        check_bf16(torch_to_np(fused), want, f"fused(S = {ranks}) {name}")
        exact, dmax = check_bf16(torch_to_np(fused), torch_to_np(split), f"fused(S = {ranks}) vs ranks {name}")
        assert dmax <= 1 and exact >= 0.999, (name, exact, dmax)
    _log(f"[parity] tensor-parallel emulation, {ranks} ranks: slices match the full-row oracle")


def test_too_wide_is_unsupported_and_writes_nothing():
    T, hq, hk = 2, 65536, 8
    x = torch.zeros((T, hq + hk), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(hq, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(qk.QKNormError) as e:
        qk.qknorm_fused(x[:, :hq], x[:, hq:], g, g[:hk].clone(), 1e-6, 1)
    assert e.value.status == 2


def test_single_token_and_empty():
    _custom_case(1, 5120, 1024, 1024, "bf16", 1, seed=61)
    _custom_case(1, 256, 256, 0, "f32", 2, seed=62)
    # T = 0: no-op, nothing written
    x = torch.full((0, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    qk.qknorm_fused(x, x.clone(), g, g, 1e-6, 1)
    qk.qknorm_partial_stats(x, x.clone(), 1)
    torch.cuda.synchronize()


def test_large_and_small_magnitudes():
    _custom_case(40, 2048, 512, 0, "bf16", 4, seed=71, scale=1e15)
    _custom_case(40, 2048, 512, 0, "bf16", 4, seed=72, scale=1e-15)
    _custom_case(40, 2048, 512, 0, "f32", 2, seed=73, scale=3e8)


def test_factor_below_the_normal_range():
    """eps = 0 (and a subnormal float32 eps) with rows of a few nonzero elements
    around 3e-19: every square is a normal float32, but the mean square lies
    below the float32 normal range, so the factor is taken on the 2^64-scaled
    value (and nothing may be flushed to zero on the way)."""
    T, hq, hk = 8, 4096, 1024
    rng = np.random.default_rng(91)
    xq, xk = np.zeros((T, hq)), np.zeros((T, hk))
    for t in range(T):
        n = 1 + t
        for x, h in ((xq, hq), (xk, hk)):
            x[t, rng.choice(h, n, replace=False)] = rng.uniform(0.5, 2.0, n) * 3e-19 * rng.choice([-1.0, 1.0], n)
    assert np.all((xq ** 2).sum(1) / hq < 1.17e-38) and np.all((xk ** 2).sum(1) / hk < 1.17e-38)
    for dtype in ("f32", "bf16"):
        inp = I.make_custom(T, hq, hk, 0, dtype, seed=91)
        enc = I.to_bf16_bits if dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
        q, k = enc(xq), enc(xk)
        for eps in (0.0, 1e-40):
            for S in (1, 2):
                _log(f"[case] factor below the normal range {dtype} eps={eps} S={S}")
                xq_d, xk_d = np_to_torch(q).to(DEV), np_to_torch(k).to(DEV)
                gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
                qk.qknorm_fused(xq_d, xk_d, gq, gk, eps, S)
                torch.cuda.synchronize()
                ref = oracle.qknorm_fused(q, k, inp.gamma_q, inp.gamma_k, dtype, eps, S)
                assert np.all(np.isfinite(ref.yq)) and np.abs(ref.yq).max() > 1.0
                _compare(inp.workload, torch_to_np(xq_d), torch_to_np(xk_d), ref,
                         f"tiny mean square {dtype} eps={eps} S={S}")


def test_degenerate_rows():
    """Zero rows give 0 with eps > 0 and NaN with eps = 0; a NaN in a row
    makes that tensor's row NaN; an Inf gives 0 elsewhere and NaN at the Inf."""
    T, hq, hk = 6, 256, 64
    for dtype in ("bf16", "f32"):
        inp = I.make_custom(T, hq, hk, 0, dtype, seed=81)
        q, k = inp.q.copy(), inp.k.copy()
        enc = I.to_bf16_bits if dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
        q[0] = enc(np.zeros(hq))
        k[1] = enc(np.zeros(hk))
        q[2, 17] = enc(np.array([np.nan]))[0] if dtype == "f32" else np.uint16(0x7FC0)
        k[3, 5] = enc(np.array([np.inf]))[0] if dtype == "f32" else np.uint16(0x7F80)
        for eps in (1e-6, 0.0):
            xq = np_to_torch(q).to(DEV)
            xk = np_to_torch(k).to(DEV)
            gq = np_to_torch(inp.gamma_q).to(DEV)
            gk = np_to_torch(inp.gamma_k).to(DEV)
            qk.qknorm_fused(xq, xk, gq, gk, eps, 1)
            torch.cuda.synchronize()
            with np.errstate(all="ignore"):
                ref = oracle.qknorm_fused(q, k, inp.gamma_q, inp.gamma_k, dtype, eps, 1)
            w = inp.workload
            _compare(w, torch_to_np(xq), torch_to_np(xk), ref, f"degenerate {dtype} eps={eps}")


def test_argument_errors_write_nothing():
    x = torch.randn(8, 96, device=DEV).to(torch.bfloat16)
    before = x.clone()
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    gk = torch.ones(32, dtype=torch.bfloat16, device=DEV)
    cases = [
        lambda: qk.qknorm_fused(x[:, :64], x[:, 64:], g, gk, -1.0, 1),            # eps < 0
        lambda: qk.qknorm_fused(x[:, :64], x[:, 64:], g, gk, 1e-6, 3),            # 64 % 3
        lambda: qk.qknorm_fused(x[:, :64], x[:, 64:], g, gk, 1e-6, 1, x[:, 32:96], x[:, 64:]),  # overlap
        lambda: qk.qknorm_apply_with_stats(x[:, :64], x[:, 64:], g, gk, 1e-6,
                                           torch.ones(1, 2, 8, device=DEV), 32, 32),  # H_full < h
    ]
    for c in cases:
        with pytest.raises(qk.QKNormError) as e:
            c()
        assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), before.view(torch.int16))


def test_runs_on_the_callers_stream():
    w = I.DECODE[3]
    inp = I.make_inputs(w)
    dev = Packed(inp)
    ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "bf16", w.eps, 4)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qk.qknorm_fused(dev.q, dev.k, dev.gq, dev.gk, w.eps, 4, dev.oq, dev.ok)
    s.synchronize()
    _compare(w, torch_to_np(dev.oq), torch_to_np(dev.ok), ref, "side stream")


def test_concurrent_callers_on_their_own_streams():
    """Four host threads, each with its own stream and buffers, call the three
    entry points repeatedly at the same time; every result equals the one the
    same call gives alone (the library keeps no shared state on the launch path)."""
    import threading
    keys = ["small_dense", "decode_t256", "decode_t64", "tiny"]
    cases = []
    for n, key in enumerate(keys):
        w = I.WORKLOADS[key]
        inp = I.make_inputs(w)
        a = Packed(inp, seed=40 + n)
        fq, fk = a.fused(2)                       # alone, on the default stream
        b = Packed(inp, seed=50 + n)
        cases.append((w, a, b, fq, fk))
    _log("[case] concurrent callers: " + ", ".join(keys))
    errors = []
    barrier = threading.Barrier(len(cases))

    def worker(w, a, b, fq, fk):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                barrier.wait()
                for _ in range(20):
                    qk.qknorm_fused(b.q, b.k, b.gq, b.gk, w.eps, 2, b.oq, b.ok)
                    part = qk.qknorm_partial_stats(b.q, b.k, 2)
                    qk.qknorm_apply_with_stats(b.q, b.k, b.gq, b.gk, w.eps, part, w.hq, w.hk, b.oq, b.ok)
            s.synchronize()
            if not (np.array_equal(torch_to_np(b.oq).view(np.uint8), fq.view(np.uint8)) and
                    np.array_equal(torch_to_np(b.ok).view(np.uint8), fk.view(np.uint8))):
                errors.append(w.key)
        except Exception as e:  # reported below, in the test's own thread
            errors.append(f"{w.key}: {e!r}")

    ts = [threading.Thread(target=worker, args=c) for c in cases]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in ts), "a caller thread did not finish"
    assert not errors, errors


def test_golden_worked_examples_on_the_gpu():
    """The hand-worked examples (tests/golden/worked_examples.json: exact
    decimals derived by hand from Eq. 1, Phase A, the split path and headwise
    heads) through the kernels with fp32, bf16 and FP8 rows: each result within
    the usual tolerance of the exact decimal (one bf16 / E4M3 step of its
    single rounding; 1e-5 relative in fp32)."""
    import json
    from decimal import Decimal
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")) as f:
        data = json.load(f)

    def enc(a, dtype, gamma=False):
        a = np.asarray(a, dtype=np.float64)
        if dtype == "f32":
            return np_to_torch(a.astype(np.float32)).to(DEV)
        if dtype == "bf16" or gamma:
            return np_to_torch(I.to_bf16_bits(a)).to(DEV)
        return np_to_torch(oracle.f64_to_fp8_bits(a)).to(DEV)

    def check(got, want, dtype, what):
        want = np.asarray(want, dtype=np.float64)
        got = torch_to_np(got)
        if dtype == "f32":
            check_f32(got, want, what)
        elif dtype == "bf16":
            check_bf16(got, oracle.f64_to_bf16_bits(want), what)
        else:
            check_fp8(got, oracle.f64_to_fp8_bits(want), what)

    exact = lambda ys: np.array([[float(Decimal(v)) for v in ys]])
    for dtype in ("f32", "bf16", "fp8"):
        for ex in data["examples"]:
            x = np.array([ex["x"]], dtype=np.float64)
            q, k = enc(x, dtype), enc(x, dtype)
            gq, gk = enc(ex["gamma"], dtype, gamma=True), enc(ex["gamma"], dtype, gamma=True)
            if ex["op"] == "fused":
                qk.qknorm_fused(q, k, gq, gk, float(ex["eps"]), ex["shards"])
            else:
                st = np.array(ex["stats"], dtype=np.float32)
                stats = torch.from_numpy(np.stack([st, st], axis=1)[:, :, None].copy()).to(DEV)  # [P][2][T=1]
                qk.qknorm_apply_with_stats(q, k, gq, gk, float(ex["eps"]), stats, ex["h_full"], ex["h_full"])
            torch.cuda.synchronize()
            check(q, exact(ex["y"]), dtype, f"{ex['name']} {dtype} Q")
            check(k, exact(ex["y"]), dtype, f"{ex['name']} {dtype} K")
        for c in data["headwise_examples"]["cases"]:
            x = np.array([c["x"]], dtype=np.float64)
            q, k = enc(x, dtype), enc(x, dtype)
            g = enc(c["gamma"], dtype, gamma=True)
            qk.qknorm_headwise(q, k, g, g, float(c["eps"]), c["head_dim"], c["gamma_head_stride"])
            torch.cuda.synchronize()
            check(q, exact(c["y"]), dtype, f"{c['name']} {dtype} Q")
            check(k, exact(c["y"]), dtype, f"{c['name']} {dtype} K")

"""GPU parity for FP8 E4M3 rows (OCP E4M3FN) with bf16 gamma and fp32
arithmetic: every call against the float64 oracle, element by element.
Acceptance: each FP8 output is the oracle's once-rounded (saturating) E4M3
result or one of its two neighbours; NaN exactly where the oracle has NaN;
V columns and guard bands untouched."""

import numpy as np
import pytest
import torch

import oracle
import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, Guarded, check_fp8, fig2b_errors, np_to_torch, torch_to_np

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _layout(inp, hv, ld_pad=0, offset=0, seed=0):
    """Packed host rows [T, hq + hk + hv + ld_pad] and guarded device copies."""
    w = inp.workload
    T, hq, hk = inp.q.shape[0], inp.q.shape[1], inp.k.shape[1]
    ld = hq + hk + hv + ld_pad
    host = np.zeros((T, ld), np.uint8)
    host[:, :hq] = inp.q
    host[:, hq:hq + hk] = inp.k
    if hv + ld_pad:
        host[:, hq + hk:] = np.random.default_rng(seed).integers(0, 0x7F, (T, hv + ld_pad)).astype(np.uint8)
    src = Guarded(host, seed=seed, offset_elems=offset)
    dst = Guarded(np.random.default_rng(seed + 9).integers(0, 0x7F, host.shape).astype(np.uint8), seed=seed + 1,
                  offset_elems=offset)
    return host, src, dst


def _compare(got, ref, what):
    hq = ref.yq.shape[1]
    eq, _ = check_fp8(got[:, :hq], ref.yq_bits, what + " Q")
    ek, _ = check_fp8(got[:, hq:hq + ref.yk.shape[1]], ref.yk_bits, what + " K")
    gold = oracle.fp8_bits_to_f64(got[:, :hq])
    e = fig2b_errors(gold, ref.yq)
    _log(f"[parity] {what}: exact FP8 match Q {eq:.5f} K {ek:.5f}; vs fp64 gold Q max/mean/rms "
         f"{e[0]:.3g}/{e[1]:.3g}/{e[2]:.3g}")


def _untouched(host, src, dst, dst_init, hq, hk):
    assert src.guards_intact() and dst.guards_intact()
    assert np.array_equal(src.host(), host)
    assert np.array_equal(dst.host()[:, hq + hk:], dst_init[:, hq + hk:])


def _fused(inp, hv, shards, eps=1e-6, **kw):
    hq, hk = inp.q.shape[1], inp.k.shape[1]
    host, src, dst = _layout(inp, hv, **kw)
    dst_init = dst.host()
    x, y = src.view(), dst.view()
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    qk.qknorm_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, eps, shards, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    out = dst.host()
    _untouched(host, src, dst, dst_init, hq, hk)
    return out, oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "fp8", eps, shards)


def test_gqa_prefill_fp8_full_size():
    w = I.GQA_PREFILL_FP8
    _log(f"[case] {w.key} plan: {qk.describe_plan(0, w.hq, w.hk, w.T, 'fp8', 1, ld=w.ld)}")
    inp = I.make_inputs(w)
    out, ref = _fused(inp, w.hv, 1)
    _compare(out, ref, w.key)


@pytest.mark.parametrize("T", [1, 64, 256])
@pytest.mark.parametrize("shards", [1, 8])
def test_decode_fp8(T, shards):
    inp = I.make_custom(T, 4096, 4096, 0, "fp8", seed=600 + T)
    out, ref = _fused(inp, 4096, shards)
    _compare(out, ref, f"decode fp8 T={T} S={shards}")


def test_rank_slice_fp8_partial_and_apply():
    w = I.RANK_SLICE_FP8
    inp = I.make_inputs(w)
    hq, hk = w.hq, w.hk
    host, src, dst = _layout(inp, w.hv)
    dst_init = dst.host()
    x, y = src.view(), dst.view()
    part = qk.qknorm_partial_stats(x[:, :hq], x[:, hq:hq + hk], 1).cpu().numpy().astype(np.float64)
    ref_p = oracle.qknorm_partial_stats(inp.q, inp.k, "fp8", 1)
    assert np.all(np.abs(part - ref_p) <= 1e-5 * ref_p)
    planes = [ref_p[0]] + [oracle.qknorm_partial_stats(inp.peer_q[p], inp.peer_k[p], "fp8", 1)[0]
                           for p in range(inp.peer_q.shape[0])]
    planes = np.stack(planes).astype(np.float32)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    qk.qknorm_apply_with_stats(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, torch.from_numpy(planes).to(DEV),
                               w.hq_full, w.hk_full, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    ref = oracle.qknorm_apply_with_stats(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "fp8", w.eps, planes,
                                         w.hq_full, w.hk_full)
    _compare(dst.host(), ref, "rank_slice_fp8 apply")
    _untouched(host, src, dst, dst_init, hq, hk)


@pytest.mark.parametrize("T,k", [(5000, 3), (6144, 3), (4100, 3)])
def test_gqa_prefill_fp8_token_loop(T, k):
    """GQA-width FP8 launches whose blocks each take several token groups
    (groups/block = k; 5000 and 4100 tokens leave some blocks one group
    short): every element against the oracle, and the split path equal to
    the fused call bit for bit."""
    w = I.GQA_PREFILL_FP8.with_T(T)
    plan = qk.describe_plan(0, w.hq, w.hk, T, "fp8", 1, ld=w.ld)
    _log(f"[case] {w.key} T={T} plan: {plan}")
    assert f"groups/block={k}" in plan
    inp = I.make_inputs(w)
    out, ref = _fused(inp, w.hv, 1)
    _compare(out, ref, f"{w.key} T={T}")
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    part = qk.qknorm_partial_stats(xq, xk, 1)
    aq, ak = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, w.eps, part, w.hq, w.hk, aq, ak)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_np(aq), out[:, :w.hq])
    assert np.array_equal(torch_to_np(ak), out[:, w.hq:w.hq + w.hk])


@pytest.mark.parametrize("T,k", [(12000, 2), (32760, 4)])
def test_rank_slice_fp8_apply_token_loop(T, k):
    """The rank-slice apply with blocks taking k groups of 8 tokens (12000
    tokens: 1500 groups over 750 blocks; 32760: 4095 groups, the last block
    one group short), 4 planes, every element against the oracle."""
    w = I.RANK_SLICE_FP8.with_T(T)
    plan = qk.describe_plan(2, w.hq, w.hk, T, "fp8", 1, ld=w.ld)
    _log(f"[case] {w.key} apply T={T} plan: {plan}")
    assert f"groups/block={k}" in plan
    inp = I.make_inputs(w)
    hq, hk = w.hq, w.hk
    host, src, dst = _layout(inp, w.hv)
    dst_init = dst.host()
    x, y = src.view(), dst.view()
    planes = [oracle.qknorm_partial_stats(inp.q, inp.k, "fp8", 1)[0]] + [
        oracle.qknorm_partial_stats(inp.peer_q[p], inp.peer_k[p], "fp8", 1)[0] for p in range(inp.peer_q.shape[0])]
    planes = np.stack(planes).astype(np.float32)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    qk.qknorm_apply_with_stats(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, torch.from_numpy(planes).to(DEV),
                               w.hq_full, w.hk_full, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    ref = oracle.qknorm_apply_with_stats(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "fp8", w.eps, planes,
                                         w.hq_full, w.hk_full)
    _compare(dst.host(), ref, f"rank_slice_fp8 apply T={T}")
    _untouched(host, src, dst, dst_init, hq, hk)


def test_fused_equals_split_fp8_bitwise():
    inp = I.make_custom(300, 2048, 512, 0, "fp8", seed=701)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    fq, fk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 4, fq, fk)
    part = qk.qknorm_partial_stats(xq, xk, 4)
    aq, ak = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, 2048, 512, aq, ak)
    torch.cuda.synchronize()
    assert torch.equal(fq.view(torch.uint8), aq.view(torch.uint8))
    assert torch.equal(fk.view(torch.uint8), ak.view(torch.uint8))


@pytest.mark.parametrize("key,T,shards", [("gqa_prefill_fp8", 1024, 1), ("gqa_prefill_fp8", 2048, 2),
                                          ("rank_slice_fp8", 4096, 1)])
def test_fused_equals_split_fp8_bitwise_with_outliers(key, T, shards):
    """Rows of 3 or 4 chunks per lane, where the fused kernel once summed FP8
    squares by fused multiply-adds and partial_stats by dot products: the
    outlier draws (x50) put large and small squares in one chunk, where the
    two roundings differ."""
    w = I.WORKLOADS[key].with_T(T)
    inp = I.make_inputs(w)
    _log(f"[case] fused == split {key} T={T} S={shards}")
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    fq, fk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, w.eps, shards, fq, fk)
    part = qk.qknorm_partial_stats(xq, xk, shards)
    aq, ak = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, w.eps, part, inp.q.shape[1], inp.k.shape[1], aq, ak)
    torch.cuda.synchronize()
    assert torch.equal(fq.view(torch.uint8), aq.view(torch.uint8))
    assert torch.equal(fk.view(torch.uint8), ak.view(torch.uint8))


def test_headwise_fp8():
    w = I.GQA_PREFILL_FP8.with_T(1024)
    inp = I.make_inputs(w)
    hq, hk = w.hq, w.hk
    host, src, dst = _layout(inp, w.hv)
    dst_init = dst.host()
    x, y = src.view(), dst.view()
    gq_h, gk_h = inp.gamma_q[:128].copy(), inp.gamma_k[:128].copy()
    qk.qknorm_headwise(x[:, :hq], x[:, hq:hq + hk], np_to_torch(gq_h).to(DEV), np_to_torch(gk_h).to(DEV), w.eps, 128,
                       0, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    ref = oracle.qknorm_headwise(inp.q, inp.k, gq_h, gk_h, "fp8", w.eps, 128, 0)
    _compare(dst.host(), ref, "headwise fp8")
    _untouched(host, src, dst, dst_init, hq, hk)


def test_fp8_saturates_instead_of_nan():
    """gamma of 300 pushes many results past 448: they must come out as +-448."""
    inp = I.make_custom(64, 512, 128, 0, "fp8", seed=801)
    inp.gamma_q[...] = I.to_bf16_bits(np.full(512, 300.0))
    out, ref = _fused(inp, 0, 1)
    big = np.abs(ref.yq) > 464
    assert big.sum() > 1000
    assert np.all((out[:, :512][big] & 0x7F) == 0x7E)
    _compare(out, ref, "fp8 saturation")


def test_fp8_nan_gamma_with_overflow():
    """A NaN gamma column next to results beyond 448: NaN stays in that
    column, everything else saturates (the clamp decision sees the NaN)."""
    inp = I.make_custom(64, 512, 128, 0, "fp8", seed=802)
    g = np.full(512, 300.0)
    g[5] = np.nan
    inp.gamma_q[...] = I.to_bf16_bits(g)
    out, ref = _fused(inp, 0, 1)
    assert np.all((out[:, 5] & 0x7F) == 0x7F)
    big = np.abs(ref.yq) > 464
    assert big.sum() > 1000
    assert np.all((out[:, :512][big] & 0x7F) == 0x7E)
    _compare(out, ref, "fp8 NaN gamma")


@pytest.mark.parametrize("op", [0, 2])
def test_fp8_gamma_in_registers_saturation_and_nan(op):
    """Looping FP8 launches hold gamma widened in registers (plan: gamma=
    registers): a gamma of 300 with one NaN column there too, fused (op 0) and
    apply_with_stats (op 2) at 4500 tokens of the GQA widths (3 groups per
    block): NaN stays in its column, results beyond 448 saturate."""
    T, hq, hk = 4500, 5120, 1024
    plan = qk.describe_plan(op, hq, hk, T, "fp8", 1, ld=hq)
    _log(f"[case] fp8 gamma in registers op={op} T={T} plan: {plan}")
    assert "groups/block=3" in plan and "gamma=registers" in plan
    inp = I.make_custom(T, hq, hk, 0, "fp8", seed=803 + op)
    g = np.full(hq, 300.0)
    g[5] = np.nan
    inp.gamma_q[...] = I.to_bf16_bits(g)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    yq, yk = torch.empty_like(xq), torch.empty_like(xk)
    if op == 0:
        qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 1, yq, yk)
        ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "fp8", 1e-6, 1)
    else:
        planes = oracle.qknorm_partial_stats(inp.q, inp.k, "fp8", 1).astype(np.float32)
        qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, torch.from_numpy(planes).to(DEV), hq, hk, yq, yk)
        ref = oracle.qknorm_apply_with_stats(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "fp8", 1e-6, planes, hq, hk)
    torch.cuda.synchronize()
    out = np.concatenate([torch_to_np(yq), torch_to_np(yk)], axis=1)
    assert np.all((out[:, 5] & 0x7F) == 0x7F)
    big = np.abs(ref.yq) > 464
    assert big.sum() > 100000
    assert np.all((out[:, :hq][big] & 0x7F) == 0x7E)
    _compare(out, ref, f"fp8 gamma in registers op={op}")


@pytest.mark.parametrize("T", [4501, 8192])
def test_fp8_headwise_two_groups_per_block(T):
    """FP8 headwise launches from 4096 tokens: blocks take two token groups
    (4501 tokens: the last block one), 128-wide heads of the GQA widths,
    every element against the oracle."""
    w = I.GQA_PREFILL_FP8.with_T(T)
    plan = qk.describe_headwise_plan(w.hq, w.hk, T, 128, "fp8", 0, ld=w.ld)
    _log(f"[case] fp8 headwise T={T} plan: {plan}")
    assert "groups/block=2" in plan
    inp = I.make_inputs(w)
    hq, hk = w.hq, w.hk
    host, src, dst = _layout(inp, w.hv)
    dst_init = dst.host()
    x, y = src.view(), dst.view()
    gq, gk = np_to_torch(inp.gamma_q[:128]).to(DEV), np_to_torch(inp.gamma_k[:128]).to(DEV)
    qk.qknorm_headwise(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, 128, 0, y[:, :hq], y[:, hq:hq + hk])
    torch.cuda.synchronize()
    ref = oracle.qknorm_headwise(inp.q, inp.k, inp.gamma_q[:128], inp.gamma_k[:128], "fp8", w.eps, 128, 0)
    _compare(dst.host(), ref, f"fp8 headwise T={T}")
    _untouched(host, src, dst, dst_init, hq, hk)


def test_fp8_elementwise_path():
    _compare(*_fused(I.make_custom(45, 40 * 8, 24, 0, "fp8", seed=901), 8, 1, offset=3), "fp8 misaligned")
    _compare(*_fused(I.make_custom(31, 1000, 200, 0, "fp8", seed=902), 0, 4, ld_pad=1), "fp8 odd stride")
    _compare(*_fused(I.make_custom(19, 120, 24, 0, "fp8", seed=903), 16, 3), "fp8 shard of 40")


def test_fp8_nan_rows():
    inp = I.make_custom(8, 256, 64, 0, "fp8", seed=1001)
    inp.q[3, 7] = 0x7F      # NaN: the whole Q row of token 3 becomes NaN
    inp.k[5, 0] = 0xFF
    out, ref = _fused(inp, 0, 1)
    assert np.all((out[3, :256] & 0x7F) == 0x7F) and np.all((out[5, 256:320] & 0x7F) == 0x7F)
    _compare(out, ref, "fp8 NaN rows")


def test_fp8_in_place_equals_out_of_place():
    inp = I.make_custom(200, 1024, 256, 0, "fp8", seed=1101)
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    oq, ok = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 2, oq, ok)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 2)          # in place
    torch.cuda.synchronize()
    assert torch.equal(xq.view(torch.uint8), oq.view(torch.uint8))
    assert torch.equal(xk.view(torch.uint8), ok.view(torch.uint8))


def test_fp8_many_shards_split_equals_fused():
    inp = I.make_custom(1100, 2048, 512, 0, "fp8", seed=1102)   # 1100 tokens: ragged last block
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    fq, fk = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_fused(xq, xk, gq, gk, 1e-6, 8, fq, fk)
    part = qk.qknorm_partial_stats(xq, xk, 8)
    aq, ak = torch.empty_like(xq), torch.empty_like(xk)
    qk.qknorm_apply_with_stats(xq, xk, gq, gk, 1e-6, part, 2048, 512, aq, ak)
    torch.cuda.synchronize()
    assert torch.equal(fq.view(torch.uint8), aq.view(torch.uint8))
    assert torch.equal(fk.view(torch.uint8), ak.view(torch.uint8))
    ref = oracle.qknorm_fused(inp.q, inp.k, inp.gamma_q, inp.gamma_k, "fp8", 1e-6, 8)
    check_fp8(torch_to_np(fq), ref.yq_bits, "S=8 Q")
    check_fp8(torch_to_np(fk), ref.yk_bits, "S=8 K")
    ref_p = oracle.qknorm_partial_stats(inp.q, inp.k, "fp8", 8)
    got_p = part.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_p - ref_p) <= 1e-5 * ref_p)


def test_fp8_subnormal_inputs_and_results():
    """E4M3 subnormals (multiples of 2^-9) in, results down to the subnormal
    range out (a small gamma)."""
    inp = I.make_custom(64, 512, 128, 0, "fp8", seed=1103)
    rng = np.random.default_rng(1104)
    inp.q[:, ::3] = rng.integers(1, 8, inp.q[:, ::3].shape).astype(np.uint8)        # +subnormals
    inp.k[:, 1::4] = (rng.integers(1, 8, inp.k[:, 1::4].shape) | 0x80).astype(np.uint8)  # -subnormals
    inp.gamma_q[...] = I.to_bf16_bits(np.full(512, 2.0 ** -8))
    out, ref = _fused(inp, 0, 1)
    sub = (ref.yq_bits & 0x78) == 0
    assert sub.sum() > 100                      # many results are E4M3 subnormals
    _compare(out, ref, "fp8 subnormals")


@pytest.mark.parametrize("head_dim,stride", [(64, 0), (64, 64), (80, 0), (72, 72)])
def test_fp8_headwise_head_sizes(head_dim, stride):
    heads_q, heads_k = 12, 4
    hq, hk = heads_q * head_dim, heads_k * head_dim
    inp = I.make_custom(77, hq, hk, 0, "fp8", seed=1200 + head_dim + stride)
    gq_h = inp.gamma_q[:head_dim].copy() if stride == 0 else inp.gamma_q
    gk_h = inp.gamma_k[:head_dim].copy() if stride == 0 else inp.gamma_k
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    oq, ok = torch.empty_like(xq), torch.empty_like(xk)
    _log(f"[case] fp8 headwise head_dim={head_dim} stride={stride} plan: "
         f"{qk.describe_headwise_plan(hq, hk, 77, head_dim, 'fp8', stride)}")
    qk.qknorm_headwise(xq, xk, np_to_torch(gq_h).to(DEV), np_to_torch(gk_h).to(DEV), 1e-6, head_dim, stride, oq, ok)
    torch.cuda.synchronize()
    ref = oracle.qknorm_headwise(inp.q, inp.k, gq_h, gk_h, "fp8", 1e-6, head_dim, stride)
    check_fp8(torch_to_np(oq), ref.yq_bits, "headwise fp8 Q")
    check_fp8(torch_to_np(ok), ref.yk_bits, "headwise fp8 K")


@pytest.mark.parametrize("head_dim,hq,hk", [(96, 3072, 768), (96, 9216, 1536), (80, 5120, 1280), (128, 16384, 2048)])
def test_fp8_headwise_prefill_layouts(head_dim, hq, hk):
    """Prefill launches of FP8 rows (T = 1024, the T = 8192 layouts): per-head
    lane groups of 1 and 2 chunks per lane, and a token-wide layout of 6 chunks."""
    T = 1024
    inp = I.make_custom(T, hq, hk, 0, "fp8", seed=1300 + head_dim + hq // 64)
    gq_h, gk_h = inp.gamma_q[:head_dim].copy(), inp.gamma_k[:head_dim].copy()
    xq, xk = np_to_torch(inp.q).to(DEV), np_to_torch(inp.k).to(DEV)
    oq, ok = torch.empty_like(xq), torch.empty_like(xk)
    _log(f"[case] fp8 headwise prefill head_dim={head_dim} {hq}/{hk} plan: "
         f"{qk.describe_headwise_plan(hq, hk, T, head_dim, 'fp8', 0)}")
    qk.qknorm_headwise(xq, xk, np_to_torch(gq_h).to(DEV), np_to_torch(gk_h).to(DEV), 1e-6, head_dim, 0, oq, ok)
    torch.cuda.synchronize()
    ref = oracle.qknorm_headwise(inp.q, inp.k, gq_h, gk_h, "fp8", 1e-6, head_dim, 0)
    check_fp8(torch_to_np(oq), ref.yq_bits, "headwise fp8 Q")
    check_fp8(torch_to_np(ok), ref.yk_bits, "headwise fp8 K")

"""Property tests of the host planners (CPU only, no kernel runs): for many
shapes, every launch the library would make fits the kernel it picks (slot
counts that exist, block sizes within that kernel's register budget, lane
groups that cover every chunk, LDS sized for the block), and a shape is
refused as unsupported only when no layout of the kernel family holds it."""

import re

import pytest
from hypothesis import given, settings, strategies as st

import layerwise_qk_norm_qknorm_amd as qk

SLOTS = (1, 2, 3, 4, 6, 8, 12, 16)
VW = {"bf16": 8, "f32": 4, "fp8": 16}
UNSUPPORTED = 2


def max_threads(v, dtype, aligned):
    lim = (3 if dtype == "fp8" else 8) if aligned else {"f32": 6, "bf16": 4, "fp8": 1}[dtype]
    return 1024 if v <= lim else 256


def max_slots(dtype, aligned):
    return 8 if (dtype == "fp8" and not aligned) else 16


def slots_for(n, dtype, aligned):
    for s in SLOTS:
        if s >= n:
            return s if s <= max_slots(dtype, aligned) else 0
    return 0


def fields(desc):
    return {k: v for k, v in re.findall(r"([a-z_/]+)=(\S+)", desc)}


def ceil_div(a, b):
    return -(-a // b)


def feasible_layerwise(nc, shards, T, dtype, aligned):
    sub_wave = shards == 1 and T >= 1024
    ls = [4, 8, 16, 32] + list(range(64, 1025, 64))
    for l in ls:
        if shards > 1 and (l & (l - 1)):
            continue
        g = shards * l
        if g > 1024 or (g % 64 and not (sub_wave and g < 64)):
            continue
        v = slots_for(ceil_div(nc, l), dtype, aligned)
        if v and g <= max_threads(v, dtype, aligned):
            return True
    return False


@settings(max_examples=400, deadline=None, derandomize=True)
@given(dtype=st.sampled_from(["bf16", "f32", "fp8"]), shards=st.sampled_from([1, 1, 2, 3, 4, 8, 16, 64]),
       hq_s=st.integers(1, 9000), hk_s=st.integers(1, 3000), T=st.sampled_from([1, 7, 100, 1023, 1024, 5000, 100000]),
       op=st.sampled_from([0, 1, 2]), unaligned=st.booleans())
def test_layerwise_plans_fit_their_kernels(dtype, shards, hq_s, hk_s, T, op, unaligned):
    vw = VW[dtype]
    if not unaligned:  # whole 16-byte chunks per shard: the 16-byte path
        hq_s, hk_s = ceil_div(hq_s, vw) * vw, ceil_div(hk_s, vw) * vw
    hq, hk = hq_s * shards, hk_s * shards
    ld = hq + hk + (1 if unaligned else 0)
    if op == 2:  # apply_with_stats takes combined statistics: one shard over the local width
        shards, hq_s, hk_s = 1, hq, hk
    nc = ceil_div(hq_s, vw) + ceil_div(hk_s, vw)
    try:
        d = qk.describe_plan(op, hq, hk, T, dtype, shards, ld=ld)
    except qk.QKNormError as e:
        assert e.status == UNSUPPORTED
        aligned = not unaligned
        assert not feasible_layerwise(nc, shards, T, dtype, aligned), "a feasible shape was refused"
        return
    f = fields(d)
    aligned = f["path"] == "16B"
    assert aligned == (not unaligned)
    lanes, slots = int(f["lanes/shard"]), int(f["slots"])
    G, tpb, lds = int(f["threads/token"]), int(f["tokens/block"]), int(f["lds"])
    assert f["chunks"] == f"({ceil_div(hq_s, vw)},{ceil_div(hk_s, vw)})"
    assert slots in SLOTS and slots <= max_slots(dtype, aligned)
    assert lanes * slots >= nc                       # every chunk has a lane slot
    assert G == shards * lanes
    if shards > 1:
        assert lanes & (lanes - 1) == 0
    if G % 64:                                       # several tokens per wave
        assert G < 64 and 64 % G == 0 and shards == 1 and T >= 1024
    assert tpb >= 1 and (tpb == 1 or G <= 64)
    if f.get("form") == "slot-waves":
        # partial_stats, one shard, a token of 32 or 64 lanes: one wave per
        # chunk slot of a wave's lanes, one wave's worth of tokens per block
        assert op == 1 and shards == 1 and aligned and lanes in (32, 64) and 2 <= slots <= 4
        assert tpb == 64 // lanes and int(f["threads/block"]) == 64 * slots and lds == 0
        assert int(f["xcd_run"]) * tpb == 128
        return
    assert tpb * G <= max_threads(slots, dtype, aligned)
    waves = ceil_div(G, 64)
    group = min(lanes, 64)
    assert lds == (2 * tpb * (G // group) * 2 * 4 if waves > 1 else 0)
    assert lds <= 64 * 1024
    # token groups per block: only FP8 rows of the fused and apply calls on
    # the 16-byte path loop, over 2 to 4 groups, and only when the launch
    # holds one to four grids of 4096 waves
    k = int(f.get("groups/block", 1))
    groups = ceil_div(T, tpb)
    cap = 4096 // ceil_div(tpb * G, 64)
    if dtype == "fp8" and aligned and op != 1 and cap < groups <= 4 * cap:
        assert k == ceil_div(groups, cap)
    else:
        assert k == 1, f
    assert 1 <= k <= 4
    # residency cap: only fused bf16 launches of one shard whose tokens fill
    # 4 waves x 3 chunks with no idle slot, from 6144 tokens
    cap = f.get("max_blocks/cu")
    if op == 0 and dtype == "bf16" and aligned and shards == 1 and (G, slots) in ((256, 3), (192, 4)) and tpb == 1 \
            and lanes * slots == nc and T >= 3072:
        assert cap == "5", f
    else:
        assert cap is None, f


def feasible_headwise(heads, nc, dtype, aligned):
    if nc > 64 * 8 or heads * 4 > 1024:
        return False
    l = 4
    while l <= 64:
        v = slots_for(ceil_div(nc, l), dtype, aligned)
        if v and ceil_div(heads * l, 64) * 64 <= max_threads(v, dtype, aligned):
            return True
        l *= 2
    return False


@settings(max_examples=300, deadline=None, derandomize=True)
@given(dtype=st.sampled_from(["bf16", "f32", "fp8"]), head_dim=st.sampled_from([8, 16, 36, 64, 72, 96, 128, 256,
                                                                               512, 2048, 4096]),
       hq_heads=st.integers(1, 128), hk_heads=st.integers(1, 32), T=st.sampled_from([1, 50, 1023, 4096]),
       stride0=st.booleans())
def test_headwise_plans_fit_their_kernels(dtype, head_dim, hq_heads, hk_heads, T, stride0):
    hq, hk = hq_heads * head_dim, hk_heads * head_dim
    vw = VW[dtype]
    nc = ceil_div(head_dim, vw)
    heads = hq_heads + hk_heads
    try:
        d = qk.describe_headwise_plan(hq, hk, T, head_dim, dtype, 0 if stride0 else head_dim)
    except qk.QKNormError as e:
        assert e.status == UNSUPPORTED
        aligned = head_dim % vw == 0
        assert not feasible_headwise(heads, nc, dtype, aligned), "a feasible headwise shape was refused"
        return
    f = fields(d)
    aligned = f["path"] == "16B"
    slots, G, tpb, threads = int(f["slots"]), int(f["threads/token"]), int(f["tokens/block"]), int(f["threads/block"])
    assert f["heads"] == f"({hq_heads},{hk_heads})" and int(f["chunks/head"]) == nc
    assert slots in SLOTS and slots <= max_slots(dtype, aligned)
    assert threads % 64 == 0 and threads >= tpb * G and threads <= max_threads(slots, dtype, aligned)
    if f["layout"] == "token-wide":
        assert nc & (nc - 1) == 0 and nc <= 64 and G % 64 == 0
        assert G * slots >= heads * nc
    else:
        lanes = int(f["lanes/head"])
        assert lanes & (lanes - 1) == 0 and lanes * slots >= nc and G == heads * lanes


# The prefill launches the planner makes for the widths of inputs.PREFILL_WIDTHS
# at T = 8192 (lanes per token, chunks per lane). Each was the fastest of every
# feasible lane layout timed on MI355X for that width and row type, or within
# 2.2% of it.
PREFILL_PLANS = {
    "bf16": [(64, 3), (128, 3), (192, 3), (256, 3), (256, 3), (320, 3), (384, 3), (448, 4), (768, 3), (448, 3)],
    "fp8": [(32, 3), (64, 3), (128, 2), (128, 3), (128, 3), (256, 2), (192, 3), (256, 4), (192, 6), (256, 3)],
    "f32": [(128, 3), (256, 3), (256, 4), (320, 4), (512, 3), (448, 4), (384, 6), (576, 6), (768, 6), (448, 6)],
}


@pytest.mark.parametrize("dtype", sorted(PREFILL_PLANS))
def test_prefill_plans_are_the_measured_best(dtype):
    from layerwise_qk_norm_qknorm_amd import inputs as I
    for (hq, hk, hv), (lanes, slots) in zip(I.PREFILL_WIDTHS, PREFILL_PLANS[dtype]):
        f = fields(qk.describe_plan(0, hq, hk, 8192, dtype, 1, ld=hq + hk + hv))
        assert (int(f["lanes/shard"]), int(f["slots"])) == (lanes, slots), (dtype, hq, hk, f)


# A mid-size fused bf16 launch (T = 1536, rows 4096/4096): the mid-size rule's
# 256 lanes x 4 chunks; the prefill rule's 384 x 3 timed 12 to 32% slower on
# MI355X for these rows (the worst case of that rule at mid sizes). partial_stats
# takes the same layout (its sums must be added as the fused call adds them);
# apply_with_stats and launches above 4096 tokens keep the prefill rule (only
# fused launches of 1024 to 4096 tokens were timed for the mid-size rule).
def test_mid_size_fused_bf16_plan():
    for op in (0, 1):
        f = fields(qk.describe_plan(op, 4096, 4096, 1536, "bf16", 1, ld=3 * 4096))
        assert (int(f["lanes/shard"]), int(f["slots"])) == (256, 4), (op, f)
    g = fields(qk.describe_plan(2, 4096, 4096, 1536, "bf16", 1, ld=3 * 4096))
    assert (int(g["lanes/shard"]), int(g["slots"])) == (384, 3), g
    h = fields(qk.describe_plan(0, 4096, 4096, 6144, "bf16", 1, ld=3 * 4096))
    assert (int(h["lanes/shard"]), int(h["slots"])) == (384, 3), h


# FP8 launches of one to four grids of 4096 waves loop each block over
# k = ceil(groups / grid) token groups (2-3% faster for the GQA prefill rows at
# 8192 tokens, 3-8% for the rank-slice apply on MI355X); larger launches,
# partial_stats, bf16 rows and the decode sizes keep one group per block.
def test_fp8_token_loop_plans():
    def k(op, hq, hk, T, dtype="fp8", ld=None):
        return int(fields(qk.describe_plan(op, hq, hk, T, dtype, 1, ld=ld or hq + hk + hk)).get("groups/block", 1))
    assert k(0, 5120, 1024, 8192) == 4        # 2-wave tokens, one per block: 8192 groups over 2048 blocks
    assert k(0, 5120, 1024, 4096) == 2
    assert k(0, 5120, 1024, 2048) == 1        # one grid of 4096 waves or less
    assert k(0, 5120, 1024, 16384) == 1       # more than four grids
    assert k(2, 1280, 256, 16384) == 2        # rank-slice apply: 8 tokens of 32 lanes per 4-wave block
    assert k(1, 1280, 256, 16384) == 1        # partial_stats never loops
    assert k(0, 5120, 1024, 8192, "bf16") == 1
    assert k(2, 1280, 256, 16384, "bf16") == 1
    assert k(0, 4096, 4096, 256) == 1         # decode sizes
    # looping launches of up to 4 slots hold gamma widened in registers
    def gr(op, hq, hk, T):
        return "gamma=registers" in qk.describe_plan(op, hq, hk, T, "fp8", 1, ld=hq + 2 * hk)
    assert gr(0, 5120, 1024, 8192) and gr(2, 1280, 256, 16384)
    assert not gr(0, 5120, 1024, 16384) and not gr(0, 5120, 1024, 2048) and not gr(1, 1280, 256, 16384)


# GQA-prefill-shaped fused bf16 launches (5120/1024: 4 waves x 3 chunks per
# token, or 3 x 4 in the mid-size layout, no idle slot) from 3072 tokens run
# at most 5 blocks per compute unit (0.9-1.8% faster on MI355X); the same token
# width with idle slots, fewer tokens, the split calls and FP8 rows keep the
# register-bound residency.
def test_gqa_prefill_residency_cap():
    def cap(op, hq, hk, T, dtype="bf16"):
        return fields(qk.describe_plan(op, hq, hk, T, dtype, 1, ld=hq + 2 * hk)).get("max_blocks/cu")
    assert cap(0, 5120, 1024, 8192) == "5"
    assert cap(0, 5120, 1024, 6144) == "5"
    assert cap(0, 5120, 1024, 16384) == "5"
    assert cap(0, 5120, 1024, 4096) == "5"     # the mid-size layout, 3 waves x 4 chunks
    assert cap(0, 5120, 1024, 3072) == "5"
    assert cap(0, 5120, 1024, 2048) is None
    assert cap(0, 4096, 1024, 8192) is None     # a sixth of the slots idle
    assert cap(1, 5120, 1024, 8192) is None     # partial_stats
    assert cap(2, 5120, 1024, 8192) is None     # apply_with_stats
    assert cap(0, 5120, 1024, 8192, "fp8") is None


# FP8 headwise launches (token-wide layout) from 4096 token groups take two
# groups per block (1-7% faster on MI355X); bf16 rows and fewer tokens one.
def test_fp8_headwise_two_groups_per_block():
    def k(hq, hk, T, dtype="fp8"):
        d = qk.describe_headwise_plan(hq, hk, T, 128, dtype, 0, ld=hq + 2 * hk)
        return int(fields(d).get("groups/block", 1))
    assert k(5120, 1024, 8192) == 2 and k(5120, 1024, 4096) == 2 and k(16384, 2048, 8192) == 2
    assert k(5120, 1024, 4095) == 1 and k(5120, 1024, 256) == 1
    assert k(5120, 1024, 8192, "bf16") == 1 and k(5120, 1024, 8192, "f32") == 1


# The split path reproduces the fused call bit for bit only if partial_stats
# adds each shard's squares in the fused call's order: the same path, lanes per
# shard and chunks per lane (which fix the in-lane order and the lane
# butterfly) for every shape, shard count, token count and alignment.
@settings(max_examples=400, deadline=None, derandomize=True)
@given(dtype=st.sampled_from(["bf16", "f32", "fp8"]), shards=st.sampled_from([1, 1, 2, 4, 8, 64]),
       hq_s=st.integers(1, 6000), hk_s=st.integers(1, 2000),
       T=st.sampled_from([1, 8, 256, 1023, 1024, 1536, 2048, 4096, 4097, 8192, 16384]), unaligned=st.booleans())
def test_partial_stats_takes_the_fused_reduction_layout(dtype, shards, hq_s, hk_s, T, unaligned):
    vw = VW[dtype]
    if not unaligned:
        hq_s, hk_s = ceil_div(hq_s, vw) * vw, ceil_div(hk_s, vw) * vw
    hq, hk = hq_s * shards, hk_s * shards
    ld = hq + hk + (1 if unaligned else 0)
    try:
        fused = fields(qk.describe_plan(0, hq, hk, T, dtype, shards, ld=ld))
    except qk.QKNormError as e:
        assert e.status == UNSUPPORTED
        with pytest.raises(qk.QKNormError):
            qk.describe_plan(1, hq, hk, T, dtype, shards, ld=ld)
        return
    stats = fields(qk.describe_plan(1, hq, hk, T, dtype, shards, ld=ld))
    for key in ("path", "shards", "chunks", "lanes/shard", "slots"):
        assert fused[key] == stats[key], (key, fused, stats)


def prefill_candidates(nc, dtype):
    """(lanes, slots, waves, idle fraction) of every feasible one-shard layout
    of a prefill launch (T >= 1024) on the 16-byte path."""
    out = []
    for l in [4, 8, 16, 32] + list(range(64, 1025, 64)):
        if l % 64 and l > 64:
            continue
        v = slots_for(ceil_div(nc, l), dtype, True)
        if v and l <= max_threads(v, dtype, True):
            out.append((l, v, ceil_div(l, 64), (l * v - nc) / (l * v)))
    return out


@settings(max_examples=300, deadline=None, derandomize=True)
@given(dtype=st.sampled_from(["bf16", "f32", "fp8"]), hq=st.integers(1, 1024), hk=st.integers(1, 256),
       T=st.sampled_from([1024, 8192, 65536]))
def test_prefill_plans_follow_the_measured_rules(dtype, hq, hk, T):
    """Whenever a layout without the measured slow features fits, the planner
    avoids them: one chunk per lane, more than a quarter of the slots idle,
    blocks of 13 or more waves, and FP8 tokens over 5 or more waves."""
    vw = VW[dtype]
    hq, hk = hq * vw, hk * vw
    nc = (hq + hk) // vw
    f = fields(qk.describe_plan(0, hq, hk, T, dtype, 1))
    l, v = int(f["lanes/shard"]), int(f["slots"])
    waves, idle = ceil_div(l, 64), (l * v - nc) / (l * v)
    cands = prefill_candidates(nc, dtype)
    assert (l, v) in [(c[0], c[1]) for c in cands]

    def good(c):
        ok = c[1] > 1 and c[3] <= 0.25 and c[2] < 13
        return ok and (c[2] <= 4 if dtype == "fp8" else True)

    if any(good(c) for c in cands):
        assert good((l, v, waves, idle)), (dtype, hq, hk, T, f)


# Few-token launches (lanes per token, chunks per lane), each the fastest
# layout timed under graph replay on MI355X or within 2.9% of it.
DECODE_PLANS = [("bf16", 4096, 4096, 512, 2), ("bf16", 8192, 1024, 384, 3), ("bf16", 2048, 512, 192, 2),
                ("fp8", 16384, 2048, 384, 3), ("fp8", 5120, 1024, 192, 2), ("fp8", 2048, 512, 192, 1)]


@pytest.mark.parametrize("T", [1, 8, 64, 256])
def test_decode_plans_are_the_measured_best(T):
    for dtype, hq, hk, lanes, slots in DECODE_PLANS:
        f = fields(qk.describe_plan(0, hq, hk, T, dtype, 1))
        assert (int(f["lanes/shard"]), int(f["slots"])) == (lanes, slots), (dtype, hq, hk, T, f)


@settings(max_examples=300, deadline=None, derandomize=True)
@given(dtype=st.sampled_from(["bf16", "f32", "fp8"]), hq=st.integers(1, 1024), hk=st.integers(1, 256),
       T=st.sampled_from([1, 8, 64, 1023]))
def test_decode_plans_stay_within_8_waves(dtype, hq, hk, T):
    """A few-token launch spreads a token over at most 8 waves whenever a
    layout of at most 8 waves, at most 3 chunks per lane and at most a
    quarter of the slots idle fits."""
    vw = VW[dtype]
    hq, hk = hq * vw, hk * vw
    nc = (hq + hk) // vw
    f = fields(qk.describe_plan(0, hq, hk, T, dtype, 1))
    waves = ceil_div(int(f["lanes/shard"]), 64)
    cands = [c for c in prefill_candidates(nc, dtype) if c[0] % 64 == 0]
    if any(c[2] <= 8 and c[1] <= 3 and c[3] <= 0.25 for c in cands):
        assert waves <= 8, (dtype, hq, hk, T, f)


# Headwise prefill launches for 128-wide heads over the same widths (threads
# per token, chunks per lane): each the fastest token width timed on MI355X
# or within 3.4% of it. The narrowest bf16 and fp32 rows, where every width
# timed the same (host-bound launches), are pinned as they are; the
# narrowest FP8 rows (10 heads of 8 chunks) take the per-head layout, 6
# tokens of 80 lanes to a block: 7.5 us against 11.2 us for the best
# token-wide launch (256 threads per token).
HEADWISE_PREFILL_PLANS = {
    "bf16": [(64, 3), (192, 2), (256, 2), (384, 2), (512, 2), (576, 2), (768, 2), (1024, 2), (1024, 3), (832, 2)],
    "fp8": [(80, 1), (192, 1), (128, 2), (192, 2), (192, 2), (256, 2), (192, 3), (256, 4), (192, 6), (256, 3)],
    "f32": [(192, 2), (384, 2), (640, 2), (832, 2), (1024, 2), (1024, 2), (1024, 3), (1024, 4), (1024, 6), (1024, 3)],
}


@pytest.mark.parametrize("dtype", sorted(HEADWISE_PREFILL_PLANS))
def test_headwise_prefill_plans_are_the_measured_best(dtype):
    from layerwise_qk_norm_qknorm_amd import inputs as I
    for (hq, hk, hv), (threads, slots) in zip(I.PREFILL_WIDTHS, HEADWISE_PREFILL_PLANS[dtype]):
        f = fields(qk.describe_headwise_plan(hq, hk, 8192, 128, dtype, 0, ld=hq + hk + hv))
        assert (int(f["threads/token"]), int(f["slots"])) == (threads, slots), (dtype, hq, hk, f)
        assert f["layout"] == ("per-head" if (dtype, hq) == ("fp8", 1024) else "token-wide"), (dtype, hq, hk, f)


# Per-head headwise prefill launches (heads whose chunk count is not a power
# of two): (lanes per head, chunks per lane), each the fastest lane group
# timed on MI355X except the fp32 3072/3072 case (within 5.2%).
PER_HEAD_PLANS = [("bf16", 96, 3072, 768, 8, 2), ("bf16", 80, 5120, 1280, 8, 2), ("fp8", 96, 3072, 768, 8, 1),
                  ("fp8", 96, 9216, 1536, 4, 2), ("fp8", 80, 5120, 1280, 4, 2), ("f32", 96, 6144, 768, 8, 3),
                  ("f32", 80, 2560, 640, 8, 3), ("f32", 96, 3072, 3072, 8, 3)]


def test_per_head_prefill_plans_are_the_measured_best():
    for dtype, hd, hq, hk, lanes, slots in PER_HEAD_PLANS:
        f = fields(qk.describe_headwise_plan(hq, hk, 8192, hd, dtype, 0, ld=hq + 2 * hk))
        assert f["layout"] == "per-head"
        assert (int(f["lanes/head"]), int(f["slots"])) == (lanes, slots), (dtype, hd, hq, hk, f)


# The large-token cases of the random GPU sweep reach every launch rule that
# only applies from thousands of tokens (checked here on the CPU, from the
# plans those cases describe).
def test_large_random_cases_cover_the_launch_rules():
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "random_shapes", os.path.join(os.path.dirname(__file__), "test_random_shapes_gpu.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    seen = set()
    for c in m.large_cases():
        ld = c["hq"] + c["hk"] + c["hv"]
        if c["op"] == "headwise":
            d = qk.describe_headwise_plan(c["hq"], c["hk"], c["T"], 128, c["dtype"], 0, ld=ld)
            seen |= {"headwise loop"} if "groups/block=2" in d else set()
        else:
            d = qk.describe_plan(0 if c["op"] == "fused" else 2, c["hq"], c["hk"], c["T"], c["dtype"], 1, ld=ld)
            seen |= {f for f in ("groups/block", "gamma=registers", "max_blocks/cu") if f in d}
            if c["op"] == "split" and "gamma=registers" in d:
                seen.add("split gamma=registers")
    assert seen >= {"headwise loop", "groups/block", "gamma=registers", "max_blocks/cu", "split gamma=registers"}, seen

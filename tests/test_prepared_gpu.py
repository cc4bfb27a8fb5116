"""PreparedCall (the binding's calls checked and marshalled once): the same
launches as the plain calls, byte for byte, on the current stream or an
explicit one, and again after the inputs change in place."""

import numpy as np
import pytest
import torch

import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, np_to_torch, torch_to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _packed(w, seed):
    inp = I.make_inputs(w)
    x = np_to_torch(inp.qkv).to(DEV)
    return inp, x


@pytest.mark.parametrize("key,shards", [("decode_t1", 1), ("decode_t64", 4), ("rank_slice", 1)])
def test_prepared_fused_equals_the_plain_call(key, shards):
    w = I.WORKLOADS[key] if key != "rank_slice" else I.WORKLOADS[key].with_T(2048)
    print(f"[case] prepared fused {key} S={shards}", flush=True)
    inp, x = _packed(w, 0)
    hq, hk = w.hq, w.hk
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    y1, y2 = torch.zeros_like(x), torch.zeros_like(x)
    qk.qknorm_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, shards, y1[:, :hq], y1[:, hq:hq + hk])
    call = qk.prepare_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, shards, y2[:, :hq], y2[:, hq:hq + hk])
    call()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # inputs changed in place: the prepared call reads the new values
    x.mul_(2)
    y2.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    call(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    qk.qknorm_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, shards, y1[:, :hq], y1[:, hq:hq + hk])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_prepared_split_path_equals_the_plain_calls():
    w = I.WORKLOADS["rank_slice"].with_T(3001)
    print("[case] prepared partial_stats + apply rank_slice T=3001", flush=True)
    inp, x = _packed(w, 0)
    hq, hk = w.hq, w.hk
    q, k = x[:, :hq], x[:, hq:hq + hk]
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    p1 = qk.qknorm_partial_stats(q, k, 1)
    p2 = torch.full_like(p1, float("nan"))
    qk.prepare_partial_stats(q, k, 1, p2)()
    torch.cuda.synchronize()
    assert torch.equal(p1.view(torch.int32), p2.view(torch.int32))
    stats = torch.cat([p1, p1 * 1.5, p1 * 0.25], dim=0).contiguous()
    y1, y2 = torch.zeros_like(x), torch.zeros_like(x)
    qk.qknorm_apply_with_stats(q, k, gq, gk, w.eps, stats, w.hq_full, w.hk_full, y1[:, :hq], y1[:, hq:hq + hk])
    out = qk.prepare_apply_with_stats(q, k, gq, gk, w.eps, stats, w.hq_full, w.hk_full, y2[:, :hq],
                                      y2[:, hq:hq + hk])()
    torch.cuda.synchronize()
    assert out[0].data_ptr() == y2.data_ptr()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert not torch_to_np(y2)[:, hq + hk:].any()   # V columns untouched


def test_prepared_call_reports_library_errors():
    w = I.WORKLOADS["decode_t1"]
    inp, x = _packed(w, 0)
    hq, hk = w.hq, w.hk
    gq, gk = np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV)
    with pytest.raises(qk.QKNormError):
        qk.prepare_fused(x[:, :hq], x[:, hq:hq + hk], gq, gk, float("nan"), 1)()   # eps must be finite


def test_prepared_headwise_equals_the_plain_call():
    w = I.WORKLOADS["decode_t64"]
    print("[case] prepared headwise decode_t64", flush=True)
    inp, x = _packed(w, 0)
    hq, hk = w.hq, w.hk
    gq, gk = np_to_torch(inp.gamma_q[:128].copy()).to(DEV), np_to_torch(inp.gamma_k[:128].copy()).to(DEV)
    y1, y2 = torch.zeros_like(x), torch.zeros_like(x)
    qk.qknorm_headwise(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, 128, 0, y1[:, :hq], y1[:, hq:hq + hk])
    qk.prepare_headwise(x[:, :hq], x[:, hq:hq + hk], gq, gk, w.eps, 128, 0, y2[:, :hq], y2[:, hq:hq + hk])()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))

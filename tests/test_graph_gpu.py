"""The entry points under HIP graph capture: qknorm_fused, the split path
(qknorm_partial_stats + qknorm_apply_with_stats) and qknorm_headwise are
captured into one graph, which is replayed several times with eager work and
synchronizations in between (new inputs written eagerly before each replay);
every replay must equal, bit for bit, the same calls made eagerly."""

import pytest
import torch

import layerwise_qk_norm_qknorm_amd as qk
from layerwise_qk_norm_qknorm_amd import inputs as I
from gpu_helpers import DEV, np_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qk.load_library()
    yield
    torch.cuda.synchronize()


def _calls(x, g, outs, hq, hk, hd):
    """The captured sequence: fused S=2, split path, headwise, on packed rows x."""
    q, k = x[:, :hq], x[:, hq:hq + hk]
    yf, ya, yh, part = outs
    qk.qknorm_fused(q, k, g[0], g[1], 1e-6, 2, yf[:, :hq], yf[:, hq:hq + hk])
    qk.qknorm_partial_stats(q, k, 2, part)
    qk.qknorm_apply_with_stats(q, k, g[0], g[1], 1e-6, part, hq, hk, ya[:, :hq], ya[:, hq:hq + hk])
    qk.qknorm_headwise(q, k, g[2], g[3], 1e-6, hd, 0, yh[:, :hq], yh[:, hq:hq + hk])


def test_graph_replays_equal_eager_calls():
    T, hq, hk, hd = 1500, 1024, 256, 128
    inp = I.make_custom(T, hq, hk, 0, "bf16", seed=4242)
    x = torch.empty((T, hq + hk), dtype=torch.bfloat16, device=DEV)
    x[:, :hq] = np_to_torch(inp.q).to(DEV)
    x[:, hq:] = np_to_torch(inp.k).to(DEV)
    g = [np_to_torch(inp.gamma_q).to(DEV), np_to_torch(inp.gamma_k).to(DEV),
         np_to_torch(inp.gamma_q[:hd]).to(DEV), np_to_torch(inp.gamma_k[:hd]).to(DEV)]
    outs = [torch.zeros_like(x), torch.zeros_like(x), torch.zeros_like(x),
            torch.zeros((2, 2, T), dtype=torch.float32, device=DEV)]
    ref = [torch.zeros_like(o) for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _calls(x, g, outs, hq, hk, hd)          # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _calls(x, g, outs, hq, hk, hd)
    torch.cuda.synchronize()

    gen = torch.Generator(device=DEV)
    for rep in range(4):
        gen.manual_seed(100 + rep)
        x.copy_(torch.randn(x.shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16))  # eager
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _calls(x, g, ref, hq, hk, hd)          # the same calls, eagerly
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), f"replay {rep}"
        assert not torch.equal(outs[0], torch.zeros_like(outs[0]))
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))  # fused == split

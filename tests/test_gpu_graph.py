"""The path under HIP graph capture: the calls allocate nothing and record no
memset, so a captured step (restore q and k, prologue in place, attention)
must replay to the same bits as the eager step, replay after replay, with
other eager work and synchronisations in between."""
import pytest

from exact_head_attention_amd import inputs as I
from tests.gpu_helpers import device_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,L", [(2, 1000), (7, 4096)])
def test_step_replays_bit_identical_under_graph_capture(gpu_lib, H, L):
    import torch
    x = I.make_inputs(I.custom_workload(H=H, L=L, n_audio=L // 8), seed=9)
    d = device_inputs(x)
    cos, sin = gpu_lib.rope_tables(d["positions"], 128, x["theta"])
    q0, k0 = d["q"].clone(), d["k"].clone()
    q, k = torch.empty_like(q0), torch.empty_like(k0)
    out = torch.empty_like(q0)

    def step():
        q.copy_(q0)
        k.copy_(k0)
        gpu_lib.qknorm_rope(q, k, d["gamma_q"], d["gamma_k"], cos, sin, x["eps"])
        gpu_lib.attention(q, k, d["v"], out=out, scale=x["scale"])

    step()
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                       # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk

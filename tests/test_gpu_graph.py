"""Decode steps captured in a HIP graph: several replays, with eager work and
synchronisations between them, each checked bit for bit against the same
steps run eagerly on a copy of the state (the replayed kernels must read the
inputs and state of every replay, not of the capture)."""
from __future__ import annotations

import numpy as np
import pytest

from linear_attention_recurrent_rule_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests import gpu_util as gu  # noqa: E402


@pytest.mark.parametrize("d,n8,B,hv,hk", [(128, 64, 16, 8, 4), (64, 32, 8, 4, 4)])
def test_graph_replays_match_eager(d, n8, B, hv, hk):
    steps = 4
    ps = wl.random_packed_state(B, hv, d, n8, seed=71 + d)
    eager = gu.make_state(B, hv, hk, d, n8)
    graphed = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(eager, ps)
    gu.load_packed(graphed, ps)
    xs = [gu.inputs_to_device(wl.draw_inputs(B, hk, hv, d, dtype="bf16", seed=71, step=t))
          for t in range(steps)]
    o_eager = torch.empty((steps, B, hv, d), dtype=torch.float32, device="cuda")
    o_graph = torch.empty_like(o_eager)
    # warm the capture stream, then capture `steps` decode launches
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    scratch = gu.make_state(B, hv, hk, d, n8)
    gu.load_packed(scratch, ps)
    with torch.cuda.stream(side):
        for t in range(steps):
            scratch.decode_step(*xs[t], o=o_graph[t])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            graphed.decode_step(*xs[t], o=o_graph[t])
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[case] graph replay {rep} d={d}", flush=True)
        for t in range(steps):
            eager.decode_step(*xs[t], o=o_eager[t])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), f"replay {rep}: readout differs"
        assert torch.equal(graphed.pool8, eager.pool8) and torch.equal(graphed.pool4, eager.pool4)
        assert torch.equal(graphed.r, eager.r)
        o_graph.zero_()  # eager work between replays

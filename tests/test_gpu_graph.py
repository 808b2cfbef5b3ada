"""moe_layer_forward captured in a HIP graph (the benchmark replays decode
steps this way): every replay must reproduce the eager result bit for bit.

Replays are separated by eager work on the same buffers and by
synchronisations, so a graph node that only works on its first replay (or
that depends on state the eager calls leave behind) shows up as a mismatch.
The path records no memset nodes: every buffer the kernels need cleared is
written by a kernel.
"""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import moe_inputs as G
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


def _setup(cfg):
    dev = torch.device("cuda", 0)
    inp = G.make_layer_inputs(cfg)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    w = M.W4Weights.from_numpy(inp["weights"], device=dev)
    dm = M.dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k)
    ws = torch.empty(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    return x, logits, w, dm, ws


@pytest.mark.parametrize("cfg", [
    G.small_config("graph_prefill_t300", T=300, d=256, f=128, E=16, k=4, seed=41, zipf_s=1.1),
    G.small_config("graph_prefill_t700", T=700, d=512, f=256, E=64, k=8, seed=42),
    G.small_config("graph_decode_t1", T=1, d=2048, f=512, E=256, k=8, seed=43),
    G.small_config("graph_decode_t5", T=5, d=512, f=256, E=64, k=8, seed=44),
    # the decode kernels' other splits: one unit per gate/up wavefront with
    # several slots per down wavefront (T = 3), one down wavefront per
    # workgroup (T = 12)
    G.small_config("graph_decode_t3", T=3, d=2048, f=512, E=256, k=8, seed=45),
    G.small_config("graph_decode_t12", T=12, d=256, f=128, E=32, k=8, seed=46),
], ids=lambda c: c.name)
def test_graph_replays_match_eager(cfg):
    say(f"[graph] {cfg.name}")
    x, logits, w, dm, ws = _setup(cfg)
    wc = w.c()
    y_eager = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=x.device)
    M.moe_layer_forward(dm, x, logits, w, y=y_eager, ws=ws, wc=wc)
    torch.cuda.synchronize()
    ref = y_eager.clone()

    y_graph = torch.full_like(y_eager, float("nan"))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        M.moe_layer_forward(dm, x, logits, w, y=y_graph, ws=ws, wc=wc, stream=s)  # warm-up on s
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            M.moe_layer_forward(dm, x, logits, w, y=y_graph, ws=ws, wc=wc, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        y_graph.fill_(float("nan"))
        # eager work on the same workspace between replays
        M.moe_layer_forward(dm, x, logits, w, y=y_eager, ws=ws, wc=wc)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref), f"replay {rep} differs from the eager result"
        assert torch.equal(y_eager, ref)

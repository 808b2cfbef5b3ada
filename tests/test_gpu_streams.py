"""Layer calls on different streams share no state: three layers of different
shapes (the grouped path, its one-row-block GEMM build, and the per-token
decode kernels), each with its own workspace, enqueued many times over on
three streams so that their kernels run side by side, give the bits of the same
calls made one at a time; the hidden-state entry runs beside them too."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import moe_inputs as G
from parity_util import dev_bits, say, upload

pytestmark = pytest.mark.gpu

CFGS = [
    G.small_config("st_t300", T=300, d=512, f=256, E=32, k=4, seed=111, zipf_s=1.1),
    G.small_config("st_t24", T=24, d=2048, f=512, E=256, k=8, seed=112),
    G.small_config("st_t5", T=5, d=1024, f=256, E=64, k=8, seed=113),
]
ROUNDS = 12


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


def test_concurrent_streams_match_serial_calls():
    runs = []
    for cfg in CFGS:
        inp = G.make_layer_inputs(cfg)
        dm, x, logits, w = upload(inp)
        ws = torch.empty(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
        y_ref = M.moe_layer_forward(dm, x, logits, w, ws=ws)
        runs.append(dict(cfg=cfg, dm=dm, x=x, logits=logits, w=w, wc=w.c(), ws=ws, y_ref=y_ref))
    # the hidden-state entry of the first shape, with its own router weights
    h = runs[0]
    wr = dev_bits(G.make_router(h["cfg"]))
    ws_h = torch.empty(M.moe_layer_workspace_bytes(h["dm"]), dtype=torch.uint8, device="cuda")
    yh_ref = M.moe_layer_forward_hidden(h["dm"], h["x"], wr, h["w"], ws=ws_h)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(len(runs) + 1)]
    outs = [[torch.full_like(r["y_ref"], float("nan")) for _ in range(ROUNDS)] for r in runs]
    outs_h = [torch.full_like(yh_ref, float("nan")) for _ in range(ROUNDS)]
    torch.cuda.synchronize()
    say(f"[streams] {ROUNDS} rounds of {len(runs)} layers and the hidden-state entry")
    for i in range(ROUNDS):
        for r, s, o in zip(runs, streams, outs):
            M.moe_layer_forward(r["dm"], r["x"], r["logits"], None, y=o[i], ws=r["ws"], wc=r["wc"],
                                stream=s)
        M.moe_layer_forward_hidden(h["dm"], h["x"], wr, h["w"], y=outs_h[i], ws=ws_h,
                                   stream=streams[-1])
    torch.cuda.synchronize()
    for r, o in zip(runs, outs):
        for i in range(ROUNDS):
            assert torch.equal(o[i], r["y_ref"]), f"{r['cfg'].name}: round {i} differs"
    for i in range(ROUNDS):
        assert torch.equal(outs_h[i], yh_ref), f"hidden-state entry: round {i} differs"

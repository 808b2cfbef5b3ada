"""moe_layer_forward captured in a HIP graph (the benchmark replays decode
steps this way): every replay must reproduce the eager result bit for bit,
and the eager result matches the CPU oracle within the layer tolerance.

Replays are separated by eager work on the same buffers and by
synchronisations, so a graph node that only works on its first replay (or
that depends on state the eager calls leave behind) shows up as a mismatch.
The path records no memset nodes: every buffer the kernels need cleared is
written by a kernel.

A whole decode sequence is captured as well: 32 steps at the batch-1 decode
shape (d=2048, f=512, E=256, top-8 + shared) in one graph, each step on its
own copy of the weights, checked step by step against the oracle.
"""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import moe_inputs as G
from oracle import moe_oracle as O
from parity_util import check_y, dev_bits, say

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
    # the small-batch routing paths: one launch (T = 24), and the route kernel
    # before the one-workgroup permutation (T = 48)
    G.small_config("graph_small_t24", T=24, d=256, f=128, E=64, k=8, seed=47),
    G.small_config("graph_small_t48", T=48, d=256, f=128, E=64, k=8, seed=48),
], ids=lambda c: c.name)
def test_graph_replays_match_eager(cfg):
    say(f"[graph] {cfg.name}")
    inp = G.make_layer_inputs(cfg)
    y_ref = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k,
                            BM=M.moe_block_m())["y"]
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
    check_y(ref.cpu().numpy(), y_ref, f"{cfg.name} y (eager and every replay)")


def _scaled_down_copy(w: "M.W4Weights", m: int) -> "M.W4Weights":
    """A copy of the weights whose down projections (routed and shared) have their
    scales and biases multiplied by 2^m. Scaling both by a power of two scales
    every dequantised weight by exactly 2^m (bf16 rounding commutes with it away
    from the range ends), so the layer's output scales by exactly 2^m."""
    def scaled(t):
        return (t.view(torch.bfloat16) * (2.0 ** m)).view(torch.int16).contiguous()
    return M.W4Weights(
        M.W4Matrix(w.w13.codes.clone(), w.w13.scales.clone(), w.w13.biases.clone()),
        M.W4Matrix(w.w2.codes.clone(), scaled(w.w2.scales), scaled(w.w2.biases)),
        M.W4Matrix(w.s13.codes.clone(), w.s13.scales.clone(), w.s13.biases.clone()),
        M.W4Matrix(w.s2.codes.clone(), scaled(w.s2.scales), scaled(w.s2.biases)))


def test_decode_sequence_graph_rotated_weights():
    """32 decode steps captured in one graph, step s on weight copy s (32 copies at
    distinct addresses, down scales x 2^(s - 16)): every replay equals the eager run
    bit for bit, and step s equals 2^(s - 16) times the oracle's output within the
    layer tolerance. The steps' logits favour 16 experts so the oracle, which
    dequantises each expert it meets once, stays fast."""
    cfg = G.CONFIGS["decode_b1"]
    n = 32
    say(f"[graph] decode sequence: {n} steps, {n} weight copies")
    steps = G.make_decode_steps(cfg, n)
    hot = np.random.default_rng(61).choice(cfg.E, 16, replace=False)
    logits_np = steps["logits"].copy()
    logits_np[:, hot] += 6.0
    weights = G.make_weights(cfg)
    base = M.W4Weights.from_numpy(weights)
    copies = [_scaled_down_copy(base, s - 16) for s in range(n)]
    del base
    wcs = [c.c() for c in copies]
    dm = M.dims(1, cfg.d, cfg.f, cfg.E, cfg.k)
    ws = torch.empty(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    x = dev_bits(steps["x"])
    logits = torch.from_numpy(logits_np).cuda()
    y_eager = torch.empty((n, cfg.d), dtype=torch.float32, device="cuda")

    def run(y, stream=None):
        for s in range(n):
            M.moe_layer_forward(dm, x[s:s + 1], logits[s:s + 1], None, y=y[s:s + 1], ws=ws,
                                wc=wcs[s], stream=stream)

    run(y_eager)
    torch.cuda.synchronize()
    ref = y_eager.clone()
    y_graph = torch.full_like(y_eager, float("nan"))
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        run(y_graph, stream=st)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            run(y_graph, stream=st)
    torch.cuda.synchronize()
    for rep in range(3):
        y_graph.fill_(float("nan"))
        run(y_eager)                      # eager steps on the same workspace in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref), f"replay {rep} differs from the eager steps"
    y_or = O.token_outputs(steps["x"], logits_np, weights, cfg.k, np.arange(n))
    got = ref.cpu().numpy()
    for s in range(n):
        check_y(got[s:s + 1] * 2.0 ** (16 - s), y_or[s:s + 1], f"step {s} (copy {s})")

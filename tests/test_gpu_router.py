"""Router projection and the layer from hidden states on the GPU, through the
C ABI, against the oracle.

Scores are compared element by element with the oracle's fp64 dot products,
within the bound of any fp32 summation order of exact products:
d * 2^-24 * sum_c |x_c w_c|. Routing decided on the GPU's fp32 scores must be
bit-identical to the oracle's routing of those same scores. Where the oracle's
own scores separate the k-th and (k+1)-th experts of a token by more than
twice the bound, the GPU must have chosen the same k experts.
"""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import moe_inputs as G
from oracle import moe_oracle as O
from parity_util import W_ABS, check_y, dev_bits, say

pytestmark = pytest.mark.gpu

CASES = [
    G.small_config("rt_t37_d192_e8", T=37, d=192, f=64, E=8, k=2, seed=51),
    G.small_config("rt_t1_d2048_e256", T=1, d=2048, f=512, E=256, k=8, seed=52),
    G.small_config("rt_t300_d2048_e256", T=300, d=2048, f=512, E=256, k=8, seed=53),
    G.small_config("rt_t130_d64_e1000", T=130, d=64, f=64, E=1000, k=8, seed=54),
    G.small_config("rt_t65_d6144_e100", T=65, d=6144, f=64, E=100, k=4, seed=55),
    # 10 K steps: one whole round of eight in flight plus a ragged round
    G.small_config("rt_t64_d640_e64", T=64, d=640, f=64, E=64, k=8, seed=56),
    # an expert count that is not a multiple of 4 (the scores' row tails)
    G.small_config("rt_t70_d320_e37", T=70, d=320, f=64, E=37, k=5, seed=59),
    # a hidden size past the layer's limit (the router projection takes any
    # multiple of 64): 129 K steps, an odd count split over the two K halves
    G.small_config("rt_t33_d8256_e24", T=33, d=8256, f=64, E=24, k=4, seed=60),
    G.small_config("rt_t4096_d2048_e256", T=4096, d=2048, f=512, E=256, k=8, seed=57),
    # Up to 128 tokens the scores are dot products on the VALU (one wavefront
    # per expert and block of 4 tokens, 2048 columns per pass), so every case
    # above with T <= 128 runs there; these also do: a ragged token block, a
    # partial pass and an expert count that leaves workgroups partly empty;
    # three whole passes; five passes, the last partial; the largest batch.
    G.small_config("rt_t5_d192_e37", T=5, d=192, f=64, E=37, k=5, seed=115),
    G.small_config("rt_t16_d6144_e64", T=16, d=6144, f=64, E=64, k=8, seed=116),
    G.small_config("rt_t3_d8256_e24", T=3, d=8256, f=64, E=24, k=4, seed=117),
    G.small_config("rt_t128_d2048_e256", T=128, d=2048, f=512, E=256, k=8, seed=118),
    # and the MFMA tiles on the shapes above that stress them: a ragged K
    # round (10 K steps), expert counts that are not a multiple of 4 (row
    # tails), an odd number of K steps over the two halves, the widest input
    G.small_config("rt_t137_d192_e8", T=137, d=192, f=64, E=8, k=2, seed=119),
    G.small_config("rt_t192_d640_e64", T=192, d=640, f=64, E=64, k=8, seed=120),
    G.small_config("rt_t170_d320_e37", T=170, d=320, f=64, E=37, k=5, seed=121),
    G.small_config("rt_t133_d8256_e24", T=133, d=8256, f=64, E=24, k=4, seed=122),
    G.small_config("rt_t165_d6144_e100", T=165, d=6144, f=64, E=100, k=4, seed=123),
]


def sum_bound(x_bits, wr_bits):
    d = x_bits.shape[1]
    return d * 2.0 ** -24 * (np.abs(O.bf16_to_f64(x_bits)) @ np.abs(O.bf16_to_f64(wr_bits)).T)


def check_scores(name, x_bits, wr_bits, got):
    ref = O.router_logits(x_bits, wr_bits)
    b = sum_bound(x_bits, wr_bits)
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  {name}: max err {err.max():.3e}, max err / bound {(err / b).max():.3e}")
    assert np.isfinite(got).all()
    assert (err <= b).all(), f"{name}: score outside the fp32 summation bound"
    return ref, b


def check_routing(cfg, got, ref, b, ids, wts):
    rid, rw = O.route(got, cfg.k)
    assert np.array_equal(ids, rid)
    assert np.abs(wts - rw).max() <= W_ABS
    if cfg.k == cfg.E:
        return
    top = -np.sort(-ref, axis=1)
    sep = top[:, cfg.k - 1] - top[:, cfg.k] > 2 * b.max(axis=1)
    oid, _ = O.route(ref.astype(np.float32), cfg.k)
    assert np.array_equal(np.sort(ids[sep], axis=1), np.sort(oid[sep], axis=1))
    say(f"  {cfg.name}: {sep.mean():.3f} of tokens clearly separated, same experts chosen")
    assert sep.mean() > 0.5


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_router_scores_and_routing(cfg):
    say(f"[router] {cfg.name}")
    x = G.make_activations(cfg)["x"]
    wr = G.make_router(cfg)
    xd, wd = dev_bits(x), dev_bits(wr)
    logits = M.moe_router_logits(xd, wd)
    ids, wts = M.moe_route(logits, cfg.k)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    ref, b = check_scores(cfg.name, x, wr, got)
    check_routing(cfg, got, ref, b, ids.cpu().numpy(), wts.cpu().numpy())
    # the same inputs give the same bits (fixed summation order)
    again = M.moe_router_logits(xd, wd)
    torch.cuda.synchronize()
    assert torch.equal(again, logits)


@pytest.mark.parametrize("T", [170, 7])
def test_router_unit_rows_copy_columns(T):
    # Wr rows with a single 1.0: each score is one hidden-state value, exactly
    # (170 tokens: the MFMA tiles; 7: the dot products)
    d, E = 256, 72
    r = np.random.default_rng(58 if T == 170 else 65)
    x = G.f32_to_bf16_bits(r.standard_normal((T, d)).astype(np.float32))
    cols = r.integers(0, d, size=E)
    w = np.zeros((E, d), np.float32)
    w[np.arange(E), cols] = 1.0
    got = M.moe_router_logits(dev_bits(x), dev_bits(G.f32_to_bf16_bits(w)))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.float64), O.bf16_to_f64(x)[:, cols])


LAYER_CASES = [
    G.small_config("hid_t300", T=300, d=256, f=128, E=16, k=4, seed=61),
    G.small_config("hid_t1_decode", T=1, d=2048, f=512, E=64, k=8, seed=62),
    G.small_config("hid_t2", T=2, d=128, f=64, E=8, k=8, seed=63),
    # the router's dot products ahead of the grouped path: the one-row-block
    # GEMM build (24 tokens) and the full-tile build (100 tokens)
    G.small_config("hid_t24", T=24, d=512, f=256, E=32, k=8, seed=124),
    G.small_config("hid_t100", T=100, d=256, f=128, E=16, k=4, seed=125),
]


@pytest.mark.parametrize("cfg", LAYER_CASES, ids=[c.name for c in LAYER_CASES])
def test_layer_forward_hidden(cfg):
    say(f"[layer from hidden states] {cfg.name}")
    inp = G.make_layer_inputs(cfg)
    wr = G.make_router(cfg)
    xd, wd = dev_bits(inp["x"]), dev_bits(wr)
    w = M.W4Weights.from_numpy(inp["weights"])
    dm = M.dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k)
    y = M.moe_layer_forward_hidden(dm, xd, wd, w)
    logits = M.moe_router_logits(xd, wd)   # the scores the layer routed on (same bits)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    check_scores(cfg.name, inp["x"], wr, got)
    ref = O.layer_forward(inp["x"], got, inp["weights"], cfg.k, BM=M.moe_block_m())
    check_y(y.cpu().numpy(), ref["y"], cfg.name)
    # and the same as the layer entry point given those scores
    y2 = M.moe_layer_forward(dm, xd, logits, w)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)

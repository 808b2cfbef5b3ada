"""Pins of the oracle's whole layer (gate/up, SiLU*up, down, combine, shared expert).

The main pin is a brute-force dense evaluation, token by token, written
independently of the oracle: its own nibble unpacking, an exact fp64 affine
step rounded once to fp32 by numpy and to bf16 by torch, torch's SiLU, a
Python sort for routing and scipy's softmax. It never permutes rows, so a
mistake in the grouped path (scatter, block map, gather, combine) shows up.
Special cases then fix what the brute force shares with the oracle's reading.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import moe_inputs as G
from oracle import moe_oracle as O


# ---------------------------------------------------------------- independent brute force

def _bf16_bits_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _nearest_bf16(v):
    """Nearest bf16 (ties to even) by testing the candidates around the truncated pattern."""
    v = np.asarray(v, np.float64)
    start = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    best_val = np.full(v.shape, np.nan)
    best_key = np.full(v.shape, np.inf)
    for delta in (-2, -1, 0, 1, 2):
        cand = (start + delta) & 0xFFFF
        val = _bf16_bits_to_f64(cand.astype(np.uint16))
        ok = np.isfinite(val) & (np.signbit(val) == np.signbit(v))
        dist = np.where(ok, np.abs(val - v), np.inf)
        key = dist
        better = (key < best_key) | ((key == best_key) & ((cand & 1) == 0))   # ties to even
        best_val = np.where(better, val, best_val)
        best_key = np.where(better, key, best_key)
    return best_val


def _bf_dequant(codes, scales, biases):
    rows, half = codes.shape
    q = np.stack([codes % 16, codes // 16], axis=-1).reshape(rows, 2 * half).astype(np.float64)
    s = _bf16_bits_to_f64(scales)[:, np.arange(2 * half) // 64]
    b = _bf16_bits_to_f64(biases)[:, np.arange(2 * half) // 64]
    exact = s * q + b                       # exact in fp64 for these magnitudes
    f32 = torch.from_numpy(exact.astype(np.float32))
    return f32.to(torch.bfloat16).to(torch.float64).numpy()


def _bf_ffn(W13, W2, xt):
    f = W13.shape[0] // 2
    gate = torch.from_numpy(W13[:f] @ xt)
    up = W13[f:] @ xt
    h = _nearest_bf16(torch.nn.functional.silu(gate).numpy() * up)
    return W2 @ h


def brute_force_layer(x_bits, logits, w, k, with_shared=True):
    x = _bf16_bits_to_f64(x_bits)
    T, E = logits.shape
    y = np.zeros((T, x.shape[1]))
    cache = {}

    def mats(name, g):
        key = (name, g)
        if key not in cache:
            a, b = ("w13", "w2") if name == "routed" else ("s13", "s2")
            cache[key] = (_bf_dequant(w[a]["codes"][g], w[a]["scales"][g], w[a]["biases"][g]),
                          _bf_dequant(w[b]["codes"][g], w[b]["scales"][g], w[b]["biases"][g]))
        return cache[key]

    for t in range(T):
        order = sorted(range(E), key=lambda e: -float(logits[t, e]))[:k]
        wt = softmax(logits[t, order].astype(np.float64))
        acc = _bf_ffn(*mats("shared", 0), x[t]) if with_shared else np.zeros(x.shape[1])
        for j, e in enumerate(order):
            acc = acc + wt[j] * _bf_ffn(*mats("routed", e), x[t])
        y[t] = acc
    return y


def _assert_close(a, b, rel=1e-12):
    scale = max(np.abs(b).max(), 1e-300)
    assert np.abs(a - b).max() <= rel * scale, np.abs(a - b).max() / scale


SMALL = [
    G.CONFIGS["tiny_t16"],
    G.small_config("s1", T=5, d=64, f=64, E=3, k=1, seed=1),
    G.small_config("s2", T=8, d=128, f=64, E=4, k=4, seed=2),
    G.small_config("s3", T=7, d=192, f=128, E=8, k=2, seed=3, zipf_s=1.1),
    G.small_config("s4", T=9, d=64, f=64, E=8, k=3, seed=4, zipf_s=1.1, n_forced_empty=2),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_layer_matches_brute_force(cfg):
    inp = G.make_layer_inputs(cfg)
    out = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=4)
    ref = brute_force_layer(inp["x"], inp["logits"], inp["weights"], cfg.k)
    _assert_close(out["y"], ref)
    # the token-at-a-time path agrees as well
    toks = np.arange(cfg.T)[::2]
    _assert_close(O.token_outputs(inp["x"], inp["logits"], inp["weights"], cfg.k, toks), ref[toks])


def test_routed_only_matches_brute_force():
    """Shared weights forced to zero (codes 8, b = -8s): y is the routed sum alone."""
    cfg = G.small_config("ro", T=6, d=128, f=64, E=5, k=2, seed=8)
    inp = G.make_layer_inputs(cfg)
    w = inp["weights"]
    for name in ("s13", "s2"):
        w[name]["codes"][:] = 0x88
    out = O.layer_forward(inp["x"], inp["logits"], w, cfg.k, BM=2)
    ref = brute_force_layer(inp["x"], inp["logits"], w, cfg.k, with_shared=False)
    _assert_close(out["y"], ref)
    assert np.abs(out["o"][cfg.T * cfg.k:]).max() == 0.0


def test_zero_weights_give_zero_output():
    cfg = G.CONFIGS["tiny_t16"]
    inp = G.make_layer_inputs(cfg)
    for m in inp["weights"].values():
        m["codes"][:] = 0x88                # code 8 everywhere, bias -8s -> w = 0
    out = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=4)
    assert (out["y"] == 0).all() and (out["h"] == 0).all()


def test_zero_input_gives_zero_output():
    cfg = G.CONFIGS["tiny_t16"]
    inp = G.make_layer_inputs(cfg)
    x0 = np.zeros_like(inp["x"])
    out = O.layer_forward(x0, inp["logits"], inp["weights"], cfg.k, BM=4)
    assert (out["y"] == 0).all()


def test_identical_experts_make_routing_irrelevant():
    cfg = G.small_config("id", T=8, d=128, f=64, E=6, k=3, seed=5)
    inp = G.make_layer_inputs(cfg)
    w = inp["weights"]
    for name in ("w13", "w2"):
        for key in ("codes", "scales", "biases"):
            w[name][key][:] = w[name][key][0:1]
    y1 = O.layer_forward(inp["x"], inp["logits"], w, cfg.k, BM=4)["y"]
    other = np.random.default_rng(99).standard_normal(inp["logits"].shape).astype(np.float32)
    y2 = O.layer_forward(inp["x"], other, w, cfg.k, BM=4)["y"]
    _assert_close(y1, y2, rel=1e-13)


def test_doubling_down_scales_and_biases_doubles_output_exactly():
    cfg = G.small_config("dbl", T=8, d=128, f=64, E=4, k=2, seed=6)
    inp = G.make_layer_inputs(cfg)
    out1 = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=4)
    w = inp["weights"]
    for name in ("w2", "s2"):
        for key in ("scales", "biases"):
            w[name][key] = G.bf16_bits_times(w[name][key], 2.0)
    out2 = O.layer_forward(inp["x"], inp["logits"], w, cfg.k, BM=4)
    assert np.array_equal(out2["o"], 2 * out1["o"])
    assert np.array_equal(out2["y"], 2 * out1["y"])
    assert np.array_equal(out2["h"], out1["h"])


def test_h_is_bf16_valued_and_shapes():
    cfg = G.CONFIGS["tiny_t16"]
    inp = G.make_layer_inputs(cfg)
    out = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=4)
    rows = cfg.T * cfg.k + cfg.T
    assert out["h"].shape == (rows, cfg.f) and out["o"].shape == (rows, cfg.d)
    assert np.array_equal(O.bf16_round(out["h"]), out["h"])
    assert out["y"].shape == (cfg.T, cfg.d)

"""Planted mistakes in the oracle must be caught by its pins.

Each case edits one line of the oracle's source on the CPU (a swapped nibble,
a dropped rounding, a wrong sign, a swapped operand, a lost term), loads the
edited copy as a separate module and runs the pin that should catch it. The
unedited oracle passes the same pins (the other test files).
"""
import os
import types

import numpy as np
import pytest
import torch

import moe_inputs as G
from oracle import moe_oracle as O

from test_oracle_layer import brute_force_layer

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "moe_oracle.py")


def mutated(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("moe_oracle_mutant")
    exec(compile(src.replace(old, new), "moe_oracle_mutant", "exec"), mod.__dict__)
    return mod


# ---------------------------------------------------------------- pins, parameterised by module

def pin_layer_brute_force(M):
    for cfg in (G.CONFIGS["tiny_t16"], G.small_config("m3", T=7, d=192, f=128, E=8, k=2, seed=3)):
        inp = G.make_layer_inputs(cfg)
        y = M.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=4)["y"]
        ref = brute_force_layer(inp["x"], inp["logits"], inp["weights"], cfg.k)
        assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def pin_route_python_sort(M):
    r = np.random.default_rng(0)
    l = (np.round(r.standard_normal((40, 16)) * 2) / 2).astype(np.float32)
    ids, w = M.route(l, 4)
    for t in range(40):
        assert list(ids[t]) == sorted(range(16), key=lambda e: -float(l[t, e]))[:4]
        sel = l[t, ids[t]].astype(np.float64)
        assert np.allclose(w[t], np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum(), atol=1e-15)


def pin_permutation(M):
    r = np.random.default_rng(1)
    ids, _ = M.route(r.standard_normal((50, 8)).astype(np.float32), 3)
    counts = M.histogram(ids, 8)
    offsets = M.exclusive_scan(counts)
    st, row_of = M.scatter(ids, offsets)
    order = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(st, order // 3)
    assert np.array_equal(row_of[order], np.arange(150))


def pin_block_map(M):
    counts = np.array([5, 0, 9], np.int32)
    offsets = M.exclusive_scan(counts)
    tiles = M.block_map(counts, offsets, T=7, k=2, BM=4)
    assert [tuple(t) for t in tiles] == [(0, 0, 4), (0, 4, 5), (2, 5, 9), (2, 9, 13),
                                          (2, 13, 14), (3, 14, 18), (3, 18, 21)]


def pin_dequant(M):
    s_val = np.array([0.01, 1.0 + 2.0 ** -7, 0.0078125, 3.0], np.float32)
    s = torch.from_numpy(s_val).to(torch.bfloat16)
    b = (s.float() * -8).to(torch.bfloat16)
    sb = s.view(torch.int16).numpy().view(np.uint16).reshape(4, 1)
    bb = b.view(torch.int16).numpy().view(np.uint16).reshape(4, 1)
    q = np.tile(np.arange(16, dtype=np.uint8), (4, 4))
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    w = M.dequant(codes, sb, bb)
    exact = s.double().numpy()[:, None] * (q.astype(np.float64) - 8)
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(w, ref)


def pin_group_extent(M):
    q = np.full((1, 256), 3, np.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    s = torch.tensor([[1.0, 2.0, 4.0, 8.0]]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    z = np.zeros_like(s)
    w = M.dequant(codes, s, z)
    assert (w[0, :64] == 3).all() and (w[0, 64:128] == 6).all() and (w[0, 192:] == 24).all()


def pin_router(M):
    r = np.random.default_rng(6)
    T, d, E = 5, 128, 7
    x = r.standard_normal((T, d)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    perm = r.permutation(d)[:E]
    w = np.zeros((E, d), np.float32)
    w[np.arange(E), perm] = 1.0
    wb = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(M.router_logits(xb, wb), M.bf16_to_f64(xb)[:, perm])


MUTATIONS = [
    ("nibble order swapped", "q[..., 0::2] = codes & np.uint8(0x0F)", "q[..., 0::2] = codes >> np.uint8(4)", pin_dequant),
    ("bias sign flipped", "w32 = (s * q) + b", "w32 = (s * q) - b", pin_dequant),
    ("weights not rounded to bf16", "return bf16_round(w32.astype(np.float64))", "return w32.astype(np.float64)", pin_dequant),
    ("scale groups interleaved", "s = np.repeat(bf16_to_f64(scales).astype(np.float32), GROUP, axis=1)",
     "s = np.tile(bf16_to_f64(scales).astype(np.float32), (1, GROUP))", pin_group_extent),
    ("h not rounded to bf16", "H = bf16_round(silu(gate) * up)", "H = silu(gate) * up", pin_layer_brute_force),
    ("gate and up swapped", "gate = X @ W13[:fs].T", "gate = X @ W13[fs:].T", pin_layer_brute_force),
    ("down weights of the wrong expert", 'W2 = dequant_expert(weights["w2"], g)',
     'W2 = dequant_expert(weights["w2"], (g + 1) % E)', pin_layer_brute_force),
    ("gathered the wrong token rows", "X = x[toks]", "X = x[np.sort(toks)[::-1]]", pin_layer_brute_force),
    ("shared expert dropped", "y = o[T * k:T * k + T].copy()", "y = np.zeros_like(o[T * k:T * k + T])", pin_layer_brute_force),
    ("silu replaced by identity", "return z / (1.0 + np.exp(-z))", "return z", pin_layer_brute_force),
    ("ties to the higher index", 'ids = np.argsort(-l, axis=1, kind="stable")[:, :k]',
     'ids = np.argsort(l, axis=1, kind="stable")[:, ::-1][:, :k]', pin_route_python_sort),
    ("softmax not normalised", "w = e / e.sum(axis=1, keepdims=True)", "w = e", pin_route_python_sort),
    ("scatter not stable", "for t in range(T):", "for t in reversed(range(T)):", pin_permutation),
    ("last tile not clipped", "tiles.append((g, off + i * BM, min(off + (i + 1) * BM, off + c)))",
     "tiles.append((g, off + i * BM, off + (i + 1) * BM))", pin_block_map),
    ("router experts in reverse order", "return bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits).T",
     "return bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits)[::-1].T", pin_router),
    ("router drops a column group", "return bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits).T",
     "return bf16_to_f64(x_bits)[:, 64:] @ bf16_to_f64(wr_bits)[:, 64:].T", pin_router),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, pin):
    pin(O)                                   # the real oracle passes the pin
    with pytest.raises(AssertionError):
        pin(mutated(old, new))               # the planted mistake does not

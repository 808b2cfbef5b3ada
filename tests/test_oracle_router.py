"""Pins of the oracle's router projection (reading R13: logits = x . Wr^T over
bf16 values). Each pin is fixed by something other than the oracle's own
formula: brute-force exact sums, unit rows that must copy one input column,
and closed forms of all-ones inputs and exact scalings."""
import math

import numpy as np
import torch

import moe_inputs as G
from oracle import moe_oracle as O


def bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def vals(b):
    return torch.from_numpy(np.asarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_router_brute_force_exact_sums():
    r = np.random.default_rng(5)
    T, d, E = 3, 64, 5
    xb = bits(r.standard_normal((T, d)))
    wb = bits(r.standard_normal((E, d)) * 0.1)
    got = O.router_logits(xb, wb)
    assert got.shape == (T, E)
    xv, wv = vals(xb), vals(wb)
    for t in range(T):
        for e in range(E):
            prods = [float(xv[t, c]) * float(wv[e, c]) for c in range(d)]
            ref = math.fsum(prods)  # exactly rounded sum of exact products
            assert abs(got[t, e] - ref) <= 1e-15 * math.fsum(abs(p) for p in prods)


def test_router_unit_rows_copy_one_column():
    # Wr[e] = 1.0 at column perm[e], 0 elsewhere: the score of expert e is x[:, perm[e]]
    r = np.random.default_rng(6)
    T, d, E = 5, 128, 7
    xb = bits(r.standard_normal((T, d)))
    perm = r.permutation(d)[:E]
    w = np.zeros((E, d), np.float32)
    w[np.arange(E), perm] = 1.0
    got = O.router_logits(xb, bits(w))
    assert np.array_equal(got, vals(xb)[:, perm])


def test_router_closed_forms():
    r = np.random.default_rng(7)
    T, d, E = 4, 192, 6
    wb = bits(r.standard_normal((E, d)))
    # all-ones hidden states: every token's score is the row sum of Wr
    ones = bits(np.ones((T, d)))
    got = O.router_logits(ones, wb)
    rowsum = np.array([math.fsum(vals(wb)[e]) for e in range(E)])
    assert np.allclose(got, np.broadcast_to(rowsum, (T, E)), rtol=0, atol=1e-12)
    # doubling Wr (exact in bf16) doubles the scores; negating x negates them
    xb = bits(r.standard_normal((T, d)))
    base = O.router_logits(xb, wb)
    assert np.array_equal(O.router_logits(xb, G.bf16_bits_times(wb, 2.0)), 2 * base)
    assert np.array_equal(O.router_logits(G.bf16_bits_times(xb, -1.0), wb), -base)


def test_generated_router_scores_are_unit_scale():
    cfg = G.small_config("r", T=256, d=2048, f=64, E=64, k=8, seed=9)
    x = G.make_activations(cfg)["x"]
    l = O.router_logits(x, G.make_router(cfg))
    assert 0.8 < l.std() < 1.2 and abs(l.mean()) < 0.1

"""Randomised layer shapes on the GPU, through the C ABI, against the oracle.

A fixed-seed sweep over shapes the hand-picked cases do not all reach: T from 1
to 300 (the per-token decode kernels up to 16 tokens, the one-workgroup
routing paths up to 64, the two-kernel permutation above), d and f multiples
of 64, 1 to 300 experts (the general selection above 256), k up to 16, Zipf
skew, forced-empty experts, and the three bias formats. For every shape:
- routing, histogram, offsets, scatter, tile map and schedule are bit-exact;
- above 16 tokens the one-call layer equals the five entry points bit for bit;
- y is within the layer tolerance: mean |err| <= 2e-3 x RMS(y) always, and
  max |err| <= 2e-2 x RMS(y) unless the stored routed outputs bound it.

The grouped path stores each routed expert's output row in bf16 before the
weighted combine (reading R10), which costs up to half a bf16 ulp of that
row, 2^-8 of its magnitude. When the routed and shared outputs of a token
nearly cancel, |o| is many times RMS(y) and that rounding alone can exceed
2e-2 x RMS(y); such inputs arise here only with general biases. So each
element's error must stay within the larger of the flat bound and the
rounding bound sum_j w_j |o_j| 2^-8 (plus 2e-3 x RMS for the rest of the
arithmetic); the sweep counts the shapes that needed it.
"""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import moe_inputs as G
from oracle import moe_oracle as O
from parity_util import W_ABS, Y_MAX_REL_RMS, Y_MEAN_REL_RMS, dev_bits, expected_schedule, say

pytestmark = pytest.mark.gpu

N_CASES = 120
SEED = 7000


def random_configs():
    rng = np.random.default_rng(SEED)
    modes = [G.BIAS_NEG8, G.BIAS_NEG8, G.BIAS_GENERAL, G.BIAS_MIXED]
    out = []
    for i in range(N_CASES):
        T = int(rng.choice([1, 2, 3, 5, 7, 12, 16, 17, 24, 33, 48, 64, 65, 100, 129, 200, 257,
                            300]))
        d = 64 * int(rng.integers(1, 9))
        f = 64 * int(rng.integers(1, 7))
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 100, 257, 300]))
        k = int(rng.integers(1, min(E, 16) + 1))
        if E > 64:  # keeps the oracle's dequantisation of the used experts small
            d, f = min(d, 192), min(f, 128)
        zipf = float(rng.choice([0.0, 0.0, 1.1]))
        empty = int(rng.integers(0, E - k)) if E - k > 0 and rng.random() < 0.2 else 0
        mode = modes[int(rng.integers(0, len(modes)))]
        out.append(G.small_config(f"rand{i}_t{T}_d{d}_f{f}_e{E}_k{k}", T=T, d=d, f=f, E=E, k=k,
                                  seed=SEED + i, zipf_s=zipf, n_forced_empty=empty,
                                  bias_mode=mode))
    return out


CASES = random_configs()
_needed_rounding_bound = []


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_random_shape(cfg):
    T, d, f, E, k = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k
    say(f"[random] {cfg.name} zipf={cfg.zipf_s} empty={cfg.n_forced_empty} bias={cfg.bias_mode}")
    inp = G.make_layer_inputs(cfg)
    ref = O.layer_forward(inp["x"], inp["logits"], inp["weights"], k, BM=M.moe_block_m())
    x = dev_bits(inp["x"])
    logits = torch.from_numpy(inp["logits"]).cuda()
    w = M.W4Weights.from_numpy(inp["weights"])
    dm = M.dims(T, d, f, E, k)
    y = M.moe_layer_forward(dm, x, logits, w)
    rp = M.moe_route_permute(dm, logits)
    torch.cuda.synchronize()

    # routing and permutation, bit for bit
    p = {key: v.cpu().numpy() for key, v in rp.items()}
    assert np.array_equal(p["ids"], ref["ids"])
    assert np.abs(p["wts"] - ref["w"]).max() <= W_ABS
    assert np.array_equal(p["counts"], ref["counts"])
    assert np.array_equal(p["offsets"], ref["offsets"])
    assert np.array_equal(p["sorted_token"][:T * k], ref["sorted_token"])
    assert np.array_equal(p["row_of"][:T * k], ref["row_of"])
    n = int(p["num_tiles"][0])
    assert n == len(ref["tiles"])
    assert np.array_equal(p["tile_map"][:n, :3], ref["tiles"])
    assert np.array_equal(p["tile_map"][:n, 3], expected_schedule(ref["tiles"]))

    # the one-call layer against the staged entry points (same kernels above
    # 16 tokens; up to 16 the layer takes the per-token decode kernels)
    if T > 16:
        ids, wts = M.moe_route(logits, k)
        perm = M.moe_permute(dm, ids)
        h, o_r, o_sh = M.moe_expert_ffn_w4(dm, x, w, perm["sorted_token"], perm["tile_map"],
                                           perm["num_tiles"])
        ys = M.moe_unpermute_combine(dm, o_r, o_sh, wts, perm["row_of"])
        torch.cuda.synchronize()
        assert torch.equal(ys, y)

    # y: the mean bound always; the max bound, or per element the bound of the
    # routed outputs' bf16 storage where that is larger (grouped path only)
    yg = y.cpu().numpy().astype(np.float64)
    assert np.isfinite(yg).all()
    yr = ref["y"]
    rms = float(np.sqrt(np.mean(yr ** 2)))
    err = np.abs(yg - yr)
    say(f"  max_err/rms={err.max() / rms:.3e} mean_err/rms={err.mean() / rms:.3e}")
    assert err.mean() <= Y_MEAN_REL_RMS * rms
    if (err <= Y_MAX_REL_RMS * rms).all():
        return
    assert T > 16, "the decode kernels keep the routed outputs in fp32"
    o_routed = np.abs(ref["o"][:T * k])[ref["row_of"]].reshape(T, k, d)
    bound = np.einsum("tk,tkd->td", ref["w"], o_routed) * 2.0 ** -8 * 1.01 + Y_MEAN_REL_RMS * rms
    assert (err <= np.maximum(Y_MAX_REL_RMS * rms, bound)).all()
    _needed_rounding_bound.append(cfg.name)
    say(f"  within the bf16 storage bound of the routed outputs "
        f"(max |o| = {o_routed.max() / rms:.1f} x RMS(y))")


def test_zz_random_shapes_summary():
    """The rounding bound is the exception: most random shapes meet the flat bound."""
    say(f"[random] {len(_needed_rounding_bound)} of {N_CASES} shapes needed the bf16 storage "
        f"bound: {_needed_rounding_bound}")
    assert len(_needed_rounding_bound) <= N_CASES // 10

"""Helpers of the GPU parity tests: device upload, read-back and the tolerance checks."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import bit_quantized_grouped_router_amd as M
from oracle import moe_oracle as O

# output tolerance: max |err| <= 2e-2 * RMS(ref), mean |err| <= 2e-3 * RMS(ref)
Y_MAX_REL_RMS = 2e-2
Y_MEAN_REL_RMS = 2e-3
# router weights: fp32 exp/sum/divide against fp64
W_ABS = 2e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 (bf16 bits) numpy -> int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def upload(inp):
    cfg = inp["cfg"]
    x = dev_bits(inp["x"])
    logits = torch.from_numpy(inp["logits"]).cuda()
    w = M.W4Weights.from_numpy(inp["weights"])
    dm = M.dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k)
    return dm, x, logits, w


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "y"):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {what}: rms={rms:.4g} max_err/rms={mx / rms:.3e} mean_err/rms={mean / rms:.3e}")
    assert mx <= Y_MAX_REL_RMS * rms, f"{what}: max err {mx / rms:.3e} x RMS"
    assert mean <= Y_MEAN_REL_RMS * rms, f"{what}: mean err {mean / rms:.3e} x RMS"
    return mx / rms, mean / rms


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def check_bf16_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str, max_frac: float = 0.01,
                     slack=0.0):
    """bf16 tensor vs an oracle (bf16-valued) tensor: every element within one bf16 ulp
    (plus ``slack``, the fp32 accumulation allowance where a sum cancels), and at most
    max_frac of them not bit-identical."""
    g = O.bf16_to_f64(gpu_bits)
    diff = np.abs(g - ref)
    ulp = bf16_ulp(np.maximum(np.abs(g), np.abs(ref)))
    frac = float(np.mean(diff > 0))
    say(f"  {what}: {frac:.2e} of elements differ, max diff {float((diff / ulp).max()):.2f} ulp")
    assert (diff <= ulp * 1.0000001 + slack).all(), f"{what}: difference above one bf16 ulp"
    assert frac <= max_frac, f"{what}: {frac:.3e} of elements differ"


def expected_schedule(tiles, block_m: int = 128, xcds: int = 8) -> np.ndarray:
    """The block map's fourth column (the order the grouped GEMMs take the tiles in,
    position i going to XCD i % xcds).

    Positions 0 .. F-1 hold the F full tiles (block_m rows). Taken in tile order,
    they are split into xcds consecutive runs whose lengths differ by at most one
    (the longer runs first), and the r-th tile of run x sits at position
    r * xcds + x, so every XCD gets a contiguous run. The partial tiles follow,
    tallest first, equal heights in tile order."""
    tiles = np.asarray(tiles)
    heights = tiles[:, 2] - tiles[:, 1]
    full = [i for i in range(len(tiles)) if heights[i] == block_m]
    runs = np.array_split(np.array(full, dtype=np.int64), xcds)
    sched = np.full(len(tiles), -1, dtype=np.int64)
    for x, run in enumerate(runs):
        for r, t in enumerate(run):
            sched[r * xcds + x] = t
    partial = sorted((i for i in range(len(tiles)) if heights[i] < block_m),
                     key=lambda i: (-int(heights[i]), i))
    sched[len(full):] = partial
    assert sorted(sched.tolist()) == list(range(len(tiles)))
    return sched


def fill_expert_cache(weights, experts, cache, threads: int = 8):
    """Dequantise the given routed experts (and the shared one) with the oracle, in
    threads (numpy releases the interpreter lock inside the large array operations),
    into ``cache`` under the keys O.token_outputs uses: g for routed expert g, -1 for
    the shared expert."""
    todo = [int(g) for g in experts if int(g) not in cache]

    def one(g):
        return g, (O.dequant_expert(weights["w13"], g), O.dequant_expert(weights["w2"], g))

    with ThreadPoolExecutor(threads) as ex:
        for g, mats in ex.map(one, todo):
            cache[g] = mats
    if -1 not in cache:
        cache[-1] = (O.dequant_expert(weights["s13"], 0), O.dequant_expert(weights["s2"], 0))

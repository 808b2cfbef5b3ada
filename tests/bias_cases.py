"""Layer shapes with general (and mixed) dequantisation biases, shared by the GPU
parity tests and the CPU check that these inputs reach every exact dequantisation
path of the kernels.

The workloads' own weights use bias = -8 * scale, for which every group takes the
kernels' fast dequantisation. The page fixes a general bf16 bias per 64 weights
(noticiai.com.br, section "Prefill e decode: onde estao os ganhos"), so these
cases draw the biases in the generator's "general" and "mixed" modes.
"""
import numpy as np

import moe_inputs as G

GENERAL, MIXED = G.BIAS_GENERAL, G.BIAS_MIXED

# grouped path (route + permute + grouped GEMMs + combine): tiles of 1..4 row blocks
GROUPED = [
    G.small_config("gb_t300_zipf", T=300, d=256, f=128, E=16, k=4, seed=81, zipf_s=1.1,
                   bias_mode=GENERAL),
    G.small_config("gb_t700_mixed", T=700, d=512, f=256, E=64, k=8, seed=82, zipf_s=1.1,
                   bias_mode=MIXED),
    # one-launch routing up to 64 tokens, every tile one row block
    G.small_config("gb_t40", T=40, d=256, f=128, E=16, k=4, seed=83, bias_mode=GENERAL),
    # the headline shape's widths and expert count
    G.small_config("gb_full_width_t300", T=300, d=2048, f=512, E=256, k=8, seed=84,
                   bias_mode=GENERAL),
    G.small_config("gb_full_width_t300_mixed", T=300, d=2048, f=512, E=256, k=8, seed=85,
                   bias_mode=MIXED),
    # up to 32 tokens: the grouped GEMMs' one-row-block build, with wavefronts
    # of both K loops in one launch
    G.small_config("gb_full_width_t24_mixed", T=24, d=2048, f=512, E=256, k=8, seed=114,
                   bias_mode=MIXED),
]
# the layer's per-token decode kernels (T <= 16) and, through the staged entry
# points, the VALU projections (T <= 6) or one-row-block grouped GEMM tiles
DECODE = [
    G.small_config("gb_t1_full_width", T=1, d=2048, f=512, E=256, k=8, seed=86,
                   bias_mode=GENERAL),
    G.small_config("gb_t3_full_width", T=3, d=2048, f=512, E=256, k=8, seed=87,
                   bias_mode=GENERAL),
    G.small_config("gb_t6_mixed", T=6, d=512, f=256, E=32, k=8, seed=88, bias_mode=MIXED),
    G.small_config("gb_t16", T=16, d=256, f=128, E=32, k=8, seed=89, bias_mode=GENERAL),
]
ALL = GROUPED + DECODE


def fast_groups(scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """True where a (scale, bias) pair lets the kernels' fast dequantisation reproduce
    fp32(s*q + b) exactly: b - 1024 s and b - 64 s exact in fp32, i.e. the exponents
    of s (20..230) and b (<= 230) within -5..21 of each other (the rule the kernels
    state next to their fast path)."""
    sb = scales.astype(np.int64) | (biases.astype(np.int64) << 16)
    es = (sb >> 7) & 0xFF
    eb = (sb >> 23) & 0xFF
    return (es >= 20) & (es <= 230) & (eb <= 230) & (eb - es >= -5) & (eb - es <= 21)


def gemm_blocks_fast(weights, f: int):
    """Per expert and per wavefront block of weight rows, whether the grouped GEMM's
    wavefront takes its fast K loop: gate/up blocks are 32 gate rows with their 32
    up rows; down blocks are 64 output rows."""
    w13, w2 = weights["w13"], weights["w2"]
    f13 = fast_groups(w13["scales"], w13["biases"]).all(axis=2)       # [E, 2f]
    n = f13.shape[0]
    gate = f13[:, :f].reshape(n, f // 32, 32).all(axis=2)
    up = f13[:, f:].reshape(n, f // 32, 32).all(axis=2)
    f2 = fast_groups(w2["scales"], w2["biases"]).all(axis=2)          # [E, d]
    d = f2.shape[1]
    down = f2.reshape(n, d // 64, 64).all(axis=2)
    return gate & up, down

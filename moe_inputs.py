"""Seeded synthetic inputs for the int4-g64 MoE expert layer.

This module is shared by the CPU oracle, the tests and the benchmark. It only
draws random numbers and stores them in the layer's storage formats; it holds
none of the layer's arithmetic (no routing, no dequantisation, no GEMM).

Workloads follow the shape of the MoE layer of Qwen3.6-35B-A3B as described on
the noticiai.com.br page ("O modelo em três formatos de carga": 256 routed
experts, 8 selected per token, one shared expert seeing every token) with the
hidden size d=2048 and expert width f=512. The weight format is the page's
4-bit group-wise affine one ("Prefill e decode: onde estão os ganhos": 64
weights share one bf16 scale and one bf16 bias).

Storage formats (canonical layout, also the C-ABI layout):
  x        bf16 bits, uint16 [T, d]
  logits   float32 [T, E]
  codes    uint8 [n, rows, cols/2]; column c lives in byte c >> 1, in the low
           nibble when c is even and in the high nibble when c is odd
  scales   bf16 bits, uint16 [n, rows, cols/64]   (group g covers columns 64g..64g+63)
  biases   bf16 bits, uint16 [n, rows, cols/64]
  w13      gate rows 0..f-1 then up rows f..2f-1, cols = d
  w2       rows = d, cols = f
  s13/s2   the shared expert, n = 1, same layout

Every tensor has its own random stream ``np.random.default_rng([seed, tag])``
so adding a tensor never changes another one.

bf16 rounding of the drawn fp32 values uses torch's CPU conversion
(round to nearest even), a library routine, not the layer's code.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

GROUP = 64

# stream tags, one per tensor
TAG_X = 1
TAG_LOGITS = 2
TAG_RANK = 3
TAG_EMPTY = 4
TAG_W13_CODES = 10
TAG_W13_SCALES = 11
TAG_W2_CODES = 12
TAG_W2_SCALES = 13
TAG_S13_CODES = 20
TAG_S13_SCALES = 21
TAG_S2_CODES = 22
TAG_S2_SCALES = 23
TAG_DEC_X = 30
TAG_DEC_LOGITS = 31
TAG_ROUTER = 40
# bias patterns of the general-bias weight modes: tag of the scale stream + this
TAG_BIAS_OFFSET = 1000

# weight bias modes (make_w4)
BIAS_NEG8 = "neg8"        # bias = -8 * scale exactly (the workloads' format)
BIAS_GENERAL = "general"  # every group draws its own bias (see make_w4)
BIAS_MIXED = "mixed"      # rows of -8 * scale groups, with some rows of general groups


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    zipf_s: float = 0.0          # 0 -> no per-expert logit bias
    n_forced_empty: int = 0      # experts whose logits are set to -inf
    decode_steps: int = 0        # >0: T=1 decode workload with this many steps
    seed: int = 0
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_mode: str = BIAS_NEG8   # how the weights' biases are drawn (make_w4)

    @property
    def f_shared(self) -> int:
        return self.f


CONFIGS: Dict[str, MoeConfig] = {
    # tiny layer: the case the oracle finishes instantly
    "tiny_t16": MoeConfig("tiny_t16", T=16, d=128, f=64, E=8, k=2),
    # Qwen3.6-35B-A3B-shaped prefill, near-uniform expert load (~16 rows/expert)
    "prefill_t512": MoeConfig("prefill_t512", T=512, d=2048, f=512, E=256, k=8),
    # same shape, T=4096, Zipf(1.1)-skewed expert load (some experts >10x mean, some empty)
    "prefill_t4096_zipf": MoeConfig("prefill_t4096_zipf", T=4096, d=2048, f=512, E=256, k=8,
                                    zipf_s=1.1),
    # batch-1 decode, 1000 independent steps, weights identical to prefill_t512
    "decode_b1": MoeConfig("decode_b1", T=1, d=2048, f=512, E=256, k=8, decode_steps=1000),
    # long prefill, Zipf-skewed plus 8 experts forced empty with -inf logits
    "prefill_t16384_zipf_empty": MoeConfig("prefill_t16384_zipf_empty", T=16384, d=2048, f=512,
                                           E=256, k=8, zipf_s=1.1, n_forced_empty=8),
}


def rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits via torch's CPU conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_times(bits: np.ndarray, factor: float) -> np.ndarray:
    """bf16 bits of (bf16 value * factor), via torch; exact when factor is a power of two."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return (t.float() * factor).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_w4(seed: int, tag_codes: int, tag_scales: int, n: int, rows: int, cols: int,
            scale_lo: float, scale_hi: float, bias_mode: str = BIAS_NEG8) -> Dict[str, np.ndarray]:
    """Random int4-g64 matrices: uniform codes 0..15 and one (scale, bias) per 64 columns.

    Uniform random bytes give two independent uniform 4-bit codes per byte.
    bias_mode:
      neg8     scale ~ U(lo, hi) in bf16 and bias = -8 * scale (exact in bf16);
      general  every group draws its own pair, all in bf16:
                 scale: |s| ~ U(lo, hi), negative for 10% of the groups; 2% of
                   the groups take a tiny scale (|s| * 2^-104) and 2% a scale
                   2^-24 times smaller than their bias (|b| ~ hi * U(1/16, 16));
                 bias: -s * U(1/16, 16) for most groups; +0 for 5% and -0 for
                   2% of them; -8 * s for 3%; -s * U(0, 2^-6) for 2%;
               no value is an fp32 subnormal;
               so both exact dequantisation paths of the kernels (and the
               switches between them) occur, while the weights keep magnitudes
               near the neg8 ones;
      mixed    neg8 rows with 1% of the weight rows (all their groups) drawn as
               in general, so a block of 64 rows is neg8-only about half the time.
    """
    assert cols % GROUP == 0
    codes = rng(seed, tag_codes).integers(0, 256, size=(n, rows, cols // 2), dtype=np.uint8)
    shape = (n, rows, cols // GROUP)
    s32 = rng(seed, tag_scales).uniform(scale_lo, scale_hi, size=shape)
    if bias_mode == BIAS_NEG8:
        scales = f32_to_bf16_bits(s32.astype(np.float32))
        biases = bf16_bits_times(scales, -8.0)
        return {"codes": codes, "scales": scales, "biases": biases}
    assert bias_mode in (BIAS_GENERAL, BIAS_MIXED), bias_mode
    r = rng(seed, tag_scales + TAG_BIAS_OFFSET)
    u_sign, u_scale, u_bias = r.random(shape), r.random(shape), r.random(shape)
    frac = r.uniform(1.0 / 16.0, 16.0, size=shape)
    small = r.uniform(0.0, 2.0 ** -6, size=shape)
    s = np.where(u_sign < 0.1, -s32, s32)
    tiny = u_scale < 0.02                      # scale exponent far below the usual range
    far = (u_scale >= 0.02) & (u_scale < 0.04)  # bias 2^24 times the scale
    s = np.where(tiny, s * 2.0 ** -104, s)
    b = -s * frac
    b = np.where(far, -np.sign(s) * frac * scale_hi, b)
    s = np.where(far, s * 2.0 ** -24, s)
    b = np.where((u_bias >= 0.10) & (u_bias < 0.12) & ~tiny & ~far, -s * small, b)
    b = np.where(u_bias < 0.05, 0.0, b)
    b = np.where((u_bias >= 0.05) & (u_bias < 0.07), -0.0, b)
    scales = f32_to_bf16_bits(s.astype(np.float32))
    biases = f32_to_bf16_bits(b.astype(np.float32))
    neg8 = (u_bias >= 0.07) & (u_bias < 0.10) & ~far
    biases = np.where(neg8, bf16_bits_times(scales, -8.0), biases)
    if bias_mode == BIAS_MIXED:
        general_row = r.random((n, rows, 1)) < 0.01
        s_neg8 = f32_to_bf16_bits(s32.astype(np.float32))
        b_neg8 = bf16_bits_times(s_neg8, -8.0)
        scales = np.where(general_row, scales, s_neg8)
        biases = np.where(general_row, biases, b_neg8)
    return {"codes": codes, "scales": scales.astype(np.uint16), "biases": biases.astype(np.uint16)}


def make_weights(cfg: MoeConfig) -> Dict[str, Dict[str, np.ndarray]]:
    s, lo, hi, bm = cfg.seed, cfg.scale_lo, cfg.scale_hi, cfg.bias_mode
    return {
        "w13": make_w4(s, TAG_W13_CODES, TAG_W13_SCALES, cfg.E, 2 * cfg.f, cfg.d, lo, hi, bm),
        "w2": make_w4(s, TAG_W2_CODES, TAG_W2_SCALES, cfg.E, cfg.d, cfg.f, lo, hi, bm),
        "s13": make_w4(s, TAG_S13_CODES, TAG_S13_SCALES, 1, 2 * cfg.f_shared, cfg.d, lo, hi, bm),
        "s2": make_w4(s, TAG_S2_CODES, TAG_S2_SCALES, 1, cfg.d, cfg.f_shared, lo, hi, bm),
    }


def make_router(cfg: MoeConfig) -> np.ndarray:
    """Router matrix Wr, bf16 bits [E, d], entries N(0, 1/d): with N(0, 1) hidden
    states the scores come out near N(0, 1), like the logits of the other workloads."""
    w = rng(cfg.seed, TAG_ROUTER).standard_normal((cfg.E, cfg.d)) / np.sqrt(cfg.d)
    return f32_to_bf16_bits(w.astype(np.float32))


def zipf_bias(cfg: MoeConfig) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank): the log of a Zipf(s) pmf over a random rank order.

    The additive constant of the log-pmf is dropped: it changes neither the
    top-k choice nor the softmax over the chosen logits.
    """
    if cfg.zipf_s == 0.0:
        return np.zeros(cfg.E, dtype=np.float64)
    rank = rng(cfg.seed, TAG_RANK).permutation(cfg.E) + 1
    return -cfg.zipf_s * np.log(rank.astype(np.float64))


def forced_empty_experts(cfg: MoeConfig) -> np.ndarray:
    if cfg.n_forced_empty == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng(cfg.seed, TAG_EMPTY).choice(cfg.E, cfg.n_forced_empty, replace=False))


def make_activations(cfg: MoeConfig, T: Optional[int] = None,
                     tag_x: int = TAG_X, tag_logits: int = TAG_LOGITS) -> Dict[str, np.ndarray]:
    T = cfg.T if T is None else T
    x = f32_to_bf16_bits(rng(cfg.seed, tag_x).standard_normal((T, cfg.d)).astype(np.float32))
    logits = rng(cfg.seed, tag_logits).standard_normal((T, cfg.E)) + zipf_bias(cfg)[None, :]
    logits = logits.astype(np.float32)
    empty = forced_empty_experts(cfg)
    if empty.size:
        logits[:, empty] = -np.inf
    return {"x": x, "logits": logits}


def make_layer_inputs(cfg: MoeConfig) -> Dict[str, object]:
    """x, logits and weights of one prefill (or single decode-step) workload."""
    out: Dict[str, object] = dict(make_activations(cfg))
    out["weights"] = make_weights(cfg)
    out["cfg"] = cfg
    return out


def make_decode_steps(cfg: MoeConfig, steps: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Independent N(0,1) x [steps, d] (bf16) and logits [steps, E] (fp32) of the decode workload."""
    steps = cfg.decode_steps if steps is None else steps
    x = f32_to_bf16_bits(rng(cfg.seed, TAG_DEC_X).standard_normal((steps, cfg.d)).astype(np.float32))
    logits = rng(cfg.seed, TAG_DEC_LOGITS).standard_normal((steps, cfg.E)).astype(np.float32)
    return {"x": x, "logits": logits}


def small_config(name: str, T: int, d: int, f: int, E: int, k: int, seed: int,
                 zipf_s: float = 0.0, n_forced_empty: int = 0,
                 bias_mode: str = BIAS_NEG8) -> MoeConfig:
    """An ad-hoc configuration for tests (random small shapes)."""
    return MoeConfig(name, T=T, d=d, f=f, E=E, k=k, zipf_s=zipf_s,
                     n_forced_empty=n_forced_empty, seed=seed, bias_mode=bias_mode)

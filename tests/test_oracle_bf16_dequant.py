"""Pins of the oracle's bf16 encoding and int4-g64 dequantisation.

Each check compares the oracle with something other than itself: torch's
bf16 conversion (a library routine), a brute-force nearest-neighbour search,
exact fp64 arithmetic, or the page's own numbers (tests/golden/page_facts.json).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_bf16_value(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- bf16 decode

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = O.bf16_to_f64(bits)
    ref = torch_bf16_value(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zeros survive
    assert np.signbit(O.bf16_to_f64(np.array([0x8000], np.uint16)))[0]


# ---------------------------------------------------------------- bf16 rounding

def _f32_patterns():
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(7).integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd]).view(np.float32)


def test_round_fp32_to_bf16_matches_torch_exhaustive_high_halves():
    f = _f32_patterns()
    ok = ~np.isnan(f)
    mine = O.round_to_bf16_bits(f[ok].astype(np.float64))
    ref = torch_bf16_bits(f[ok])
    assert np.array_equal(mine, ref)
    assert (O.round_to_bf16_bits(f[~ok].astype(np.float64)) == 0x7FC0).all()


def _brute_force_bf16_bits(v):
    """Nearest bf16 by searching the neighbours of a nearby pattern; ties to even."""
    out = np.empty(v.shape, np.uint16)
    for i, x in enumerate(v):
        start = int(np.float32(x).view(np.uint32) >> 16)
        best = None
        for cand in range(start - 2, start + 3):
            cand &= 0xFFFF
            val = float(O.bf16_to_f64(np.array([cand], np.uint16))[0])
            if not np.isfinite(val) or np.signbit(val) != np.signbit(x):
                continue
            key = (abs(val - x), cand & 1)
            if best is None or key < best[0]:
                best = (key, cand)
        out[i] = best[1]
    return out


def test_round_fp64_to_bf16_single_rounding_brute_force():
    r = np.random.default_rng(11)
    v = r.standard_normal(3000) * np.exp2(r.integers(-40, 40, 3000))
    # midpoints between adjacent bf16 values nudged by less than half an fp32 ulp:
    # a double rounding (fp64 -> fp32 -> bf16) would see an exact tie here
    base = O.bf16_to_f64(r.integers(0x3000, 0x5000, 500).astype(np.uint16))
    nxt = O.bf16_to_f64((O.round_to_bf16_bits(base) + 1).astype(np.uint16))
    mid = (base + nxt) / 2
    nudged = np.concatenate([mid + (nxt - base) * 2.0 ** -30, mid - (nxt - base) * 2.0 ** -30, mid])
    v = np.concatenate([v, nudged, -nudged])
    assert np.array_equal(O.round_to_bf16_bits(v), _brute_force_bf16_bits(v))
    # the nudged-up midpoints must round up (a double rounding would tie to even)
    up = O.round_to_bf16_bits(nudged[:500])
    assert np.array_equal(up, O.round_to_bf16_bits(nxt))


def test_round_overflow_underflow_special():
    big = np.array([3.5e38, -3.5e38, np.inf, -np.inf, 0.0, -0.0, 2.0 ** -140, 2.0 ** -134 * 1.5])
    bits = O.round_to_bf16_bits(big)
    assert bits[0] == 0x7F80 and bits[1] == 0xFF80
    assert bits[2] == 0x7F80 and bits[3] == 0xFF80
    assert bits[4] == 0x0000 and bits[5] == 0x8000
    assert bits[6] == 0x0000                          # below half the smallest subnormal
    # 1.5 * 2^-134 is 0.75 of the subnormal step 2^-133: nearest is one step
    assert bits[7] == 0x0001
    assert bits[7] == torch_bf16_bits(np.array([2.0 ** -134 * 1.5], np.float32))[0]


# ---------------------------------------------------------------- dequantisation

def _pack_cols(q):
    """Pack codes [rows, cols] (0..15) into bytes: column c -> byte c//2, low nibble for even c."""
    q = np.asarray(q, np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def test_nibble_order_hand_case():
    # byte 0x21: column 0 holds code 1 (low nibble), column 1 holds code 2 (high nibble)
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x21
    codes[0, 31] = 0xF0            # column 62 -> 0, column 63 -> 15
    one = torch_bf16_bits(np.array([1.0], np.float32))
    zero = torch_bf16_bits(np.array([0.0], np.float32))
    w = O.dequant(codes, one.reshape(1, 1), zero.reshape(1, 1))
    assert w[0, 0] == 1.0 and w[0, 1] == 2.0
    assert w[0, 62] == 0.0 and w[0, 63] == 15.0
    assert (w[0, 2:62] == 0.0).all()


def test_dequant_exhaustive_scales_symmetric_bias():
    """All 16 codes x every bf16 scale whose 16*s is finite, bias = -8*s.

    Expected value, computed independently: s*(q-8) exactly in fp64, rounded to
    bf16 by torch (round to nearest even). With b = -8s the fp32 step is exact.
    """
    s_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s_val = torch_bf16_value(s_bits)
    keep = np.isfinite(s_val) & (np.abs(s_val) < 2.0 ** 120)
    s_bits = s_bits[keep]
    s_val = s_val[keep]
    b_bits = torch_bf16_bits((s_val * -8.0).astype(np.float32))
    assert np.array_equal(torch_bf16_value(b_bits), -8.0 * s_val)      # -8s exact in bf16
    n = len(s_bits)
    q = np.tile(np.arange(16, dtype=np.uint8), (n, 4))                 # one group of 64 per row
    w = O.dequant(_pack_cols(q), s_bits.reshape(n, 1), b_bits.reshape(n, 1))
    exact = s_val[:, None] * (q.astype(np.float64) - 8.0)
    ref = torch_bf16_value(torch_bf16_bits(exact.astype(np.float32)))
    assert np.array_equal(np.asarray(exact, np.float32).astype(np.float64), exact)
    same = (w == ref) | (np.isnan(w) & np.isnan(ref))
    assert same.all()
    # the bf16 step really rounds for some inputs (e.g. s = 1 + 2^-7, q - 8 = 7)
    assert (w != exact).any()
    s1 = torch_bf16_bits(np.array([1.0 + 2.0 ** -7], np.float32))
    w1 = O.dequant(_pack_cols(np.full((1, 64), 15, np.uint8)), s1.reshape(1, 1),
                   torch_bf16_bits(np.array([-8.0 * (1 + 2.0 ** -7)], np.float32)).reshape(1, 1))
    # exact 7 + 7/128 = 7.0546875 lies 0.75 of the way between the bf16 neighbours
    # 7.03125 and 7.0625 (step 2^-5), so it rounds up to 7.0625
    assert w1[0, 0] == 7.0625


def test_dequant_random_bias_single_fp32_rounding():
    """General biases: fp32(s*q + b) must be ONE rounding of the exact value.

    The reference computes s*q + b exactly in fp64 (exponents are kept close so
    it is exact), rounds once to fp32 with numpy, then to bf16 with torch.
    """
    r = np.random.default_rng(3)
    rows = 4096
    s_bits = torch_bf16_bits(r.uniform(0.005, 0.02, (rows, 2)).astype(np.float32))
    b_bits = torch_bf16_bits((r.uniform(-0.3, 0.3, (rows, 2))).astype(np.float32))
    q = r.integers(0, 16, (rows, 128)).astype(np.uint8)
    w = O.dequant(_pack_cols(q), s_bits, b_bits)
    s = np.repeat(torch_bf16_value(s_bits), 64, axis=1)
    b = np.repeat(torch_bf16_value(b_bits), 64, axis=1)
    exact = s * q + b
    # exactness of the fp64 reference: the fp64 sum equals the sum of its parts
    assert np.array_equal(exact - b, s * q)
    f32 = exact.astype(np.float32)
    ref = torch_bf16_value(torch_bf16_bits(f32))
    assert np.array_equal(w, ref)


def test_one_scale_and_bias_cover_exactly_64_consecutive_inputs():
    """Changing the scale and bias of group j of row r changes exactly columns 64j..64j+63 of row r."""
    r = np.random.default_rng(5)
    rows, cols = 6, 256
    q = r.integers(1, 16, (rows, cols)).astype(np.uint8)
    s = torch_bf16_bits(r.uniform(0.005, 0.02, (rows, cols // 64)).astype(np.float32))
    b = torch_bf16_bits(r.uniform(-0.2, -0.1, (rows, cols // 64)).astype(np.float32))
    base = O.dequant(_pack_cols(q), s, b)
    for (rr, j) in [(0, 0), (3, 2), (5, 3)]:
        s2, b2 = s.copy(), b.copy()
        s2[rr, j] = torch_bf16_bits(np.array([0.5], np.float32))[0]
        b2[rr, j] = torch_bf16_bits(np.array([1.0], np.float32))[0]
        changed = O.dequant(_pack_cols(q), s2, b2) != base
        expect = np.zeros_like(changed)
        expect[rr, 64 * j:64 * (j + 1)] = True
        assert np.array_equal(changed, expect)


def test_format_size_matches_page_checkpoint():
    """4-bit codes plus one bf16 scale and one bf16 bias per 64 weights reproduce the
    page's ~70 GB (bf16) -> 19.4 GB (4-bit) within 2%; a scale-only format would not."""
    facts = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
    g = facts["quant_group"]["value"]
    assert g == O.GROUP
    rows, cols = 8, 4 * g
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // g), np.uint16)
    w = O.dequant(codes, scales, scales)                 # shapes accepted by the oracle
    assert w.shape == (rows, cols)
    bits_per_weight = 8.0 * (codes.nbytes + 2 * scales.nbytes) / w.size
    assert bits_per_weight == 4.5
    ratio = bits_per_weight / 16.0
    predicted = facts["bf16_checkpoint_gb"]["value"] * ratio
    assert abs(predicted - facts["w4_checkpoint_gb"]["value"]) / facts["w4_checkpoint_gb"]["value"] < 0.02
    scale_only = facts["bf16_checkpoint_gb"]["value"] * (4 + 16 / g) / 16.0
    assert abs(scale_only - facts["w4_checkpoint_gb"]["value"]) / facts["w4_checkpoint_gb"]["value"] > 0.03


def test_scaling_scale_and_bias_by_two_doubles_weights_exactly():
    r = np.random.default_rng(9)
    q = r.integers(0, 16, (16, 128)).astype(np.uint8)
    s = torch_bf16_bits(r.uniform(0.005, 0.02, (16, 2)).astype(np.float32))
    b = torch_bf16_bits(r.uniform(-0.2, 0.1, (16, 2)).astype(np.float32))
    s2 = torch_bf16_bits((torch_bf16_value(s) * 2).astype(np.float32))
    b2 = torch_bf16_bits((torch_bf16_value(b) * 2).astype(np.float32))
    assert np.array_equal(O.dequant(_pack_cols(q), s2, b2), 2 * O.dequant(_pack_cols(q), s, b))

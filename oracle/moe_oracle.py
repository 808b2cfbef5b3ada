"""CPU oracle of the int4-g64 grouped MoE expert layer (plain numpy, fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module. The product path (the HIP library and
its Python binding) never calls it, and this module imports nothing from the
product path: the two share no code, tables or helpers.

Source of the method. The noticiai.com.br page on Perplexity's Lily engine
(https://noticiai.com.br/?p=12593) describes the layer:
  * section "O modelo em três formatos de carga": a router scores 256 experts
    and keeps eight, and one shared expert sees every token;
  * section "Prefill e decode: onde estão os ganhos": weights are 4-bit affine
    codes in groups of 64 that share one bf16 scale and one bf16 bias; the
    tensor units consume bf16, so weights are rebuilt to bf16 one tile at a
    time inside the grouped GEMM with fp32 accumulation; the routing
    histogram, prefix scan, scatter and block map stay on the GPU.

The result is quantised, routed and rounded at defined points, so the oracle
walks the method's steps in order rather than a dense closed form. Where the
page is silent, the readings taken here are:
  R1  router weights: softmax over the k selected logits (= full softmax
      renormalised over the top k); selection on fp32 logits, descending,
      ties to the lower expert index, -0 equal to +0;
  R2  shared expert weight 1.0 (no gate), added to every token;
  R3  dropless: every assignment is computed;
  R4  dequantisation w = s*q + b with unsigned q in 0..15, groups of 64 along
      the input (column) dimension, computed in fp32 and rounded once to bf16
      (round to nearest even);
  R5  expert FFN is the gated SiLU form down(SiLU(gate x) * (up x)); the page
      names experts but not their FFN, and this is the Qwen3 MoE family's form;
  R6  the activation h fed to the down projection is rounded to bf16, because
      the tensor units take bf16 operands;
  R7  o and y are kept unrounded (fp64 here);
  R8  block map: per group, ceil(count/BM) tiles of at most BM rows, groups in
      order 0..E-1 then the shared group E.
  R13 router projection (the step before routing, for callers that start
      from hidden states): the router's score of expert e for token t is the
      dot product of the token's bf16 hidden state with row e of a bf16
      matrix Wr [E, d]; the page says only that the router scores the 256
      experts, and a bias-free linear projection is the plainest reading.
Accumulation is fp64 over the exactly decoded bf16 operands.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

GROUP = 64

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# --------------------------------------------------------------------------
# bf16 encoding (O0 and the rounding used by R4 and R6)
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit pattern of the nearest bf16 to each value (ties to even).

    bf16 keeps 8 significant bits (7 stored). In the normal range the fp64
    significand is rounded at its 45th bit (52 - 7 stored bits), half to even;
    a carry out of the significand moves into the exponent, as IEEE intends.
    Below 2^-126 the bf16 grid is fixed at 2^-133 (subnormals) and the value
    is rounded on that grid instead. Magnitudes that round above the largest
    finite bf16 become infinity. NaN becomes the quiet NaN 0x7FC0.
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    bits = v.view(np.uint64)
    mag = bits & np.uint64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    mag += np.uint64((1 << 44) - 1)
    mag += lsb
    mag >>= np.uint64(45)
    mag <<= np.uint64(45)
    val = mag.view(np.float64)
    a = np.abs(v)
    small = a < 2.0 ** -126
    if small.any():
        val[small] = np.rint(a[small] * 2.0 ** 133) * 2.0 ** -133
    over = val > BF16_MAX
    if over.any():
        val[over] = np.inf
    out = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out |= ((bits >> np.uint64(48)) & np.uint64(0x8000)).astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Value of the nearest bf16, as fp64."""
    return bf16_to_f64(round_to_bf16_bits(v))


# --------------------------------------------------------------------------
# O7: dequantisation of one int4-g64 matrix (R4)
# --------------------------------------------------------------------------

def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] codes; column c is byte c>>1, low nibble for even c."""
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    q[..., 0::2] = codes & np.uint8(0x0F)
    q[..., 1::2] = codes >> np.uint8(4)
    return q


def dequant(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """bf16 weights (as fp64) of one matrix: w = bf16_rne(fp32(s*q + b)).

    codes [rows, cols/2] uint8, scales/biases [rows, cols/64] bf16 bits.
    Group j of a row covers columns 64j .. 64j+63 (the page's 64-weight groups
    along the input dimension). s*q is exact in fp32 (8-bit times 4-bit
    significands), so the fp32 step rounds once, at the addition.
    """
    q = unpack_codes(codes).astype(np.float32)
    rows, cols = q.shape
    assert scales.shape == (rows, cols // GROUP) and biases.shape == scales.shape
    s = np.repeat(bf16_to_f64(scales).astype(np.float32), GROUP, axis=1)
    b = np.repeat(bf16_to_f64(biases).astype(np.float32), GROUP, axis=1)
    w32 = (s * q) + b                            # numpy fp32 ops: IEEE round to nearest
    assert w32.dtype == np.float32
    return bf16_round(w32.astype(np.float64))


def dequant_expert(wt: Dict[str, np.ndarray], g: int) -> np.ndarray:
    return dequant(wt["codes"][g], wt["scales"][g], wt["biases"][g])


# --------------------------------------------------------------------------
# O1-O2: router (R1)
# --------------------------------------------------------------------------

def route(logits: np.ndarray, k: int):
    """Top-k experts per token and their softmax weights.

    Order: fp32 logit descending, ties to the lower expert index, -0 == +0.
    Weights: exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k slots, fp64.
    Precondition: no NaN and at least k finite logits per token.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    assert 1 <= k <= E
    assert not np.isnan(l).any(), "router logits must not be NaN"
    assert (np.isfinite(l).sum(axis=1) >= k).all(), "need at least k finite logits per token"
    l = np.where(l == 0.0, 0.0, l)               # -0 -> +0
    ids = np.argsort(-l, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(l, ids, axis=1)
    e = np.exp(sel - sel[:, :1])
    w = e / e.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


# --------------------------------------------------------------------------
# O3-O6: histogram, exclusive scan, stable scatter, block map
# --------------------------------------------------------------------------

def histogram(ids: np.ndarray, E: int) -> np.ndarray:
    return np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int32)


def exclusive_scan(counts: np.ndarray) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off.astype(np.int32)


def scatter(ids: np.ndarray, offsets: np.ndarray):
    """Counting-sort placement: for t ascending then slot j ascending, the
    assignment (t, j) to expert e takes row offsets[e] + (rows already given to e).

    Returns sorted_token [T*k] (token of each permuted row) and
    row_of [T*k] (permuted row of assignment t*k + j).
    """
    T, k = ids.shape
    cursor = np.zeros(len(offsets) - 1, dtype=np.int64)
    sorted_token = np.full(T * k, -1, dtype=np.int32)
    row_of = np.full(T * k, -1, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            p = int(offsets[e]) + int(cursor[e])
            cursor[e] += 1
            sorted_token[p] = t
            row_of[t * k + j] = p
    return sorted_token, row_of


def block_map(counts: np.ndarray, offsets: np.ndarray, T: int, k: int, BM: int) -> np.ndarray:
    """Tiles (group, row_begin, row_end) of at most BM rows (R8).

    Routed groups 0..E-1 cover their segments of the permuted rows; the shared
    group E covers rows T*k .. T*k+T-1 (one row per token, token order).
    """
    E = len(counts)
    tiles = []
    groups = [(g, int(offsets[g]), int(counts[g])) for g in range(E)] + [(E, T * k, T)]
    for g, off, c in groups:
        n = (c + BM - 1) // BM
        for i in range(n):
            tiles.append((g, off + i * BM, min(off + (i + 1) * BM, off + c)))
    return np.array(tiles, dtype=np.int32).reshape(-1, 3)


# --------------------------------------------------------------------------
# O8-O9: expert FFNs over the permuted rows (R5, R6, R7)
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, sorted_token: np.ndarray, counts: np.ndarray,
               offsets: np.ndarray, weights: Dict[str, Dict[str, np.ndarray]],
               T: int, k: int):
    """h [T*k+T, f] (bf16 values) and o [T*k+T, d] (fp64) for every permuted row.

    Row p of routed group g multiplies token sorted_token[p]; shared row T*k+t
    multiplies token t. gate = W13[:f] x, up = W13[f:] x, h = bf16(silu(gate)*up),
    o = W2 h, all accumulated in fp64 over bf16 operands.
    """
    E = len(counts)
    d = x.shape[1]
    f = weights["w13"]["codes"].shape[1] // 2
    rows = T * k + T
    h = np.zeros((rows, f), dtype=np.float64)
    o = np.zeros((rows, d), dtype=np.float64)
    for g in range(E + 1):
        if g < E:
            c, off = int(counts[g]), int(offsets[g])
            if c == 0:
                continue
            toks = sorted_token[off:off + c]
            W13 = dequant_expert(weights["w13"], g)
            W2 = dequant_expert(weights["w2"], g)
        else:
            c, off = T, T * k
            toks = np.arange(T)
            W13 = dequant_expert(weights["s13"], 0)
            W2 = dequant_expert(weights["s2"], 0)
        X = x[toks]
        fs = W13.shape[0] // 2
        gate = X @ W13[:fs].T
        up = X @ W13[fs:].T
        H = bf16_round(silu(gate) * up)
        h[off:off + c, :fs] = H
        o[off:off + c] = H @ W2.T
    return h, o


# --------------------------------------------------------------------------
# O10: unpermute and weighted combine with the shared expert (R2)
# --------------------------------------------------------------------------

def combine(o: np.ndarray, w: np.ndarray, row_of: np.ndarray, T: int, k: int) -> np.ndarray:
    """y[t] = o[T*k + t] + sum_j w[t, j] * o[row_of[t*k + j]]."""
    y = o[T * k:T * k + T].copy()
    for j in range(k):
        y += w[:, j:j + 1] * o[row_of.reshape(T, k)[:, j]]
    return y


# --------------------------------------------------------------------------
# router projection (R13)
# --------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """R13: logits[t, e] = sum over c of x[t, c] * Wr[e, c], in fp64 over the
    exactly decoded bf16 values (section "O modelo em três formatos de carga":
    the router scores every expert for every token). x is [T, d], Wr is [E, d];
    the result is [T, E]."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits).T


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------

def layer_forward(x_bits: np.ndarray, logits: np.ndarray,
                  weights: Dict[str, Dict[str, np.ndarray]], k: int, BM: int) -> Dict[str, np.ndarray]:
    """Every step of the layer; returns all intermediates and y [T, d] (fp64)."""
    T, E = logits.shape
    x = bf16_to_f64(x_bits)
    ids, w = route(logits, k)
    counts = histogram(ids, E)
    offsets = exclusive_scan(counts)
    sorted_token, row_of = scatter(ids, offsets)
    tiles = block_map(counts, offsets, T, k, BM)
    h, o = expert_ffn(x, sorted_token, counts, offsets, weights, T, k)
    y = combine(o, w, row_of, T, k)
    return {"ids": ids, "w": w, "counts": counts, "offsets": offsets,
            "sorted_token": sorted_token, "row_of": row_of, "tiles": tiles,
            "h": h, "o": o, "y": y}


def token_outputs(x_bits: np.ndarray, logits: np.ndarray,
                  weights: Dict[str, Dict[str, np.ndarray]], k: int,
                  tokens: np.ndarray, cache: Dict | None = None) -> np.ndarray:
    """y for a subset of tokens, one token at a time (for layers too large to run whole).

    Row-wise the layer is per token: y[t] = shared(x_t) + sum_j w_j expert_{id_j}(x_t),
    with the same roundings as expert_ffn. ``cache`` keeps dequantised experts.
    """
    cache = {} if cache is None else cache
    ids, w = route(logits[tokens], k)
    x = bf16_to_f64(x_bits[tokens])

    def mats(g):
        if g not in cache:
            if g < 0:
                cache[g] = (dequant_expert(weights["s13"], 0), dequant_expert(weights["s2"], 0))
            else:
                cache[g] = (dequant_expert(weights["w13"], g), dequant_expert(weights["w2"], g))
        return cache[g]

    def ffn(g, xt):
        W13, W2 = mats(g)
        fs = W13.shape[0] // 2
        H = bf16_round(silu(W13[:fs] @ xt) * (W13[fs:] @ xt))
        return W2 @ H

    y = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    for i in range(len(tokens)):
        y[i] = ffn(-1, x[i])
        for j in range(k):
            y[i] += w[i, j] * ffn(int(ids[i, j]), x[i])
    return y

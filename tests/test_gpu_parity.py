"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Routing ids, histogram, offsets, permutation and block map: bit-exact.
Router weights: |w - w_ref| <= 2e-6. Layer output y (fp32): max |err| <=
2e-2 RMS(y_ref) and mean |err| <= 2e-3 RMS(y_ref). Intermediates (diagnostic):
h within one bf16 ulp of the oracle's on all but a small fraction of
elements; the down GEMM and the combine checked in isolation from the GPU's
own inputs.
"""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import bias_cases
import moe_inputs as G
from oracle import moe_oracle as O
from parity_util import (W_ABS, check_bf16_close, check_y, dev_bits, expected_schedule, host_bits, say,
                         upload)

pytestmark = pytest.mark.gpu

# tokens up to which moe_layer_forward runs the per-token decode kernels
# (one grid row per token) rather than the routed, permuted grouped path
DECODE_MAX_T = 16

SMALL = [
    G.CONFIGS["tiny_t16"],
    G.small_config("ragged_t37_d192", T=37, d=192, f=128, E=5, k=3, seed=11),
    G.small_config("k1_t130", T=130, d=128, f=64, E=4, k=1, seed=12),
    G.small_config("kE_t40", T=40, d=256, f=64, E=6, k=6, seed=13),
    G.small_config("e1_t20", T=20, d=128, f=64, E=1, k=1, seed=14),
    G.small_config("t2_full_width", T=2, d=2048, f=512, E=256, k=8, seed=15),
    G.small_config("skew_empty_t300", T=300, d=256, f=128, E=32, k=4, seed=16, zipf_s=1.1,
                   n_forced_empty=3),
    G.small_config("multi_tile_t700", T=700, d=128, f=128, E=2, k=1, seed=17),
    # the widest inputs the grouped GEMMs take (their LDS scale tables for
    # K = 6144 leave room for one workgroup per CU)
    G.small_config("max_d6144_t40", T=40, d=6144, f=64, E=3, k=2, seed=18),
    G.small_config("max_f6144_t40", T=40, d=64, f=6144, E=3, k=2, seed=19),
    # up to 6 tokens the expert projections run on the VALU kernels (a few
    # weight rows per wavefront); f / 32 lanes per down row: 2, 4, 16, 32, 64
    G.small_config("gemv_t3_f64", T=3, d=64, f=64, E=4, k=2, seed=20),
    G.small_config("gemv_t5_d192", T=5, d=192, f=128, E=5, k=3, seed=21),
    G.small_config("gemv_t6_full_width", T=6, d=2048, f=512, E=256, k=8, seed=22),
    G.small_config("gemv_t6_f1024", T=6, d=512, f=1024, E=16, k=4, seed=24),
    G.small_config("gemv_t4_f2048", T=4, d=256, f=2048, E=8, k=2, seed=23),
    # decode kernels with more slots than the down kernel's 16 wavefronts
    # (wavefronts take two or three slots each), and f / 32 = 8 lanes per row
    G.small_config("decode_k20_f256", T=3, d=128, f=256, E=40, k=20, seed=25),
    G.small_config("decode_k32_t16", T=16, d=64, f=64, E=64, k=32, seed=26),
    # decode kernels over the widest input (three 2048-column passes per row)
    G.small_config("decode_d6144_t2", T=2, d=6144, f=64, E=4, k=2, seed=27),
    # the most experts and the largest k the library takes, grouped path
    G.small_config("max_e1024_k32_t40", T=40, d=64, f=64, E=1024, k=32, seed=28),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


_inputs = {}
_oracle = {}


def inputs(cfg):
    if cfg.name not in _inputs:
        _inputs[cfg.name] = G.make_layer_inputs(cfg)
    return _inputs[cfg.name]


def oracle(cfg):
    if cfg.name not in _oracle:
        inp = inputs(cfg)
        _oracle[cfg.name] = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k,
                                            BM=M.moe_block_m())
    return _oracle[cfg.name]


def staged(cfg):
    """Run the five entry points one after the other; return device tensors."""
    inp = inputs(cfg)
    dm, x, logits, w = upload(inp)
    ids, wts = M.moe_route(logits, cfg.k)
    perm = M.moe_permute(dm, ids)
    h, o_r, o_sh = M.moe_expert_ffn_w4(dm, x, w, perm["sorted_token"], perm["tile_map"],
                                       perm["num_tiles"])
    y = M.moe_unpermute_combine(dm, o_r, o_sh, wts, perm["row_of"])
    torch.cuda.synchronize()
    return dict(dm=dm, x=x, logits=logits, w=w, ids=ids, wts=wts, perm=perm, h=h, o_r=o_r,
                o_sh=o_sh, y=y)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_route_permute_bit_exact(cfg):
    say(f"[route/permute] {cfg.name}")
    ref = oracle(cfg)
    r = staged(cfg)
    assert np.array_equal(r["ids"].cpu().numpy(), ref["ids"])
    assert np.abs(r["wts"].cpu().numpy() - ref["w"]).max() <= W_ABS
    p = {k: v.cpu().numpy() for k, v in r["perm"].items()}
    assert np.array_equal(p["counts"], ref["counts"])
    assert np.array_equal(p["offsets"], ref["offsets"])
    assert np.array_equal(p["sorted_token"][:cfg.T * cfg.k], ref["sorted_token"])
    assert np.array_equal(p["row_of"][:cfg.T * cfg.k], ref["row_of"])
    n = int(p["num_tiles"][0])
    assert n == len(ref["tiles"]) <= M.moe_tile_capacity(r["dm"])
    assert np.array_equal(p["tile_map"][:n, :3], ref["tiles"])
    assert np.array_equal(p["tile_map"][:n, 3], expected_schedule(ref["tiles"]))


# Up to 64 tokens: one launch when each of the workgroup's wavefronts has at
# most 16 selection rounds (general selection above 256 experts counted 4x),
# else the route kernel and then the one-workgroup permutation.
ROUTE_PERMUTE = [
    G.small_config("rp_t1", T=1, d=64, f=64, E=256, k=8, seed=71),       # one launch
    G.small_config("rp_t2", T=2, d=64, f=64, E=256, k=8, seed=72),       # one launch
    G.small_config("rp_t32", T=32, d=64, f=64, E=256, k=8, seed=79),     # one launch, 16 rounds
    G.small_config("rp_t33", T=33, d=64, f=64, E=256, k=8, seed=80),     # route + permutation
    G.small_config("rp_t37_e5", T=37, d=64, f=64, E=5, k=3, seed=73),    # one launch
    G.small_config("rp_t16_e1000_k4", T=16, d=64, f=64, E=1000, k=4, seed=95),  # one launch
    G.small_config("rp_t64_kE", T=64, d=64, f=64, E=8, k=8, seed=74),    # route + permutation
    G.small_config("rp_t64_e1000", T=64, d=64, f=64, E=1000, k=32, seed=75),
    G.small_config("rp_t50_zipf_empty", T=50, d=64, f=64, E=256, k=8, seed=76, zipf_s=1.1,
                   n_forced_empty=8),
    G.small_config("rp_t65", T=65, d=64, f=64, E=256, k=8, seed=77),     # two-kernel path
    G.small_config("rp_t300_zipf", T=300, d=64, f=64, E=64, k=4, seed=78, zipf_s=1.1),
]


@pytest.mark.parametrize("cfg", ROUTE_PERMUTE, ids=lambda c: c.name)
def test_route_permute_one_call(cfg):
    """moe_route_permute (its one-workgroup paths up to 64 tokens) against the oracle, bit
    for bit, and against moe_route followed by moe_permute."""
    say(f"[route_permute] {cfg.name}")
    a = G.make_activations(cfg)
    logits = torch.from_numpy(a["logits"]).cuda()
    dm = M.dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k)
    r = M.moe_route_permute(dm, logits)
    ids, wts = M.moe_route(logits, cfg.k)
    perm = M.moe_permute(dm, ids)
    torch.cuda.synchronize()
    p = {k: v.cpu().numpy() for k, v in r.items()}
    rid, rw = O.route(a["logits"], cfg.k)
    counts = O.histogram(rid, cfg.E)
    offsets = O.exclusive_scan(counts)
    st, row_of = O.scatter(rid, offsets)
    tiles = O.block_map(counts, offsets, cfg.T, cfg.k, M.moe_block_m())
    assert np.array_equal(p["ids"], rid)
    assert np.abs(p["wts"] - rw).max() <= W_ABS
    assert np.array_equal(p["counts"], counts)
    assert np.array_equal(p["offsets"], offsets)
    assert np.array_equal(p["sorted_token"][:cfg.T * cfg.k], st)
    assert np.array_equal(p["row_of"][:cfg.T * cfg.k], row_of)
    n = int(p["num_tiles"][0])
    assert n == len(tiles)
    assert np.array_equal(p["tile_map"][:n, :3], tiles)
    assert np.array_equal(p["tile_map"][:n, 3], expected_schedule(tiles))
    # the same bits as the two entry points
    assert torch.equal(r["ids"], ids) and torch.equal(r["wts"], wts)
    for key in ("counts", "offsets", "sorted_token", "row_of"):
        assert torch.equal(r[key], perm[key]), key
    assert torch.equal(r["tile_map"][:n], perm["tile_map"][:n])


def _h_slack(cfg, inp, ref):
    T, k = cfg.T, cfg.k
    x = O.bf16_to_f64(inp["x"])
    slack = np.zeros((T * k + T, cfg.f))
    for g in range(cfg.E + 1):
        lo, hi = (ref["offsets"][g], ref["offsets"][g + 1]) if g < cfg.E else (T * k, T * k + T)
        if hi == lo:
            continue
        toks = ref["sorted_token"][lo:hi] if g < cfg.E else np.arange(T)
        W = O.dequant_expert(inp["weights"]["w13"] if g < cfg.E else inp["weights"]["s13"],
                             g if g < cfg.E else 0)
        X = x[toks]
        gate, up = X @ W[:cfg.f].T, X @ W[cfg.f:].T
        g_abs, u_abs = np.abs(X) @ np.abs(W[:cfg.f]).T, np.abs(X) @ np.abs(W[cfg.f:]).T
        # |d silu(z)/dz| <= 1.1
        slack[lo:hi] = 1e-5 * (1.1 * np.abs(up) * g_abs + np.abs(O.silu(gate)) * u_abs)
    return slack


# general and mixed dequantisation biases (the plain K loops of both grouped
# GEMMs at every row-block count, and the per-group plain branch of the decode
# and small-batch kernels)
GENERAL_BIAS = bias_cases.ALL


@pytest.mark.parametrize("cfg", SMALL + GENERAL_BIAS, ids=lambda c: c.name)
def test_expert_ffn_and_combine(cfg):
    say(f"[ffn] {cfg.name}")
    ref = oracle(cfg)
    r = staged(cfg)
    T, k = cfg.T, cfg.k
    inp = inputs(cfg)
    # gate/up + SiLU*up against the oracle's h; where gate or up cancels, allow the
    # fp32 accumulation error (relative to the sum of |terms|) to move h
    h = host_bits(r["h"])
    check_bf16_close(h, ref["h"], "h", max_frac=0.02, slack=_h_slack(cfg, inp, ref))
    # down GEMM from the GPU's own h: o = W2_g h_p, exact in fp64
    hg = O.bf16_to_f64(h)
    o_ref = np.zeros((T * k + T, cfg.d))
    o_abs = np.zeros((T * k + T, cfg.d))        # sum of |terms|: scale of fp32 rounding
    for g in range(cfg.E + 1):
        lo, hi = (ref["offsets"][g], ref["offsets"][g + 1]) if g < cfg.E else (T * k, T * k + T)
        if hi == lo:
            continue
        W2 = O.dequant_expert(inp["weights"]["w2"] if g < cfg.E else inp["weights"]["s2"],
                              g if g < cfg.E else 0)
        o_ref[lo:hi] = hg[lo:hi] @ W2.T
        o_abs[lo:hi] = np.abs(hg[lo:hi]) @ np.abs(W2).T
    o_r = host_bits(r["o_r"])[:T * k]
    check_bf16_close(o_r, O.bf16_round(o_ref[:T * k]), "o_routed", max_frac=0.02,
                     slack=1e-5 * o_abs[:T * k])
    o_sh = r["o_sh"].cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(o_ref[T * k:] ** 2))
    assert np.abs(o_sh - o_ref[T * k:]).max() <= 1e-5 * rms
    # combine from the GPU's own o and weights
    orr = O.bf16_to_f64(o_r)
    wts = r["wts"].cpu().numpy().astype(np.float64)
    row_of = ref["row_of"].reshape(T, k)
    y_ref = o_sh.copy()
    for j in range(k):
        y_ref += wts[:, j:j + 1] * orr[row_of[:, j]]
    y = r["y"].cpu().numpy().astype(np.float64)
    assert np.abs(y - y_ref).max() <= 1e-5 * np.sqrt(np.mean(y_ref ** 2))


@pytest.mark.parametrize("cfg", SMALL + GENERAL_BIAS + [G.CONFIGS["prefill_t512"]],
                         ids=lambda c: c.name)
def test_layer_forward_matches_oracle(cfg):
    say(f"[layer] {cfg.name}")
    inp = inputs(cfg)
    ref = oracle(cfg)
    dm, x, logits, w = upload(inp)
    y = M.moe_layer_forward(dm, x, logits, w)
    torch.cuda.synchronize()
    check_y(y.cpu().numpy(), ref["y"])
    if cfg.T > DECODE_MAX_T:
        # one call runs exactly the staged kernels: identical bits
        assert torch.equal(y, staged(cfg)["y"])
    else:
        # up to DECODE_MAX_T tokens the layer takes the per-token decode
        # kernels instead; the staged path agrees within the same tolerance
        check_y(staged(cfg)["y"].cpu().numpy(), ref["y"], "staged y")


def test_dequant_bit_exact_exhaustive_scales():
    say("[dequant] every bf16 scale x 16 codes, bias -8s; random biases")
    s_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s_val = O.bf16_to_f64(s_bits)
    keep = np.isfinite(s_val) & (np.abs(s_val) < 2.0 ** 120)
    s_bits = s_bits[keep]
    b_bits = O.round_to_bf16_bits(-8.0 * O.bf16_to_f64(s_bits))
    r = np.random.default_rng(21)
    n = len(s_bits)
    rand_b = O.round_to_bf16_bits(r.uniform(-1, 1, n) * np.abs(O.bf16_to_f64(s_bits)) * 16)
    for biases in (b_bits, rand_b):
        q = np.tile(np.arange(16, dtype=np.uint8), (n, 4))
        r.permuted(q, axis=1, out=q)
        codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        m = M.W4Matrix(torch.from_numpy(codes).cuda(), dev_bits(s_bits.reshape(n, 1)),
                       dev_bits(biases.reshape(n, 1)))
        out = host_bits(M.moe_dequant_w4(m))
        ref = O.round_to_bf16_bits(O.dequant(codes, s_bits.reshape(n, 1), biases.reshape(n, 1)))
        nan = np.isnan(O.bf16_to_f64(ref))
        bad = np.nonzero((out != ref) & ~nan)
        for r_, c_ in list(zip(*bad))[:8]:
            say(f"  mismatch s=0x{s_bits[r_]:04x} b=0x{biases[r_]:04x} q={q[r_, c_]} "
                f"gpu=0x{out[r_, c_]:04x} ref=0x{ref[r_, c_]:04x}")
        assert len(bad[0]) == 0, f"{len(bad[0])} mismatching weights"
    # signed zeros: s in {+0, -0} x b in {+0, -0} and b = -0 with normal scales
    zs = np.array([0x0000, 0x8000, 0x3C00, 0xBC00, 0x0000, 0x8000], np.uint16)
    zb = np.array([0x0000, 0x8000, 0x8000, 0x8000, 0x8000, 0x0000], np.uint16)
    q = np.tile(np.arange(16, dtype=np.uint8), (6, 4))
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    m = M.W4Matrix(torch.from_numpy(codes).cuda(), dev_bits(zs.reshape(6, 1)),
                   dev_bits(zb.reshape(6, 1)))
    out = host_bits(M.moe_dequant_w4(m))
    ref = O.round_to_bf16_bits(O.dequant(codes, zs.reshape(6, 1), zb.reshape(6, 1)))
    assert np.array_equal(out, ref)


def test_dequant_matches_oracle_on_layer_weights():
    say("[dequant] expert matrices of the Qwen3.6-35B-A3B-shaped layer")
    inp = inputs(G.CONFIGS["prefill_t512"])
    w = M.W4Weights.from_numpy(inp["weights"])
    for name, g in (("w13", 0), ("w13", 255), ("w2", 7), ("s13", 0), ("s2", 0)):
        out = host_bits(M.moe_dequant_w4(getattr(w, name), index=g))
        ref = O.round_to_bf16_bits(O.dequant_expert(inp["weights"][name], g))
        assert np.array_equal(out, ref), name


@pytest.mark.parametrize("E,k", [(256, 8), (1000, 8), (64, 1), (8, 8), (300, 32)])
def test_route_ties_zeros_and_inf(E, k):
    say(f"[route ties] E={E} k={k}")
    r = np.random.default_rng(E + k)
    T = 257
    l = (np.round(r.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    l[r.random((T, E)) < 0.2] = -0.0
    l[r.random((T, E)) < 0.2] = 0.0
    ninf = r.random((T, E)) < 0.3
    ninf[:, :k] = False
    l[ninf] = -np.inf
    l[5] = 0.0                       # a row of all-equal zeros (mixed signs below)
    l[5, ::3] = -0.0
    ids, wts = M.moe_route(torch.from_numpy(l).cuda(), k)
    rid, rw = O.route(l, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(wts.cpu().numpy() - rw).max() <= W_ABS
    assert list(ids[5].cpu().numpy()) == list(range(k))


def test_route_nan_stays_in_range():
    """NaN logits break the precondition; ids must still be distinct and in range."""
    say("[route nan]")
    l = np.random.default_rng(3).standard_normal((64, 256)).astype(np.float32)
    l[::2, ::3] = np.nan
    l[1] = np.nan
    ids, _ = M.moe_route(torch.from_numpy(l).cuda(), 8)
    ids = ids.cpu().numpy()
    assert ((ids >= 0) & (ids < 256)).all()
    assert all(len(set(row)) == 8 for row in ids)


def test_zero_tokens_is_noop():
    say("[T=0]")
    cfg = G.CONFIGS["tiny_t16"]
    _, x, logits, w = upload(inputs(cfg))
    dm = M.dims(0, cfg.d, cfg.f, cfg.E, cfg.k)
    y = torch.full((1, cfg.d), 7.0, device="cuda")
    M.moe_layer_forward(dm, x, logits, w, y=y, ws=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert (y == 7.0).all()


# A block map whose groups have more rows than there are tokens, as ids that
# repeat an expert within a token would give. moe_permute requires distinct
# ids per token, so the map is built here from the oracle's steps and handed
# to the grouped GEMMs directly. Up to 32 tokens the GEMMs run the kernel
# compiled for one-row-block tiles, which takes a taller tile in 32-row
# passes. The largest group here: 61 rows (one tile, two passes), 256 rows
# (two full tiles, four passes each) and 108 rows (four passes).
REPEAT_IDS = [
    G.small_config("rep_t24_k4_e4", T=24, d=128, f=64, E=4, k=4, seed=96),
    G.small_config("rep_t32_k8_e8_all0", T=32, d=192, f=128, E=8, k=8, seed=97),
    G.small_config("rep_t17_k8_e8", T=17, d=2048, f=512, E=8, k=8, seed=98, bias_mode=G.BIAS_MIXED),
]


def _repeat_ids(cfg):
    r = np.random.default_rng(cfg.seed)
    T, k, E = cfg.T, cfg.k, cfg.E
    if cfg.name.endswith("all0"):
        return np.zeros((T, k), dtype=np.int32)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    ids[r.random((T, k)) < 0.7] = 0
    return ids


@pytest.mark.parametrize("cfg", REPEAT_IDS, ids=lambda c: c.name)
def test_tall_groups_from_repeated_ids(cfg):
    say(f"[tall groups] {cfg.name}")
    T, k, E = cfg.T, cfg.k, cfg.E
    inp = inputs(cfg)
    ids = _repeat_ids(cfg)
    r = np.random.default_rng(cfg.seed + 1)
    wts = r.random((T, k)).astype(np.float32)
    wts /= wts.sum(axis=1, keepdims=True)
    counts = O.histogram(ids, E)
    offsets = O.exclusive_scan(counts)
    sorted_token, row_of = O.scatter(ids, offsets)
    tiles = O.block_map(counts, offsets, T, k, M.moe_block_m())
    assert counts.max() > 32  # some tile needs more than one pass
    h_ref, o_ref = O.expert_ffn(O.bf16_to_f64(inp["x"]), sorted_token, counts, offsets,
                                inp["weights"], T, k)
    y_ref = O.combine(o_ref, wts.astype(np.float64), row_of, T, k)

    dm, x, _, w = upload(inp)
    tmap = np.zeros((M.moe_tile_capacity(dm), 4), dtype=np.int32)
    tmap[:len(tiles), :3] = tiles
    tmap[:len(tiles), 3] = expected_schedule(tiles)
    dev_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    h, o_r, o_sh = M.moe_expert_ffn_w4(dm, x, w, dev_i32(sorted_token), dev_i32(tmap),
                                       dev_i32([len(tiles), 0, 0, 0]))
    y = M.moe_unpermute_combine(dm, o_r, o_sh, torch.from_numpy(wts).cuda(), dev_i32(row_of))
    torch.cuda.synchronize()
    ref = dict(offsets=offsets, sorted_token=sorted_token)
    check_bf16_close(host_bits(h), h_ref, "h", max_frac=0.02, slack=_h_slack(cfg, inp, ref))
    check_y(y.cpu().numpy(), y_ref)


# Routing built so that every expert a token block picks gets exactly 128 rows: token
# block b (128 tokens) picks experts k*b .. k*b + k - 1, and the tokens past the last
# whole block pick the next k experts. The full tiles F (routed, then the shared
# expert's) then fall on each side of the XCD runs' edge cases: fewer than 8, exactly
# 8, one and two past a multiple of 8, with and without partial tiles after them.
FULL_RUNS = [
    ("runs_f7_t128_k6", 128, 6, 8, 126),    # 6 + 1 full tiles: seven runs of one
    ("runs_f8_t128_k7", 128, 7, 8, 127),    # 7 + 1: one tile per run
    ("runs_f9_t128_k8", 128, 8, 16, 128),   # 8 + 1: run 0 holds two
    ("runs_f18_t293_k8", 293, 8, 32, 129),  # 16 + 2, then nine 37-row tiles
]


@pytest.mark.parametrize("case", FULL_RUNS, ids=lambda c: c[0])
def test_schedule_runs_of_full_tiles(case):
    name, T, k, E, seed = case
    say(f"[full-tile runs] {name}")
    cfg = G.small_config(name, T=T, d=128, f=64, E=E, k=k, seed=seed)
    inp = dict(G.make_layer_inputs(cfg))
    logits = np.asarray(inp["logits"], dtype=np.float32) * np.float32(0.01)
    for t in range(T):
        b = t // 128
        logits[t, [(k * b + j) % E for j in range(k)]] += np.float32(4.0 + 0.1 * np.arange(k))
    inp["logits"] = logits
    ref = O.layer_forward(inp["x"], logits, inp["weights"], k, BM=M.moe_block_m())
    counts = ref["counts"]
    assert sorted(set(counts.tolist()) - {0}) == sorted({128} | ({T % 128} - {0}))
    dm, x, lg, w = upload(inp)
    ids, wts = M.moe_route(lg, k)
    perm = M.moe_permute(dm, ids)
    h, o_r, o_sh = M.moe_expert_ffn_w4(dm, x, w, perm["sorted_token"], perm["tile_map"],
                                       perm["num_tiles"])
    y = M.moe_unpermute_combine(dm, o_r, o_sh, wts, perm["row_of"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    p = {kk: v.cpu().numpy() for kk, v in perm.items()}
    n = int(p["num_tiles"][0])
    assert n == len(ref["tiles"])
    assert np.array_equal(p["tile_map"][:n, :3], ref["tiles"])
    sched = expected_schedule(ref["tiles"])
    assert np.array_equal(p["tile_map"][:n, 3], sched)
    full = int(((ref["tiles"][:, 2] - ref["tiles"][:, 1]) == 128).sum())
    assert full == {126: 7, 127: 8, 128: 9, 129: 18}[seed]
    check_y(y.cpu().numpy(), ref["y"])

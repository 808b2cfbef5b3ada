"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one moe_layer_forward call per layer), plus robustness.

The oracle cannot run the whole T=4096 / T=16384 layers in test time, so:
routing, histogram, offsets, permutation and block map are compared in full
(bit-exact); y is compared on sampled tokens computed one by one by the
oracle; every output must be finite. Decode (T=1): routing on all 1000
steps, y on a seeded subset of steps.
"""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import moe_inputs as G
from oracle import moe_oracle as O
from parity_util import (W_ABS, check_y, dev_bits, expected_schedule, fill_expert_cache, say,
                         upload)

pytestmark = pytest.mark.gpu

_cache = {}      # dequantised experts, shared: these workloads use identical weights


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


def _check_routing(cfg, inp, dm, logits):
    ids, wts = M.moe_route(logits, cfg.k)
    perm = M.moe_permute(dm, ids)
    torch.cuda.synchronize()
    rid, rw = O.route(inp["logits"], cfg.k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(wts.cpu().numpy() - rw).max() <= W_ABS
    counts = O.histogram(rid, cfg.E)
    offsets = O.exclusive_scan(counts)
    st, row_of = O.scatter(rid, offsets)
    tiles = O.block_map(counts, offsets, cfg.T, cfg.k, M.moe_block_m())
    p = {k: v.cpu().numpy() for k, v in perm.items()}
    assert np.array_equal(p["counts"], counts)
    assert np.array_equal(p["offsets"], offsets)
    assert np.array_equal(p["sorted_token"], st)
    assert np.array_equal(p["row_of"], row_of)
    n = int(p["num_tiles"][0])
    assert n == len(tiles) <= M.moe_tile_capacity(dm)
    assert np.array_equal(p["tile_map"][:n, :3], tiles)
    assert np.array_equal(p["tile_map"][:n, 3], expected_schedule(tiles))
    return counts


@pytest.mark.parametrize("name", ["prefill_t4096_zipf", "prefill_t16384_zipf_empty"])
def test_full_size_prefill(name):
    cfg = G.CONFIGS[name]
    say(f"[full size] {name}: routing + permutation")
    inp = G.make_layer_inputs(cfg)
    dm, x, logits, w = upload(inp)
    counts = _check_routing(cfg, inp, dm, logits)
    if cfg.n_forced_empty:
        assert (counts[G.forced_empty_experts(cfg)] == 0).all()
    assert counts.max() > 10 * counts.mean() and (counts == 0).any()   # skew really present
    say(f"[full size] {name}: layer forward")
    y = M.moe_layer_forward(dm, x, logits, w)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all()
    r = np.random.default_rng(5)
    # sampled tokens: for every non-empty expert, the token of its last permuted
    # row (so the last, possibly partial, tile of every group is checked: every
    # tile between 33 and 127 rows is such a tile), of its first row and of one
    # random row; tokens routed to the most loaded expert; the first and last
    # tokens, and 20 random ones
    rid, _ = O.route(inp["logits"], cfg.k)
    offsets = O.exclusive_scan(counts)
    st, _ = O.scatter(rid, offsets)
    picks = [r.choice(cfg.T, 20, replace=False), [0, cfg.T - 1]]
    for g in np.nonzero(counts)[0]:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        picks.append([st[lo], st[hi - 1], st[r.integers(lo, hi)]])
    top = int(np.argmax(counts))
    heavy = np.nonzero((rid == top).any(axis=1))[0]
    picks += [heavy[:4], heavy[-4:]]
    toks = np.unique(np.concatenate([np.asarray(p, dtype=np.int64) for p in picks]))
    # every non-empty expert is checked on at least one of its rows
    checked = np.unique(rid[toks])
    assert set(np.nonzero(counts)[0]) <= set(checked.tolist())
    say(f"[full size] {name}: oracle on {len(toks)} tokens covering all "
        f"{int((counts > 0).sum())} non-empty experts")
    fill_expert_cache(inp["weights"], checked, _cache)
    ref = O.token_outputs(inp["x"], inp["logits"], inp["weights"], cfg.k, toks, cache=_cache)
    check_y(yh[toks], ref, f"y[{len(toks)} sampled tokens]")


# Many tokens at narrow widths: a million tokens over 4,097 permutation
# blocks (each placement workgroup scans every earlier block's counts), and
# 262,144 Zipf-routed tokens over 256 experts (1,025 blocks); routing,
# permutation and block map in full, y on sampled tokens.
MANY = [
    G.small_config("many_t1m_e8_k2", T=1 << 20, d=128, f=64, E=8, k=2, seed=101),
    G.small_config("many_t262k_e256_k8", T=1 << 18, d=64, f=64, E=256, k=8, seed=102,
                   zipf_s=1.1),
]


@pytest.mark.parametrize("cfg", MANY, ids=lambda c: c.name)
def test_many_tokens(cfg):
    say(f"[many tokens] {cfg.name}: routing + permutation")
    inp = G.make_layer_inputs(cfg)
    dm, x, logits, w = upload(inp)
    counts = _check_routing(cfg, inp, dm, logits)
    say(f"[many tokens] {cfg.name}: layer forward")
    y = M.moe_layer_forward(dm, x, logits, w)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all()
    r = np.random.default_rng(cfg.seed)
    rid, _ = O.route(inp["logits"], cfg.k)
    offsets = O.exclusive_scan(counts)
    st, _ = O.scatter(rid, offsets)
    picks = [r.choice(cfg.T, 24, replace=False), [0, cfg.T - 1]]
    for g in np.nonzero(counts)[0]:
        picks.append([st[int(offsets[g])], st[int(offsets[g + 1]) - 1]])
    toks = np.unique(np.concatenate([np.asarray(p, dtype=np.int64) for p in picks]))
    ref = O.token_outputs(inp["x"], inp["logits"], inp["weights"], cfg.k, toks)
    check_y(yh[toks], ref, f"y[{len(toks)} sampled tokens]")


def test_decode_b1():
    cfg = G.CONFIGS["decode_b1"]
    say("[decode] routing of all 1000 steps")
    steps = G.make_decode_steps(cfg)
    weights = G.make_weights(cfg)
    logits_all = torch.from_numpy(steps["logits"]).cuda()
    ids, wts = M.moe_route(logits_all, cfg.k)
    rid, rw = O.route(steps["logits"], cfg.k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(wts.cpu().numpy() - rw).max() <= W_ABS
    say("[decode] y on 64 seeded steps through the T=1 path")
    w = M.W4Weights.from_numpy(weights)
    dm = M.dims(1, cfg.d, cfg.f, cfg.E, cfg.k)
    ws = torch.empty(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    x_all = dev_bits(steps["x"])
    pick = np.sort(np.random.default_rng(7).choice(cfg.decode_steps, 64, replace=False))
    ys = []
    for s in pick:
        ys.append(M.moe_layer_forward(dm, x_all[s:s + 1], logits_all[s:s + 1], w, ws=ws).clone())
    torch.cuda.synchronize()
    y = torch.cat(ys).cpu().numpy()
    fill_expert_cache(weights, np.unique(rid[pick]), _cache)
    ref = O.token_outputs(steps["x"], steps["logits"], weights, cfg.k, pick, cache=_cache)
    check_y(y, ref, "decode y")
    # the T=1 path agrees with the prefill kernels run on the same single token
    s = int(pick[0])
    dm1 = M.dims(1, cfg.d, cfg.f, cfg.E, cfg.k)
    idsd, wd = M.moe_route(logits_all[s:s + 1], cfg.k)
    perm = M.moe_permute(dm1, idsd)
    h, o_r, o_sh = M.moe_expert_ffn_w4(dm1, x_all[s:s + 1], w, perm["sorted_token"],
                                       perm["tile_map"], perm["num_tiles"])
    yp = M.moe_unpermute_combine(dm1, o_r, o_sh, wd, perm["row_of"])
    torch.cuda.synchronize()
    check_y(yp.cpu().numpy(), ref[:1], "prefill kernels at T=1")


def test_small_decode_shapes():
    for cfg in (G.small_config("dec_small", T=1, d=128, f=64, E=8, k=2, seed=31),
                G.small_config("dec_k1", T=1, d=256, f=128, E=16, k=1, seed=32),
                G.small_config("dec_wide", T=1, d=4096, f=256, E=64, k=4, seed=33)):
        say(f"[decode small] {cfg.name}")
        inp = G.make_layer_inputs(cfg)
        dm, x, logits, w = upload(inp)
        y = M.moe_layer_forward(dm, x, logits, w)
        torch.cuda.synchronize()
        ref = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=M.moe_block_m())
        check_y(y.cpu().numpy(), ref["y"], cfg.name)


def test_deterministic_bits():
    cfg = G.CONFIGS["prefill_t4096_zipf"]
    say("[determinism] two runs of the T=4096 layer")
    inp = G.make_layer_inputs(cfg)
    dm, x, logits, w = upload(inp)
    ws = torch.empty(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    y1 = M.moe_layer_forward(dm, x, logits, w, ws=ws).clone()
    ws.fill_(0xAB)
    y2 = M.moe_layer_forward(dm, x, logits, w, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ids, _ = M.moe_route(logits, cfg.k)
    p1 = M.moe_permute(dm, ids)
    p2 = M.moe_permute(dm, ids)
    torch.cuda.synchronize()
    n = int(p1["num_tiles"][0])
    assert torch.equal(p1["tile_map"][:n], p2["tile_map"][:n])
    for key in ("counts", "offsets", "sorted_token", "row_of", "num_tiles"):
        assert torch.equal(p1[key], p2[key]), key


def test_nan_scales_of_empty_experts_are_never_read():
    cfg = G.small_config("nan_empty", T=200, d=256, f=128, E=32, k=4, seed=41, zipf_s=1.1,
                         n_forced_empty=4)
    say(f"[robust] {cfg.name}")
    inp = G.make_layer_inputs(cfg)
    dm, x, logits, w = upload(inp)
    y1 = M.moe_layer_forward(dm, x, logits, w).clone()
    counts = O.histogram(O.route(inp["logits"], cfg.k)[0], cfg.E)
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) >= 4
    for name in ("w13", "w2"):
        for key in ("scales", "biases"):
            getattr(w, name).__dict__[key][torch.from_numpy(empty).cuda()] = 0x7FC0  # bf16 NaN
    y2 = M.moe_layer_forward(dm, x, logits, w)
    torch.cuda.synchronize()
    assert torch.isfinite(y2).all()
    assert torch.equal(y1, y2)


def test_guard_canaries_around_outputs():
    cfg = G.small_config("canary", T=77, d=192, f=128, E=8, k=2, seed=51)
    say(f"[robust] {cfg.name}")
    inp = G.make_layer_inputs(cfg)
    dm, x, logits, w = upload(inp)
    G_ = 64
    n = cfg.T * cfg.d
    ybuf = torch.full((n + 2 * G_,), 12345.0, device="cuda")
    wsn = M.moe_layer_workspace_bytes(dm)
    wsbuf = torch.full((wsn + 2 * 256,), 0x5A, dtype=torch.uint8, device="cuda")
    y = ybuf[G_:G_ + n].view(cfg.T, cfg.d)
    M.moe_layer_forward(dm, x, logits, w, y=y, ws=wsbuf[256:256 + wsn])
    torch.cuda.synchronize()
    assert (ybuf[:G_] == 12345.0).all() and (ybuf[G_ + n:] == 12345.0).all()
    assert (wsbuf[:256] == 0x5A).all() and (wsbuf[256 + wsn:] == 0x5A).all()
    ref = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k, BM=M.moe_block_m())
    check_y(y.cpu().numpy(), ref["y"], "canary y")

"""The general-bias test inputs reach every exact dequantisation path the
kernels have (CPU only: a property of the inputs, checked before any GPU test
relies on it)."""
import numpy as np

import moe_inputs as G
from bias_cases import DECODE, GROUPED, fast_groups, gemm_blocks_fast
from oracle import moe_oracle as O


def _used_experts(cfg, inp):
    ids, _ = O.route(inp["logits"], cfg.k)
    return np.unique(ids)


def test_neg8_weights_take_only_the_fast_path():
    cfg = G.CONFIGS["tiny_t16"]
    w = G.make_weights(cfg)
    for m in w.values():
        assert fast_groups(m["scales"], m["biases"]).all()


def test_grouped_cases_reach_the_plain_k_loop():
    for cfg in GROUPED:
        inp = G.make_layer_inputs(cfg)
        used = _used_experts(cfg, inp)
        gate_up, down = gemm_blocks_fast(inp["weights"], cfg.f)
        s_gate_up, s_down = gemm_blocks_fast({"w13": inp["weights"]["s13"],
                                              "w2": inp["weights"]["s2"]}, cfg.f)
        gu = np.concatenate([gate_up[used].ravel(), s_gate_up.ravel()])
        dn = np.concatenate([down[used].ravel(), s_down.ravel()])
        # some wavefronts take the plain K loop in both GEMMs
        assert (~gu).any() and (~dn).any(), cfg.name
        if cfg.bias_mode == G.BIAS_MIXED:
            # and others the fast one, in the same launch
            assert gu.any() and dn.any(), cfg.name


def test_decode_cases_mix_both_paths_per_group():
    for cfg in DECODE:
        inp = G.make_layer_inputs(cfg)
        used = _used_experts(cfg, inp)
        for name in ("w13", "w2"):
            m = inp["weights"][name]
            fg = fast_groups(m["scales"][used], m["biases"][used])
            assert fg.any() and (~fg).any(), (cfg.name, name)


def test_general_biases_hold_the_special_values():
    w = G.make_w4(3, 10, 11, 8, 64, 2048, 0.005, 0.02, G.BIAS_GENERAL)
    s, b = O.bf16_to_f64(w["scales"]), O.bf16_to_f64(w["biases"])
    assert (w["biases"] == 0x0000).any() and (w["biases"] == 0x8000).any()   # +0 and -0
    assert (s < 0).any()                                                   # negative scales
    assert (np.abs(s) < 2.0 ** -100).any()                                 # tiny scales
    assert (np.abs(b) > 2.0 ** 20 * np.abs(s)).any()                       # bias far above scale
    # weights stay normal fp32 numbers (no subnormal from cancellation)
    W = O.dequant(w["codes"][0], w["scales"][0], w["biases"][0])
    assert not ((W != 0) & (np.abs(W) < 2.0 ** -126)).any()

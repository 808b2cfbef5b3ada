"""Regression guard for the grouped GEMMs' LDS ordering.

The build also makes libmoe_w4_schedcheck.so: the same sources, with the
grouped GEMMs compiled with a scheduling barrier after each K step's loads.
That schedule leaves more of a step's A-fragment LDS reads in flight towards
the step's end; the activation DMA issued right after the next barrier
refills the stage those reads come from. The results stay correct only while
each barrier of the K loop also waits for the wavefront's own LDS reads. So
the check library must give the same bits as the main library, and match the
oracle.
"""
import os

import numpy as np
import pytest
import torch

import bit_quantized_grouped_router_amd as M
import bias_cases
import moe_inputs as G
from bit_quantized_grouped_router_amd import build as B
from oracle import moe_oracle as O
from parity_util import check_y, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    assert os.path.exists(B.SCHEDCHECK_PATH), "the build makes the schedule-check library"
    yield
    torch.cuda.synchronize()


CASES = [G.CONFIGS["prefill_t4096_zipf"],
         [c for c in bias_cases.GROUPED if c.name == "gb_t700_mixed"][0]]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_schedule_check_build_is_bit_identical(cfg):
    say(f"[schedcheck] {cfg.name}")
    inp = G.make_layer_inputs(cfg)
    dm, x, logits, w = upload(inp)
    y_main = M.moe_layer_forward(dm, x, logits, w)
    torch.cuda.synchronize()
    with M.using_library(B.SCHEDCHECK_PATH):
        y_check = M.moe_layer_forward(dm, x, logits, w)
        torch.cuda.synchronize()
    diff = (y_main - y_check).abs().max().item()
    say(f"  max |main - check| = {diff:.3e}")
    assert torch.equal(y_main, y_check)
    if cfg.T <= 1024:
        ref = O.layer_forward(inp["x"], inp["logits"], inp["weights"], cfg.k,
                              BM=M.moe_block_m())["y"]
        check_y(y_check.cpu().numpy(), ref, f"{cfg.name} y (check library)")

"""The C-ABI library loads, exports every declared entry point, and validates
arguments on the host before touching the GPU (no GPU needed: every call
below returns before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import bit_quantized_grouped_router_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        from bit_quantized_grouped_router_amd import build
        build.build()
    return M.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_are_all_exported(L):
    names = declared_functions()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", M.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(M.EXPORTS) == set(names)
    for n in names:
        getattr(L, n)


def test_library_has_gfx950_code_only():
    out = subprocess.run(["/opt/rocm/bin/roc-obj-ls", M.LIB_PATH], capture_output=True, text=True)
    if out.returncode != 0:
        pytest.skip("roc-obj-ls unavailable")
    assert "gfx950" in out.stdout
    assert not re.search(r"gfx9[0-4]\d\b", out.stdout.replace("gfx950", ""))


def _dims(T=16, d=128, f=64, E=8, k=2, f_shared=None):
    return M.MoeDims(T, d, f, E, k, f if f_shared is None else f_shared)


def test_block_m_and_capacity(L):
    BM = L.moe_block_m()
    assert BM == 128
    for (T, E, k) in [(16, 8, 2), (4096, 256, 8), (16384, 256, 8), (1, 256, 8), (3, 5, 5)]:
        dm = _dims(T=T, d=2048, f=512, E=E, k=k)
        tk = T * k
        routed = min(tk, (tk + min(E, tk) * (BM - 1)) // BM)
        assert L.moe_tile_capacity(ctypes.byref(dm)) == routed + -(-T // BM)


def test_status_strings(L):
    for st in (OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP):
        assert L.moe_status_string(st)
    assert L.moe_last_hip_error() == 0


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def test_route_validation(L):
    assert L.moe_route(None, 0, 8, 2, None, None, None) == OK          # T == 0: no-op
    assert L.moe_route(None, 4, 8, 2, FAKE, FAKE, None) == INVALID     # null logits
    assert L.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, None) == INVALID     # k > E
    assert L.moe_route(FAKE, 4, 8, 0, FAKE, FAKE, None) == INVALID
    assert L.moe_route(FAKE, -1, 8, 2, FAKE, FAKE, None) == INVALID
    assert L.moe_route(FAKE, 4, 2048, 8, FAKE, FAKE, None) == UNSUPPORTED
    assert L.moe_route(FAKE, 4, 64, 33, FAKE, FAKE, None) == UNSUPPORTED
    assert L.moe_route(FAKE + 4, 4, 8, 2, FAKE, FAKE, None) == ALIGN


def test_dims_validation(L):
    f = L.moe_layer_workspace_bytes
    assert f(ctypes.byref(_dims(d=100))) == 0
    assert f(ctypes.byref(_dims(f=96))) == 0
    assert f(ctypes.byref(_dims(E=2000))) == 0
    assert f(ctypes.byref(_dims(k=9))) == 0
    assert f(ctypes.byref(_dims(f_shared=0))) == 0
    assert f(ctypes.byref(_dims())) > 0
    assert L.moe_tile_capacity(ctypes.byref(_dims(d=100))) == -1
    # the largest batch: T * (k + 1) rows of max(d, 2f) elements under 2^31
    # (116,508 tokens at the headline widths)
    assert f(ctypes.byref(_dims(T=116508, d=2048, f=512, E=256, k=8))) > 0
    assert f(ctypes.byref(_dims(T=116509, d=2048, f=512, E=256, k=8))) == 0
    # workspace grows with T
    a = f(ctypes.byref(_dims(T=100, d=2048, f=512, E=256, k=8)))
    b = f(ctypes.byref(_dims(T=200, d=2048, f=512, E=256, k=8)))
    assert b > a > 0


def _weights(base=FAKE):
    m = M.MoeW4Matrix(base, base, base)
    return M.MoeW4Weights(m, m, m, m)


def test_layer_forward_validation(L):
    w = _weights()
    dm = _dims()
    need = L.moe_layer_workspace_bytes(ctypes.byref(dm))
    fw = L.moe_layer_forward
    assert fw(ctypes.byref(_dims(T=0)), None, None, ctypes.byref(w), None, None, 0, None) == OK
    assert fw(ctypes.byref(_dims(d=100)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need, None) == UNSUPPORTED
    # the grouped GEMMs keep a tile's scales for every K group in LDS: K <= 6144
    assert fw(ctypes.byref(_dims(d=6208)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need, None) == UNSUPPORTED
    assert fw(ctypes.byref(_dims(f=6208)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need, None) == UNSUPPORTED
    assert fw(ctypes.byref(dm), FAKE, FAKE, None, FAKE, FAKE, need, None) == INVALID
    # the shared expert's width: another width is a valid layer these kernels do not run
    assert fw(ctypes.byref(_dims(f_shared=128)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need,
              None) == UNSUPPORTED
    assert fw(ctypes.byref(_dims(f_shared=0)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need,
              None) == INVALID
    assert fw(ctypes.byref(_dims(f_shared=-64)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need,
              None) == INVALID
    assert L.moe_tile_capacity(ctypes.byref(_dims(f_shared=128))) == -1
    assert fw(ctypes.byref(dm), None, FAKE, ctypes.byref(w), FAKE, FAKE, need, None) == INVALID
    assert fw(ctypes.byref(dm), FAKE, FAKE, ctypes.byref(_weights(FAKE + 2)), FAKE, FAKE, need, None) == ALIGN
    assert fw(ctypes.byref(dm), FAKE, FAKE, ctypes.byref(w), FAKE + 8, FAKE, need, None) == ALIGN
    assert fw(ctypes.byref(dm), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need - 1, None) == WORKSPACE
    bad = M.MoeW4Weights(w.w13, w.w2, M.MoeW4Matrix(FAKE, None, FAKE), w.s2)
    assert fw(ctypes.byref(dm), FAKE, FAKE, ctypes.byref(bad), FAKE, FAKE, need, None) == INVALID


def test_permute_and_ffn_validation(L):
    dm = _dims(T=300, d=256, f=128, E=16, k=4)
    need = L.moe_permute_workspace_bytes(ctypes.byref(dm))
    assert need == 2 * 16 * 4                     # two blocks of 256 tokens x E counters
    p = L.moe_permute
    args = [FAKE] * 7
    assert p(ctypes.byref(dm), *args, FAKE, need - 4, None) == WORKSPACE
    assert p(ctypes.byref(dm), None, *args[1:], FAKE, need, None) == INVALID
    w = _weights()
    assert L.moe_expert_gate_up_w4(ctypes.byref(dm), FAKE, ctypes.byref(w), FAKE, FAKE, FAKE,
                                   None, None) == INVALID
    assert L.moe_expert_down_w4(ctypes.byref(dm), FAKE, ctypes.byref(w), FAKE, FAKE, FAKE + 1,
                                FAKE, None) == ALIGN
    assert L.moe_unpermute_combine(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, None, None) == INVALID
    assert L.moe_expert_ffn_w4(ctypes.byref(_dims(T=0)), None, None, None, None, None, None,
                               None, None, None) == OK
    m = M.MoeW4Matrix(FAKE, FAKE, FAKE)
    assert L.moe_dequant_w4(ctypes.byref(m), 4, 100, FAKE, None) == UNSUPPORTED
    assert L.moe_dequant_w4(ctypes.byref(m), 0, 128, FAKE, None) == OK
    assert L.moe_dequant_w4(None, 4, 128, FAKE, None) == INVALID


def test_route_permute_validation(L):
    rp = L.moe_route_permute
    dm = _dims(T=300, d=256, f=128, E=16, k=4)
    need = L.moe_permute_workspace_bytes(ctypes.byref(dm))
    args = [FAKE] * 9
    assert rp(ctypes.byref(_dims(T=0)), *([None] * 10), 0, None) == OK
    assert rp(ctypes.byref(dm), None, *args[1:], FAKE, need, None) == INVALID
    assert rp(ctypes.byref(dm), *args[:4], FAKE + 4, *args[5:], FAKE, need, None) == ALIGN
    assert rp(ctypes.byref(dm), *args, FAKE, need - 4, None) == WORKSPACE
    assert rp(ctypes.byref(_dims(k=9)), *args, FAKE, need, None) == INVALID


def test_router_validation(L):
    r = L.moe_router_logits
    assert r(None, None, 0, 64, 8, None, None) == OK                   # T == 0: no-op
    assert r(FAKE, FAKE, -1, 64, 8, FAKE, None) == INVALID
    assert r(FAKE, FAKE, 4, 0, 8, FAKE, None) == INVALID
    assert r(FAKE, FAKE, 4, 64, 0, FAKE, None) == INVALID
    assert r(FAKE, FAKE, 4, 100, 8, FAKE, None) == UNSUPPORTED         # d % 64 != 0
    assert r(FAKE, FAKE, 4, 64, 1025, FAKE, None) == UNSUPPORTED
    assert r(FAKE, FAKE, 1 << 19, 4096, 8, FAKE, None) == UNSUPPORTED   # T*d = 2^31
    assert r(None, FAKE, 4, 64, 8, FAKE, None) == INVALID
    assert r(FAKE, FAKE, 4, 64, 8, None, None) == INVALID
    assert r(FAKE, FAKE + 8, 4, 64, 8, FAKE, None) == ALIGN


def test_layer_forward_hidden_validation(L):
    w = _weights()
    dm = _dims()
    need = L.moe_layer_workspace_bytes(ctypes.byref(dm))
    fh = L.moe_layer_forward_hidden
    assert fh(ctypes.byref(_dims(T=0)), None, None, ctypes.byref(w), None, None, 0, None) == OK
    assert fh(ctypes.byref(_dims(d=100)), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need, None) == UNSUPPORTED
    assert fh(ctypes.byref(dm), FAKE, None, ctypes.byref(w), FAKE, FAKE, need, None) == INVALID
    assert fh(ctypes.byref(dm), FAKE, FAKE + 4, ctypes.byref(w), FAKE, FAKE, need, None) == ALIGN
    assert fh(ctypes.byref(dm), FAKE, FAKE, None, FAKE, FAKE, need, None) == INVALID
    assert fh(ctypes.byref(dm), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, need - 1, None) == WORKSPACE
    # the workspace holds the router scores too: it grows with E
    a = L.moe_layer_workspace_bytes(ctypes.byref(_dims(T=64, E=8)))
    b = L.moe_layer_workspace_bytes(ctypes.byref(_dims(T=64, E=64)))
    assert b >= a + 64 * 56 * 4


def test_binding_refuses_cpu_tensors(L):
    import torch
    with pytest.raises(M.MoeError):
        M.moe_route(torch.zeros((4, 8)), 2)


def test_binding_checks_buffer_sizes(L):
    """The binding refuses a tensor smaller than the dims imply (the kernels would
    index past its end) before it looks at the device; the size check runs on
    CPU tensors too."""
    import torch

    T, d, f, E, k = 4, 128, 64, 8, 2
    dm = M.dims(T, d, f, E, k)
    # routing (T and E come from the logits' shape): an output one column short
    with pytest.raises(M.MoeError, match="topk_ids holds"):
        M.moe_route(torch.zeros((T, E), dtype=torch.float32), k,
                    topk_ids=torch.zeros((T, k - 1), dtype=torch.int32),
                    topk_w=torch.zeros((T, k), dtype=torch.float32))
    # right sizes get past the size check and stop at the device check
    with pytest.raises(M.MoeError, match="GPU memory"):
        M.moe_route(torch.zeros((T, E), dtype=torch.float32), k,
                    topk_ids=torch.zeros((T, k), dtype=torch.int32),
                    topk_w=torch.zeros((T, k), dtype=torch.float32))

    def weights(short=None):
        def mat(n, rows, cols, cut):
            c = torch.zeros(n * rows * cols // 2 - (16 if cut else 0), dtype=torch.uint8)
            s = torch.zeros(n * rows * cols // 64, dtype=torch.int16)
            return M.W4Matrix(c, s, s.clone())
        return M.W4Weights(mat(E, 2 * f, d, short == "w13"), mat(E, d, f, short == "w2"),
                           mat(1, 2 * f, d, short == "s13"), mat(1, d, f, short == "s2"))

    x = torch.zeros((T, d), dtype=torch.int16)
    logits = torch.zeros((T, E), dtype=torch.float32)
    y = torch.zeros((T, d), dtype=torch.float32)
    ws = torch.zeros(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8)
    for short in ("w13", "w2", "s13", "s2"):
        with pytest.raises(M.MoeError, match=f"{short}.codes holds"):
            M.moe_layer_forward(dm, x, logits, weights(short), y=y, ws=ws)
    with pytest.raises(M.MoeError, match="y holds"):
        M.moe_layer_forward(dm, x, logits, weights(), y=torch.zeros((T, d - 1)), ws=ws)
    with pytest.raises(M.MoeError, match="GPU memory"):
        M.moe_layer_forward(dm, x, logits, weights(), y=y, ws=ws)
    # the combine: o_routed one row short
    with pytest.raises(M.MoeError, match="o_routed holds"):
        M.moe_unpermute_combine(dm, torch.zeros((T * k - 1, d), dtype=torch.int16),
                                torch.zeros((T, d)), torch.zeros((T, k)),
                                torch.zeros(T * k, dtype=torch.int32), y=y)
    # dequant: matrix index past the stack
    m = weights().w13
    with pytest.raises(M.MoeError, match="outside"):
        M.moe_dequant_w4(M.W4Matrix(m.codes.view(E, 2 * f, d // 2), m.scales.view(E, 2 * f, d // 64),
                                    m.biases.view(E, 2 * f, d // 64)), index=E)


def test_binding_checks_element_types(L):
    """Each tensor is read as one fixed element type; a tensor of another type (an
    fp32 x would have its bits read as bf16) is refused before any device access."""
    import torch

    T, d, f, E, k = 4, 128, 64, 8, 2
    dm = M.dims(T, d, f, E, k)
    with pytest.raises(M.MoeError, match="logits has dtype"):
        M.moe_route(torch.zeros((T, E), dtype=torch.float64), k)
    with pytest.raises(M.MoeError, match="topk_ids has dtype"):
        M.moe_route(torch.zeros((T, E)), k, topk_ids=torch.zeros((T, k), dtype=torch.int64),
                    topk_w=torch.zeros((T, k)))
    with pytest.raises(M.MoeError, match="x has dtype"):
        M.moe_router_logits(torch.zeros((T, d), dtype=torch.float32),
                            torch.zeros((E, d), dtype=torch.bfloat16))
    with pytest.raises(M.MoeError, match="x has dtype"):
        M.moe_router_logits(torch.zeros((T, d), dtype=torch.float16),
                            torch.zeros((E, d), dtype=torch.bfloat16))
    # the router matrix must have x's width and E full rows
    with pytest.raises(M.MoeError, match="columns"):
        M.moe_router_logits(torch.zeros((T, d), dtype=torch.bfloat16),
                            torch.zeros((E, d - 64), dtype=torch.bfloat16))
    with pytest.raises(M.MoeError, match="GPU memory"):
        M.moe_router_logits(torch.zeros((T, d), dtype=torch.bfloat16),
                            torch.zeros((E, d), dtype=torch.bfloat16))
    # dequant: scales and biases sized and typed
    codes = torch.zeros((1, 2 * f, d // 2), dtype=torch.uint8)
    sc = torch.zeros((1, 2 * f, d // 64), dtype=torch.int16)
    with pytest.raises(M.MoeError, match="scales holds"):
        M.moe_dequant_w4(M.W4Matrix(codes, sc[:, :f], sc))
    with pytest.raises(M.MoeError, match="biases has dtype"):
        M.moe_dequant_w4(M.W4Matrix(codes, sc, sc.float()))
    # the layer: an fp32 x
    ws = torch.zeros(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8)
    with pytest.raises(M.MoeError, match="x has dtype"):
        M.moe_layer_forward(dm, torch.zeros((T, d)), torch.zeros((T, E)), None,
                            y=torch.zeros((T, d)), ws=ws)


def test_noalloc_validation(L):
    """The no-allocation layer call validates like moe_layer_forward and refuses, before
    any HIP call, a layer whose scratch exceeds the library's static array."""
    w = _weights()
    fn = L.moe_layer_forward_noalloc
    assert fn(ctypes.byref(_dims(T=0)), None, None, ctypes.byref(w), None, None) == OK
    assert fn(ctypes.byref(_dims(d=100)), FAKE, FAKE, ctypes.byref(w), FAKE, None) == UNSUPPORTED
    assert fn(ctypes.byref(_dims()), None, FAKE, ctypes.byref(w), FAKE, None) == INVALID
    assert fn(ctypes.byref(_dims()), FAKE, FAKE, ctypes.byref(w), FAKE + 4, None) == ALIGN
    limit = 64 << 20
    big = _dims(T=1308, d=2048, f=512, E=256, k=8)
    assert L.moe_layer_workspace_bytes(ctypes.byref(big)) > limit
    assert fn(ctypes.byref(big), FAKE, FAKE, ctypes.byref(w), FAKE, None) == WORKSPACE
    fits = _dims(T=1307, d=2048, f=512, E=256, k=8)
    assert L.moe_layer_workspace_bytes(ctypes.byref(fits)) <= limit
    header = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)" in header

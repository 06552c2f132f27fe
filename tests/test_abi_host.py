"""Host-side checks of the C ABI (no GPU needed, no kernel launched): the
library loads, exports every symbol include/tmx.h declares, the ctypes
struct matches the C layout, and validation fails before any launch."""
import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import datagen as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tmx.h")


@pytest.fixture(scope="module")
def tmx():
    from token_moe_amd import tmx as t
    if not os.path.exists(t.LIB_PATH):
        from token_moe_amd.build import build
        build()
    t.load_library()
    return t


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tmx_[a-z_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("tmx_create", "tmx_load_weights", "tmx_block_stack_forward", "tmx_moe_route",
              "tmx_destroy", "tmx_last_error", "tmx_sublayer_forward", "tmx_debug_permute"):
        assert n in names


def test_library_exports_every_declared_symbol(tmx):
    lib = tmx.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(tmx.EXPORTED)


def test_config_struct_layout_matches_c(tmx):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    fields = [f for f, _ in tmx.tmx_config._fields_]
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"tmx.h\"\nint main(void){\n"
    prog += 'printf("%zu\\n", sizeof(tmx_config));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof(tmx_config, {f}));\n'
    prog += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(prog)
        exe = os.path.join(d, "t")
        subprocess.run([gcc, "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = [int(v) for v in subprocess.run([exe], check=True, capture_output=True,
                                              text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(tmx.tmx_config)
    for f, off in zip(fields, out[1:]):
        assert getattr(tmx.tmx_config, f).offset == off, f


def test_status_and_enum_values_match_header(tmx):
    src = open(HEADER).read()
    for name, val in [("TMX_OK", 0), ("TMX_ERR_INVALID_ARG", 1), ("TMX_ERR_UNSUPPORTED", 2),
                      ("TMX_ERR_OOM", 3), ("TMX_ERR_DEVICE", 4), ("TMX_ERR_STATE", 5),
                      ("TMX_W_NORM_GAIN", dg.K_NORM_GAIN), ("TMX_W_UP", dg.K_UP),
                      ("TMX_W_GATE", dg.K_GATE), ("TMX_W_DOWN", dg.K_DOWN),
                      ("TMX_W_ROUTER", dg.K_ROUTER), ("TMX_W_EXP_UP", dg.K_EXP_UP),
                      ("TMX_W_EXP_GATE", dg.K_EXP_GATE), ("TMX_W_EXP_DOWN", dg.K_EXP_DOWN),
                      ("TMX_W_SH_UP", dg.K_SH_UP), ("TMX_W_SH_GATE", dg.K_SH_GATE),
                      ("TMX_W_SH_DOWN", dg.K_SH_DOWN), ("TMX_MIX", 0), ("TMX_REVERT", 1),
                      ("TMX_F32", 0), ("TMX_BF16", 1), ("TMX_MXFP8", 2),
                      ("TMX_W_NORM_BIAS", dg.K_NORM_BIAS), ("TMX_W_BIAS_UP", dg.K_BIAS_UP),
                      ("TMX_W_BIAS_DOWN", dg.K_BIAS_DOWN), ("TMX_BLOCK_TOKENMIXER_LARGE", 0),
                      ("TMX_BLOCK_RANKMIXER", tmx.TMX_BLOCK_RANKMIXER),
                      ("TMX_W_EXP_BIAS_UP", dg.K_EXP_BIAS_UP), ("TMX_W_EXP_BIAS_DOWN", dg.K_EXP_BIAS_DOWN),
                      ("TMX_W_TOK_UP", dg.K_TOK_UP), ("TMX_W_TOK_DOWN", dg.K_TOK_DOWN),
                      ("TMX_W_HEAD_UP", dg.K_HEAD_UP), ("TMX_W_HEAD_DOWN", dg.K_HEAD_DOWN)]:
        m = re.search(rf"\b{name}\s*=\s*(\d+)", src)
        assert m and int(m.group(1)) == val, name


def _create(tmx, **kw):
    base = dict(B_max=16, T=4, H=4, D=32, L=1, hidden_mix=64, hidden_rev=64, dtype=tmx.TMX_F32)
    base.update(kw)
    cfg = tmx.make_config(**base)
    h = ctypes.c_void_p()
    lib = tmx.load_library()
    st = lib.tmx_create(ctypes.byref(cfg), 0, ctypes.byref(h))
    return st, h, lib.tmx_last_error(None).decode()


@pytest.mark.parametrize("kw,status", [
    (dict(D=30, H=4), "INVALID_ARG"),            # D % H
    (dict(T=0), "INVALID_ARG"),
    (dict(L=0), "INVALID_ARG"),
    (dict(B_max=0), "INVALID_ARG"),
    (dict(eps=0.0), "INVALID_ARG"),
    (dict(eps=-1.0), "INVALID_ARG"),
    (dict(inter_residual_gap=-1), "INVALID_ARG"),
    (dict(hidden_mix=0), "INVALID_ARG"),
    (dict(dtype=7), "INVALID_ARG"),
    (dict(E=4, top_k=5, expert_hidden=8, shared_hidden=8), "INVALID_ARG"),   # k > E
    (dict(E=4, top_k=0, expert_hidden=8, shared_hidden=8), "INVALID_ARG"),
    (dict(E=4, top_k=2, expert_hidden=0, shared_hidden=8), "INVALID_ARG"),
    (dict(E=4, top_k=2, expert_hidden=8, shared_hidden=8, alpha=-1.0), "INVALID_ARG"),
    (dict(E=-1), "INVALID_ARG"),
    # bf16 fast path shape limits
    (dict(dtype=1, D=32, H=8, T=16, hidden_mix=64, hidden_rev=64), "UNSUPPORTED"),     # dh = 4
    (dict(dtype=1, D=96, H=4, T=4, hidden_mix=64, hidden_rev=64), "UNSUPPORTED"),      # W = 96
    (dict(dtype=1, D=128, H=4, T=4, hidden_mix=100, hidden_rev=64), "UNSUPPORTED"),    # hidden % 128
    (dict(dtype=1, D=128, H=4, T=4, E=8, top_k=2, expert_hidden=64, shared_hidden=64), "UNSUPPORTED"),
    # MXFP8: dense sub-layers at W = 256 or 512, MoE at W = 512, hidden <= 1024
    (dict(dtype=2, D=768, H=16, T=16, hidden_mix=256, hidden_rev=256), "UNSUPPORTED"),
    (dict(dtype=2, D=128, H=4, T=4, hidden_mix=256, hidden_rev=256), "UNSUPPORTED"),
    (dict(dtype=2, D=256, H=16, T=16, hidden_mix=2048, hidden_rev=256), "UNSUPPORTED"),
    (dict(dtype=2, D=256, H=16, T=16, E=16, top_k=4, expert_hidden=256, shared_hidden=512), "UNSUPPORTED"),
    (dict(dtype=2, D=512, H=16, T=16, E=16, top_k=4, expert_hidden=256, shared_hidden=2048), "UNSUPPORTED"),
    (dict(dtype=2, D=512, H=16, T=16, E=12, top_k=4, expert_hidden=256, shared_hidden=512), "UNSUPPORTED"),
    (dict(dtype=2, D=512, H=16, T=16, E=16, top_k=10, expert_hidden=256, shared_hidden=512), "UNSUPPORTED"),
    (dict(dtype=2, D=768, H=32, T=32, E=32, top_k=4, expert_hidden=384, shared_hidden=1024), "UNSUPPORTED"),
    (dict(dtype=3), "INVALID_ARG"),
    # MXFP8 capability checks come after every shape check: H = 0 or D % H != 0
    # must be INVALID_ARG, never a division by zero in the MXFP8 width check
    (dict(dtype=2, D=256, H=0, T=16, hidden_mix=256, hidden_rev=256), "INVALID_ARG"),
    (dict(dtype=2, D=256, H=7, T=16, hidden_mix=256, hidden_rev=256), "INVALID_ARG"),
    (dict(dtype=2, D=256, H=16, T=0, hidden_mix=256, hidden_rev=256), "INVALID_ARG"),
    (dict(dtype=2, D=256, H=16, T=16, hidden_mix=0, hidden_rev=256), "INVALID_ARG"),
    (dict(block=2), "INVALID_ARG"),
    # RankMixer: H == T, no mix hidden, no inter-residual; bf16 dense, D 256 / 512
    (dict(block=1, dtype=1, D=256, H=8, T=16, hidden_mix=0, hidden_rev=1024, inter_residual_gap=0), "INVALID_ARG"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=1024, hidden_rev=1024, inter_residual_gap=0),
     "INVALID_ARG"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=1024, inter_residual_gap=2), "INVALID_ARG"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=0, inter_residual_gap=0), "INVALID_ARG"),
    (dict(block=1, dtype=0, D=256, H=16, T=16, hidden_mix=0, hidden_rev=1024, inter_residual_gap=0), "UNSUPPORTED"),
    (dict(block=1, dtype=1, D=128, H=16, T=16, hidden_mix=0, hidden_rev=1024, inter_residual_gap=0), "UNSUPPORTED"),
    (dict(block=1, dtype=1, D=256, H=64, T=64, hidden_mix=0, hidden_rev=1024, inter_residual_gap=0), "UNSUPPORTED"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=1000, inter_residual_gap=0), "UNSUPPORTED"),
    (dict(block=1, dtype=1, D=512, H=16, T=16, hidden_mix=0, hidden_rev=384, inter_residual_gap=0), "UNSUPPORTED"),
    # RankMixer ReLU-routed experts: hidden_rev 0, top_k 0 (variable count); D 256, E 16 / 32, h_e % 128
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=1024, inter_residual_gap=0, E=16, top_k=0,
          expert_hidden=128), "INVALID_ARG"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=0, inter_residual_gap=0, E=16, top_k=4,
          expert_hidden=128), "INVALID_ARG"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=0, inter_residual_gap=0, E=16, top_k=0,
          expert_hidden=0), "INVALID_ARG"),
    (dict(block=1, dtype=1, D=512, H=16, T=16, hidden_mix=0, hidden_rev=0, inter_residual_gap=0, E=16, top_k=0,
          expert_hidden=128), "UNSUPPORTED"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=0, inter_residual_gap=0, E=8, top_k=0,
          expert_hidden=128), "UNSUPPORTED"),
    (dict(block=1, dtype=1, D=256, H=16, T=16, hidden_mix=0, hidden_rev=0, inter_residual_gap=0, E=16, top_k=0,
          expert_hidden=96), "UNSUPPORTED"),
    # x_hat workspace (B_max*T*D bf16) must stay under 4 GiB
    (dict(dtype=1, B_max=1 << 21, D=512, H=16, T=16, E=16, top_k=4, expert_hidden=256, shared_hidden=512),
     "UNSUPPORTED"),
])
def test_create_validation(tmx, kw, status):
    st, h, msg = _create(tmx, **kw)
    assert tmx.STATUS_NAMES[st] == status, msg
    assert h.value is None
    assert msg


@pytest.mark.parametrize("kw", [
    dict(),
    # MXFP8 shapes that pass validation: dense W 512 / 256 (uneven mixing),
    # MoE at W 512 and at W 768 (hidden 768 = the most W 768 allows)
    dict(dtype=2, T=16, H=8, D=256, hidden_mix=1024, hidden_rev=1024),
    dict(dtype=2, T=16, H=16, D=512, E=16, top_k=4, expert_hidden=256, shared_hidden=1024),
    dict(dtype=2, T=32, H=32, D=768, E=32, top_k=4, expert_hidden=384, shared_hidden=768),
])
def test_create_without_device_reports_device_error(tmx, kw):
    """Valid configurations get past validation and fail only for want of a
    device."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h, msg = _create(tmx, **kw)
    assert st == tmx.TMX_ERR_DEVICE and h.value is None and msg


def test_null_context_calls(tmx):
    lib = tmx.load_library()
    assert lib.tmx_destroy(None) == tmx.TMX_OK
    assert lib.tmx_block_stack_forward(None, None, None, 1, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_load_weights(None, 0, 0, 1, None, 0, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_moe_route(None, 0, 0, None, 1, None, None, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_sublayer_forward(None, 0, 0, None, None, None, None, 1, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_debug_permute(None, None, None, 1, 0, 0, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_relu_route(None, 0, None, 1, None, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_moe_buckets(None, 0, 0, None, 1, None, None, None, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_set_kernel_timing(None, 1) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_kernel_times(None, None, None, 0) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_set_model_io(None, None, 0, 128, 128) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_load_io_weights(None, 16, None, 0, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_tokenize(None, None, None, 1, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_head(None, None, None, 1, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_model_forward(None, None, None, 1, None) == tmx.TMX_ERR_INVALID_ARG
    assert lib.tmx_last_error(None)


def test_python_errors_carry_status(tmx):
    with pytest.raises(tmx.TmxError) as e:
        tmx.Context(tmx.make_config(B_max=1, T=4, H=3, D=32, L=1, hidden_mix=8, hidden_rev=8))
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG


def test_bulk_bf16_quantisation_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    a = np.concatenate([a, np.float32(1.0) + np.arange(2000, dtype=np.float32) * np.float32(2 ** -8)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(dg.f32_to_bf16_bits(a), want)
    np.testing.assert_array_equal(dg.bf16_bits_to_f32(want), dg.to_bf16_values(a))


def test_bank_generation_is_worker_independent():
    cfg = dg.WORKLOADS[4].with_(L=1, B=8)
    a = dg.weight_banks(cfg, workers=1)
    b = dg.weight_banks(cfg, workers=8)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    ws = dg.WeightSource(cfg, a)
    np.testing.assert_array_equal(ws(1, 1, dg.K_EXP_UP, 3), dg.weight_slice(cfg, 1, 1, dg.K_EXP_UP, 3))


def test_rankmixer_bank_generation_is_worker_independent():
    """RankMixer banks (dense FFN and ReLU-routed experts, with drawn norm
    parameters): the same values for any worker count, and each slice equal
    to its direct draw."""
    for wl in (dg.RANKMIXER_WORKLOADS["rankmixer_d256"], dg.RANKMIXER_WORKLOADS["rankmixer_moe_d256"]):
        cfg = wl.with_(L=1, B=8, T=4, H=4, random_norm=True)
        a = dg.weight_banks(cfg, workers=1)
        b = dg.weight_banks(cfg, workers=8)
        assert a.keys() == b.keys()
        for k in a:
            np.testing.assert_array_equal(a[k], b[k])
        kinds = {k[2] for k in a}
        assert dg.K_NORM_BIAS in kinds and (dg.K_EXP_BIAS_DOWN in kinds) == cfg.moe
        ws = dg.WeightSource(cfg, a)
        kind = dg.K_EXP_UP if cfg.moe else dg.K_UP
        np.testing.assert_array_equal(ws(1, 1, kind, 2), dg.weight_slice(cfg, 1, 1, kind, 2))

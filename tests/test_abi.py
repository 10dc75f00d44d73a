"""Host-side checks of the C ABI (no GPU work is launched).

The library is loaded and every function declared in include/h3dit.h must be
exported. Argument validation runs on the host before any HIP call, so each
error path is exercised here with placeholder (never dereferenced) pointers.
"""
import ctypes
import os
import re

import pytest

from joint_attention_dit_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3dit.h")

# placeholder device addresses: aligned, disjoint, never touched
P = {name: 0x100000000 * (i + 1) for i, name in enumerate(
    ["x", "cond", "pos", "out", "ws", "w_ada", "w_qkv", "w_o", "w_up", "w_down", "mod", "h"])}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3dit_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in h3dit.h but not exported"
    assert set(names) == set(B.EXPORTED)


def test_config_struct_layout():
    assert ctypes.sizeof(B.Config) == 32
    assert ctypes.sizeof(B.Weights) == 40


def full_cfg(**kw):
    c = B.make_config(5376, 56, 14336, 16896)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_size_plan():
    n = B.h3dit_workspace_size(full_cfg())
    T, D, A, F = 16896, 5376, 7168, 14336
    Tp = B.h3dit_padded_tokens(T)
    assert Tp == 16896 and B.h3dit_padded_tokens(288) == 320 and B.h3dit_padded_tokens(1) == 64
    lower = 6 * D * 8 + 128 * T * 4 + 2 * T * D + 4 * T * A + 2 * A * Tp + 2 * T * A + 4 * T * D + 2 * T * F
    # plus the scratch for K slices of a GEMM's last wave (the largest of the four):
    # at 16896 tokens the QKV GEMM has 84 x 66 = 5544 tiles, 168 of them in the
    # last wave of 256 CUs, each cut into three 256 x 256 fp32 slices (two waves
    # of thirds instead of one whole wave); MLP up has 112 left, cut in two
    split = max(168 * 3, 112 * 2) * 256 * 256 * 4
    # plus the attention's key-range pieces: 56 heads x 66 query tiles = 3696
    # workgroups, 112 of them past the last whole round of 256 CUs, each cut in
    # two pieces of (256 x 128 outputs + 256 sums + 256 shifts) fp32
    att = 112 * 2 * 256 * 130 * 4
    assert lower + split + att <= n <= lower + split + att + 10 * 256
    assert B.h3dit_workspace_size(B.make_config(256, 2, 1024, 1)) > 0


def _forward(lib, cfg, ws_bytes=1 << 40, **override):
    p = dict(P)
    p.update(override)
    w = B.Weights(p["w_ada"], p["w_qkv"], p["w_o"], p["w_up"], p["w_down"])
    return lib.h3dit_block_forward(ctypes.byref(cfg), p["x"], p["cond"], ctypes.byref(w), p["pos"],
                                   p["out"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, B.H3DIT_EUNSUPPORTED),
    ("hidden", 5377, B.H3DIT_EUNSUPPORTED),
    ("hidden", 0, B.H3DIT_EUNSUPPORTED),
    ("ffn", 100, B.H3DIT_EUNSUPPORTED),
    ("heads", 0, B.H3DIT_EINVAL),
    ("n_tokens", 0, B.H3DIT_EINVAL),
    ("n_tokens", (1 << 20) + 1, B.H3DIT_EINVAL),
    ("x_dtype", 7, B.H3DIT_EINVAL),
    ("eps", -1.0, B.H3DIT_EINVAL),
    ("rope_base", 0.0, B.H3DIT_EINVAL),
])
def test_config_validation(lib, field, value, status):
    assert _forward(lib, full_cfg(**{field: value})) == status
    assert lib.h3dit_last_error().decode() != ""


def test_null_misaligned_workspace_overlap(lib):
    cfg = full_cfg()
    assert _forward(lib, cfg, x=None) == B.H3DIT_EINVAL
    assert "x is NULL" in lib.h3dit_last_error().decode()
    assert _forward(lib, cfg, w_down=0) == B.H3DIT_EINVAL
    assert _forward(lib, cfg, cond=P["cond"] + 4) == B.H3DIT_EALIGN
    assert _forward(lib, cfg, ws_bytes=1000) == B.H3DIT_EWORKSPACE
    assert _forward(lib, cfg, out=P["x"]) == B.H3DIT_EINVAL
    assert "overlaps" in lib.h3dit_last_error().decode()
    assert lib.h3dit_block_forward(None, P["x"], P["cond"], None, P["pos"], P["out"], P["ws"],
                                   1 << 40, None) == B.H3DIT_EINVAL


def test_timed_variant_validates_events(lib):
    cfg = full_cfg()
    w = B.Weights(P["w_ada"], P["w_qkv"], P["w_o"], P["w_up"], P["w_down"])
    ev = (ctypes.c_void_p * 10)(*([0x1000] * 10))
    assert lib.h3dit_block_forward_timed(ctypes.byref(cfg), P["x"], P["cond"], ctypes.byref(w),
                                         P["pos"], P["out"], P["ws"], 1 << 40, None, ev,
                                         9) == B.H3DIT_EINVAL
    ev[3] = None
    assert lib.h3dit_block_forward_timed(ctypes.byref(cfg), P["x"], P["cond"], ctypes.byref(w),
                                         P["pos"], P["out"], P["ws"], 1 << 40, None, ev,
                                         10) == B.H3DIT_EINVAL


def test_stage_validation(lib):
    cfg = full_cfg()
    assert lib.h3dit_modulation(ctypes.byref(cfg), None, P["cond"], P["mod"], None) == B.H3DIT_EINVAL
    assert lib.h3dit_rmsnorm_modulate(ctypes.byref(cfg), P["x"], 5, P["mod"], P["mod"], P["h"],
                                      None) == B.H3DIT_EINVAL
    assert lib.h3dit_attention(ctypes.byref(full_cfg(head_dim=96)), P["x"], P["x"], P["h"],
                               None) == B.H3DIT_EUNSUPPORTED
    assert lib.h3dit_out_proj_residual(ctypes.byref(cfg), P["x"], P["w_o"], P["x"], 3, P["mod"],
                                       P["out"], None) == B.H3DIT_EINVAL
    # the MXFP8 attention entry: null codes / scales, unsupported head size,
    # misaligned codes (all rejected on the host, before any HIP call)
    assert lib.h3dit_attention_mxfp8(ctypes.byref(cfg), P["x"], P["x"], P["h"], None, P["mod"],
                                     None) == B.H3DIT_EINVAL
    assert lib.h3dit_attention_mxfp8(ctypes.byref(cfg), P["x"], P["x"], P["h"], P["out"], None,
                                     None) == B.H3DIT_EINVAL
    assert lib.h3dit_attention_mxfp8(ctypes.byref(full_cfg(head_dim=96)), P["x"], P["x"], P["h"],
                                     P["out"], P["mod"], None) == B.H3DIT_EUNSUPPORTED
    assert lib.h3dit_attention_mxfp8(ctypes.byref(cfg), P["x"], P["x"], P["h"], P["out"] + 4,
                                     P["mod"], None) == B.H3DIT_EALIGN


def test_fault_injection_reports_hip_error(lib, monkeypatch):
    monkeypatch.setenv("H3DIT_FAULT_INJECT", "launch")
    assert _forward(lib, full_cfg()) == B.H3DIT_EHIP
    assert "injected" in lib.h3dit_last_error().decode()
    with pytest.raises(B.H3ditError):
        B._check(B.H3DIT_EHIP, "h3dit_block_forward")


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.h3dit_status_string(s).startswith(b"H3DIT_")
    assert b"unknown" in lib.h3dit_status_string(42)


# ---------------------------------------------------------------- DiT stack
def stack_cfg(n_blocks=2, text=256, grid=64):
    return B.StackConfig(n_blocks, 24, 2, grid, grid, text)


def test_stack_struct_layout_and_workspace():
    assert ctypes.sizeof(B.StackConfig) == 24
    assert ctypes.sizeof(B.StackWeights) == 32
    cfg = B.make_config(5376, 56, 14336, 4352, B.H3DIT_F32)
    n = B.h3dit_stack_workspace_size(cfg, stack_cfg())
    T, D, Ti, F = 4352, 5376, 4096, 96
    extra = 2 * 4 * T * D + 4 * Ti * F + 16 * D + 4 * Ti * D + 4 * Ti * F
    blk = B.h3dit_workspace_size(cfg)
    assert blk + extra <= n <= blk + extra + 8 * 256


def test_stack_shape_validation():
    cfg = B.make_config(256, 2, 1024, 24)
    with pytest.raises(B.H3ditError) as ei:     # 8 text + 5 x 4 image tokens != 24
        B.h3dit_stack_workspace_size(cfg, B.StackConfig(1, 4, 2, 5, 4, 8))
    assert ei.value.status == B.H3DIT_EINVAL
    with pytest.raises(B.H3ditError) as ei:     # 3 features per patch (not a multiple of 4)
        B.h3dit_stack_workspace_size(cfg, B.StackConfig(1, 3, 1, 4, 4, 8))
    assert ei.value.status == B.H3DIT_EUNSUPPORTED
    with pytest.raises(B.H3ditError) as ei:
        B.h3dit_stack_workspace_size(cfg, B.StackConfig(-1, 4, 2, 4, 4, 8))
    assert ei.value.status == B.H3DIT_EINVAL


def _dit(lib, cfg, st, ws_bytes=1 << 40, blocks=2, **override):
    p = {k: 0x100000000 * (i + 1) for i, k in enumerate(
        ["latent", "text", "cond", "pos", "v", "ws", "wp", "wa", "wf"])}
    p.update(override)
    arr = (B.Weights * blocks)(*[B.Weights(*[0x20000000000 + 0x1000000000 * (5 * b + j)
                                             for j in range(5)]) for b in range(blocks)])
    sw = B.StackWeights(p["wp"], p["wa"], p["wf"], ctypes.cast(arr, ctypes.POINTER(B.Weights)))
    return lib.h3dit_dit_forward(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), p["latent"],
                                 p["text"], p["cond"], p["pos"], p["v"], p["ws"], ws_bytes, None)


def test_dit_forward_validation(lib):
    cfg = B.make_config(5376, 56, 14336, 4352, B.H3DIT_F32)
    st = stack_cfg()
    assert _dit(lib, cfg, st, latent=None) == B.H3DIT_EINVAL
    assert _dit(lib, cfg, st, wf=0x100000004) == B.H3DIT_EALIGN
    assert _dit(lib, cfg, st, ws_bytes=4096) == B.H3DIT_EWORKSPACE
    assert _dit(lib, cfg, st, v=0x100000000 * 6 + 64) == B.H3DIT_EINVAL      # inside the workspace
    assert "overlaps" in lib.h3dit_last_error().decode()
    bad = B.StackWeights(0x100000000 * 7, 0x100000000 * 8, 0x100000000 * 9, None)
    assert lib.h3dit_dit_forward(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(bad),
                                 0x100000000, 0x200000000, 0x300000000, 0x400000000, 0x500000000,
                                 0x600000000, 1 << 40, None) == B.H3DIT_EINVAL
    assert "blocks is NULL" in lib.h3dit_last_error().decode()


def test_latent_step_validation(lib):
    assert lib.h3dit_latent_step(None, 0x100000000, 0.5, 10, None) == B.H3DIT_EINVAL
    assert lib.h3dit_latent_step(0x100000000, 0x200000000, 0.5, 0, None) == B.H3DIT_EINVAL
    assert lib.h3dit_latent_step(0x100000000, 0x200000000, float("nan"), 4, None) == B.H3DIT_EINVAL


def test_modulation_table_validation(lib):
    cfg = B.make_config(256, 2, 1024, 24)
    a, c, m = 0x100000000, 0x200000000, 0x300000000
    assert lib.h3dit_modulation_table(ctypes.byref(cfg), a, c, 0, m, None) == B.H3DIT_EINVAL
    assert lib.h3dit_modulation_table(ctypes.byref(cfg), a, c, 4097, m, None) == B.H3DIT_EINVAL
    assert lib.h3dit_modulation_table(ctypes.byref(cfg), None, c, 6, m, None) == B.H3DIT_EINVAL
    assert lib.h3dit_modulation_table(ctypes.byref(cfg), a, c, 6, m + 8, None) == B.H3DIT_EALIGN


def test_dit_modulation_table_and_forward_mod_validation(lib):
    cfg = B.make_config(5376, 56, 14336, 4352, B.H3DIT_F32)
    st = stack_cfg()
    arr = (B.Weights * 2)(*[B.Weights(*[0x20000000000 + 0x1000000000 * (5 * b + j)
                                        for j in range(5)]) for b in range(2)])
    sw = B.StackWeights(0x100000000, 0x200000000, 0x300000000,
                        ctypes.cast(arr, ctypes.POINTER(B.Weights)))
    conds, table = 0x400000000, 0x500000000
    tab = lib.h3dit_dit_modulation_table
    assert tab(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), conds, 0, table, None) == B.H3DIT_EINVAL
    assert tab(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), None, 6, table, None) == B.H3DIT_EINVAL
    arr[1].w_ada = 0x20000000004  # misaligned block weight
    assert tab(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), conds, 6, table, None) == B.H3DIT_EALIGN
    arr[1].w_ada = None
    assert tab(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), conds, 6, table, None) == B.H3DIT_EINVAL
    assert "w_ada" in lib.h3dit_last_error().decode()
    # with a table the AdaLN weights are not needed, but the table is
    fwd = lib.h3dit_dit_forward_mod
    args = (0x600000000, 0x700000000)  # latent, text
    assert fwd(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), *args, None, 0x800000000,
               0x900000000, 0xa00000000, 1 << 40, None) == B.H3DIT_EINVAL
    assert "mods" in lib.h3dit_last_error().decode()
    assert fwd(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), *args, 0xb00000000,
               0x800000000, 0x900000000, 0xa00000000, 4096, None) == B.H3DIT_EWORKSPACE


# ------------------------------------------------------------------ MXFP8
def test_mxfp8_struct_and_scale_bytes():
    assert ctypes.sizeof(B.MxWeights) == 64
    assert B.h3dit_mxfp8_scale_bytes(300, 384) == 512 * 12
    assert B.h3dit_mxfp8_scale_bytes(256, 128) == 1024
    assert B.h3dit_mxfp8_scale_bytes(16896, 14336) == 16896 * 448
    for rows, K in ((0, 128), (10, 100), (10, 0), (-1, 256)):
        assert B.h3dit_mxfp8_scale_bytes(rows, K) == 0


def test_mxfp8_workspace_adds_quantised_operand():
    cfg = full_cfg()
    T, D, A, F = 16896, 5376, 7168, 14336
    bf = B.h3dit_workspace_size(cfg)
    mx = B.h3dit_workspace_size_mxfp8(cfg)
    # codes and scales of the widest linear input (u, [T, F]); the split scratch
    # follows the MXFP8 GEMM's 128-wide K tiles
    assert mx - bf >= T * F + T * F // 32 - 112 * 2 * 256 * 256 * 4


def test_mxfp8_quantize_and_linear_validation(lib):
    x, c, s = P["x"], P["h"], P["mod"]
    assert lib.h3dit_mxfp8_quantize(x, 10, 100, c, s, None) == B.H3DIT_EUNSUPPORTED
    assert lib.h3dit_mxfp8_quantize(x, 0, 128, c, s, None) == B.H3DIT_EUNSUPPORTED
    assert lib.h3dit_mxfp8_quantize(x, 10, 128, None, s, None) == B.H3DIT_EINVAL
    assert lib.h3dit_mxfp8_quantize(x, 10, 128, c, s + 8, None) == B.H3DIT_EALIGN
    y = P["out"]
    assert lib.h3dit_linear_mxfp8(x, s, c, s, 4, 8, 192, y, None) == B.H3DIT_EUNSUPPORTED
    assert lib.h3dit_linear_mxfp8(x, s, c, s, 4, 6, 128, y, None) == B.H3DIT_EUNSUPPORTED
    assert lib.h3dit_linear_mxfp8(x, None, c, s, 4, 8, 128, y, None) == B.H3DIT_EINVAL


def _forward_mx(lib, cfg, q=None, ws_bytes=1 << 40):
    w = B.Weights(P["w_ada"], 0, 0, 0, 0)  # the bf16 linear weights are not read
    if q is None:
        q = B.MxWeights(*[0x200000000 * (i + 20) for i in range(8)])
    return lib.h3dit_block_forward_mxfp8(ctypes.byref(cfg), P["x"], P["cond"], ctypes.byref(w),
                                         ctypes.byref(q) if q is not False else None, P["pos"],
                                         P["out"], P["ws"], ws_bytes, None)


def test_mxfp8_forward_validation(lib):
    with_fault = os.environ.get("H3DIT_FAULT_INJECT")
    assert with_fault is None
    assert _forward_mx(lib, full_cfg(), q=False) == B.H3DIT_EINVAL
    assert _forward_mx(lib, full_cfg(hidden=5312)) == B.H3DIT_EUNSUPPORTED  # 83 * 64
    assert "multiples of 128" in lib.h3dit_last_error().decode()
    assert _forward_mx(lib, full_cfg(ffn=14400)) == B.H3DIT_EUNSUPPORTED
    q = B.MxWeights(*[0x200000000 * (i + 20) for i in range(8)])
    q.w_down_scale = None
    assert _forward_mx(lib, full_cfg(), q=q) == B.H3DIT_EINVAL
    need = B.h3dit_workspace_size_mxfp8(full_cfg())
    assert _forward_mx(lib, full_cfg(), ws_bytes=need - 1) == B.H3DIT_EWORKSPACE


def _dit_mx(lib, cfg, st, q="ok", ws_bytes=1 << 40, blocks=2):
    p = {k: 0x100000000 * (i + 1) for i, k in enumerate(
        ["latent", "text", "cond", "pos", "v", "ws", "wp", "wa", "wf"])}
    arr = (B.Weights * blocks)(*[B.Weights(0x20000000000 + 0x1000000000 * b, 0, 0, 0, 0)
                                 for b in range(blocks)])
    sw = B.StackWeights(p["wp"], p["wa"], p["wf"], ctypes.cast(arr, ctypes.POINTER(B.Weights)))
    qarr = (B.MxWeights * blocks)(*[B.MxWeights(*[0x40000000000 + 0x1000000000 * (8 * b + j)
                                                  for j in range(8)]) for b in range(blocks)])
    if q == "null_scale":
        qarr[blocks - 1].w_up_scale = None
    qp = None if q is None else ctypes.cast(qarr, ctypes.POINTER(B.MxWeights))
    return lib.h3dit_dit_forward_mxfp8(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), qp,
                                       p["latent"], p["text"], p["cond"], p["pos"], p["v"],
                                       p["ws"], ws_bytes, None)


def test_dit_forward_mxfp8_validation(lib):
    cfg = B.make_config(5376, 56, 14336, 4352, B.H3DIT_F32)
    st = stack_cfg()
    assert _dit_mx(lib, cfg, st, q=None) == B.H3DIT_EINVAL
    assert "q is NULL" in lib.h3dit_last_error().decode()
    assert _dit_mx(lib, cfg, st, q="null_scale") == B.H3DIT_EINVAL
    assert "block 1" in lib.h3dit_last_error().decode()
    assert _dit_mx(lib, B.make_config(5312, 56, 14336, 4352, B.H3DIT_F32), st) == \
        B.H3DIT_EUNSUPPORTED
    need = B.h3dit_stack_workspace_size_mxfp8(cfg, st)
    assert need > B.h3dit_stack_workspace_size(cfg, st)
    assert _dit_mx(lib, cfg, st, ws_bytes=need - 1) == B.H3DIT_EWORKSPACE

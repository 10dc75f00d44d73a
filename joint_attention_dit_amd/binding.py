"""Thin ctypes binding of libh3dit.so (include/h3dit.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a negative status becomes an exception.
Every step of the block runs in the library's HIP kernels; there is no
fallback. Importing this module on a machine without the built library
raises at once.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh3dit.so")

H3DIT_OK, H3DIT_EINVAL, H3DIT_EUNSUPPORTED, H3DIT_EWORKSPACE, H3DIT_EALIGN, H3DIT_EHIP = \
    0, -1, -2, -3, -4, -5
H3DIT_BF16, H3DIT_F32 = 0, 1

EXPORTED = (
    "h3dit_workspace_size", "h3dit_block_forward", "h3dit_block_forward_timed",
    "h3dit_modulation", "h3dit_rmsnorm_modulate", "h3dit_rope_table", "h3dit_qkv_rope",
    "h3dit_attention", "h3dit_out_proj_residual", "h3dit_mlp_up_gelu",
    "h3dit_mlp_down_residual", "h3dit_linear_f32", "h3dit_stack_workspace_size",
    "h3dit_dit_forward", "h3dit_latent_step", "h3dit_padded_tokens", "h3dit_status_string",
    "h3dit_last_error", "h3dit_modulation_table", "h3dit_dit_modulation_table",
    "h3dit_dit_forward_mod", "h3dit_mxfp8_scale_bytes", "h3dit_mxfp8_quantize",
    "h3dit_linear_mxfp8", "h3dit_workspace_size_mxfp8", "h3dit_block_forward_mxfp8",
    "h3dit_block_forward_mxfp8_timed", "h3dit_workspace_layout", "h3dit_stack_workspace_size_mxfp8",
    "h3dit_dit_forward_mxfp8", "h3dit_dit_forward_mod_mxfp8", "h3dit_attention_mxfp8",
    "h3dit_block_forward_noalloc",
)
NOALLOC_SCRATCH_BYTES = 256 << 20   # H3DIT_NOALLOC_SCRATCH_BYTES


class H3ditError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} failed: {detail or 'no detail'} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_tokens", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [("w_ada", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


class MxWeights(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("w_qkv_scale", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("w_o_scale", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_up_scale", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("w_down_scale", ctypes.c_void_p)]


class WorkspaceMap(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("mod", "table", "h", "qk", "vt", "o", "x1", "u",
                                                "q_h2", "q_h2_scale", "q_u", "q_u_scale")]


class StackConfig(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("patch", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("text_tokens", ctypes.c_int32)]


class StackWeights(ctypes.Structure):
    _fields_ = [("w_patch", ctypes.c_void_p), ("w_ada_final", ctypes.c_void_p),
                ("w_final", ctypes.c_void_p), ("blocks", ctypes.POINTER(Weights))]


_lib: Optional[ctypes.CDLL] = None


def load_library() -> ctypes.CDLL:
    """Load libh3dit.so from the package directory (fails loudly if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m joint_attention_dit_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(Config)
    sigs = {
        "h3dit_workspace_size": [cfgp, ctypes.POINTER(sz)],
        "h3dit_block_forward": [cfgp, vp, vp, ctypes.POINTER(Weights), vp, vp, vp, sz, vp],
        "h3dit_block_forward_noalloc": [cfgp, vp, vp, ctypes.POINTER(Weights), vp, vp, vp],
        "h3dit_block_forward_timed": [cfgp, vp, vp, ctypes.POINTER(Weights), vp, vp, vp, sz, vp,
                                      ctypes.POINTER(vp), ctypes.c_int],
        "h3dit_modulation": [cfgp, vp, vp, vp, vp],
        "h3dit_rmsnorm_modulate": [cfgp, vp, i32, vp, vp, vp, vp],
        "h3dit_rope_table": [cfgp, vp, vp, vp],
        "h3dit_qkv_rope": [cfgp, vp, vp, vp, vp, vp, vp],
        "h3dit_attention": [cfgp, vp, vp, vp, vp],
        "h3dit_out_proj_residual": [cfgp, vp, vp, vp, i32, vp, vp, vp],
        "h3dit_mlp_up_gelu": [cfgp, vp, vp, vp, vp],
        "h3dit_mlp_down_residual": [cfgp, vp, vp, vp, vp, vp, vp],
        "h3dit_linear_f32": [vp, vp, i32, i32, i32, vp, vp],
        "h3dit_stack_workspace_size": [cfgp, ctypes.POINTER(StackConfig), ctypes.POINTER(sz)],
        "h3dit_dit_forward": [cfgp, ctypes.POINTER(StackConfig), ctypes.POINTER(StackWeights),
                              vp, vp, vp, vp, vp, vp, sz, vp],
        "h3dit_latent_step": [vp, vp, ctypes.c_float, ctypes.c_int64, vp],
        "h3dit_modulation_table": [cfgp, vp, vp, ctypes.c_int, vp, vp],
        "h3dit_dit_modulation_table": [cfgp, ctypes.POINTER(StackConfig),
                                       ctypes.POINTER(StackWeights), vp, ctypes.c_int, vp, vp],
        "h3dit_dit_forward_mod": [cfgp, ctypes.POINTER(StackConfig), ctypes.POINTER(StackWeights),
                                  vp, vp, vp, vp, vp, vp, sz, vp],
        "h3dit_mxfp8_quantize": [vp, ctypes.c_int64, ctypes.c_int64, vp, vp, vp],
        "h3dit_attention_mxfp8": [cfgp, vp, vp, vp, vp, vp, vp],
        "h3dit_linear_mxfp8": [vp, vp, vp, vp, i32, i32, i32, vp, vp],
        "h3dit_workspace_size_mxfp8": [cfgp, ctypes.POINTER(sz)],
        "h3dit_workspace_layout": [cfgp, i32, ctypes.POINTER(WorkspaceMap)],
        "h3dit_stack_workspace_size_mxfp8": [cfgp, ctypes.POINTER(StackConfig), ctypes.POINTER(sz)],
        "h3dit_dit_forward_mxfp8": [cfgp, ctypes.POINTER(StackConfig), ctypes.POINTER(StackWeights),
                                    ctypes.POINTER(MxWeights), vp, vp, vp, vp, vp, vp, sz, vp],
        "h3dit_dit_forward_mod_mxfp8": [cfgp, ctypes.POINTER(StackConfig),
                                        ctypes.POINTER(StackWeights), ctypes.POINTER(MxWeights),
                                        vp, vp, vp, vp, vp, vp, sz, vp],
        "h3dit_block_forward_mxfp8": [cfgp, vp, vp, ctypes.POINTER(Weights),
                                      ctypes.POINTER(MxWeights), vp, vp, vp, sz, vp],
        "h3dit_block_forward_mxfp8_timed": [cfgp, vp, vp, ctypes.POINTER(Weights),
                                            ctypes.POINTER(MxWeights), vp, vp, vp, sz, vp,
                                            ctypes.POINTER(vp), ctypes.c_int],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.h3dit_mxfp8_scale_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
    lib.h3dit_mxfp8_scale_bytes.restype = ctypes.c_size_t
    lib.h3dit_padded_tokens.argtypes = [ctypes.c_int64]
    lib.h3dit_padded_tokens.restype = ctypes.c_int64
    lib.h3dit_status_string.argtypes = [ctypes.c_int]
    lib.h3dit_status_string.restype = ctypes.c_char_p
    lib.h3dit_last_error.argtypes = []
    lib.h3dit_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, name: str) -> None:
    if status != H3DIT_OK:
        detail = load_library().h3dit_last_error().decode()
        raise H3ditError(status, name, detail)


def make_config(hidden: int, heads: int, ffn: int, n_tokens: int, x_dtype: int = H3DIT_BF16,
                eps: float = 1e-6, rope_base: float = 10000.0, head_dim: int = 128) -> Config:
    return Config(hidden, heads, head_dim, ffn, n_tokens, x_dtype, eps, rope_base)


def config_from(block_cfg) -> Config:
    """Config for a joint_attention_dit_amd.inputs.BlockConfig."""
    return make_config(block_cfg.hidden, block_cfg.heads, block_cfg.ffn, block_cfg.n_tokens,
                       H3DIT_F32 if block_cfg.x_dtype == "fp32" else H3DIT_BF16,
                       block_cfg.eps, block_cfg.rope_base, block_cfg.head_dim)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return H3DIT_BF16
    if t.dtype == torch.float32:
        return H3DIT_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ ABI calls
def h3dit_workspace_size(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().h3dit_workspace_size(ctypes.byref(cfg), ctypes.byref(n)),
           "h3dit_workspace_size")
    return n.value


def h3dit_padded_tokens(n_tokens: int) -> int:
    return int(load_library().h3dit_padded_tokens(n_tokens))


def weights_struct(w: Dict[str, torch.Tensor]) -> Weights:
    return Weights(_ptr(w["w_ada"]), _ptr(w["w_qkv"]), _ptr(w["w_o"]), _ptr(w["w_up"]),
                   _ptr(w["w_down"]))


def h3dit_block_forward(cfg: Config, x: torch.Tensor, cond: torch.Tensor,
                        w: Dict[str, torch.Tensor], positions: torch.Tensor, out: torch.Tensor,
                        workspace: torch.Tensor, stream=None) -> None:
    ws = weights_struct(w)
    _check(load_library().h3dit_block_forward(
        ctypes.byref(cfg), _ptr(x), _ptr(cond), ctypes.byref(ws), _ptr(positions), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
        "h3dit_block_forward")


def h3dit_block_forward_noalloc(cfg: Config, x: torch.Tensor, cond: torch.Tensor,
                                w: Dict[str, torch.Tensor], positions: torch.Tensor,
                                out: torch.Tensor, stream=None) -> None:
    ws = weights_struct(w)
    _check(load_library().h3dit_block_forward_noalloc(
        ctypes.byref(cfg), _ptr(x), _ptr(cond), ctypes.byref(ws), _ptr(positions), _ptr(out),
        _stream(stream)), "h3dit_block_forward_noalloc")


def h3dit_block_forward_timed(cfg: Config, x, cond, w, positions, out, workspace,
                              events: Sequence[int], stream=None) -> None:
    ws = weights_struct(w)
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(load_library().h3dit_block_forward_timed(
        ctypes.byref(cfg), _ptr(x), _ptr(cond), ctypes.byref(ws), _ptr(positions), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
        arr, len(events)), "h3dit_block_forward_timed")


def h3dit_modulation(cfg: Config, w_ada, cond, mod, stream=None) -> None:
    _check(load_library().h3dit_modulation(ctypes.byref(cfg), _ptr(w_ada), _ptr(cond), _ptr(mod),
                                           _stream(stream)), "h3dit_modulation")


def h3dit_modulation_table(cfg: Config, w_ada, conds, mods, stream=None) -> None:
    """conds [n, D] fp32 -> mods [n, 6D] fp64 (one pass over w_ada)."""
    _check(load_library().h3dit_modulation_table(ctypes.byref(cfg), _ptr(w_ada), _ptr(conds),
                                                 int(conds.shape[0]), _ptr(mods), _stream(stream)),
           "h3dit_modulation_table")


def h3dit_rmsnorm_modulate(cfg: Config, x, shift, scale, h, stream=None) -> None:
    _check(load_library().h3dit_rmsnorm_modulate(ctypes.byref(cfg), _ptr(x), _dtype_code(x),
                                                 _ptr(shift), _ptr(scale), _ptr(h),
                                                 _stream(stream)), "h3dit_rmsnorm_modulate")


def h3dit_rope_table(cfg: Config, positions, table, stream=None) -> None:
    _check(load_library().h3dit_rope_table(ctypes.byref(cfg), _ptr(positions), _ptr(table),
                                           _stream(stream)), "h3dit_rope_table")


def h3dit_qkv_rope(cfg: Config, h, w_qkv, table, qk, vt, stream=None) -> None:
    _check(load_library().h3dit_qkv_rope(ctypes.byref(cfg), _ptr(h), _ptr(w_qkv), _ptr(table),
                                         _ptr(qk), _ptr(vt), _stream(stream)), "h3dit_qkv_rope")


def h3dit_attention(cfg: Config, qk, vt, o, stream=None) -> None:
    _check(load_library().h3dit_attention(ctypes.byref(cfg), _ptr(qk), _ptr(vt), _ptr(o),
                                          _stream(stream)), "h3dit_attention")


def h3dit_attention_mxfp8(cfg: Config, qk, vt, o, o_codes, o_scales, stream=None) -> None:
    _check(load_library().h3dit_attention_mxfp8(ctypes.byref(cfg), _ptr(qk), _ptr(vt), _ptr(o),
                                                _ptr(o_codes), _ptr(o_scales), _stream(stream)),
           "h3dit_attention_mxfp8")


def h3dit_out_proj_residual(cfg: Config, o, w_o, resid, gate, x1, stream=None) -> None:
    _check(load_library().h3dit_out_proj_residual(ctypes.byref(cfg), _ptr(o), _ptr(w_o),
                                                  _ptr(resid), _dtype_code(resid), _ptr(gate),
                                                  _ptr(x1), _stream(stream)),
           "h3dit_out_proj_residual")


def h3dit_mlp_up_gelu(cfg: Config, h2, w_up, u, stream=None) -> None:
    _check(load_library().h3dit_mlp_up_gelu(ctypes.byref(cfg), _ptr(h2), _ptr(w_up), _ptr(u),
                                            _stream(stream)), "h3dit_mlp_up_gelu")


def h3dit_mlp_down_residual(cfg: Config, u, w_down, x1, gate, out, stream=None) -> None:
    _check(load_library().h3dit_mlp_down_residual(ctypes.byref(cfg), _ptr(u), _ptr(w_down),
                                                  _ptr(x1), _ptr(gate), _ptr(out),
                                                  _stream(stream)), "h3dit_mlp_down_residual")


def h3dit_linear_f32(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    M, K = x.shape
    N = w.shape[0]
    _check(load_library().h3dit_linear_f32(_ptr(x), _ptr(w), M, N, K, _ptr(y), _stream(stream)),
           "h3dit_linear_f32")


def h3dit_stack_workspace_size(cfg: Config, st: StackConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().h3dit_stack_workspace_size(ctypes.byref(cfg), ctypes.byref(st),
                                                     ctypes.byref(n)),
           "h3dit_stack_workspace_size")
    return n.value


def h3dit_dit_forward(cfg: Config, st: StackConfig, w_patch, w_ada_final, w_final,
                      blocks: Sequence[Dict[str, torch.Tensor]], latent, text, cond, positions,
                      v, workspace, stream=None) -> None:
    arr = (Weights * max(len(blocks), 1))(*[weights_struct(b) for b in blocks])
    sw = StackWeights(_ptr(w_patch), _ptr(w_ada_final), _ptr(w_final),
                      ctypes.cast(arr, ctypes.POINTER(Weights)))
    _check(load_library().h3dit_dit_forward(
        ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), _ptr(latent), _ptr(text),
        _ptr(cond), _ptr(positions), _ptr(v), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "h3dit_dit_forward")


def _stack_weights(w_patch, w_ada_final, w_final, blocks):
    arr = (Weights * max(len(blocks), 1))(*[weights_struct(b) for b in blocks])
    sw = StackWeights(_ptr(w_patch), _ptr(w_ada_final), _ptr(w_final),
                      ctypes.cast(arr, ctypes.POINTER(Weights)))
    return sw, arr  # the array must outlive the call


def h3dit_dit_modulation_table(cfg: Config, st: StackConfig, w_ada_final,
                               blocks: Sequence[Dict[str, torch.Tensor]], conds, table,
                               stream=None) -> None:
    """conds [S, D] fp32 -> table [S, n_blocks + 1, 6D] fp64."""
    sw, arr = _stack_weights(None, w_ada_final, None, blocks)
    _check(load_library().h3dit_dit_modulation_table(
        ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), _ptr(conds), int(conds.shape[0]),
        _ptr(table), _stream(stream)), "h3dit_dit_modulation_table")


def h3dit_dit_forward_mod(cfg: Config, st: StackConfig, w_patch, w_final,
                          blocks: Sequence[Dict[str, torch.Tensor]], latent, text, mods, positions,
                          v, workspace, stream=None) -> None:
    """h3dit_dit_forward with the modulation from one step's table row mods."""
    sw, arr = _stack_weights(w_patch, None, w_final, blocks)
    _check(load_library().h3dit_dit_forward_mod(
        ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw), _ptr(latent), _ptr(text),
        _ptr(mods), _ptr(positions), _ptr(v), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "h3dit_dit_forward_mod")


def h3dit_stack_workspace_size_mxfp8(cfg: Config, st: StackConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().h3dit_stack_workspace_size_mxfp8(ctypes.byref(cfg), ctypes.byref(st),
                                                           ctypes.byref(n)),
           "h3dit_stack_workspace_size_mxfp8")
    return n.value


def quantize_blocks(blocks: Sequence[Dict[str, torch.Tensor]], stream=None):
    """MXFP8 codes + scales of every block's four linear weights (on their device)."""
    out = []
    for b in blocks:
        q = {}
        for k in MX_LINEARS:
            q[k], q[k + "_scale"] = mxfp8_quantize(b[k], stream)
        out.append(q)
    return out


def _mx_array(qblocks):
    return (MxWeights * max(len(qblocks), 1))(*[mx_weights_struct(q) for q in qblocks])


def h3dit_dit_forward_mxfp8(cfg: Config, st: StackConfig, w_patch, w_ada_final, w_final,
                            blocks: Sequence[Dict[str, torch.Tensor]], qblocks, latent, text,
                            cond, positions, v, workspace, stream=None) -> None:
    """h3dit_dit_forward with MXFP8 linears; blocks supply w_ada, qblocks the
    quantised linears (quantize_blocks)."""
    sw, arr = _stack_weights(w_patch, w_ada_final, w_final, [_ada_only(b) for b in blocks])
    qa = _mx_array(qblocks)
    _check(load_library().h3dit_dit_forward_mxfp8(
        ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw),
        ctypes.cast(qa, ctypes.POINTER(MxWeights)) if qblocks else None, _ptr(latent), _ptr(text),
        _ptr(cond), _ptr(positions), _ptr(v), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "h3dit_dit_forward_mxfp8")


def h3dit_dit_forward_mod_mxfp8(cfg: Config, st: StackConfig, w_patch, w_final,
                                blocks: Sequence[Dict[str, torch.Tensor]], qblocks, latent, text,
                                mods, positions, v, workspace, stream=None) -> None:
    sw, arr = _stack_weights(w_patch, None, w_final, [_ada_only(b) for b in blocks])
    qa = _mx_array(qblocks)
    _check(load_library().h3dit_dit_forward_mod_mxfp8(
        ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(sw),
        ctypes.cast(qa, ctypes.POINTER(MxWeights)) if qblocks else None, _ptr(latent), _ptr(text),
        _ptr(mods), _ptr(positions), _ptr(v), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)),
        "h3dit_dit_forward_mod_mxfp8")


def _ada_only(b: Dict[str, torch.Tensor]) -> Dict[str, Optional[torch.Tensor]]:
    """A block's weight dict for the MXFP8 stack: only w_ada is read."""
    return {"w_ada": b.get("w_ada"), "w_qkv": None, "w_o": None, "w_up": None, "w_down": None}


def h3dit_latent_step(latent: torch.Tensor, v: torch.Tensor, dt: float, stream=None) -> None:
    _check(load_library().h3dit_latent_step(_ptr(latent), _ptr(v), float(dt), latent.numel(),
                                            _stream(stream)), "h3dit_latent_step")


def h3dit_mxfp8_scale_bytes(rows: int, K: int) -> int:
    return int(load_library().h3dit_mxfp8_scale_bytes(rows, K))


def h3dit_mxfp8_quantize(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                         stream=None) -> None:
    """bf16 x [rows, K] -> codes uint8 [rows, K] + scales uint8 (1 KB block layout)."""
    rows, K = x.shape
    _check(load_library().h3dit_mxfp8_quantize(_ptr(x), rows, K, _ptr(codes), _ptr(scales),
                                               _stream(stream)), "h3dit_mxfp8_quantize")


def h3dit_linear_mxfp8(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                       y: torch.Tensor, stream=None) -> None:
    M, K = xq.shape
    N = wq.shape[0]
    _check(load_library().h3dit_linear_mxfp8(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K,
                                             _ptr(y), _stream(stream)), "h3dit_linear_mxfp8")


def h3dit_workspace_size_mxfp8(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().h3dit_workspace_size_mxfp8(ctypes.byref(cfg), ctypes.byref(n)),
           "h3dit_workspace_size_mxfp8")
    return n.value


def h3dit_workspace_layout(cfg: Config, linears: str = "bf16") -> WorkspaceMap:
    m = WorkspaceMap()
    _check(load_library().h3dit_workspace_layout(ctypes.byref(cfg), 1 if linears == "mxfp8" else 0,
                                                 ctypes.byref(m)), "h3dit_workspace_layout")
    return m


def mxfp8_quantize(x: torch.Tensor, stream=None):
    """Allocate and fill (codes, scales) for the bf16 matrix x [rows, K]."""
    rows, K = x.shape
    codes = torch.empty(rows, K, dtype=torch.uint8, device=x.device)
    scales = torch.empty(h3dit_mxfp8_scale_bytes(rows, K), dtype=torch.uint8, device=x.device)
    h3dit_mxfp8_quantize(x, codes, scales, stream)
    return codes, scales


MX_LINEARS = ("w_qkv", "w_o", "w_up", "w_down")


def mx_weights_struct(q: Dict[str, torch.Tensor]) -> MxWeights:
    """q holds '<name>' codes and '<name>_scale' scales for each of MX_LINEARS."""
    args = []
    for k in MX_LINEARS:
        args += [_ptr(q[k]), _ptr(q[k + "_scale"])]
    return MxWeights(*args)


def h3dit_block_forward_mxfp8(cfg: Config, x, cond, w, q, positions, out, workspace,
                              stream=None) -> None:
    ws, qs = weights_struct(w), mx_weights_struct(q)
    _check(load_library().h3dit_block_forward_mxfp8(
        ctypes.byref(cfg), _ptr(x), _ptr(cond), ctypes.byref(ws), ctypes.byref(qs),
        _ptr(positions), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "h3dit_block_forward_mxfp8")


def h3dit_block_forward_mxfp8_timed(cfg: Config, x, cond, w, q, positions, out, workspace,
                                    events: Sequence[int], stream=None) -> None:
    ws, qs = weights_struct(w), mx_weights_struct(q)
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(load_library().h3dit_block_forward_mxfp8_timed(
        ctypes.byref(cfg), _ptr(x), _ptr(cond), ctypes.byref(ws), ctypes.byref(qs),
        _ptr(positions), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream), arr, len(events)), "h3dit_block_forward_mxfp8_timed")


# ------------------------------------------------------------------ helpers
class Block:
    """Device-resident inputs + workspace for repeated h3dit_block_forward calls."""

    def __init__(self, block_cfg, inputs: Dict[str, torch.Tensor], device: str = "cuda",
                 linears: str = "bf16"):
        """linears: "bf16", or "mxfp8" (weights quantised once here, on the GPU)."""
        if linears not in ("bf16", "mxfp8"):
            raise ValueError(f"linears must be 'bf16' or 'mxfp8' (got {linears!r})")
        self.block_cfg = block_cfg
        self.cfg = config_from(block_cfg)
        self.linears = linears
        self.dev = {k: v.to(device).contiguous() for k, v in inputs.items()}
        self.weights = {k: self.dev[k] for k in ("w_ada", "w_qkv", "w_o", "w_up", "w_down")}
        T, D = block_cfg.n_tokens, block_cfg.hidden
        self.out = torch.empty(T, D, dtype=torch.float32, device=device)
        self.mx = None
        if linears == "mxfp8":
            self.mx = {}
            for k in MX_LINEARS:
                self.mx[k], self.mx[k + "_scale"] = mxfp8_quantize(self.weights[k])
            nbytes = h3dit_workspace_size_mxfp8(self.cfg)
        else:
            nbytes = h3dit_workspace_size(self.cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def forward(self, stream=None) -> torch.Tensor:
        d = self.dev
        if self.mx is not None:
            h3dit_block_forward_mxfp8(self.cfg, d["x"], d["cond"], self.weights, self.mx,
                                      d["positions"], self.out, self.workspace, stream)
        else:
            h3dit_block_forward(self.cfg, d["x"], d["cond"], self.weights, d["positions"],
                                self.out, self.workspace, stream)
        return self.out

    def intermediates(self) -> Dict[str, torch.Tensor]:
        """Views of the intermediate tensors the last forward left in the workspace
        (h3dit_workspace_layout): mod, table, h (= h2), qk, vt, o, x1, u."""
        c = self.block_cfg
        T, D, A, F, H = c.n_tokens, c.hidden, c.attn_width, c.ffn, c.heads
        Tp = h3dit_padded_tokens(T)
        m = h3dit_workspace_layout(self.cfg, self.linears)
        ws = self.workspace

        def view(off, n, dtype, shape):
            nb = n * torch.tensor([], dtype=dtype).element_size()
            return ws[off:off + nb].view(dtype).reshape(shape)

        out = {}
        if self.linears == "mxfp8":
            sd, sf = h3dit_mxfp8_scale_bytes(T, D), h3dit_mxfp8_scale_bytes(T, F)
            out.update({"q_h2": view(m.q_h2, T * D, torch.uint8, (T, D)),
                        "q_h2_scale": view(m.q_h2_scale, sd, torch.uint8, (sd,)),
                        "q_u": view(m.q_u, T * F, torch.uint8, (T, F)),
                        "q_u_scale": view(m.q_u_scale, sf, torch.uint8, (sf,))})
        return {**out, "mod": view(m.mod, 6 * D, torch.float64, (6 * D,)),
                "table": view(m.table, T * 128, torch.float32, (T, 64, 2)),
                "h": view(m.h, T * D, torch.bfloat16, (T, D)),
                "qk": view(m.qk, T * 2 * A, torch.bfloat16, (T, 2 * A)),
                "vt": view(m.vt, A * Tp, torch.bfloat16, (H, 128, Tp)),
                "o": view(m.o, T * A, torch.bfloat16, (T, A)),
                "x1": view(m.x1, T * D, torch.float32, (T, D)),
                "u": view(m.u, T * F, torch.bfloat16, (T, F))}

    def forward_timed(self, events: Sequence[int], stream=None) -> torch.Tensor:
        d = self.dev
        if self.mx is not None:
            h3dit_block_forward_mxfp8_timed(self.cfg, d["x"], d["cond"], self.weights, self.mx,
                                            d["positions"], self.out, self.workspace, events,
                                            stream)
        else:
            h3dit_block_forward_timed(self.cfg, d["x"], d["cond"], self.weights, d["positions"],
                                      self.out, self.workspace, events, stream)
        return self.out

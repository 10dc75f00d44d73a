"""CPU oracle for one MiniMax-H3-Image DiT block forward pass (float64).

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library. Only
the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the library never calls it and has no CPU fallback.

What it computes is the plain definition of the block, step by step, in the
order of the architecture diagram on the apxml.com spec page ("Architecture
Diagram": AdaLN modulation -> RMSNorm -> joint attention -> residual ->
AdaLN modulation -> RMSNorm -> GELU MLP -> residual), with the shapes of the
Hugging Face model card ("Model Architecture": hidden 5376, 56 heads of 128,
FFN 14336) and these readings of what the pages leave open:

  * one weight set for text and image tokens; no biases anywhere;
  * modulation = W_ada . cond split into six rows of width D:
    shift1, scale1, gate1, shift2, scale2, gate2; no SiLU on cond;
  * RMSNorm without a learned weight, eps = 1e-6, mean over the hidden dim;
    modulated as norm(x) * (1 + scale) + shift;
  * 2D axial RoPE: within each head, dims 0..63 turn with the row position and
    dims 64..127 with the column position; adjacent pairs (2i, 2i+1) inside
    each half share frequency base**(-2i/64); text tokens at (0, 0);
    applied to q and k only;
  * bidirectional attention over the whole packed sequence, scale 1/sqrt(128),
    no mask;
  * GELU in its tanh form;
  * x1 and the block output kept at full precision (float64 here).

Two modes:
  * ``"exact"``: every value is float64; softmax is the plain softmax.
  * ``"contract"``: the same math, but values are rounded to bf16 exactly
    where the GPU path stores a bf16 matrix-core operand (h1, v, the
    rotated q and k, the unnormalised attention weights, the attention
    output o, h2 and the GELU output u). q and k are rounded once, after
    the rotation; the stored q also carries the softmax scale:
    q = bf16(rope(q) * log2(e) / sqrt(128)), so a score s = q.k is already
    in base-2 units. The attention
    weights are P = bf16(2 ** (s - ceil(max_j s))), normalised by the sum of
    the rounded P. Mathematically this equals the softmax; the integer shift
    only makes the bf16 weights independent of the order in which keys are
    visited, so the GPU result can be mirrored.

All arithmetic other than the bf16 rounding points is float64.
Parity pins: every function here is checked in the CPU test-suite against
closed forms, invariants, library routines or brute force.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

LOG2E = 1.4426950408889634  # log2(e)


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), float64 in -> float64 out
# ----------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even).

    bf16 keeps 8 significant bits and float32's exponent range. A value with
    binary exponent e (x = m * 2**e, 0.5 <= |m| < 1) is rounded on the grid
    2**(e - 8); below the smallest normal (2**-126) the grid is fixed at
    2**-133 (subnormals). numpy's rint rounds halves to even.
    Overflow past the largest finite bf16 is not handled (inputs never reach it).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)          # -125 - 8 = -133: subnormal grid
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def _round(x: np.ndarray, mode: str) -> np.ndarray:
    return bf16_round(x) if mode == "contract" else x


# ----------------------------------------------------------------------------
# step a1: AdaLN modulation (spec page diagram, "AdaLN Modulation")
# ----------------------------------------------------------------------------
def modulation(w_ada: np.ndarray, cond: np.ndarray) -> np.ndarray:
    """mod[6D] = W_ada[6D, D] . cond[D]  (float64)."""
    return w_ada @ cond


def split_modulation(mod: np.ndarray, D: int) -> Dict[str, np.ndarray]:
    names = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")
    return {n: mod[i * D:(i + 1) * D] for i, n in enumerate(names)}


# ----------------------------------------------------------------------------
# steps a2 / a7: RMSNorm + modulation (spec page "RMS Normalization")
# ----------------------------------------------------------------------------
def rms_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis, no learned weight."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def modulated_norm(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, eps: float,
                   mode: str) -> np.ndarray:
    return _round(rms_normalize(x, eps) * (1.0 + scale) + shift, mode)


# ----------------------------------------------------------------------------
# step a4: 2D axial RoPE
# ----------------------------------------------------------------------------
def rope_frequencies(base: float, half_dim: int = 64) -> np.ndarray:
    """theta_i = base ** (-2 i / half_dim), i = 0 .. half_dim/2 - 1."""
    i = np.arange(half_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / half_dim)


def apply_rope(t: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate t[..., tokens, heads, 128] by the 2D axial positions pos[tokens, 2].

    Half a (a = 0: row, a = 1: column) covers dims 64a .. 64a + 63; inside it
    the pair (64a + 2i, 64a + 2i + 1) turns by angle pos[:, a] * theta_i:
        (u, w) -> (u cos - w sin, u sin + w cos).
    """
    T, H, dh = t.shape
    assert dh == 128 and pos.shape == (T, 2)
    theta = rope_frequencies(base, dh // 2)                     # [32]
    out = np.empty_like(t)
    for a in range(2):
        ang = pos[:, a].astype(np.float64)[:, None] * theta[None, :]   # [T, 32]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        u = t[:, :, 64 * a + 0:64 * a + 64:2]
        w = t[:, :, 64 * a + 1:64 * a + 64:2]
        out[:, :, 64 * a + 0:64 * a + 64:2] = u * c - w * s
        out[:, :, 64 * a + 1:64 * a + 64:2] = u * s + w * c
    return out


# ----------------------------------------------------------------------------
# step a5: joint bidirectional attention
# ----------------------------------------------------------------------------
def scaled_query(q: np.ndarray) -> np.ndarray:
    """Contract-mode stored query: bf16(q * log2(e) / sqrt(dh)), rounded once.

    Folding the softmax scale (1/sqrt(dh), and the change of base from e to 2)
    into the query before its single bf16 rounding keeps one rounding per
    stored element, as for k; softmax(q.k / sqrt(dh)) = 2^(q'.k) / sum 2^(q'.k).
    """
    return bf16_round(q * (LOG2E / math.sqrt(q.shape[-1])))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mode: str) -> np.ndarray:
    """o[Tq, H, dh] for queries q[Tq, H, dh] against all keys k, v[Tk, H, dh].

    exact:    o = softmax(q k^T / sqrt(dh)) v
    contract: q already carries the factor log2(e) / sqrt(dh) (see
              scaled_query), so s = q k^T is the base-2 exponent;
              P = bf16(2**(s - ceil(max s)));  o = bf16( (P v) / sum(P) )
    """
    Tq, H, dh = q.shape
    out = np.empty((Tq, H, dh), dtype=np.float64)
    for h in range(H):
        scores = q[:, h, :] @ k[:, h, :].T                       # [Tq, Tk]
        if mode == "contract":
            s = scores
            m = np.ceil(np.max(s, axis=1, keepdims=True))
            p = bf16_round(np.exp2(s - m))
            out[:, h, :] = bf16_round((p @ v[:, h, :]) / np.sum(p, axis=1, keepdims=True))
        else:
            s = scores / math.sqrt(dh)
            s = s - np.max(s, axis=1, keepdims=True)
            p = np.exp(s)
            out[:, h, :] = (p @ v[:, h, :]) / np.sum(p, axis=1, keepdims=True)
    return out


# ----------------------------------------------------------------------------
# step a8: GELU, tanh form (Hendrycks & Gimpel, 2016)
# ----------------------------------------------------------------------------
def gelu_tanh(z: np.ndarray) -> np.ndarray:
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


# ----------------------------------------------------------------------------
# the whole block (steps a1 .. a9)
# ----------------------------------------------------------------------------
def block_forward(x: np.ndarray, cond: np.ndarray, w: Dict[str, np.ndarray], pos: np.ndarray,
                  heads: int, eps: float = 1e-6, rope_base: float = 10000.0,
                  mode: str = "contract", rows: Optional[np.ndarray] = None,
                  linears: str = "bf16") -> Dict[str, np.ndarray]:
    """One DiT block. All array inputs float64 (bf16 / fp32 values widened exactly).

    x [T, D], cond [D], w: w_ada [6D, D], w_qkv [3A, D], w_o [D, A],
    w_up [F, D], w_down [D, F]; pos int [T, 2].
    rows: optional sorted token indices; then every per-token output is
    computed for those rows only (keys and values still cover all T tokens).
    Returns the intermediates (mod, h1, q, k, v for the rows that matter,
    o, x1, h2, u, out) as float64.
    """
    assert mode in ("exact", "contract")
    assert linears in ("bf16", "mxfp8")
    # the four linears: plain products, or both operands quantised to MXFP8
    # along K first (oracle/mxfp8.py; contract mode only, where the inputs are
    # the bf16 operands of the GPU path)
    if linears == "mxfp8":
        assert mode == "contract"
        from . import mxfp8
        lin = mxfp8.linear
    else:
        lin = lambda a, b: a @ b.T
    T, D = x.shape
    A = w["w_qkv"].shape[0] // 3
    dh = A // heads
    r = np.arange(T) if rows is None else np.asarray(rows)

    mod = modulation(w["w_ada"], cond)
    mv = split_modulation(mod, D)

    # a2: h1 for every token (keys and values need all of them)
    h1 = modulated_norm(x, mv["shift1"], mv["scale1"], eps, mode)

    # a3: projections; k and v over all tokens, q over the requested rows
    w_q, w_k, w_v = w["w_qkv"][:A], w["w_qkv"][A:2 * A], w["w_qkv"][2 * A:]
    q = lin(h1[r], w_q).reshape(len(r), heads, dh)
    k = lin(h1, w_k).reshape(T, heads, dh)
    v = _round(lin(h1, w_v), mode).reshape(T, heads, dh)

    # a4: RoPE on q and k; each is rounded to bf16 once, after the rotation
    # (and, for q, after the softmax scale)
    q = apply_rope(q, pos[r], rope_base)
    q = scaled_query(q) if mode == "contract" else q
    k = _round(apply_rope(k, pos, rope_base), mode)

    # a5: attention of the requested queries against every key
    o = attention(q, k, v, mode).reshape(len(r), A)

    # a6: output projection + gated residual
    x1 = x[r] + mv["gate1"] * lin(o, w["w_o"])

    # a7 .. a9: modulated norm, GELU MLP, gated residual
    h2 = modulated_norm(x1, mv["shift2"], mv["scale2"], eps, mode)
    u = _round(gelu_tanh(lin(h2, w["w_up"])), mode)
    out = x1 + mv["gate2"] * lin(u, w["w_down"])

    return dict(mod=mod, h1=h1, q=q.reshape(len(r), A), k=k.reshape(T, A), v=v.reshape(T, A),
                o=o, x1=x1, h2=h2, u=u, out=out, rows=r)


# ----------------------------------------------------------------------------
# the DiT around the blocks (model card, "Model Architecture": latent patches
# become the image tokens of the packed sequence; spec page,
# "Specifications": 50 layers). Readings where the pages are silent: the
# patch embedding and the final projection are plain fp32 linears without
# bias; the final layer is a modulated RMSNorm (shift, scale from its own
# AdaLN linear of cond) followed by the projection, like the blocks' norms;
# the same cond feeds every block of one evaluation.
# ----------------------------------------------------------------------------
def patchify(latent: np.ndarray, p: int) -> np.ndarray:
    """latent [C, H, W] -> patches [(H/p)(W/p), C p p]; token t = gy (W/p) + gx,
    feature c p p + dy p + dx holds latent[c, gy p + dy, gx p + dx]."""
    C, H, W = latent.shape
    gh, gw = H // p, W // p
    return latent.reshape(C, gh, p, gw, p).transpose(1, 3, 0, 2, 4).reshape(gh * gw, C * p * p)


def unpatchify(vt: np.ndarray, C: int, p: int, gh: int, gw: int) -> np.ndarray:
    """Inverse of patchify: per-token rows [gh gw, C p p] -> [C, gh p, gw p]."""
    return vt.reshape(gh, gw, C, p, p).transpose(2, 0, 3, 1, 4).reshape(C, gh * p, gw * p)


def final_layer(x_img: np.ndarray, cond: np.ndarray, w_ada_final: np.ndarray,
                w_final: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """(rmsnorm(x) * (1 + scale) + shift) . w_final^T with (shift, scale) = w_ada_final . cond."""
    D = x_img.shape[1]
    mod = w_ada_final @ cond
    shift, scale = mod[:D], mod[D:2 * D]
    return (rms_normalize(x_img, eps) * (1.0 + scale) + shift) @ w_final.T


def dit_forward(latent: np.ndarray, text: np.ndarray, cond: np.ndarray, w_patch: np.ndarray,
                w_ada_final: np.ndarray, w_final: np.ndarray, blocks, pos: np.ndarray,
                heads: int, patch: int, eps: float = 1e-6, rope_base: float = 10000.0,
                mode: str = "contract", linears: str = "bf16") -> np.ndarray:
    """One DiT evaluation: v [C, H, W] for latent [C, H, W] (see module notes).
    linears="mxfp8": every block's four linears in MXFP8 (see block_forward)."""
    C, H, W = latent.shape
    x = np.concatenate([text, patchify(latent, patch) @ w_patch.T], axis=0)
    for w in blocks:
        x = block_forward(x, cond, w, pos, heads=heads, eps=eps, rope_base=rope_base,
                          mode=mode, linears=linears)["out"]
    vt = final_layer(x[text.shape[0]:], cond, w_ada_final, w_final, eps)
    return unpatchify(vt, C, patch, H // patch, W // patch)


def euler_sample(latent: np.ndarray, conds, dt: float, **dit_kwargs) -> np.ndarray:
    """Explicit Euler steps latent <- latent + dt * v(latent, cond_k), one per cond.
    The pages do not give the sampler's schedule; this fixed-step update is a
    stand-in that exercises the repeated evaluation, not the model's sampler."""
    for cond in conds:
        latent = latent + dt * dit_forward(latent, cond=cond, **dit_kwargs)
    return latent

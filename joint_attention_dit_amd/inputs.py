"""Seeded synthetic inputs for one MiniMax-H3-Image DiT block.

This module holds the workload shapes and the seeded input generators that
both the HIP path and the CPU oracle consume. It holds none of the block's
arithmetic: it only draws random numbers, lays out token positions and picks
sample rows.

Shapes follow the model card (Hugging Face card, section "Model Architecture":
hidden 5376, 56 heads, FFN 14336; one token per 2x2 latent patch, i.e. per
32x32 pixels) and the spec page's list (apxml.com spec page, "Specifications":
head dimension 128, 56 query and 56 key-value heads). Token geometry: a
4096x4096 canvas is 128x128 = 16,384 image tokens (vLLM blog, "Inference
Optimizations").

Generation rules (the pages' serving guide fixes a CPU generator with a fixed
seed so that every machine sees the same noise; the same practice is used
here):
  * CPU ``torch.Generator``, seed 0 unless stated.
  * Draw order: w_ada, w_qkv, w_o, w_up, w_down, x, cond.
  * Weights ~ N(0, 0.02^2), rounded to bf16 (round-to-nearest-even).
  * x ~ N(0, 1): fp32 for the tiny block, bf16 for the full-width blocks.
  * cond ~ N(0, 1), fp32.
  * Sample rows: a separate generator, seed 1, drawn without replacement.

Token order inside the packed joint sequence: text tokens first, then the
target image (row-major), then each reference image (row-major). Text tokens
sit at RoPE position (0, 0). Image token (r, c) of the target sits at (r, c);
reference image k (k = 1, 2, ...) sits at (row_offset_k + r, c) with
row_offset_k = 64 * k for the edit-shaped workload.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class BlockConfig:
    name: str
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    text_tokens: int
    # one (rows, cols, row_offset) triple per image: target first, then refs
    images: Tuple[Tuple[int, int, int], ...]
    x_dtype: str  # "fp32" or "bf16"
    eps: float = 1e-6
    rope_base: float = 10000.0
    description: str = ""

    @property
    def attn_width(self) -> int:
        return self.heads * self.head_dim

    @property
    def image_tokens(self) -> int:
        return sum(r * c for r, c, _ in self.images)

    @property
    def n_tokens(self) -> int:
        return self.text_tokens + self.image_tokens


_FULL = dict(hidden=5376, heads=56, head_dim=128, ffn=14336)

CONFIGS: Dict[str, BlockConfig] = {
    "tiny": BlockConfig(
        "tiny", hidden=256, heads=2, head_dim=128, ffn=1024, text_tokens=32,
        images=((16, 16, 0),), x_dtype="fp32",
        description="tiny block: hidden 256, 2x128 heads, FFN 1024, 16x16 image + 32 text = 288 tokens"),
    "2048": BlockConfig(
        "2048", text_tokens=256, images=((64, 64, 0),), x_dtype="bf16",
        description="full-width block, 2048x2048 canvas: 64x64 = 4096 image + 256 text = 4352 tokens",
        **_FULL),
    "4096": BlockConfig(
        "4096", text_tokens=512, images=((128, 128, 0),), x_dtype="bf16",
        description="full-width block, 4096x4096 canvas: 128x128 = 16384 image + 512 text = 16896 tokens",
        **_FULL),
    "edit": BlockConfig(
        "edit", text_tokens=1024,
        images=((64, 64, 0), (64, 64, 64), (64, 64, 128), (64, 64, 192), (64, 64, 256)),
        x_dtype="bf16",
        description="edit-shaped block: 2048x2048 target + 4 references of 64x64 + 1024 text = 21504 tokens",
        **_FULL),
    # one GPU's token share of the 4096x4096 block under G-way Ulysses sequence
    # parallelism (vLLM blog, "Inference Optimizations", and the serving
    # recipe's deployment profiles: SP4 is the default layout): T / G tokens
    # through the per-token kernels, laid out as 512 / G text tokens and
    # 128-column image rows of the canvas
    "share4": BlockConfig(
        "share4", text_tokens=128, images=((32, 128, 0),), x_dtype="bf16",
        description="4-way Ulysses share of the 4096x4096 block: 128 text + 32x128 image = 4224 tokens",
        **_FULL),
    "share8": BlockConfig(
        "share8", text_tokens=64, images=((16, 128, 0),), x_dtype="bf16",
        description="8-way Ulysses share of the 4096x4096 block: 64 text + 16x128 image = 2112 tokens",
        **_FULL),
    # non-square canvas (2720x1536 -> 85x48 tokens): ragged tiles everywhere
    "nonsquare": BlockConfig(
        "nonsquare", text_tokens=256, images=((48, 85, 0),), x_dtype="bf16",
        description="full-width block, 2720x1536 canvas: 48x85 = 4080 image + 256 text = 4336 tokens",
        **_FULL),
}


def small_config(name: str, *, hidden: int, heads: int, ffn: int, text_tokens: int,
                 images: Tuple[Tuple[int, int, int], ...], x_dtype: str = "fp32") -> BlockConfig:
    """A reduced-width block (head_dim stays 128) for quick parity cases."""
    return BlockConfig(name, hidden=hidden, heads=heads, head_dim=128, ffn=ffn,
                       text_tokens=text_tokens, images=images, x_dtype=x_dtype,
                       description=f"{name}: hidden {hidden}, {heads}x128 heads, FFN {ffn}")


def positions(cfg: BlockConfig) -> np.ndarray:
    """Integer RoPE positions (row, col), int32 [T, 2], in packed token order."""
    parts = [np.zeros((cfg.text_tokens, 2), dtype=np.int32)]
    for rows, cols, row_off in cfg.images:
        r, c = np.meshgrid(np.arange(rows, dtype=np.int32), np.arange(cols, dtype=np.int32),
                           indexing="ij")
        parts.append(np.stack([r.reshape(-1) + row_off, c.reshape(-1)], axis=1).astype(np.int32))
    return np.ascontiguousarray(np.concatenate(parts, axis=0))


def make_inputs(cfg: BlockConfig, seed: int = 0) -> Dict[str, torch.Tensor]:
    """All block inputs as CPU tensors (weights bf16 [out, in] row-major)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    D, A, F = cfg.hidden, cfg.attn_width, cfg.ffn
    T = cfg.n_tokens

    def w(rows: int, cols: int) -> torch.Tensor:
        return (torch.randn(rows, cols, generator=g, dtype=torch.float32) * 0.02).to(torch.bfloat16)

    out: Dict[str, torch.Tensor] = {}
    out["w_ada"] = w(6 * D, D)
    out["w_qkv"] = w(3 * A, D)
    out["w_o"] = w(D, A)
    out["w_up"] = w(F, D)
    out["w_down"] = w(D, F)
    x = torch.randn(T, D, generator=g, dtype=torch.float32)
    out["x"] = x if cfg.x_dtype == "fp32" else x.to(torch.bfloat16)
    out["cond"] = torch.randn(D, generator=g, dtype=torch.float32)
    out["positions"] = torch.from_numpy(positions(cfg))
    return out


# ---------------------------------------------------------------- DiT stack
@dataclass(frozen=True)
class StackConfig:
    """The DiT around the blocks: n_blocks blocks of shape `block` (one target
    image, text first), latents of `channels` channels cut into patch x patch
    patches (one image token each), `steps` denoising steps."""
    name: str
    block: BlockConfig
    n_blocks: int
    channels: int
    patch: int
    steps: int
    description: str = ""

    @property
    def grid(self) -> Tuple[int, int]:
        rows, cols, _ = self.block.images[0]
        return rows, cols

    @property
    def latent_shape(self) -> Tuple[int, int, int]:
        rows, cols = self.grid
        return self.channels, rows * self.patch, cols * self.patch

    @property
    def patch_features(self) -> int:
        return self.channels * self.patch * self.patch


STACK_CONFIGS: Dict[str, StackConfig] = {
    "tiny_stack": StackConfig(
        "tiny_stack",
        block=small_config("tiny_stack", hidden=256, heads=2, ffn=1024, text_tokens=8,
                           images=((4, 4, 0),)),
        n_blocks=3, channels=4, patch=2, steps=2,
        description="tiny DiT: 3 blocks of hidden 256, 4-channel 8x8 latent (4x4 tokens) + 8 text, 2 steps"),
    "dit_2048": StackConfig(
        "dit_2048", block=CONFIGS["2048"], n_blocks=50, channels=24, patch=2, steps=6,
        description=("full DiT: 50 blocks, 6 denoising steps at 2048x2048 (24-channel 128x128 latent, "
                     "64x64 image tokens + 256 text tokens)")),
}


def make_stack_inputs(scfg: StackConfig, seed: int = 0, device: str = "cpu",
                      n_blocks: int = -1) -> Dict[str, object]:
    """Seeded DiT-stack inputs. Draw order (one generator, `seed`): for every
    block w_ada, w_qkv, w_o, w_up, w_down (bf16, N(0, 0.02^2)); then w_patch
    (fp32 [D, C p p], N(0, 0.02^2)), w_ada_final (bf16 [2D, D]), w_final (fp32
    [C p p, D], N(0, 0.02^2)), the latent (fp32, N(0, 1)) and the text tokens
    (fp32 [text, D], N(0, 1)). Step k's cond vector (fp32 [D], N(0, 1)) comes
    from its own generator seeded k. `device` "cuda" draws on the GPU (a
    different stream of numbers than the CPU generator) for the full-size
    stack; n_blocks < 0 means scfg.n_blocks."""
    nb = scfg.n_blocks if n_blocks < 0 else n_blocks
    b = scfg.block
    D, A, F = b.hidden, b.attn_width, b.ffn
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def rnd(*shape, scale=1.0, dtype=torch.float32):
        return (torch.randn(*shape, generator=g, dtype=torch.float32, device=device) * scale).to(dtype)

    blocks = []
    for _ in range(nb):
        blocks.append({"w_ada": rnd(6 * D, D, scale=0.02, dtype=torch.bfloat16),
                       "w_qkv": rnd(3 * A, D, scale=0.02, dtype=torch.bfloat16),
                       "w_o": rnd(D, A, scale=0.02, dtype=torch.bfloat16),
                       "w_up": rnd(F, D, scale=0.02, dtype=torch.bfloat16),
                       "w_down": rnd(D, F, scale=0.02, dtype=torch.bfloat16)})
    P = scfg.patch_features
    out: Dict[str, object] = {"blocks": blocks}
    out["w_patch"] = rnd(D, P, scale=0.02)
    out["w_ada_final"] = rnd(2 * D, D, scale=0.02, dtype=torch.bfloat16)
    out["w_final"] = rnd(P, D, scale=0.02)
    out["latent"] = rnd(*scfg.latent_shape)
    out["text"] = rnd(b.text_tokens, D)
    conds = []
    for k in range(scfg.steps):
        gk = torch.Generator(device=device)
        gk.manual_seed(k)
        conds.append(torch.randn(D, generator=gk, dtype=torch.float32, device=device))
    out["conds"] = conds
    out["positions"] = torch.from_numpy(positions(b)).to(device)
    return out


def sample_rows(n_tokens: int, n: int = 256, seed: int = 1) -> np.ndarray:
    """Sorted token indices for sampled-row parity; all rows when n >= T."""
    if n >= n_tokens:
        return np.arange(n_tokens, dtype=np.int64)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    idx = torch.randperm(n_tokens, generator=g)[:n]
    return np.sort(idx.numpy().astype(np.int64))


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 / fp32 CPU tensor to a float64 array."""
    return t.detach().to("cpu").to(torch.float64).numpy()

"""GPU parity of the DiT stack (patch embedding, blocks, modulated final
projection, Euler steps) against the float64 CPU oracle, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from joint_attention_dit_amd import binding as B
from joint_attention_dit_amd.inputs import (STACK_CONFIGS, BlockConfig, StackConfig,
                                            make_stack_inputs, to_numpy_f64)
from tests._common import assert_block_parity, errors

import oracle as O

pytestmark = pytest.mark.gpu

DT = 1.0 / 6.0
_FULL = dict(hidden=5376, heads=56, head_dim=128, ffn=14336)


def say(msg):
    print(msg, flush=True)


def full_width(name, n_blocks, text, grid, steps=1):
    blk = BlockConfig(name, text_tokens=text, images=((grid, grid, 0),), x_dtype="fp32", **_FULL)
    return StackConfig(name, block=blk, n_blocks=n_blocks, channels=24, patch=2, steps=steps,
                       description=f"{name}: full width, {n_blocks} blocks, {grid}x{grid} + {text}")


def gpu_stack(scfg: StackConfig, inp, blocks=None):
    """Runs the denoising loop on the GPU; returns (v of every step, final latent)."""
    cfg = B.config_from(scfg.block)
    blocks = inp["blocks"] if blocks is None else blocks
    gh, gw = scfg.grid
    st = B.StackConfig(len(blocks), scfg.channels, scfg.patch, gh, gw, scfg.block.text_tokens)
    ws = torch.empty(B.h3dit_stack_workspace_size(cfg, st), dtype=torch.uint8, device="cuda")
    dev = lambda t: t.to("cuda").contiguous()
    dblocks = [{k: dev(v) for k, v in b.items()} for b in blocks]
    latent = dev(inp["latent"]).clone()
    text = dev(inp["text"]) if scfg.block.text_tokens > 0 else None
    pos = dev(inp["positions"])
    v = torch.empty_like(latent)
    vs = []
    for cond in inp["conds"]:
        B.h3dit_dit_forward(cfg, st, dev(inp["w_patch"]), dev(inp["w_ada_final"]),
                            dev(inp["w_final"]), dblocks, latent, text, dev(cond), pos, v, ws)
        vs.append(v.cpu().double().numpy())
        B.h3dit_latent_step(latent, v, DT)
    torch.cuda.synchronize()
    return vs, latent.cpu().double().numpy()


def oracle_stack(scfg: StackConfig, inp, mode="contract", blocks=None):
    blocks = inp["blocks"] if blocks is None else blocks
    kw = dict(text=to_numpy_f64(inp["text"]), w_patch=to_numpy_f64(inp["w_patch"]),
              w_ada_final=to_numpy_f64(inp["w_ada_final"]), w_final=to_numpy_f64(inp["w_final"]),
              blocks=[{k: to_numpy_f64(t) for k, t in b.items()} for b in blocks],
              pos=inp["positions"].numpy(), heads=scfg.block.heads, patch=scfg.patch,
              eps=scfg.block.eps, rope_base=scfg.block.rope_base, mode=mode)
    latent = to_numpy_f64(inp["latent"])
    vs = []
    for cond in inp["conds"]:
        v = O.dit_forward(latent, cond=to_numpy_f64(cond), **kw)
        vs.append(v)
        latent = latent + DT * v
    return vs, latent


def test_stack_tiny_all_steps():
    scfg = STACK_CONFIGS["tiny_stack"]
    say(f"[stack] {scfg.description}")
    inp = make_stack_inputs(scfg, seed=0)
    g_vs, g_lat = gpu_stack(scfg, inp)
    r_vs, r_lat = oracle_stack(scfg, inp)
    for k, (g, r) in enumerate(zip(g_vs, r_vs)):
        assert_block_parity(g, r, f"tiny stack v step {k}")
    lat0 = to_numpy_f64(inp["latent"])
    assert_block_parity((g_lat - lat0) / DT, (r_lat - lat0) / DT, "tiny stack latent displacement")


def test_stack_without_blocks_full_width():
    """Patch embedding + final layer only (fp32 linears): close to float64."""
    scfg = full_width("embed_final", 0, text=16, grid=8)
    say(f"[stack] {scfg.description}")
    inp = make_stack_inputs(scfg, seed=1, n_blocks=0)
    g_vs, _ = gpu_stack(scfg, inp)
    r_vs, _ = oracle_stack(scfg, inp, mode="exact")
    e = errors(g_vs[0], r_vs[0])
    say(f"[parity] embed+final v: rel_l2={e['rel_l2']:.3e} max_abs/rms={e['max_abs_over_rms']:.3e}")
    assert e["rel_l2"] < 1e-5 and e["max_abs_over_rms"] < 1e-4


def test_stack_identity_blocks_match_no_blocks_bitwise():
    """Blocks with zero gates return their input exactly, so two of them in the
    chain leave the DiT output bit-identical to the chain without blocks."""
    scfg = full_width("identity_blocks", 2, text=16, grid=8)
    say(f"[stack] {scfg.description}")
    inp = make_stack_inputs(scfg, seed=2)
    D = scfg.block.hidden
    blocks = []
    for b in inp["blocks"]:
        w_ada = b["w_ada"].clone()
        w_ada[2 * D:3 * D] = 0
        w_ada[5 * D:6 * D] = 0
        blocks.append(dict(b, w_ada=w_ada))
    g_id, _ = gpu_stack(scfg, inp, blocks=blocks)
    g_none, _ = gpu_stack(scfg, inp, blocks=[])
    assert np.array_equal(g_id[0], g_none[0])


def test_stack_one_block_full_width():
    scfg = full_width("one_block", 1, text=32, grid=16)
    say(f"[stack] {scfg.description}")
    inp = make_stack_inputs(scfg, seed=3)
    g_vs, _ = gpu_stack(scfg, inp)
    r_vs, _ = oracle_stack(scfg, inp)
    assert_block_parity(g_vs[0], r_vs[0], "full-width one-block DiT v")


def test_modulation_table_bitwise_equals_one_vector_calls():
    """Several conditioning vectors per pass over W_ada (9: two passes of 8 and 1)
    give exactly the per-vector results."""
    scfg = STACK_CONFIGS["tiny_stack"]
    inp = make_stack_inputs(scfg, seed=3)
    cfg = B.config_from(scfg.block)
    D = scfg.block.hidden
    w_ada = inp["blocks"][0]["w_ada"].cuda()
    g = torch.Generator().manual_seed(11)
    conds = (torch.randn(9, D, generator=g) * 3).cuda()
    table = torch.empty(9, 6 * D, dtype=torch.float64, device="cuda")
    B.h3dit_modulation_table(cfg, w_ada, conds, table)
    for s in range(9):
        one = torch.empty(6 * D, dtype=torch.float64, device="cuda")
        B.h3dit_modulation(cfg, w_ada, conds[s].contiguous(), one)
        assert torch.equal(table[s], one), s


def test_stack_with_modulation_table_bitwise_equals_stack():
    """All steps of the tiny stack: the modulation taken from the precomputed
    table (every AdaLN weight read once) leaves every v and the final latent
    bit-identical."""
    scfg = STACK_CONFIGS["tiny_stack"]
    say(f"[stack] modulation table, {scfg.description}")
    inp = make_stack_inputs(scfg, seed=0)
    g_vs, g_lat = gpu_stack(scfg, inp)
    cfg = B.config_from(scfg.block)
    gh, gw = scfg.grid
    nb = len(inp["blocks"])
    st = B.StackConfig(nb, scfg.channels, scfg.patch, gh, gw, scfg.block.text_tokens)
    ws = torch.empty(B.h3dit_stack_workspace_size(cfg, st), dtype=torch.uint8, device="cuda")
    dev = lambda t: t.to("cuda").contiguous()
    dblocks = [{k: dev(v) for k, v in b.items()} for b in inp["blocks"]]
    conds = torch.stack([c for c in inp["conds"]]).cuda().contiguous()
    D = scfg.block.hidden
    table = torch.full((len(inp["conds"]), nb + 1, 6 * D), float("nan"), dtype=torch.float64,
                       device="cuda")
    B.h3dit_dit_modulation_table(cfg, st, dev(inp["w_ada_final"]), dblocks, conds, table)
    latent = dev(inp["latent"]).clone()
    v = torch.empty_like(latent)
    for k in range(len(inp["conds"])):
        B.h3dit_dit_forward_mod(cfg, st, dev(inp["w_patch"]), dev(inp["w_final"]), dblocks, latent,
                                dev(inp["text"]), table[k].contiguous(), dev(inp["positions"]), v,
                                ws)
        assert np.array_equal(v.cpu().double().numpy(), g_vs[k]), k
        B.h3dit_latent_step(latent, v, DT)
    assert np.array_equal(latent.cpu().double().numpy(), g_lat)

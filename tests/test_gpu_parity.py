"""GPU parity of the HIP path against the float64 CPU oracle (contract mode).

Stage tests feed each entry point the oracle's own inputs for that step, so a
failure names the step. Block tests run h3dit_block_forward end to end and
compare the output element by element (all rows for small blocks, 256 seeded
rows for the full-width blocks) against the bar: max |err| <= 2e-2 * RMS(out)
and relative L2 <= 5e-3.
"""
import numpy as np
import pytest
import torch

import oracle as O
from joint_attention_dit_amd import binding as B
from joint_attention_dit_amd.inputs import CONFIGS, make_inputs, sample_rows, small_config

from tests._common import (assert_bf16_close, assert_block_parity, bf16_ulp_diff, cached_case,
                           errors, oracle_inputs, oracle_reference)

pytestmark = pytest.mark.gpu

MID = small_config("mid", hidden=512, heads=4, ffn=1536, text_tokens=35, images=((23, 29, 0),),
                   x_dtype="bf16")
MID32 = small_config("mid32", hidden=384, heads=3, ffn=1024, text_tokens=10, images=((9, 13, 0),),
                     x_dtype="fp32")
SMALL_CASES = [CONFIGS["tiny"], MID, MID32]


def say(msg):
    print(msg, flush=True)


def dev(t, dtype=None):
    t = t if dtype is None else t.to(dtype)
    return t.contiguous().cuda()


def bf16_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


def f64_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).cuda()


def unswap_vt(vt):
    """vt holds token t in column t with bits 4, 3, 2 moved to bits 2, 4, 3
    (a permutation within each group of 32 keys); return it in token order."""
    t = np.arange(vt.shape[-1])
    src = (t & ~28) | ((t & 12) << 1) | ((t & 16) >> 2)
    return vt[..., src]


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().to(torch.float64).numpy()


# ------------------------------------------------------------------ stages
@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_stage_modulation(cfg):
    inp = cached_case(cfg)
    say(f"[stage] modulation {cfg.name} D={cfg.hidden}")
    c = B.config_from(cfg)
    mod = torch.empty(6 * cfg.hidden, dtype=torch.float64, device="cuda")
    B.h3dit_modulation(c, dev(inp["w_ada"]), dev(inp["cond"]), mod)
    x, cond, w, pos = oracle_inputs(inp)
    np.testing.assert_allclose(host(mod), O.modulation(w["w_ada"], cond), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_stage_rmsnorm_modulate(cfg):
    inp = cached_case(cfg)
    say(f"[stage] rmsnorm {cfg.name} T={cfg.n_tokens} D={cfg.hidden} x={cfg.x_dtype}")
    x, cond, w, pos = oracle_inputs(inp)
    mv = O.split_modulation(O.modulation(w["w_ada"], cond), cfg.hidden)
    c = B.config_from(cfg)
    h = torch.empty(cfg.n_tokens, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    B.h3dit_rmsnorm_modulate(c, dev(inp["x"]), f64_dev(mv["shift1"]), f64_dev(mv["scale1"]), h)
    ref = O.modulated_norm(x, mv["shift1"], mv["scale1"], cfg.eps, "contract")
    ulp = bf16_ulp_diff(host(h), ref)
    assert ulp.max() <= 1 and np.mean(ulp > 0) < 1e-3, (ulp.max(), np.mean(ulp > 0))


@pytest.mark.parametrize("cfg", [MID, MID32], ids=lambda c: c.name)
def test_stage_rmsnorm_rounds_like_fp64_beside_bf16_midpoints(cfg):
    """Shifts chosen so that, in each column, one element's fp64 value lies
    2^-28 (relative) above or below a midpoint between two bf16 values: its
    rounding to fp32 lands on the midpoint, and only the fp64 value says which
    way the bf16 rounding goes. The kernel's output must be the oracle's, bit
    for bit, on those elements and on every other one."""
    inp = cached_case(cfg)
    say(f"[stage] rmsnorm midpoints {cfg.name} T={cfg.n_tokens} D={cfg.hidden} x={cfg.x_dtype}")
    x, cond, w, pos = oracle_inputs(inp)
    T, D = x.shape
    scale = O.split_modulation(O.modulation(w["w_ada"], cond), D)["scale1"]
    rng = np.random.default_rng(7)
    rows, cols = rng.integers(0, T, size=D), np.arange(D)
    prod = O.rms_normalize(x, cfg.eps)[rows, cols] * (1.0 + scale)
    # the midpoint above a bf16 value a (in magnitude): a's bits with bit 15 set
    u = (rng.standard_normal(D) * np.maximum(np.abs(prod), 0.5)).astype(np.float32)
    mid = ((u.view(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32).astype(np.float64)
    side = rng.choice([-1.0, 1.0], size=D)
    shift = mid * (1.0 + side * 2.0 ** -28) - prod
    value = O.rms_normalize(x, cfg.eps)[rows, cols] * (1.0 + scale) + shift
    assert np.mean(value.astype(np.float32) == mid) > 0.99  # fp32 lands on the midpoint
    c = B.config_from(cfg)
    h = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    B.h3dit_rmsnorm_modulate(c, dev(inp["x"]), f64_dev(shift), f64_dev(scale), h)
    ref = O.modulated_norm(x, shift, scale, cfg.eps, "contract")
    up = np.abs(ref[rows, cols]) > np.abs(mid)
    assert 0.3 < np.mean(up) < 0.7, np.mean(up)  # both directions are exercised
    ulp = bf16_ulp_diff(host(h), ref)
    assert ulp[rows, cols].max() == 0 and ulp.max() == 0, (ulp[rows, cols].max(), ulp.max())


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_stage_rope_table(cfg):
    inp = cached_case(cfg)
    say(f"[stage] rope table {cfg.name} T={cfg.n_tokens}")
    c = B.config_from(cfg)
    table = torch.empty(cfg.n_tokens, 64, 2, dtype=torch.float32, device="cuda")
    B.h3dit_rope_table(c, dev(inp["positions"]), table)
    pos = inp["positions"].numpy().astype(np.float64)
    theta = O.rope_frequencies(cfg.rope_base)
    ang = np.concatenate([pos[:, 0:1] * theta[None], pos[:, 1:2] * theta[None]], axis=1)
    got = host(table)
    np.testing.assert_allclose(got[..., 0], np.cos(ang), atol=1e-7, rtol=0)
    np.testing.assert_allclose(got[..., 1], np.sin(ang), atol=1e-7, rtol=0)


def _qkv_stage(cfg, inp):
    x, cond, w, pos = oracle_inputs(inp)
    mv = O.split_modulation(O.modulation(w["w_ada"], cond), cfg.hidden)
    h1 = O.modulated_norm(x, mv["shift1"], mv["scale1"], cfg.eps, "contract")
    c = B.config_from(cfg)
    T, A = cfg.n_tokens, cfg.attn_width
    Tp = B.h3dit_padded_tokens(T)
    table = torch.empty(T, 64, 2, dtype=torch.float32, device="cuda")
    B.h3dit_rope_table(c, dev(inp["positions"]), table)
    qk = torch.empty(T, 2 * A, dtype=torch.bfloat16, device="cuda")
    vt = torch.full((cfg.heads, 128, Tp), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.h3dit_qkv_rope(c, bf16_dev(h1), dev(inp["w_qkv"]), table, qk, vt)
    return h1, w, pos, qk, vt


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_stage_qkv_rope(cfg):
    inp = cached_case(cfg)
    say(f"[stage] qkv+rope {cfg.name} T={cfg.n_tokens}")
    h1, w, pos, qk, vt = _qkv_stage(cfg, inp)
    T, A, H = cfg.n_tokens, cfg.attn_width, cfg.heads
    wq, wk, wv = w["w_qkv"][:A], w["w_qkv"][A:2 * A], w["w_qkv"][2 * A:]
    q = O.scaled_query(O.apply_rope((h1 @ wq.T).reshape(T, H, 128), pos, cfg.rope_base))
    k = O.bf16_round(O.apply_rope((h1 @ wk.T).reshape(T, H, 128), pos, cfg.rope_base))
    v = O.bf16_round(h1 @ wv.T).reshape(T, H, 128)
    g_qk = host(qk)
    g_vt = unswap_vt(host(vt))
    for name, got, ref in (("q", g_qk[:, :A], q.reshape(T, A)), ("k", g_qk[:, A:], k.reshape(T, A)),
                           ("v", g_vt[:, :, :T].transpose(2, 0, 1).reshape(T, A), v.reshape(T, A))):
        # a one-ulp difference in a bf16 input of the rotation can cancel into
        # many ulps of a small output, so q and k errors are measured against
        # the norm of their rotation pair (which RoPE preserves)
        if name == "v":
            assert_bf16_close(got, ref, "v", ulps=1, floor_over_rms=1e-4)
            continue
        frac = float(np.mean(got != ref))
        pair = np.sqrt(ref[:, 0::2] ** 2 + ref[:, 1::2] ** 2).repeat(2, axis=1)
        rel = np.abs(got - ref) / np.maximum(pair, 1e-30)
        say(f"  {name}: max |err|/pair-norm {rel.max():.2e}, mismatch fraction {frac:.2e}")
        assert rel.max() <= 2 ** -7 and frac < 1e-2, (name, rel.max(), frac)
    assert np.all(g_vt[:, :, T:] == 0.0), "vt padding must be zero"


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_stage_attention(cfg):
    inp = cached_case(cfg)
    say(f"[stage] attention {cfg.name} T={cfg.n_tokens} H={cfg.heads}")
    h1, w, pos, qk, vt = _qkv_stage(cfg, inp)
    T, A, H = cfg.n_tokens, cfg.attn_width, cfg.heads
    o = torch.empty(T, A, dtype=torch.bfloat16, device="cuda")
    B.h3dit_attention(B.config_from(cfg), qk, vt, o)
    g_qk, g_vt = host(qk), unswap_vt(host(vt))
    q = g_qk[:, :A].reshape(T, H, 128)
    k = g_qk[:, A:].reshape(T, H, 128)
    v = g_vt[:, :, :T].transpose(2, 0, 1)
    ref = O.attention(q, k, v, "contract").reshape(T, A)
    got = host(o)
    e = errors(got, ref)
    say(f"  o: rel_l2 {e['rel_l2']:.2e}")
    assert e["rel_l2"] < 1e-3
    assert_bf16_close(got, ref, "o", ulps=2, floor_over_rms=1e-3, max_mismatch=2e-2)


def test_attention_single_token_returns_v():
    say("[stage] attention T=1")
    cfg = small_config("one", hidden=256, heads=2, ffn=256, text_tokens=1, images=())
    c = B.config_from(cfg)
    g = torch.Generator().manual_seed(5)
    qk = (torch.randn(1, 512, generator=g) * 4).to(torch.bfloat16).cuda()
    vt = torch.zeros(2, 128, 64, dtype=torch.bfloat16)
    vt[:, :, 0] = torch.randn(2, 128, generator=g).to(torch.bfloat16)
    vt = vt.cuda()
    o = torch.empty(1, 256, dtype=torch.bfloat16, device="cuda")
    B.h3dit_attention(c, qk, vt, o)
    assert torch.equal(o.cpu(), vt[:, :, 0].reshape(1, 256).cpu())


def _vt_from_tokens(v: torch.Tensor, Tp: int) -> torch.Tensor:
    """[T, H, 128] values -> [H, 128, Tp] in the kernel's column order."""
    T, H, _ = v.shape
    vt = torch.zeros(H, 128, Tp, dtype=v.dtype)
    t = np.arange(T)
    cols = (t & ~28) | ((t & 12) << 1) | ((t & 16) >> 2)
    vt[:, :, torch.from_numpy(cols)] = v.permute(1, 2, 0)
    return vt


@pytest.mark.parametrize("case", ["planted", "ramp"])
def test_attention_shift_rise(case):
    """Scores far above the first key tile's maximum force the rise of the
    shift (the kernel runs the key loop again with the raised shift): planted
    keys in an early, a middle and the ragged last tile for queries of
    different workgroups, or keys whose norm grows along the sequence so that
    every row's maximum lies far past its first tile (weights of the first
    pass overflow). The oracle takes the single shift ceil(max s) per row."""
    T, H = 700, 2
    say(f"[stage] attention shift rise {case} T={T} H={H}")
    g = torch.Generator().manual_seed(11)
    q = torch.randn(T, H, 128, generator=g) * 0.5
    k = torch.randn(T, H, 128, generator=g) * 0.5   # scores ~N(0, 2.8^2), base 2
    if case == "planted":
        for qi, ki in ((5, 100), (300, 650), (520, 695), (699, 64)):
            for h in range(H):
                k[ki, h] = q[qi, h] * (160.0 / float(q[qi, h].square().sum()))
    else:
        k *= (0.2 + 40.0 * torch.arange(T, dtype=torch.float32) / T).reshape(T, 1, 1)
    v = torch.randn(T, H, 128, generator=g)
    qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    Tp = B.h3dit_padded_tokens(T)
    qk = torch.cat([qb.reshape(T, H * 128), kb.reshape(T, H * 128)], dim=1).contiguous().cuda()
    vt = _vt_from_tokens(vb, Tp).cuda()
    o = torch.empty(T, H * 128, dtype=torch.bfloat16, device="cuda")
    cfg = small_config("shift", hidden=256, heads=H, ffn=256, text_tokens=T, images=())
    B.h3dit_attention(B.config_from(cfg), qk, vt, o)
    f = lambda t: t.to(torch.float64).numpy()
    s_max = max(float((f(qb)[:, h] @ f(kb)[:, h].T).max()) for h in range(H))
    first = max(float((f(qb)[:, h] @ f(kb)[:64, h].T).max()) for h in range(H))
    say(f"  max score {s_max:.1f}, first tile max {first:.1f}")
    assert s_max > first + 130, "the case must push scores far past the first tile"
    ref = O.attention(f(qb), f(kb), f(vb), "contract").reshape(T, H * 128)
    got = host(o)
    e = errors(got, ref)
    say(f"  o: rel_l2 {e['rel_l2']:.2e}")
    assert np.all(np.isfinite(got))
    assert e["rel_l2"] < 1e-3
    # Per element: two bf16 ulps of the output, plus what a one-ulp difference
    # in any weight's bf16 rounding (fp32 scores on the GPU, fp64 in the
    # oracle) moves: |dP_i| <= 2^-7 P_i, so |do| <= 2^-7 (sum P_i |v_i| / sum P
    # + |o|). Peaked rows with cancelling values need that second term.
    flip = np.empty_like(ref)
    for h in range(H):
        sc = f(qb)[:, h] @ f(kb)[:, h].T
        P = O.bf16_round(np.exp2(sc - np.ceil(sc.max(axis=1, keepdims=True))))
        flip[:, h * 128:(h + 1) * 128] = (P @ np.abs(f(vb)[:, h])) / P.sum(axis=1, keepdims=True)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 2 * 2.0 ** -7 * np.abs(ref) + 2.0 ** -7 * (flip + np.abs(ref)) + 1e-4 * rms
    excess = np.abs(got - ref) / bound
    say(f"  o: max err/bound {excess.max():.3f}, mismatch fraction {np.mean(got != ref):.2e}")
    assert excess.max() <= 1.0


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_stage_projections_and_mlp(cfg):
    inp = cached_case(cfg)
    say(f"[stage] out-proj / mlp {cfg.name} T={cfg.n_tokens}")
    ref = oracle_reference(cfg, inp)
    mv = O.split_modulation(ref["mod"], cfg.hidden)
    c = B.config_from(cfg)
    T, D, F = cfg.n_tokens, cfg.hidden, cfg.ffn
    x1 = torch.empty(T, D, dtype=torch.float32, device="cuda")
    B.h3dit_out_proj_residual(c, bf16_dev(ref["o"]), dev(inp["w_o"]), dev(inp["x"]),
                              f64_dev(mv["gate1"]), x1)
    e = errors(host(x1), ref["x1"])
    say(f"  x1: rel_l2 {e['rel_l2']:.2e} max_abs/rms {e['max_abs_over_rms']:.2e}")
    assert e["rel_l2"] < 1e-5 and e["max_abs_over_rms"] < 1e-4

    u = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    B.h3dit_mlp_up_gelu(c, bf16_dev(ref["h2"]), dev(inp["w_up"]), u)
    assert_bf16_close(host(u), ref["u"], "u", ulps=1, floor_over_rms=1e-4)

    out = torch.empty(T, D, dtype=torch.float32, device="cuda")
    B.h3dit_mlp_down_residual(c, bf16_dev(ref["u"]), dev(inp["w_down"]),
                              torch.from_numpy(ref["x1"]).to(torch.float32).cuda(),
                              f64_dev(mv["gate2"]), out)
    e = errors(host(out), ref["out"])
    say(f"  out: rel_l2 {e['rel_l2']:.2e} max_abs/rms {e['max_abs_over_rms']:.2e}")
    assert e["rel_l2"] < 1e-5 and e["max_abs_over_rms"] < 1e-4


# ------------------------------------------------------------------ whole block
def run_block(cfg, inp):
    blk = B.Block(cfg, inp)
    out = blk.forward()
    return host(out), blk


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_block_small_all_rows(cfg):
    inp = cached_case(cfg)
    say(f"[block] {cfg.name} T={cfg.n_tokens} all rows")
    got, _ = run_block(cfg, inp)
    ref = oracle_reference(cfg, inp)
    assert_block_parity(got, ref["out"], f"{cfg.name} out")
    ex = oracle_reference(cfg, inp, mode="exact")
    e = errors(got, ex["out"])
    say(f"  (info) vs exact fp64: rel_l2 {e['rel_l2']:.2e} max_abs/rms {e['max_abs_over_rms']:.2e}")


@pytest.mark.parametrize("T_text,grid", [(1, ()), (64, ()), (65, ()), (3, ((1, 1, 0),)),
                                         (0, ((8, 16, 0),))], ids=["T1", "T64", "T65", "T4", "T128"])
def test_block_edge_token_counts(T_text, grid):
    cfg = small_config("edge", hidden=256, heads=2, ffn=512, text_tokens=T_text, images=grid)
    inp = make_inputs(cfg, seed=11)
    say(f"[block] edge T={cfg.n_tokens}")
    got, _ = run_block(cfg, inp)
    assert_block_parity(got, oracle_reference(cfg, inp)["out"], f"edge T={cfg.n_tokens}")


def test_block_zero_gates_return_input_bitwise():
    cfg = MID
    inp = dict(cached_case(cfg))
    D = cfg.hidden
    w_ada = inp["w_ada"].clone()
    w_ada[2 * D:3 * D] = 0
    w_ada[5 * D:6 * D] = 0
    inp["w_ada"] = w_ada
    say("[block] zero gates")
    got, _ = run_block(cfg, inp)
    assert np.array_equal(got, inp["x"].to(torch.float64).numpy())


def test_block_deterministic():
    cfg = MID
    inp = cached_case(cfg)
    say("[block] determinism")
    blk = B.Block(cfg, inp)
    a = blk.forward().clone()
    b = blk.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attention_key_pieces_in_block():
    """The block's attention when its last, partial round of workgroups is cut
    along the keys (here 16 heads x 17 query tiles = 272 workgroups: 16 past
    the first round of 256, each cut into key-range pieces whose partial sums
    a second kernel merges, every piece with its own shift). o from the
    block's workspace against the oracle's attention of the block's own q, k,
    v on every row, and the block output against the oracle at the block bar."""
    cfg = small_config("pieces", hidden=256, heads=16, ffn=512, text_tokens=44,
                       images=((48, 89, 0),), x_dtype="bf16")
    T, A, H = cfg.n_tokens, cfg.attn_width, cfg.heads
    say(f"[block] attention key pieces T={T} H={H}")
    inp = cached_case(cfg)
    blk = B.Block(cfg, inp)
    out = host(blk.forward())
    it = blk.intermediates()
    g_qk, g_vt, g_o = host(it["qk"]), unswap_vt(host(it["vt"])), host(it["o"])
    q = g_qk[:, :A].reshape(T, H, 128)
    k = g_qk[:, A:].reshape(T, H, 128)
    v = g_vt[:, :, :T].transpose(2, 0, 1)
    ref = O.attention(q, k, v, "contract").reshape(T, A)
    e = errors(g_o, ref)
    flip = np.empty_like(ref)
    for h in range(H):
        sc = q[:, h] @ k[:, h].T
        P = O.bf16_round(np.exp2(sc - np.ceil(sc.max(axis=1, keepdims=True))))
        flip[:, h * 128:(h + 1) * 128] = (P @ np.abs(v[:, h])) / P.sum(axis=1, keepdims=True)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 2 * 2.0 ** -7 * np.abs(ref) + 2.0 ** -7 * (flip + np.abs(ref)) + 1e-4 * rms
    excess = np.abs(g_o - ref) / bound
    say(f"  o: rel_l2 {e['rel_l2']:.2e}, max err/bound {excess.max():.3f}")
    assert e["rel_l2"] < 1e-3 and excess.max() <= 1.0
    # (the pieces are head 15's query tiles 1..16, rows 256 .. T - 1 of its columns)
    assert_block_parity(out, oracle_reference(cfg, inp)["out"], "pieces out")


@pytest.mark.slow
def test_attention_shift_rise_full_length_rows():
    """The second pass at the full 4096x4096 sequence length (16,896 tokens,
    8 heads: 528 workgroups, the last partial round cut into key-range pieces
    when the split plan takes it): keys whose norm grows along the sequence,
    so every workgroup finds its rows' maxima and runs its key loop again.
    Against the oracle on 256 seeded query rows over all keys, with the
    per-element bound of the short-sequence shift tests."""
    T, H = 16896, 8
    say(f"[stage] attention shift rise full length T={T} H={H}")
    g = torch.Generator().manual_seed(12)
    q = torch.randn(T, H, 128, generator=g) * (12.0 / 128 ** 0.5)
    k = torch.randn(T, H, 128, generator=g)
    k *= (0.2 + 40.0 * torch.arange(T, dtype=torch.float32) / T).reshape(T, 1, 1)
    v = torch.randn(T, H, 128, generator=g)
    qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    del q, k, v
    Tp = B.h3dit_padded_tokens(T)
    qk = torch.cat([qb.reshape(T, H * 128), kb.reshape(T, H * 128)], dim=1).contiguous().cuda()
    vt = _vt_from_tokens(vb, Tp).cuda()
    o = torch.empty(T, H * 128, dtype=torch.bfloat16, device="cuda")
    B.h3dit_attention(B.make_config(256, H, 256, T), qk, vt, o)
    torch.cuda.synchronize()
    rows = sample_rows(T, 256, seed=1)
    f = lambda t: t.to(torch.float64).numpy()
    fq, fk, fv = f(qb[rows]), f(kb), f(vb)
    first = max(float((fq[:, h] @ fk[:64, h].T).max()) for h in range(H))
    s_max = max(float((fq[:, h] @ fk[:, h].T).max()) for h in range(H))
    say(f"  max score {s_max:.1f}, first tile max {first:.1f}")
    assert s_max > first + 130, "the case must push scores far past the first tile"
    ref = O.attention(fq, fk, fv, "contract").reshape(len(rows), H * 128)
    got = host(o)[rows]
    e = errors(got, ref)
    flip = np.empty_like(ref)
    for h in range(H):
        sc = fq[:, h] @ fk[:, h].T
        P = O.bf16_round(np.exp2(sc - np.ceil(sc.max(axis=1, keepdims=True))))
        flip[:, h * 128:(h + 1) * 128] = (P @ np.abs(fv[:, h])) / P.sum(axis=1, keepdims=True)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 2 * 2.0 ** -7 * np.abs(ref) + 2.0 ** -7 * (flip + np.abs(ref)) + 1e-4 * rms
    excess = np.abs(got - ref) / bound
    say(f"  o: rel_l2 {e['rel_l2']:.2e}, max err/bound {excess.max():.3f}")
    assert np.all(np.isfinite(got)) and e["rel_l2"] < 1e-3
    assert excess.max() <= 1.0


def test_attention_second_pass_cost_bounded():
    """Scores that rise along the sequence make every workgroup find its rows'
    maxima (a scores-only pass) and repeat the key loop: the kernel then takes
    at most 2.6x its time on ordinary scores (about 1 + 0.3 + 1 passes). Times
    are the fastest of five calls each, 4352 tokens, 16 heads."""
    T, H = 4352, 16
    say(f"[stage] attention second-pass cost T={T} H={H}")
    c = B.make_config(256, H, 256, T)
    g = torch.Generator(device="cuda").manual_seed(3)
    o = torch.empty(T, H * 128, dtype=torch.bfloat16, device="cuda")
    times = {}
    for rising in (False, True):
        q = torch.randn(T, H * 128, device="cuda", generator=g) * (12.0 / 128 ** 0.5)
        k = torch.randn(T, H * 128, device="cuda", generator=g)
        if rising:
            k *= (0.2 + 40.0 * torch.arange(T, device="cuda", dtype=torch.float32) / T).reshape(T, 1)
        qk = torch.cat([q, k], dim=1).to(torch.bfloat16).contiguous()
        vt = torch.randn(H, 128, T, device="cuda", generator=g).to(torch.bfloat16)
        B.h3dit_attention(c, qk, vt, o)
        best = float("inf")
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.h3dit_attention(c, qk, vt, o)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        assert torch.isfinite(o.float()).all()
        times[rising] = best
    ratio = times[True] / times[False]
    say(f"  ordinary {times[False]:.3f} ms, rising {times[True]:.3f} ms: {ratio:.2f}x")
    assert ratio <= 2.6

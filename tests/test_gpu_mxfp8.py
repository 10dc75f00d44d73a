"""MXFP8 linears on the GPU against the float64 oracle (oracle/mxfp8.py).

* quantisation: codes and scales bit-exact, including zero blocks, bf16
  subnormals, saturation, ties and ragged row counts;
* h3dit_linear_mxfp8: every element within the bound of the scaled E4M3
  product's fp32 accumulation, |err| <= 2^-12 * sum_k |x_k w_k| (the matrix
  cores add the 128 products of one K step with a narrower internal sum than
  IEEE fp32; the measured worst case is about 8e-5 of the sum of magnitudes);
* the block with MXFP8 linears: for small blocks, the block-output bar
  against the oracle's block with linears="mxfp8" on all rows; for the
  full-width blocks (256 seeded rows), each stage against the oracle's step
  applied to the GPU's own input for it (teacher forcing), the codes the
  producers write bit-exact, and end to end a looser bound fixed in advance:
  the GPU block's relative L2 distance from the oracle's MXFP8 block at most a
  third of the distance between the oracle's MXFP8 and bf16 blocks (quantising
  every linear must be what moves the result; a linear left in bf16 or a
  wrong composition would use up most of that gap).
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import mxfp8 as MX
from joint_attention_dit_amd import binding as B
from joint_attention_dit_amd.inputs import CONFIGS, make_inputs, sample_rows, small_config

from tests._common import assert_block_parity, cached_case, errors, oracle_inputs

pytestmark = pytest.mark.gpu

# |err| <= LINEAR_BOUND * sum_k |x_k w_k| for the MXFP8 product
LINEAR_BOUND = 2.0 ** -12


def say(msg):
    print(msg, flush=True)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def unpack_scales(buf: np.ndarray, rows: int, K: int) -> np.ndarray:
    """[rows, K / 32] scale bytes from the 1 KB block layout of include/h3dit.h:
    block (p, t) at (p * K / 128 + t) * 1024, byte (kb * 16 + r) * 16 + b for
    row 256 p + 16 b + r and K block 4 t + kb."""
    P, KT = -(-rows // 256), K // 128
    a = buf.reshape(P, KT, 4, 16, 16)          # p, t, kb, r, b
    a = a.transpose(0, 4, 3, 1, 2)             # p, b, r, t, kb
    return a.reshape(P * 256, KT * 4)


def quantize_gpu(x_bf16: torch.Tensor):
    codes, scales = B.mxfp8_quantize(x_bf16.cuda().contiguous())
    rows, K = x_bf16.shape
    return host(codes), unpack_scales(host(scales), rows, K)


def special_matrix(rows: int, K: int, seed: int) -> torch.Tensor:
    """Random bf16 rows over a wide range of magnitudes, with special blocks."""
    g = np.random.default_rng(seed)
    v = g.standard_normal((rows, K)) * np.exp2(g.integers(-40, 40, size=(rows, 1)))
    v[0, 0:32] = 0.0                                   # all-zero block
    v[0, 32:64] = -0.0                                 # negative zeros
    v[1, 0:32] = g.standard_normal(32) * 2.0 ** -130   # bf16 subnormals only
    v[1, 32:64] = g.standard_normal(32) * 2.0 ** -120  # subnormal and normal mixed
    v[1, 33] = 2.0 ** -118
    v[2, 0:32] = g.standard_normal(32) * 1e30          # large values
    # exact ties of the E4M3 grid after scaling: block max 1.0 (X = -8), so an
    # element m * 2^-8 becomes m; 1.0625 = 17 / 16 lies between 1 and 1.125
    v[3, 0:32] = 0.0
    v[3, 0] = 1.0
    v[3, 1:9] = np.array([1.0625, 1.1875, 3.25, 3.75, 0.5 * 2 ** -9, 1.5 * 2 ** -9, -1.0625,
                          -1.5 * 2 ** -9]) * 2.0 ** -8
    # saturation: the block max 1.99 * 2^k scales to 509 > 448
    v[4, 0:32] = 0.01
    v[4, 5] = -1.99 * 2.0 ** 7
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("rows,K", [(300, 384), (256, 128), (1, 256), (513, 640)])
def test_quantize_bit_exact(rows, K):
    say(f"[mxfp8] quantize rows={rows} K={K}")
    x = special_matrix(max(rows, 5), K, seed=rows + K)[:rows].contiguous()
    codes, scales = quantize_gpu(x)
    ref_c, ref_s = MX.quantize(x.to(torch.float64).numpy())
    assert np.array_equal(codes, ref_c), int(np.sum(codes != ref_c))
    assert np.array_equal(scales[:rows], ref_s), int(np.sum(scales[:rows] != ref_s))
    assert np.all(scales[rows:] == 0), "scale rows past the matrix must be 0"


def _linear_case(M, N, K, seed, exact_ints=False):
    g = np.random.default_rng(seed)
    if exact_ints:
        x = g.integers(-14, 15, size=(M, K)).astype(np.float32)
        w = g.integers(-14, 15, size=(N, K)).astype(np.float32)
    else:
        x = (g.standard_normal((M, K)) * np.exp2(g.integers(-3, 4, size=(M, K // 32)).repeat(32, 1)))
        w = g.standard_normal((N, K)) * 0.02
    return (torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16),
            torch.from_numpy(np.asarray(w, np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("M,N,K", [(300, 260, 640), (256, 256, 128), (1, 4, 256), (600, 520, 1152)])
def test_linear_mxfp8_bound(M, N, K):
    say(f"[mxfp8] linear M={M} N={N} K={K}")
    x, w = _linear_case(M, N, K, seed=M * 7 + N)
    xq, xs = B.mxfp8_quantize(x.cuda())
    wq, ws = B.mxfp8_quantize(w.cuda())
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.h3dit_linear_mxfp8(xq, xs, wq, ws, y)
    got = host(y).astype(np.float64)
    xd = MX.dequantize(*MX.quantize(x.to(torch.float64).numpy()))
    wd = MX.dequantize(*MX.quantize(w.to(torch.float64).numpy()))
    ref = xd @ wd.T
    mag = np.abs(xd) @ np.abs(wd).T
    ratio = np.abs(got - ref) / np.maximum(mag, 1e-300)
    e = errors(got, ref)
    say(f"  max |err| / sum|terms| = {ratio.max():.3e}, mean signed err / sum|terms| = "
        f"{np.mean((got - ref) / np.maximum(mag, 1e-300)):.2e}, rel_l2 {e['rel_l2']:.2e}")
    assert np.all(np.isfinite(got))
    assert ratio.max() <= LINEAR_BOUND, ratio.max()


def test_linear_mxfp8_small_integers():
    """Integers in [-14, 14] are exact in MXFP8; products and their sums (< 2^24)
    are exact in fp32 if the scaled product keeps every bit of them."""
    M, N, K = 64, 64, 512
    x, w = _linear_case(M, N, K, seed=3, exact_ints=True)
    xq, xs = B.mxfp8_quantize(x.cuda())
    wq, ws = B.mxfp8_quantize(w.cuda())
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.h3dit_linear_mxfp8(xq, xs, wq, ws, y)
    got = host(y).astype(np.float64)
    ref = x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
    mag = np.abs(x.to(torch.float64).numpy()) @ np.abs(w.to(torch.float64).numpy()).T
    say(f"[mxfp8] integer linear: {int(np.sum(got != ref))} of {got.size} differ, "
        f"max |err|/sum|terms| {np.max(np.abs(got - ref) / mag):.2e}")
    assert np.max(np.abs(got - ref) / mag) <= LINEAR_BOUND


MID = small_config("mid", hidden=512, heads=4, ffn=1536, text_tokens=35, images=((23, 29, 0),),
                   x_dtype="bf16")
MID32 = small_config("mid32", hidden=384, heads=3, ffn=1024, text_tokens=10, images=((9, 13, 0),),
                     x_dtype="fp32")


def mx_reference(cfg, inp, rows=None, linears="mxfp8"):
    x, cond, w, pos = oracle_inputs(inp)
    return O.block_forward(x, cond, w, pos, heads=cfg.heads, eps=cfg.eps, rope_base=cfg.rope_base,
                           mode="contract", rows=rows, linears=linears)


@pytest.mark.parametrize("cfg", [CONFIGS["tiny"], MID, MID32], ids=lambda c: c.name)
def test_block_mxfp8_small_all_rows(cfg):
    inp = cached_case(cfg)
    say(f"[mxfp8] block {cfg.name} T={cfg.n_tokens} all rows")
    blk = B.Block(cfg, inp, linears="mxfp8")
    got = host(blk.forward()).astype(np.float64)
    ref = mx_reference(cfg, inp)
    assert_block_parity(got, ref["out"], f"{cfg.name} mxfp8 out")
    e = errors(got, mx_reference(cfg, inp, linears="bf16")["out"])
    say(f"  (info) vs bf16-linear oracle: rel_l2 {e['rel_l2']:.2e} "
        f"max_abs/rms {e['max_abs_over_rms']:.2e}")


@pytest.mark.parametrize("T_text,grid", [(1, ()), (65, ()), (0, ((8, 16, 0),))],
                         ids=["T1", "T65", "T128"])
def test_block_mxfp8_edge_token_counts(T_text, grid):
    """Token counts below one 256-row panel, ragged against it, and exactly
    half of it, at the block bar against the oracle's MXFP8 block."""
    cfg = small_config("edge", hidden=256, heads=2, ffn=512, text_tokens=T_text, images=grid)
    inp = make_inputs(cfg, seed=11)
    say(f"[mxfp8] edge T={cfg.n_tokens}")
    blk = B.Block(cfg, inp, linears="mxfp8")
    got = host(blk.forward()).astype(np.float64)
    assert_block_parity(got, mx_reference(cfg, inp)["out"], f"mxfp8 edge T={cfg.n_tokens}")


def test_block_mxfp8_deterministic_and_weights_unchanged():
    cfg = MID
    inp = cached_case(cfg)
    blk = B.Block(cfg, inp, linears="mxfp8")
    a = blk.forward().clone()
    b = blk.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for k in B.MX_LINEARS:  # the forward never writes its weights
        c, s = B.mxfp8_quantize(blk.weights[k])
        assert torch.equal(c, blk.mx[k]) and torch.equal(s, blk.mx[k + "_scale"])


@pytest.mark.parametrize("T,H", [(1, 1), (288, 2), (700, 3)])
def test_attention_mxfp8_codes_bit_exact(T, H):
    """The attention kernel's MXFP8 epilogue (o's codes for the MXFP8 output
    projection): o bitwise equal to h3dit_attention's, codes and scales bitwise
    equal to h3dit_mxfp8_quantize of that o, including the zero scale bytes of
    the last panel's rows past T. V is scaled per dimension by 2^-20..2^20 so
    that the blocks of 32 take many scale bytes."""
    say(f"[mxfp8] attention epilogue codes T={T} H={H}")
    A = H * 128
    Tp = B.h3dit_padded_tokens(T)
    g = torch.Generator().manual_seed(1000 + T + H)
    qk = (torch.randn(T, 2 * A, generator=g) * 0.4).to(torch.bfloat16).cuda()
    dim_scale = torch.exp2(torch.arange(128, dtype=torch.float32) % 41 - 20.0)
    vt = (torch.randn(H, 128, Tp, generator=g) * dim_scale.reshape(1, 128, 1)).to(torch.bfloat16)
    vt = vt.cuda()
    cfg = B.make_config(256, H, 256, T)
    o1 = torch.empty(T, A, dtype=torch.bfloat16, device="cuda")
    B.h3dit_attention(cfg, qk, vt, o1)
    o2 = torch.empty_like(o1)
    codes = torch.empty(T, A, dtype=torch.uint8, device="cuda")
    scales = torch.full((B.h3dit_mxfp8_scale_bytes(T, A),), 77, dtype=torch.uint8, device="cuda")
    B.h3dit_attention_mxfp8(cfg, qk, vt, o2, codes, scales)
    rc, rs = B.mxfp8_quantize(o1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "o differs from h3dit_attention"
    nc = int((codes != rc).sum())
    ns = int((scales != rs).sum())
    say(f"  codes differ: {nc}, scale bytes differ: {ns} of {scales.numel()}")
    assert nc == 0 and ns == 0


def _unswap_vt(vt):
    t = np.arange(vt.shape[-1])
    return vt[..., (t & ~28) | ((t & 12) << 1) | ((t & 16) >> 2)]


def _check_linear(got, resid, gate, xd, wd, what, post=None):
    """got = resid + gate * (xd . wd^T) elementwise within the MXFP8 product's
    bound (LINEAR_BOUND * sum |terms|) plus fp32 rounding of the residual add;
    with post (GELU), got = bf16(post(xd . wd^T)) within the product bound
    carried through post (slope below 1.2) plus one bf16 rounding."""
    lin = xd @ wd.T
    mag = LINEAR_BOUND * (np.abs(xd) @ np.abs(wd).T)
    if post is None:
        ref = resid + gate * lin
        bound = np.abs(gate) * mag + 2.0 ** -22 * (np.abs(resid) + np.abs(gate * lin)) + 1e-30
    else:
        ref = post(lin)
        bound = 1.2 * mag + 2.0 ** -8 * np.abs(ref) + 1e-30
    r = np.abs(got - ref) / bound
    e = errors(got, ref)
    say(f"  {what}: max err/bound {r.max():.3f}, rel_l2 {e['rel_l2']:.2e}")
    assert np.all(np.isfinite(got)) and r.max() <= 1.0, (what, r.max())


@pytest.mark.slow
@pytest.mark.parametrize("name", ["2048", "4096", "nonsquare"])
def test_block_mxfp8_full_width_stages(name):
    """Full-width MXFP8 block, stage by stage on 256 seeded rows: each linear
    against the oracle's MXFP8 linear of the GPU's own bf16 input for it (its
    E4M3 codes are bit-exact, so only accumulation can differ). Each E4M3
    quantisation turns a one-ulp difference of its bf16 input into a whole
    E4M3 step, and four of them in a row amplify the few-ulp differences that
    fp32 accumulation order leaves upstream: end to end the GPU block and the
    oracle's MXFP8 block differ by about 2 % at 2048 x 2048 (the MXFP8 linears
    themselves move the block by about 15 % from the bf16 linears on these
    random weights), so full width is checked per stage."""
    cfg = CONFIGS[name]
    T, D, A, H, F = cfg.n_tokens, cfg.hidden, cfg.attn_width, cfg.heads, cfg.ffn
    say(f"[mxfp8] block {name} T={T} stages on 256 sampled rows")
    inp = make_inputs(cfg, seed=0)
    blk = B.Block(cfg, inp, linears="mxfp8")
    out = host(blk.forward()).astype(np.float64)
    iv = {k: v.detach().cpu() for k, v in blk.intermediates().items()}
    # h1 as the block computed it: the same normalisation kernel on the same inputs
    h1 = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    mod = blk.intermediates()["mod"]
    B.h3dit_rmsnorm_modulate(blk.cfg, blk.dev["x"], mod[0:D].contiguous(), mod[D:2 * D].contiguous(), h1)
    h1 = h1.cpu()
    del blk
    torch.cuda.empty_cache()
    f64 = lambda t: t.to(torch.float64).numpy()
    rows = sample_rows(T, 256, seed=1)
    x, cond, w, pos = oracle_inputs(inp)
    mv = O.split_modulation(O.modulation(w["w_ada"], cond), D)
    np.testing.assert_allclose(f64(iv["mod"]), O.modulation(w["w_ada"], cond), rtol=1e-11, atol=1e-12)
    deq = lambda a: MX.dequantize(*MX.quantize(a))

    # QKV + RoPE from the block's h1
    hq = deq(f64(h1)[rows])
    wqkv = deq(w["w_qkv"])
    qkv = hq @ wqkv.T
    mag = LINEAR_BOUND * (np.abs(hq) @ np.abs(wqkv).T)
    q = O.scaled_query(O.apply_rope(qkv[:, :A].reshape(-1, H, 128), pos[rows], cfg.rope_base))
    k = O.bf16_round(O.apply_rope(qkv[:, A:2 * A].reshape(-1, H, 128), pos[rows], cfg.rope_base))
    v = O.bf16_round(qkv[:, 2 * A:])
    g_qk = f64(iv["qk"])[rows]
    g_v = _unswap_vt(f64(iv["vt"]))[:, :, rows].transpose(2, 0, 1).reshape(-1, A)
    # the rotation mixes the pair (2i, 2i + 1): each output carries both
    # products' bounds (times the softmax factor for q), then one bf16 rounding
    sc = 1.4426950408889634 / np.sqrt(128.0)
    for nm, got, ref, mg, f in (("q", g_qk[:, :A], q.reshape(-1, A), mag[:, :A], sc),
                                ("k", g_qk[:, A:], k.reshape(-1, A), mag[:, A:2 * A], 1.0),
                                ("v", g_v, v, mag[:, 2 * A:], None)):
        pb = mg if f is None else f * (mg[:, 0::2] + mg[:, 1::2]).repeat(2, axis=1)
        r = np.abs(got - ref) / (pb + 2.0 ** -7 * np.abs(ref) + 1e-30)
        say(f"  {nm}: max err/bound {r.max():.3f}, mismatch {np.mean(got != ref):.2e}")
        assert r.max() <= 1.0, (nm, r.max())

    # attention over the block's q, k, v
    qk_all = f64(iv["qk"])
    v_all = _unswap_vt(f64(iv["vt"]))[:, :, :T].transpose(2, 0, 1)
    o_ref = O.attention(qk_all[rows, :A].reshape(-1, H, 128), qk_all[:, A:].reshape(T, H, 128),
                        v_all, "contract").reshape(-1, A)
    o = f64(iv["o"])[rows]
    e = errors(o, o_ref)
    say(f"  o: rel_l2 {e['rel_l2']:.2e}")
    assert e["rel_l2"] < 1e-3

    # the three remaining linears from the block's own o, h2 and u
    x1 = f64(iv["x1"])[rows]
    _check_linear(x1, x[rows], mv["gate1"], deq(o), deq(w["w_o"]), "x1 (output projection)")
    h2_ref = O.modulated_norm(x1, mv["shift2"], mv["scale2"], cfg.eps, "contract")
    h2 = f64(iv["h"])[rows]
    assert np.max(np.abs(h2 - h2_ref) / (2.0 ** -8 * np.abs(h2_ref) + 1e-30)) <= 1.0
    u = f64(iv["u"])[rows]
    _check_linear(u, None, None, deq(h2), deq(w["w_up"]), "u (MLP up + GELU)", post=O.gelu_tanh)
    # the normalisation and the GELU epilogue also write their output as MXFP8
    # codes: bit-exact against the oracle's quantisation of the same bf16 values
    for nm, bf, K in (("h2", h2, D), ("u", u, F)):
        rc, rs = MX.quantize(bf)
        gc = iv["q_" + nm].numpy()[rows]
        gs = unpack_scales(iv["q_" + nm + "_scale"].numpy(), T, K)[rows]
        say(f"  {nm} codes: {int(np.sum(gc != rc))} differ, scales: {int(np.sum(gs != rs))} differ")
        assert np.array_equal(gc, rc) and np.array_equal(gs, rs), nm
    _check_linear(out[rows], x1, mv["gate2"], deq(u), deq(w["w_down"]), "out (MLP down)")

    # end to end against the oracle's MXFP8 block (see the module notes)
    kw = dict(heads=H, eps=cfg.eps, rope_base=cfg.rope_base, rows=rows)
    r_mx = O.block_forward(x, cond, w, pos, linears="mxfp8", **kw)["out"]
    r_bf = O.block_forward(x, cond, w, pos, **kw)["out"]
    d_gpu = errors(out[rows], r_mx)["rel_l2"]
    d_eff = errors(r_bf, r_mx)["rel_l2"]
    say(f"  end to end: GPU vs MXFP8 oracle rel_l2 {d_gpu:.3e}; MXFP8 vs bf16 oracle "
        f"{d_eff:.3e} (ratio {d_gpu / d_eff:.3f}, bar 1/3)")
    assert d_gpu <= d_eff / 3


@pytest.mark.parametrize("K", [1024, 5376, 14336])
def test_linear_mxfp8_long_sums_exact(K):
    """All-ones operands: every partial sum is an integer below 2^24, exact in
    fp32, so the K / 128 accumulating products must return exactly K."""
    M = N = 256
    x = torch.ones(M, K, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(N, K, dtype=torch.bfloat16, device="cuda")
    xq, xs = B.mxfp8_quantize(x)
    wq, ws = B.mxfp8_quantize(w)
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.h3dit_linear_mxfp8(xq, xs, wq, ws, y)
    got = host(y)
    say(f"[mxfp8] all-ones K={K}: min {got.min()} max {got.max()} (exact {K})")
    assert np.all(got == K)


@pytest.mark.parametrize("K", [5376, 7168, 14336])
def test_linear_mxfp8_full_width_k(K):
    """The full-width reduction lengths on a narrow N, 4352 tokens, checked on
    128 sampled rows."""
    M, N = 4352, 512
    g = np.random.default_rng(K)
    x = torch.from_numpy((g.standard_normal((M, K)) * 1.5).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((g.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    xq, xs = B.mxfp8_quantize(x.cuda())
    wq, ws = B.mxfp8_quantize(w.cuda())
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.h3dit_linear_mxfp8(xq, xs, wq, ws, y)
    rows = sample_rows(M, 128, seed=2)
    got = host(y)[rows].astype(np.float64)
    xd = MX.dequantize(*MX.quantize(x[rows].to(torch.float64).numpy()))
    wd = MX.dequantize(*MX.quantize(w.to(torch.float64).numpy()))
    ref = xd @ wd.T
    mag = np.abs(xd) @ np.abs(wd).T
    ratio = np.abs(got - ref) / mag
    e = errors(got, ref)
    say(f"[mxfp8] K={K}: max |err|/sum|terms| {ratio.max():.3e}, rel_l2 {e['rel_l2']:.3e}, "
        f"mean signed err/|ref| {np.mean((got - ref) * np.sign(ref)) / np.mean(np.abs(ref)):.2e}")
    assert ratio.max() <= LINEAR_BOUND

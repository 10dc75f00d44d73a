"""Pins for how the oracle composes the block in contract mode and with MXFP8
linears (no GPU).

The block is the architecture diagram of the apxml.com spec page "MiniMax H3
Image" ("Architecture Diagram") with the shapes of the Hugging Face model card
"MiniMax-H3-Image" ("Model Architecture"). Contract mode rounds to bf16 at
exactly the points where the GPU stores a bf16 matrix-core operand: h1, v, the
rotated q (which also carries the softmax factor log2(e)/sqrt(128)) and k, the
attention weights P = bf16(2^(s - ceil(max s))), o = bf16(sum P v / sum P), h2
and u; everything else is float64. The MXFP8 variant (vLLM blog "H3-Image Day-0
Support", "Inference Optimizations": the DiT's linears in MXFP8) quantises both
operands of each of the four linears along K, in the OCP MX format (E4M3
elements, one power-of-two scale per 32).

Each test rebuilds the block in plain Python loops, with a scalar bf16 rounding
and a scalar MX quantiser written here from those definitions (no numpy
rounding, no call into the oracle), and requires every intermediate of
``oracle.block_forward`` to agree element by element. A missing or extra
rounding anywhere (an unrounded v, u or o, k rounded before its rotation as
well as after, one linear left unquantised) moves some element by at least a
bf16 or E4M3 step, far outside the float64 tolerance used here.
"""
import math

import numpy as np
import pytest

import oracle as O

LOG2E = math.log2(math.e)


# ------------------------------------------------------------------ scalar roundings
def bf16_scalar(x: float) -> float:
    """Round to the nearest bf16 value, ties to even (8 significant bits; the
    grid stops at 2^-133 below the smallest normal). math.frexp gives the
    binade, Python's round() rounds halves to even."""
    if x == 0.0:
        return 0.0
    _, e = math.frexp(x)
    e = max(e, -125)
    return round(x * 2.0 ** (8 - e)) * 2.0 ** (e - 8)


def e4m3_scalar(t: float) -> float:
    """Value of the OCP E4M3 number nearest to t (ties to even), saturating at
    +-448. Normal binades [2^e, 2^(e+1)) for e >= -6 carry 3 mantissa bits
    (step 2^(e-3)); below 2^-6 the subnormal step is 2^-9."""
    a = abs(t)
    if a == 0.0:
        return 0.0
    e = -6
    while a >= 2.0 ** (e + 1):       # binade by repeated doubling (no log)
        e += 1
    step = 2.0 ** (e - 3)            # for a < 2^-6 the loop leaves e = -6: step 2^-9
    q = min(round(a / step) * step, 448.0)
    return math.copysign(q, t)


def mx_dequant_row(row):
    """A row (length a multiple of 32) after MXFP8 quantisation and back: per
    block of 32, X = floor(log2(max |v|)) - 8 (the largest E4M3 binade is 2^8),
    each element e4m3(v / 2^X) * 2^X; an all-zero block stays zero."""
    out = []
    for b in range(0, len(row), 32):
        blk = row[b:b + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out.extend(0.0 for _ in blk)
            continue
        fl = 0                        # floor(log2(amax)) by stepping
        while 2.0 ** fl > amax:
            fl -= 1
        while 2.0 ** (fl + 1) <= amax:
            fl += 1
        s = 2.0 ** (fl - 8)
        out.extend(e4m3_scalar(v / s) * s for v in blk)
    return out


def test_scalar_roundings_against_fixed_values():
    """The scalar helpers themselves, against values the formats fix."""
    u = 2.0 ** -8
    assert bf16_scalar(1 + u) == 1.0 and bf16_scalar(1 + 3 * u) == 1 + 4 * u
    assert bf16_scalar(-(1 + u + 2.0 ** -30)) == -(1 + 2 * u)
    assert bf16_scalar(2.0 ** -133 * 0.75) == 2.0 ** -133
    # E4M3: 1.0625 ties to 1.0, 1.1875 to 1.25, 432 to 448, 500 saturates,
    # 2^-10 ties to 0 and 3 * 2^-10 to 2^-8, 240 exact, 17 -> 16 (step 2 at 16)
    assert [e4m3_scalar(v) for v in (1.0625, 1.1875, 432.0, 500.0, 2.0 ** -10, 3 * 2.0 ** -10,
                                      240.0, 17.0)] == [1.0, 1.25, 448.0, 448.0, 0.0, 2.0 ** -8,
                                                        240.0, 16.0]
    # MX: a block whose maximum is 1 gets scale 2^-8; 1.99 * 2^20 saturates to 448 * 2^12
    row = [0.0] * 32
    row[0], row[1] = 1.0, 0.3
    d = mx_dequant_row(row)
    assert d[0] == 1.0 and d[1] == e4m3_scalar(0.3 * 256) / 256
    row[0] = 1.99 * 2.0 ** 20
    assert mx_dequant_row(row)[0] == 448 * 2.0 ** 12


# ------------------------------------------------------------------ the scalar block
def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def _matvec(w, vec):
    return [_dot(row, vec) for row in w]


def scalar_contract_block(x, cond, w, pos, H, eps=1e-6, base=10000.0, linears="bf16"):
    """The block in contract mode, plain Python loops. linears="mxfp8" routes
    every linear's two operands through mx_dequant_row first."""
    T, D = len(x), len(x[0])
    A = H * 128
    B = bf16_scalar
    if linears == "mxfp8":
        def lin(rows, wmat):
            wq = [mx_dequant_row(list(r)) for r in wmat]
            return [_matvec(wq, mx_dequant_row(list(r))) for r in rows]
    else:
        def lin(rows, wmat):
            return [_matvec(wmat, list(r)) for r in rows]

    mod = _matvec(w["w_ada"], cond)
    sh1, sc1, g1, sh2, sc2, g2 = (mod[i * D:(i + 1) * D] for i in range(6))

    def mnorm(row, sh, sc):
        ms = sum(v * v for v in row) / len(row)
        d = math.sqrt(ms + eps)
        return [B(row[j] / d * (1 + sc[j]) + sh[j]) for j in range(len(row))]

    def rope(vec, p):
        out = list(vec)
        for h in range(H):
            for a in range(2):
                for i in range(32):
                    d = h * 128 + 64 * a + 2 * i
                    ang = p[a] * base ** (-2.0 * i / 64)
                    c, s = math.cos(ang), math.sin(ang)
                    out[d] = vec[d] * c - vec[d + 1] * s
                    out[d + 1] = vec[d] * s + vec[d + 1] * c
        return out

    h1 = [mnorm(list(x[t]), sh1, sc1) for t in range(T)]
    wq, wk, wv = w["w_qkv"][:A], w["w_qkv"][A:2 * A], w["w_qkv"][2 * A:]
    pq, pk, pv = lin(h1, wq), lin(h1, wk), lin(h1, wv)
    c = LOG2E / math.sqrt(128)
    q = [[B(z * c) for z in rope(pq[t], pos[t])] for t in range(T)]
    k = [[B(z) for z in rope(pk[t], pos[t])] for t in range(T)]
    v = [[B(z) for z in pv[t]] for t in range(T)]

    o = [[0.0] * A for _ in range(T)]
    for h in range(H):
        sl = slice(h * 128, (h + 1) * 128)
        for i in range(T):
            s = [_dot(q[i][sl], k[j][sl]) for j in range(T)]
            m = math.ceil(max(s))
            p = [B(2.0 ** (z - m)) for z in s]
            zsum = sum(p)
            for d in range(128):
                o[i][h * 128 + d] = B(sum(p[j] * v[j][h * 128 + d] for j in range(T)) / zsum)
    proj = lin(o, w["w_o"])
    x1 = [[x[t][n] + g1[n] * proj[t][n] for n in range(D)] for t in range(T)]
    h2 = [mnorm(x1[t], sh2, sc2) for t in range(T)]
    up = lin(h2, w["w_up"])
    u = []
    for t in range(T):
        u.append([B(0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3))))
                  for z in up[t]])
    down = lin(u, w["w_down"])
    out = [[x1[t][n] + g2[n] * down[t][n] for n in range(D)] for t in range(T)]
    return dict(h1=h1, q=q, k=k, v=v, o=o, x1=x1, h2=h2, u=u, out=out)


def _inputs(T=6, D=8, H=2, Fd=16, seed=7):
    """bf16-valued weights (as the GPU path takes them), float64 activations,
    RoPE positions with text at (0, 0) and a 2x2 image grid."""
    r = np.random.default_rng(seed)
    A = H * 128
    bf = np.vectorize(bf16_scalar)
    w = dict(w_ada=bf(r.standard_normal((6 * D, D)) * 0.3),
             w_qkv=bf(r.standard_normal((3 * A, D)) * 0.3),
             w_o=bf(r.standard_normal((D, A)) * 0.05),
             w_up=bf(r.standard_normal((Fd, D)) * 0.3),
             w_down=bf(r.standard_normal((D, Fd)) * 0.3))
    x = r.standard_normal((T, D))
    cond = r.standard_normal(D)
    pos = np.array([[0, 0]] * 2 + [[a, b] for a in range(2) for b in range(2)])[:T]
    return x, cond, w, pos, H


KEYS = ("h1", "q", "k", "v", "o", "x1", "h2", "u", "out")


def _compare(got, ref):
    for key in KEYS:
        a = np.asarray(got[key], dtype=np.float64).reshape(np.asarray(ref[key]).shape)
        b = np.asarray(ref[key], dtype=np.float64)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13 * max(1.0, np.abs(b).max()),
                                   err_msg=key)


def test_contract_block_matches_scalar_rounding_sites():
    x, cond, w, pos, H = _inputs()
    ref = scalar_contract_block(x.tolist(), cond.tolist(), {k: v.tolist() for k, v in w.items()},
                                pos.tolist(), H)
    got = O.block_forward(x, cond, w, pos, heads=H, mode="contract")
    _compare(got, ref)
    # the roundings are live on these inputs: each rounded tensor differs from
    # its unrounded value somewhere (a pin that no rounding could fail is vacuous)
    ex = O.block_forward(x, cond, w, pos, heads=H, mode="exact")
    for key in ("h1", "v", "o", "h2", "u", "out"):
        assert not np.array_equal(got[key], ex[key]), key


def test_contract_block_scalar_second_case():
    # more tokens than the first case, a wider image grid and larger activations
    x, cond, w, pos, H = _inputs(T=9, seed=11)
    pos = np.array([[0, 0], [0, 0], [0, 0], [0, 1], [0, 2], [1, 0], [1, 1], [1, 2], [2, 0]])
    x = x * 3.0
    ref = scalar_contract_block(x.tolist(), cond.tolist(), {k: v.tolist() for k, v in w.items()},
                                pos.tolist(), H)
    got = O.block_forward(x, cond, w, pos, heads=H, mode="contract")
    _compare(got, ref)


@pytest.mark.parametrize("seed", [5, 6])
def test_mxfp8_block_matches_scalar_composition(seed):
    # every linear's K must be a multiple of 32: D = 32, A = 256, F = 64
    x, cond, w, pos, H = _inputs(T=5, D=32, Fd=64, seed=seed)
    ref = scalar_contract_block(x.tolist(), cond.tolist(), {k: v.tolist() for k, v in w.items()},
                                pos.tolist(), H, linears="mxfp8")
    got = O.block_forward(x, cond, w, pos, heads=H, mode="contract", linears="mxfp8")
    _compare(got, ref)
    # quantisation is live in every linear: the bf16-linear block differs in each
    # linear's output-dependent tensor
    plain = O.block_forward(x, cond, w, pos, heads=H, mode="contract")
    for key in ("k", "v", "x1", "u", "out"):
        assert not np.allclose(got[key], plain[key], rtol=1e-6, atol=0), key


# ------------------------------------------------------------------ the DiT around the blocks
def scalar_dit(latent, text, cond, w_patch, w_ada_final, w_final, blocks, pos, H, p, eps=1e-6):
    """One DiT evaluation in plain loops: patch rows (feature c p p + dy p + dx of
    token gy gw + gx is latent[c][gy p + dy][gx p + dx]), fp64 patch embedding
    after the text rows, the blocks in order, the modulated final norm and
    projection of the image rows, and the rows put back into latent order."""
    C, Hh, Ww = len(latent), len(latent[0]), len(latent[0][0])
    gh, gw = Hh // p, Ww // p
    patches = []
    for gy in range(gh):
        for gx in range(gw):
            patches.append([latent[c][gy * p + dy][gx * p + dx]
                            for c in range(C) for dy in range(p) for dx in range(p)])
    x = [list(r) for r in text] + [_matvec(w_patch, r) for r in patches]
    for w in blocks:
        x = scalar_contract_block(x, cond, w, pos, H, eps=eps)["out"]
    D = len(x[0])
    mod = _matvec(w_ada_final, cond)
    v = [[[0.0] * Ww for _ in range(Hh)] for _ in range(C)]
    for i, row in enumerate(x[len(text):]):
        d = math.sqrt(sum(z * z for z in row) / D + eps)
        hrow = [row[j] / d * (1 + mod[D + j]) + mod[j] for j in range(D)]
        y = _matvec(w_final, hrow)
        gy, gx = divmod(i, gw)
        for c in range(C):
            for dy in range(p):
                for dx in range(p):
                    v[c][gy * p + dy][gx * p + dx] = y[c * p * p + dy * p + dx]
    return v


def test_dit_forward_and_euler_match_scalar_composition():
    """Two blocks with different weights (so their order matters), patch size 2
    over a 2 x 3 grid of latent patches, two text tokens, two Euler steps with
    different conditioning vectors, contract mode throughout."""
    r = np.random.default_rng(21)
    D, H, Fd, C, p, gh, gw, ntext = 8, 2, 16, 2, 2, 2, 3, 2
    blocks = []
    for b in range(2):
        _, _, w, _, _ = _inputs(T=1, D=D, H=H, Fd=Fd, seed=30 + b)
        blocks.append(w)
    latent = r.standard_normal((C, gh * p, gw * p))
    text = r.standard_normal((ntext, D))
    conds = [r.standard_normal(D), r.standard_normal(D)]
    w_patch = r.standard_normal((D, C * p * p)) * 0.5
    w_ada_final = np.vectorize(bf16_scalar)(r.standard_normal((2 * D, D)) * 0.3)
    w_final = r.standard_normal((C * p * p, D)) * 0.5
    pos = np.array([[0, 0]] * ntext + [[a, b] for a in range(gh) for b in range(gw)])
    kw = dict(text=text, w_patch=w_patch, w_ada_final=w_ada_final, w_final=w_final,
              blocks=blocks, pos=pos, heads=H, patch=p)
    lists = lambda a: np.asarray(a).tolist()
    sblocks = [{k: lists(v) for k, v in w.items()} for w in blocks]

    got = O.dit_forward(latent, cond=conds[0], mode="contract", **kw)
    ref = scalar_dit(lists(latent), lists(text), lists(conds[0]), lists(w_patch),
                     lists(w_ada_final), lists(w_final), sblocks, lists(pos), H, p)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-13)
    # block order is part of the definition: the reversed stack differs
    rev = O.dit_forward(latent, cond=conds[0], mode="contract", **dict(kw, blocks=blocks[::-1]))
    assert not np.allclose(rev, got, rtol=1e-6, atol=0)

    dt = 1.0 / 6
    lat = lists(latent)
    for cnd in conds:
        vv = scalar_dit(lat, lists(text), lists(cnd), lists(w_patch), lists(w_ada_final),
                        lists(w_final), sblocks, lists(pos), H, p)
        lat = [[[lat[c][y][x] + dt * vv[c][y][x] for x in range(len(lat[0][0]))]
                for y in range(len(lat[0]))] for c in range(len(lat))]
    got2 = O.euler_sample(latent, conds, dt, mode="contract", **kw)
    np.testing.assert_allclose(got2, np.array(lat), rtol=1e-12, atol=1e-13)

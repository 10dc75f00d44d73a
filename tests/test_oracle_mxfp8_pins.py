"""Pins for the MXFP8 oracle (oracle/mxfp8.py) against values fixed by the OCP
FP8 / MX definitions and by arithmetic, not by the oracle's own formulas."""
import numpy as np
import pytest

from oracle import mxfp8 as X


def test_e4m3_table_points():
    # values of the OCP E4M3 table: zero, smallest subnormal, largest subnormal,
    # smallest normal, one, 1.5, two, the largest finite value, NaN, negative max
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x78: 256.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    got = X.decode_e4m3(np.array(list(known), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(known.values())))
    assert np.isnan(X.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_finite_codes_increase_and_round_trip():
    pos = X.decode_e4m3(np.arange(0, 127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                     # 127 distinct increasing magnitudes
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(X.encode_e4m3(X.decode_e4m3(codes)), codes)


def test_e4m3_ties_to_even_and_saturation():
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A: midpoints go to the even code
    assert X.encode_e4m3(1.0625) == 0x38 and X.encode_e4m3(1.1875) == 0x3A
    assert X.encode_e4m3(1.0624) == 0x38 and X.encode_e4m3(1.0626) == 0x39
    # subnormal grid 2**-9: half of the smallest subnormal ties to zero, 1.5 steps to 2 steps
    assert X.encode_e4m3(2.0 ** -10) == 0x00 and X.encode_e4m3(3 * 2.0 ** -10) == 0x02
    assert X.encode_e4m3(-2.0 ** -11) == 0x80               # sign kept when rounding to zero
    for v in (448.0, 460.0, 480.0, 1e6):
        assert X.encode_e4m3(v) == 0x7E and X.encode_e4m3(-v) == 0xFE
    # spacing near the top: 416 = 1.625 * 256, 448; 432 is the midpoint -> even code (448 = ...110)
    assert X.decode_e4m3(X.encode_e4m3(432.0)) == 448.0


def test_mx_scale_selection():
    # largest magnitude 1.0 -> X = 0 - 8 = -8 (byte 119); 1.0 scales to 256, exactly E4M3 0x78
    v = np.zeros(32)
    v[3] = 1.0
    v[7] = -0.5
    q, s = X.quantize(v[None, :])
    assert s[0, 0] == 127 - 8 and q[0, 3] == 0x78 and X.decode_e4m3(q[0, 7]) == -128.0
    # largest magnitude 1.75 * 2**20 -> X = 20 - 8 = 12; it scales to 448 exactly
    v[3] = 1.75 * 2.0 ** 20
    q, s = X.quantize(v[None, :])
    assert s[0, 0] == 127 + 12 and q[0, 3] == 0x7E
    # 1.99 * 2**20 scales to 509.4 and saturates to 448 (the MX clamp)
    v[3] = 1.99 * 2.0 ** 20
    q, s = X.quantize(v[None, :])
    assert q[0, 3] == 0x7E and X.dequantize(q, s)[0, 3] == 448 * 2.0 ** 12
    # a zero block takes the smallest scale and all-zero elements
    q, s = X.quantize(np.zeros((2, 64)))
    assert np.all(s == 0) and np.all(q == 0)


def test_mx_quantisation_error_bound():
    """Each element is within half an E4M3 step of its scaled value, unless it saturated."""
    g = np.random.default_rng(0)
    v = g.standard_normal((64, 256)) * np.exp2(g.integers(-20, 20, size=(64, 1)))
    q, s = X.quantize(v)
    d = X.dequantize(q, s)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    t = np.abs(v) / scale                                  # magnitude in E4M3 units
    _, e = np.frexp(np.maximum(t, 2.0 ** -6))
    half_step = np.exp2(e - 1 - 3) / 2 * scale             # half the spacing of the binade
    sat = t > 448
    assert np.all(np.abs(d - v)[~sat] <= half_step[~sat])
    assert np.all(np.abs(d[sat]) == 448 * scale[sat])
    assert np.mean(sat) < 0.01


def test_mx_linear_matches_loops_and_exact_cases():
    g = np.random.default_rng(1)
    x = g.standard_normal((3, 64))
    w = g.standard_normal((5, 64))
    y = X.linear(x, w)
    xd = X.dequantize(*X.quantize(x))
    wd = X.dequantize(*X.quantize(w))
    for i in range(3):
        for j in range(5):
            assert y[i, j] == pytest.approx(sum(xd[i, k] * wd[j, k] for k in range(64)), rel=1e-13)
    # integers up to 14 have at most 4 significant bits and scale to at most 448
    # (14 * 2**5): they are stored exactly, so the product is the exact one
    xi = g.integers(-14, 15, size=(4, 96)).astype(np.float64)
    wi = g.integers(-14, 15, size=(6, 96)).astype(np.float64)
    assert np.array_equal(X.linear(xi, wi), xi @ wi.T)
    # 15 scales to 480 and saturates: the pin above is not vacuous
    v = np.full((1, 32), 15.0)
    assert X.dequantize(*X.quantize(v))[0, 0] == 14.0


def test_block_with_mxfp8_linears():
    """The MXFP8 block is the contract block with each linear replaced by the
    quantised product: equal to it when every operand is exactly representable,
    and close to it (about E4M3's 2**-4 relative step, averaged) otherwise."""
    import oracle as O
    from joint_attention_dit_amd.inputs import CONFIGS, make_inputs
    from tests._common import oracle_inputs, errors
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, seed=0)
    x, cond, w, pos = oracle_inputs(inp)
    kw = dict(heads=cfg.heads, eps=cfg.eps, rope_base=cfg.rope_base, rows=np.arange(0, 288, 7))
    ref = O.block_forward(x, cond, w, pos, **kw)
    q8 = O.block_forward(x, cond, w, pos, linears="mxfp8", **kw)
    e = errors(q8["out"], ref["out"])
    assert 1e-4 < e["rel_l2"] < 5e-2, e
    # weights whose rows are small integers (exact in MXFP8): only the activations move
    wi = dict(w)
    g = np.random.default_rng(3)
    for k in ("w_qkv", "w_o", "w_up", "w_down"):
        wi[k] = g.integers(-3, 4, size=w[k].shape).astype(np.float64) / 64
    a = O.block_forward(x, cond, wi, pos, **kw)
    b = O.block_forward(x, cond, wi, pos, linears="mxfp8", **kw)
    assert not np.array_equal(a["out"], b["out"])          # the activations are quantised
    assert np.array_equal(X.dequantize(*X.quantize(wi["w_up"])), wi["w_up"])  # weights exact

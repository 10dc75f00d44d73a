"""MXFP8 quantisation and linears, float64 CPU oracle.

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library. Only
the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the library never calls it and has no CPU fallback.

The vLLM blog ("H3-Image Day-0 Support", section Inference Optimizations)
runs the DiT's linears in MXFP8; the pages do not define the format. This
module follows the public OCP definitions of it:

  * FP8 E4M3 elements (OCP 8-bit floating point): 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    m/8 * 2**-6; there are no infinities; S.1111.111 is NaN, so the largest
    finite magnitude is S.1111.110 = 1.75 * 2**8 = 448.
  * MX blocks (OCP Microscaling): 32 consecutive elements along the reduction
    dimension share one E8M0 scale 2**X, X in [-127, 127], stored as the byte
    X + 127 (255 would be NaN and is never produced). For a block with
    largest magnitude a > 0, X = floor(log2(a)) - 8, where 8 is the largest
    exponent of E4M3; each element is stored as e4m3(v / 2**X).

Readings where the definitions leave a choice: the
element conversion rounds to nearest with ties to even and saturates to
+-448 (a block's largest element can exceed 448 after scaling by at most a
factor 512/448); a block of zeros takes X = -127; a negative value that
rounds to zero keeps its sign (byte 0x80); the inputs are the bf16 tensors
of the bf16 path (h1, o, h2, u and the bf16 weights), so quantisation is
the only difference between the two paths.
"""
import numpy as np

BLOCK = 32          # elements per shared scale
E4M3_MAX = 448.0    # largest finite E4M3 magnitude
E4M3_EMAX = 8       # exponent of the largest E4M3 binade
SCALE_BIAS = 127    # E8M0 stores X + 127


def _e4m3_magnitudes() -> np.ndarray:
    """Magnitude of every 7-bit code 0..127 (code 127 is NaN)."""
    out = np.empty(128)
    for c in range(128):
        e, m = c >> 3, c & 7
        if c == 127:
            out[c] = np.nan
        elif e == 0:
            out[c] = m / 8.0 * 2.0 ** -6
        else:
            out[c] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_MAG = _e4m3_magnitudes()
_FINITE = _MAG[:127]          # codes 0..126, strictly increasing


def decode_e4m3(codes) -> np.ndarray:
    """Bytes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = _MAG[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def encode_e4m3(x) -> np.ndarray:
    """float64 -> E4M3 bytes: round to nearest, ties to even, saturate to +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    i = np.clip(np.searchsorted(_FINITE, a), 1, 126)   # _FINITE[i-1] <= a <= _FINITE[i] (inside)
    lo, hi = _FINITE[i - 1], _FINITE[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((i & 1) == 0))
    code = np.where(pick_hi, i, i - 1)
    code = np.where(a >= E4M3_MAX, 126, code)              # saturation
    code = np.where(a <= 0.0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def block_scale_exponent(a) -> np.ndarray:
    """X = floor(log2(a)) - 8 for a block maximum a > 0, -127 for a == 0, clamped."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                  # a = f * 2**e, f in [0.5, 1)  ->  floor(log2 a) = e - 1
    x = np.where(a > 0, e - 1 - E4M3_EMAX, -SCALE_BIAS)
    return np.clip(x, -SCALE_BIAS, SCALE_BIAS).astype(np.int64)


def quantize(v: np.ndarray):
    """MXFP8 along the last axis (length a multiple of 32).

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K / 32])."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % BLOCK == 0, K
    blocks = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    X = block_scale_exponent(np.max(np.abs(blocks), axis=-1))
    codes = encode_e4m3(blocks * np.exp2(-X.astype(np.float64))[..., None])
    return codes.reshape(v.shape), (X + SCALE_BIAS).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of quantize up to rounding: e4m3 value * 2**(scale byte - 127)."""
    K = codes.shape[-1]
    vals = decode_e4m3(codes).reshape(codes.shape[:-1] + (K // BLOCK, BLOCK))
    f = np.exp2(np.asarray(scales, dtype=np.float64) - SCALE_BIAS)
    return (vals * f[..., None]).reshape(codes.shape)


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x . w^T with both operands quantised to MXFP8 along K (float64 product)."""
    xq, xs = quantize(x)
    wq, ws = quantize(w)
    return dequantize(xq, xs) @ dequantize(wq, ws).T

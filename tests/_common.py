"""Shared helpers of the test-suite: GPU availability, seeded cases, error metrics."""
from __future__ import annotations

import functools
from typing import Dict

import numpy as np
import pytest
import torch

from joint_attention_dit_amd.inputs import BlockConfig, make_inputs, to_numpy_f64

import oracle as O

WEIGHTS = ("w_ada", "w_qkv", "w_o", "w_up", "w_down")

# block-output parity bar: max |err| <= 2e-2 * RMS(out) and rel L2 <= 5e-3
MAX_ABS_OVER_RMS = 2e-2
REL_L2 = 5e-3


def gpu_available() -> bool:
    return torch.cuda.is_available()


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")


def oracle_inputs(inp: Dict[str, torch.Tensor]):
    """float64 numpy views of the seeded inputs (exact widening)."""
    w = {k: to_numpy_f64(inp[k]) for k in WEIGHTS}
    return to_numpy_f64(inp["x"]), to_numpy_f64(inp["cond"]), w, inp["positions"].numpy()


@functools.lru_cache(maxsize=4)
def cached_case(cfg: BlockConfig, seed: int = 0):
    return make_inputs(cfg, seed=seed)


def errors(got: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    rms = float(np.sqrt(np.mean(ref * ref)))
    return {
        "rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)),
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rms": rms,
        "max_abs_over_rms": float(np.max(np.abs(d)) / rms) if d.size and rms > 0 else 0.0,
    }


def assert_block_parity(got: np.ndarray, ref: np.ndarray, what: str = "out") -> Dict[str, float]:
    e = errors(got, ref)
    print(f"[parity] {what}: rel_l2={e['rel_l2']:.3e} max_abs/rms={e['max_abs_over_rms']:.3e} "
          f"rms={e['rms']:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e["rel_l2"] <= REL_L2, f"{what}: rel L2 {e['rel_l2']:.3e} > {REL_L2}"
    assert e["max_abs_over_rms"] <= MAX_ABS_OVER_RMS, \
        f"{what}: max abs / rms {e['max_abs_over_rms']:.3e} > {MAX_ABS_OVER_RMS}"
    return e


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between two arrays of bf16 values."""
    ia = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).view(torch.int32).numpy() >> 16
    ib = torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).view(torch.int32).numpy() >> 16
    # map sign-magnitude to a monotone integer line
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia.astype(np.int64) - ib.astype(np.int64))


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str, ulps: float = 1.0,
                      floor_over_rms: float = 1e-4, max_mismatch: float = 1e-2) -> None:
    """bf16 results against the oracle's rounded values.

    Element bound: |got - ref| <= ulps * 2^-7 * |ref| + floor_over_rms * RMS(ref)
    (2^-7 |ref| is at least one bf16 ulp at |ref|; the floor covers values that
    are tiny because of cancellation, where fp32 accumulation order decides
    the low bits). At most max_mismatch of the elements may differ at all.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = ulps * 2.0 ** -7 * np.abs(ref) + floor_over_rms * rms
    excess = np.abs(got - ref) / bound
    frac = float(np.mean(got != ref))
    print(f"  {what}: max err/bound {excess.max():.3f}, mismatch fraction {frac:.2e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert excess.max() <= 1.0, f"{what}: error exceeds bound ({excess.max():.3f}x)"
    assert frac <= max_mismatch, f"{what}: mismatch fraction {frac:.2e} > {max_mismatch}"


def oracle_reference(cfg: BlockConfig, inp, rows=None, mode: str = "contract"):
    x, cond, w, pos = oracle_inputs(inp)
    return O.block_forward(x, cond, w, pos, heads=cfg.heads, eps=cfg.eps,
                           rope_base=cfg.rope_base, mode=mode, rows=rows)

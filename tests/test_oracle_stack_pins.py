"""CPU pins of the DiT-stack part of the oracle (patchify, final layer, DiT
evaluation, Euler steps) against definitions written out element by element,
invariants and special cases (model card, "Model Architecture": latent patches
are the image tokens)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(7)


def test_patchify_matches_elementwise_definition():
    C, p, gh, gw = 3, 2, 3, 4
    z = RNG.standard_normal((C, gh * p, gw * p))
    got = O.patchify(z, p)
    assert got.shape == (gh * gw, C * p * p)
    for gy in range(gh):
        for gx in range(gw):
            t = gy * gw + gx
            for c in range(C):
                for dy in range(p):
                    for dx in range(p):
                        assert got[t, c * p * p + dy * p + dx] == z[c, gy * p + dy, gx * p + dx]


def test_unpatchify_inverts_patchify_both_ways():
    for C, p, gh, gw in ((4, 2, 4, 4), (24, 2, 3, 5), (2, 3, 2, 2)):
        z = RNG.standard_normal((C, gh * p, gw * p))
        np.testing.assert_array_equal(O.unpatchify(O.patchify(z, p), C, p, gh, gw), z)
        rows = RNG.standard_normal((gh * gw, C * p * p))
        np.testing.assert_array_equal(O.patchify(O.unpatchify(rows, C, p, gh, gw), p), rows)


def test_final_layer_matches_scalar_loops():
    n, D, P = 3, 8, 5
    x = RNG.standard_normal((n, D))
    cond = RNG.standard_normal(D)
    wa = RNG.standard_normal((2 * D, D)) * 0.3
    wf = RNG.standard_normal((P, D))
    eps = 1e-6
    got = O.final_layer(x, cond, wa, wf, eps)
    mod = [sum(wa[r, k] * cond[k] for k in range(D)) for r in range(2 * D)]
    for i in range(n):
        r = 1.0 / math.sqrt(sum(v * v for v in x[i]) / D + eps)
        h = [x[i, d] * r * (1.0 + mod[D + d]) + mod[d] for d in range(D)]
        for j in range(P):
            assert got[i, j] == pytest.approx(sum(h[d] * wf[j, d] for d in range(D)), rel=1e-12,
                                              abs=1e-12)


def test_final_layer_special_cases():
    n, D, P = 4, 16, 6
    x = RNG.standard_normal((n, D)) * 5
    wf = RNG.standard_normal((P, D))
    cond = RNG.standard_normal(D)
    # no modulation: the projection of the plain RMS-normalised rows (RMS
    # sqrt(ms / (ms + eps)))
    got = O.final_layer(x, cond, np.zeros((2 * D, D)), wf)
    h = O.rms_normalize(x, 1e-6)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(h * h, axis=1)), np.sqrt(ms / (ms + 1e-6)),
                               rtol=1e-12)
    np.testing.assert_allclose(got, h @ wf.T, rtol=1e-13, atol=1e-13)
    # with eps = 0, scaling a row leaves its output unchanged (RMSNorm is scale-invariant)
    z = np.zeros((2 * D, D))
    np.testing.assert_allclose(O.final_layer(3.0 * x, cond, z, wf, eps=0.0),
                               O.final_layer(x, cond, z, wf, eps=0.0), rtol=1e-12, atol=1e-12)


def _tiny_stack(n_blocks=2, zero_gates=False, seed=3):
    rng = np.random.default_rng(seed)
    D, H, F, C, p, gh, gw, text = 256, 2, 512, 4, 2, 3, 3, 4
    A = 128 * H
    blocks = []
    for _ in range(n_blocks):
        w = {"w_ada": O.bf16_round(rng.standard_normal((6 * D, D)) * 0.02),
             "w_qkv": O.bf16_round(rng.standard_normal((3 * A, D)) * 0.02),
             "w_o": O.bf16_round(rng.standard_normal((D, A)) * 0.02),
             "w_up": O.bf16_round(rng.standard_normal((F, D)) * 0.02),
             "w_down": O.bf16_round(rng.standard_normal((D, F)) * 0.02)}
        if zero_gates:
            w["w_ada"][2 * D:3 * D] = 0.0   # gate1
            w["w_ada"][5 * D:6 * D] = 0.0   # gate2
        blocks.append(w)
    pos = np.concatenate([np.zeros((text, 2), np.int64),
                          np.stack(np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij"),
                                   -1).reshape(-1, 2)])
    kw = dict(text=rng.standard_normal((text, D)), w_patch=rng.standard_normal((D, C * p * p)) * 0.02,
              w_ada_final=O.bf16_round(rng.standard_normal((2 * D, D)) * 0.02),
              w_final=rng.standard_normal((C * p * p, D)) * 0.02, blocks=blocks, pos=pos, heads=H,
              patch=p)
    latent = rng.standard_normal((C, gh * p, gw * p))
    cond = rng.standard_normal(D)
    return latent, cond, kw


@pytest.mark.parametrize("mode", ["exact", "contract"])
def test_dit_with_identity_blocks_is_embed_then_final(mode):
    """Zero gates make every block return its input exactly, so the DiT reduces
    to the final layer of the patch embedding (text tokens then play no part)."""
    latent, cond, kw = _tiny_stack(n_blocks=2, zero_gates=True)
    got = O.dit_forward(latent, cond=cond, mode=mode, **kw)
    C, H, W = latent.shape
    emb = O.patchify(latent, kw["patch"]) @ kw["w_patch"].T
    ref = O.unpatchify(O.final_layer(emb, cond, kw["w_ada_final"], kw["w_final"]), C, kw["patch"],
                       H // kw["patch"], W // kw["patch"])
    np.testing.assert_array_equal(got, ref)
    kw2 = dict(kw, text=kw["text"] * 7.0 + 1.0)
    np.testing.assert_array_equal(O.dit_forward(latent, cond=cond, mode=mode, **kw2), ref)


def test_dit_zero_blocks_equals_identity_blocks():
    latent, cond, kw = _tiny_stack(n_blocks=2, zero_gates=True)
    a = O.dit_forward(latent, cond=cond, **kw)
    b = O.dit_forward(latent, cond=cond, **dict(kw, blocks=[]))
    np.testing.assert_array_equal(a, b)


def test_dit_output_is_linear_in_the_final_projection():
    latent, cond, kw = _tiny_stack(n_blocks=1)
    a = O.dit_forward(latent, cond=cond, mode="exact", **kw)
    b = O.dit_forward(latent, cond=cond, mode="exact", **dict(kw, w_final=2.5 * kw["w_final"]))
    np.testing.assert_allclose(b, 2.5 * a, rtol=1e-12, atol=1e-12)


def test_dit_contract_close_to_exact():
    latent, cond, kw = _tiny_stack(n_blocks=2)
    a = O.dit_forward(latent, cond=cond, mode="exact", **kw)
    b = O.dit_forward(latent, cond=cond, mode="contract", **kw)
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert 0 < rel < 2e-2


def test_euler_steps():
    latent, cond, kw = _tiny_stack(n_blocks=1)
    # zero final projection: v = 0, the latent does not move
    kw0 = dict(kw, w_final=np.zeros_like(kw["w_final"]))
    np.testing.assert_array_equal(O.euler_sample(latent, [cond, cond], 0.5, **kw0), latent)
    # one step is latent + dt v
    v = O.dit_forward(latent, cond=cond, **kw)
    np.testing.assert_allclose(O.euler_sample(latent, [cond], 1.0 / 6, **kw), latent + v / 6,
                               rtol=0, atol=1e-15)

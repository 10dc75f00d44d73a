"""One GPU's attention share under Ulysses sequence parallelism (vLLM blog
"H3-Image Day-0 Support", "Inference Optimizations": the DiT runs
sequence-parallel over 4 GPUs; serving recipe "MiniMax-H3-Image", deployment
profiles: SP4 is the default). With G GPUs, an all-to-all hands each GPU H / G
heads of q, k and v over all T tokens; its attention is then h3dit_attention
with H / G heads at the full sequence length.

Here, on the 4096x4096 block (T = 16,896): the block's own rotated q, k and
transposed v (from its workspace) for heads 0 .. H/G - 1 (G = 4: 14 heads,
G = 8: 7 heads) go through h3dit_attention with H / G heads; the result must be
bitwise the block's o for those heads (heads are independent), and within the
attention bound of the oracle's contract-mode attention on 256 sampled query
rows (seed 1) against all keys. The per-token kernels of a share are the
full-width blocks share4 / share8 in test_gpu_wide_blocks.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
from joint_attention_dit_amd import binding as B
from joint_attention_dit_amd.inputs import CONFIGS, make_inputs, sample_rows

from tests._common import errors

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def block4096():
    cfg = CONFIGS["4096"]
    say(f"[ulysses] 4096 block T={cfg.n_tokens}: forward for q, k, v and o")
    blk = B.Block(cfg, make_inputs(cfg, seed=0))
    blk.forward()
    torch.cuda.synchronize()
    it = blk.intermediates()
    keep = {k: it[k].clone() for k in ("qk", "vt", "o")}
    del blk, it
    torch.cuda.empty_cache()
    return cfg, keep


def unswap_vt(vt):
    t = np.arange(vt.shape[-1])
    src = (t & ~28) | ((t & 12) << 1) | ((t & 16) >> 2)
    return vt[..., src]


@pytest.mark.parametrize("G", [4, 8])
def test_ulysses_share_attention(block4096, G):
    cfg, t = block4096
    T, H, A = cfg.n_tokens, cfg.heads, cfg.attn_width
    Hs = H // G
    As = Hs * 128
    say(f"[ulysses] G={G}: attention of {Hs} heads over T={T}")
    qk_s = torch.cat([t["qk"][:, :As], t["qk"][:, A:A + As]], dim=1).contiguous()
    vt_s = t["vt"][:Hs].contiguous()
    o_s = torch.empty(T, As, dtype=torch.bfloat16, device="cuda")
    B.h3dit_attention(B.make_config(cfg.hidden, Hs, cfg.ffn, T), qk_s, vt_s, o_s)
    torch.cuda.synchronize()
    assert torch.equal(o_s, t["o"][:, :As]), "share attention differs from the block's heads"

    rows = sample_rows(T, 256, seed=1)
    f = lambda x: x.detach().cpu().to(torch.float64).numpy()
    q = f(qk_s[:, :As]).reshape(T, Hs, 128)
    k = f(qk_s[:, As:]).reshape(T, Hs, 128)
    v = unswap_vt(f(vt_s))[:, :, :T].transpose(2, 0, 1)
    ref = O.attention(q[rows], k, v, "contract").reshape(len(rows), As)
    got = f(o_s)[rows]
    e = errors(got, ref)
    say(f"  o: rel_l2 {e['rel_l2']:.2e}, mismatch fraction {np.mean(got != ref):.2e}")
    assert np.all(np.isfinite(got)) and e["rel_l2"] < 1e-3
    # two bf16 ulps of the output plus what a one-ulp flip of any weight's
    # bf16 rounding moves (|dP_i| <= 2^-7 P_i): 2^-7 (sum P |v| / sum P + |o|)
    flip = np.empty_like(ref)
    for h in range(Hs):
        sc = q[rows, h] @ k[:, h].T
        P = O.bf16_round(np.exp2(sc - np.ceil(sc.max(axis=1, keepdims=True))))
        flip[:, h * 128:(h + 1) * 128] = (P @ np.abs(v[:, h])) / P.sum(axis=1, keepdims=True)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 2 * 2.0 ** -7 * np.abs(ref) + 2.0 ** -7 * (flip + np.abs(ref)) + 1e-4 * rms
    excess = np.abs(got - ref) / bound
    say(f"  o: max err/bound {excess.max():.3f}")
    assert excess.max() <= 1.0

"""The largest sequence the boundary accepts: 2^20 = 1,048,576 tokens (1,024 text
tokens and a 1,023 x 1,024 image grid), at reduced width (hidden 256, two heads
of 128, FFN 512) so that the float64 oracle stays cheap. Every index the kernels
form grows with the token count (attention over a million keys, 4,096 GEMM token
tiles, a 512 MB RoPE table, V^T rows of a million columns), so this is where an
overflow of 32-bit arithmetic or of the attention's weight sums would show.

Against the oracle on 256 seeded rows plus the first and last token, at the
block bar (the oracle's attention still runs over all 2^20 keys).
"""
import numpy as np
import pytest
import torch

from joint_attention_dit_amd import binding as B
from joint_attention_dit_amd.inputs import make_inputs, sample_rows, small_config

from tests._common import assert_block_parity, oracle_reference

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def say(msg):
    print(msg, flush=True)


def test_block_at_the_token_limit():
    cfg = small_config("max_tokens", hidden=256, heads=2, ffn=512, text_tokens=1024,
                       images=((1023, 1024, 0),), x_dtype="bf16")
    T = cfg.n_tokens
    assert T == 1 << 20
    say(f"[block] token limit T={T} D={cfg.hidden} H={cfg.heads} F={cfg.ffn}")
    inp = make_inputs(cfg, seed=0)
    blk = B.Block(cfg, inp)
    out = blk.forward()
    torch.cuda.synchronize()
    rows = np.union1d(sample_rows(T, 256, seed=1), np.array([0, T - 1]))
    got = out[torch.from_numpy(rows).cuda()].cpu().to(torch.float64).numpy()
    del blk, out
    torch.cuda.empty_cache()
    ref = oracle_reference(cfg, inp, rows=rows)
    assert_block_parity(got, ref["out"], "token limit out")

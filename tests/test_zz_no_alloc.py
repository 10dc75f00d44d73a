"""h3dit_block_forward_noalloc (the block forward whose scratch is the
library's static device array) against h3dit_block_forward through the C ABI:
bitwise equal outputs on two calls in a row, the second with a smaller block,
and the size limit rejected on the host before any HIP call."""
import ctypes

import pytest
import torch

from joint_attention_dit_amd import binding as B
from joint_attention_dit_amd.inputs import CONFIGS, make_inputs, small_config

pytestmark = pytest.mark.gpu

MID = small_config("mid", hidden=512, heads=4, ffn=1536, text_tokens=35, images=((23, 29, 0),),
                   x_dtype="bf16")


def say(msg):
    print(msg, flush=True)


def _both(cfg, seed):
    inp = make_inputs(cfg, seed=seed)
    blk = B.Block(cfg, inp)
    ref = blk.forward().clone()
    d = blk.dev
    out = torch.full_like(ref, float("nan"))
    B.h3dit_block_forward_noalloc(blk.cfg, d["x"], d["cond"], blk.weights, d["positions"], out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_forward_two_calls():
    # first the larger block, then a smaller one: the second call must not
    # depend on what the first left in the shared scratch
    for cfg, seed in ((MID, 3), (CONFIGS["tiny"], 4)):
        need = B.h3dit_workspace_size(B.config_from(cfg))
        say(f"[noalloc] {cfg.name} T={cfg.n_tokens} D={cfg.hidden}: scratch {need} of "
            f"{B.NOALLOC_SCRATCH_BYTES} bytes")
        assert need < B.NOALLOC_SCRATCH_BYTES
        ref, out = _both(cfg, seed)
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref), f"{cfg.name}: differs from h3dit_block_forward"
    # and the larger block again after the smaller one
    ref, out = _both(MID, 5)
    assert torch.equal(out, ref)


def test_noalloc_rejects_blocks_beyond_the_scratch():
    lib = B.load_library()
    cfg = B.make_config(5376, 56, 14336, 4352)   # the 2048x2048 block needs about 0.6 GB
    assert B.h3dit_workspace_size(cfg) > B.NOALLOC_SCRATCH_BYTES
    w = B.Weights(*(0x100000000 * (i + 1) for i in range(5)))
    st = lib.h3dit_block_forward_noalloc(ctypes.byref(cfg), 0x700000000, 0x800000000,
                                         ctypes.byref(w), 0x900000000, 0xA00000000, None)
    assert st == B.H3DIT_EWORKSPACE, st
    assert b"static scratch" in lib.h3dit_last_error()

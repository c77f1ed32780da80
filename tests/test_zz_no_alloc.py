"""vswin_block_fwd_noalloc (the entry point that allocates nothing) against
vswin_block_fwd on the same inputs: the same kernels run on the library's
static scratch array instead of a caller workspace, so the outputs must be
bitwise equal.  Two calls in a row, the second on a smaller input (the
array keeps the first call's contents), then a block too large for the
array, which must be refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
import shifted_window_attention_amd as vs

from helpers import dev, dev_params, say

pytestmark = pytest.mark.gpu


def _block(shape, shift, seed):
    B, T, H, W, C = shape
    heads = C // 32
    p = synth.gen_block_params(C, heads, 15 * 13 * 13, 4, np.random.SeedSequence(seed), "bf16", "stress")
    x = synth.round_bf16(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))
    return dev(x, "bf16"), dev_params(p, "bf16"), heads, (8, 7, 7), shift


def test_noalloc_matches_workspace_entry_two_calls():
    cases = [((1, 16, 56, 56, 96), (4, 3, 3), 71),     # Swin-T stage 1, shifted
             ((1, 16, 14, 21, 96), (0, 0, 0), 72)]     # smaller, regular, after it
    for shape, shift, seed in cases:
        say(f"noalloc block {shape} shift {shift}")
        x, w, heads, window, sh = _block(shape, shift, seed)
        ref = vs.vswin_block_fwd(x, w, heads, window, sh)
        got = vs.vswin_block_fwd_noalloc(x, w, heads, window, sh)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), f"{shape}: max diff {(got.float() - ref.float()).abs().max().item()}"


def test_noalloc_refuses_blocks_beyond_its_scratch():
    say("noalloc: a block beyond the static scratch is refused")
    x = torch.zeros((8, 16, 60, 60, 128), dtype=torch.bfloat16, device="cuda")
    p = dev_params(synth.gen_block_params(128, 4, 15 * 13 * 13, 4, np.random.SeedSequence(3), "bf16"), "bf16")
    y = torch.full_like(x, 7.0)
    with pytest.raises(vs.VswinError) as e:
        vs.vswin_block_fwd_noalloc(x, p, 4, (8, 7, 7), (4, 3, 3), out=y)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())          # untouched: nothing was enqueued

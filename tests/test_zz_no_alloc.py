"""The allocation-free key mean (attn_key_mean_noalloc) against attn_key_mean, which takes
a caller workspace: two calls in a row on one GPU, the second with a smaller input, each
bit for bit equal to the workspace entry point's result (the same kernels and the same
fixed summation order).  Each call prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import bf16_causal_flashattention_amd as cfa
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_key_mean_noalloc_matches_workspace_entry_point():
    cases = [((2, 5000, 3, 192), 81), ((1, 1300, 2, 128), 82)]  # the second call is smaller
    for (B, S, H, D), seed in cases:
        print("CASE key_mean_noalloc", B, S, H, D, flush=True)
        k = torch.from_numpy(synth.gaussian(B, S, H, D, D, seed)[1]).to(DEV)
        k += 3.0  # a common offset, the component K smoothing removes
        ref = cfa.key_mean(k)
        out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device=DEV)
        cfa.key_mean_noalloc(k, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        want = k.double().mean(dim=1).float()
        assert torch.allclose(out, want, rtol=0, atol=1e-6)

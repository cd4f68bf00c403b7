"""moe_permute_noalloc (the permutation for callers that cannot allocate,
its histogram in the library's fixed scratch array) against moe_permute
with a caller workspace: identical offsets, permutation and gathered rows,
bit for bit, on calls in a row that reuse the array -- a large batch, then a
smaller one (the array keeps the first call's contents), then one small
enough for the single-block sort, which uses no scratch."""

import numpy as np
import pytest
import torch

import mixture_experts_layer_40_amd as moe
import synth
from gpu_parity import say

pytestmark = pytest.mark.gpu


def _ids(T, K, E, seed):
    """K distinct expert ids per token, skewed like a routed batch."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    w = torch.rand((T, E), generator=g, device="cuda") + torch.linspace(0, 2, E, device="cuda")
    return torch.topk(w, K, dim=1).indices.to(torch.int32).contiguous()


@pytest.mark.parametrize("seq", [((60000, 8, 256), (9000, 6, 64), (300, 8, 256))])
def test_permute_noalloc_matches_permute_on_calls_in_a_row(seq):
    d = 128
    for i, (T, K, E) in enumerate(seq):
        say(f"[noalloc] call {i}: T={T} K={K} E={E}")
        spec = synth.scaled_config("v3_prefill_bf16", name="noalloc", T=T, d=d, E=E, K=K, I=64, Is=64)
        cfg = moe.config_of(spec)
        idx = _ids(T, K, E, 100 + i)
        x = torch.randn((T, d), device="cuda").to(torch.bfloat16)
        TK = T * K
        off_a = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        off_b = off_a.clone()
        perm_a = torch.full((TK,), -7, dtype=torch.int32, device="cuda")
        perm_b = perm_a.clone()
        xp_a = torch.empty((TK, d), dtype=torch.bfloat16, device="cuda")
        xp_b = torch.empty_like(xp_a)
        ws = torch.empty(max(moe.moe_workspace_size(cfg, moe.MOE_WS_PERMUTE), 256), dtype=torch.uint8,
                         device="cuda")
        moe.moe_permute(cfg, idx, x, off_a, perm_a, xp_a, ws=ws)
        moe.moe_permute_noalloc(cfg, idx, x, off_b, perm_b, xp_b)
        torch.cuda.synchronize()
        assert torch.equal(off_a, off_b), "expert offsets differ"
        assert torch.equal(perm_a, perm_b), "permutation differs"
        assert torch.equal(xp_a, xp_b), "gathered rows differ"
        # and both are the stable counting sort of the ids
        flat = idx.reshape(-1).cpu().numpy()
        want = np.argsort(flat, kind="stable")
        assert np.array_equal(perm_b.cpu().numpy(), want)
        assert np.array_equal(off_b.cpu().numpy()[1:], np.cumsum(np.bincount(flat, minlength=E)))

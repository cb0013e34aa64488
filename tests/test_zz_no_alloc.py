"""The allocation-free routing entry point (moe_route_capacity_align_noalloc,
its routing map in the library's own per-device scratch array) against the
workspace entry point it varies (moe_route_capacity_align): every output bit
for bit, on two calls in a row -- the DeepSeek-sized routing (a 10 MiB map)
and then a smaller skewed layer, so the second call runs on scratch that the
first left full of its own map."""

import numpy as np
import pytest
import torch

import moe_inputs
from gpu_support import say
from mixture_experts_expert_amd import MoEBuffers, MoEError, moe_route_capacity_align_noalloc
from conftest import load_golden

pytestmark = pytest.mark.gpu

OUTS = ("topk_ids", "topk_probs", "route_slot", "expert_count", "sorted_slot_ids", "slot_probs",
        "expert_ids", "block_start", "token_routes", "token_route_count", "num_tokens_post_padded")


def _noalloc(buf, logits):
    moe_route_capacity_align_noalloc(logits, buf.K, buf.C, buf.topk_ids, buf.topk_probs,
                                     buf.route_slot, buf.expert_count, buf.sorted_slot_ids,
                                     buf.slot_probs, buf.expert_ids, buf.block_start,
                                     buf.token_routes, buf.token_route_count,
                                     buf.num_tokens_post_padded)


def _same(a, b, what):
    for k in OUTS:
        x, y = getattr(a, k), getattr(b, k)
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"{what}: {k} differs from the workspace call"


def test_noalloc_equals_workspace_call_twice():
    alpha = load_golden("skew_alpha.json")["alpha"]
    cases = [("deepseek routing", 8192, 256, 8, 1.0, None, 4),
             ("smaller skewed layer", 3000, 128, 8, 1.0, alpha, 3)]
    for what, N, E, K, F, skew, seed in cases:
        say(f"[noalloc] {what}: N={N} E={E} K={K} F={F}")
        logits = torch.from_numpy(moe_inputs.make_logits(N, E, seed, skew)).to("cuda")
        a = MoEBuffers(N, 64, 64, E, K, F, "cuda")
        b = MoEBuffers(N, 64, 64, E, K, F, "cuda")
        for t in OUTS:                      # the two sides start from different garbage
            getattr(b, t).fill_(-7)
        a.route_capacity_align(logits)
        _noalloc(b, logits)
        torch.cuda.synchronize()
        _same(a, b, what)
        dropped = int((a.token_routes < 0).sum())
        say(f"  bitwise equal; {dropped} of {N * K} routes dropped")
        assert dropped > 0                  # both cases exercise the over-capacity selection


def test_noalloc_rejects_maps_beyond_its_scratch():
    # 5 bytes per expert and token: N=16384, E=256 needs 20 MiB > 16 MiB
    buf = MoEBuffers(16384, 64, 64, 256, 8, 1.0, "cuda")
    logits = torch.zeros((16384, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(MoEError) as ei:
        _noalloc(buf, logits)
    assert ei.value.status == -2

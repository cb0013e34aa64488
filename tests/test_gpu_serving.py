"""GPU tests of variable-N serving ([BK] "What this adds"): routing with a
device-side live-token count, and the bucket ladder of captured graphs.

Bars: routing and layout outputs bit-exact; a replayed item's output equals
the eager forward of the same item bit for bit (same route list, same tiles,
same float32 order); outputs against the oracle within the forward's bars.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import assert_bf16_close, host, say
from mixture_experts_expert_amd import (DroplessBuffers, ServingLadder, moe_dropless_bound,
                                        moe_route_dropless, moe_route_dropless_live)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _route(buf, logits, K, n_live=None):
    args = (buf.topk_ids, buf.topk_probs, buf.route_within, buf.route_counts, buf.sorted_slot_ids,
            buf.slot_probs, buf.expert_ids, buf.block_start, buf.token_routes,
            buf.token_route_count, buf.num_tokens_post_padded, buf.workspace)
    if n_live is None:
        moe_route_dropless(logits, K, *args)
    else:
        moe_route_dropless_live(logits, K, n_live, *args)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n_live", [700, 0, 1, 1024, 5000, -3])
def test_live_routing_equals_routing_the_live_prefix(n_live):
    Ncap, E, K = 1024, 64, 6
    lg = torch.from_numpy(moe_inputs.make_logits(Ncap, E, 11)).to(DEV)
    n = min(max(n_live, 0), Ncap)
    a = DroplessBuffers(Ncap, 64, 64, E, K, DEV)
    # stale contents must not leak into the result
    for t in (a.topk_ids, a.token_routes, a.sorted_slot_ids):
        t.fill_(12345)
    _route(a, lg, K, torch.tensor([n_live], dtype=torch.int32, device=DEV))
    ids, probs = host(a.topk_ids), host(a.topk_probs)
    assert np.all(ids[n:] == -1) and np.all(probs[n:] == 0)
    assert np.all(host(a.token_routes)[n:] == -1) and np.all(host(a.token_route_count)[n:] == 0)
    if n == 0:
        assert int(host(a.num_tokens_post_padded)[0]) == 0
        assert np.all(host(a.route_counts) == 0)
        return
    b = DroplessBuffers(n, 64, 64, E, K, DEV)
    _route(b, lg[:n].contiguous(), K)
    for k in ("topk_ids", "topk_probs", "token_routes", "token_route_count"):
        assert np.array_equal(host(getattr(a, k))[:n], host(getattr(b, k))), k
    for k in ("route_counts", "block_start", "num_tokens_post_padded"):
        assert np.array_equal(host(getattr(a, k)), host(getattr(b, k))), k
    ext = int(host(b.num_tokens_post_padded)[0])
    Rb = moe_dropless_bound(n, K, E)
    # pad slots name the buffers' sentinel row (Ncap: rows n..Ncap-1 of a
    # bucket's x are stale but real rows), the prefix call names n
    ssi_b = host(b.sorted_slot_ids)[:ext]
    assert np.array_equal(host(a.sorted_slot_ids)[:ext], np.where(ssi_b == n, Ncap, ssi_b))
    assert np.array_equal(host(a.slot_probs)[:ext].view(np.uint32), host(b.slot_probs)[:ext].view(np.uint32))
    assert np.array_equal(host(a.expert_ids)[:Rb // 32], host(b.expert_ids))
    # the oracle's dropless layout of the live tokens
    m = oracle.dropless_align(host(b.topk_ids), host(b.topk_probs), n, E)
    ssi_o = m["sorted_slot_ids"][:ext]
    assert np.array_equal(host(a.sorted_slot_ids)[:ext], np.where(ssi_o == n, Ncap, ssi_o))
    assert np.array_equal(host(a.token_routes)[:n], m["token_routes"])


def _ladder_case():
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    T = moe_inputs.make_tensors(w, DEV)
    lg = torch.from_numpy(moe_inputs.make_logits(1024, w.E, 23)).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(23)
    x = torch.randn(1024, w.H, generator=g, device=DEV).to(torch.bfloat16)
    return w, T, lg, x


def test_serving_replay_equals_eager_and_oracle():
    w, T, lg, x = _ladder_case()
    lad = ServingLadder(T["w1"], T["w2"], w.K, expected=512, max_tokens=1024, device=DEV,
                        reserve_bytes=0)
    caps = lad.capture()
    say(f"  buckets {lad.ladder.sizes}, captured {caps}")
    assert caps == lad.ladder.sizes
    eager = ServingLadder(T["w1"], T["w2"], w.K, expected=512, max_tokens=1024, device=DEV,
                          reserve_bytes=0)     # never captured: every item runs eagerly
    for n in (1, 37, 256, 300, 460, 511, 512, 600, 700, 1000, 1024):
        y = lad.run(lg[:n], x[:n]).clone()
        ye = eager.run(lg[:n], x[:n]).clone()
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"n={n}: replay differs from eager"
        if n in (37, 512, 700, 1024):
            o = oracle.dropless_forward(host(lg[:n]), host(x[:n]), host(T["w1"]), host(T["w2"]), w.K)
            assert_bf16_close(host(y), o["y"], f"y (n={n}) vs oracle")
    say(f"  counts {lad.counts}")
    assert lad.counts["eager"] >= 2           # n = 1 and n = 37 pad beyond the ratio
    assert sum(v for k, v in lad.counts.items() if k != "eager") >= 8
    assert eager.counts["eager"] == 11


def test_serving_capture_stops_at_memory_reserve():
    w, T, lg, x = _ladder_case()
    free = [40 << 30]

    def fake_mem():
        free[0] -= 1 << 30          # each query sees 1 GiB less
        return free[0], 80 << 30

    lad = ServingLadder(T["w1"], T["w2"], w.K, expected=512, max_tokens=1024, device=DEV,
                        reserve_bytes=35 << 30, mem_get_info=fake_mem)
    caps = lad.capture()
    say(f"  captured {caps} of {lad.ladder.sizes}")
    assert 0 < len(caps) < len(lad.ladder.sizes)
    assert caps == sorted(lad.ladder.capture_order()[:len(caps)])   # the largest ones
    ref = ServingLadder(T["w1"], T["w2"], w.K, expected=512, max_tokens=1024, device=DEV,
                        reserve_bytes=0)
    for n in (260, 520, 1000):      # some replayed, some eager
        assert torch.equal(lad.run(lg[:n], x[:n]).clone(), ref.run(lg[:n], x[:n]).clone())


def test_serving_qwen_shape_item_against_oracle():
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    T = moe_inputs.make_tensors(w, DEV)
    lad = ServingLadder(T["w1"], T["w2"], w.K, expected=4096, max_tokens=8192, device=DEV,
                        reserve_bytes=0)
    lad.capture()
    eager = ServingLadder(T["w1"], T["w2"], w.K, expected=4096, max_tokens=8192, device=DEV,
                          reserve_bytes=0)
    n = 3000
    y = lad.run(T["logits"][:n], T["x"][:n]).clone()
    ye = eager.run(T["logits"][:n], T["x"][:n]).clone()
    torch.cuda.synchronize()
    assert lad.counts.get(lad.ladder.pick(n), 0) == 1 and eager.counts["eager"] == 1
    bad = (~torch.isfinite(y.float())).any(dim=1).nonzero().flatten().tolist()
    say(f"  rows with non-finite values: {len(bad)} {bad[:10]}")
    assert torch.equal(y, ye), "replay differs from eager"
    o = oracle.dropless_forward(host(T["logits"][:n]), host(T["x"][:n]), host(T["w1"]),
                                host(T["w2"]), w.K)
    assert_bf16_close(host(y), o["y"], "y (n=3000 in its bucket) vs oracle")

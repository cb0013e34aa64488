"""The dispatch side of an expert-parallel exchange on one GPU
(moe_dispatch_rows): the send buffer holds each slot's token row in route
order, pads as zero rows.

* bit-exact against oracle.dispatch_rows on every workload shape that fits
  and on a ragged layer with pads (N = 77, H = 192);
* loopback at the Qwen3-30B-A3B shape: dispatched rows -> the grouped FFN
  with the identity route list (what a receiving rank runs) -> the
  gather-combine through the original inverse map gives act, route_out and y
  bit for bit equal to the permute-free forward (same per-slot rows, same
  kernels, same K order), i.e. the permuted path equals the permute-free one.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import host, run_steps, say
from mixture_experts_expert_amd import (MoEBuffers, moe_dispatch_rows, moe_gather_combine,
                                        moe_grouped_fc1_swiglu, moe_grouped_fc2)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _forward(w, skew_alpha=None):
    T = moe_inputs.make_tensors(w, DEV, skew_alpha=skew_alpha)
    buf = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    run_steps(buf, T["logits"], T["x"], T["w1"], T["w2"])
    return T, buf


def _dispatch(x, ssi):
    rows = torch.full((ssi.shape[0], x.shape[1]), 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe_dispatch_rows(x, ssi, rows)
    torch.cuda.synchronize()
    return rows


@pytest.mark.parametrize("name", ["tiny_n64_h64_e4_k2", "small_qwen3moe_n1024_h512_e8_k2",
                                  "qwen3_30b_a3b_n4096_h2048_e128_k8",
                                  "skew_zipf_n4096_e128_k8_f1.5"])
def test_dispatch_rows_bitwise(name, skew_alpha):
    w = moe_inputs.WORKLOADS[name]
    T, buf = _forward(w, skew_alpha if w.skew else None)
    rows = _dispatch(T["x"], buf.sorted_slot_ids)
    ssi = host(buf.sorted_slot_ids)
    ref = oracle.dispatch_rows(host(T["x"]), ssi)
    assert np.array_equal(host(rows), ref)
    pads = ssi == w.N
    say(f"  {name}: {rows.shape[0]} slot rows, {int(pads.sum())} pads")
    assert np.all(host(rows)[pads] == 0)


def test_dispatch_rows_ragged_with_pads():
    N, H, E, K, F = 77, 192, 6, 3, 1.6
    w = moe_inputs.Workload("ragged_dispatch", N, H, E, K, F, 64, 31)
    T, buf = _forward(w)
    ssi = host(buf.sorted_slot_ids)
    assert (ssi == N).sum() > 0
    rows = _dispatch(T["x"], buf.sorted_slot_ids)
    assert np.array_equal(host(rows), oracle.dispatch_rows(host(T["x"]), ssi))


def test_rank_loopback_equals_permute_free_forward():
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    T, buf = _forward(w)
    rows = _dispatch(T["x"], buf.sorted_slot_ids)
    R = rows.shape[0]
    ident = torch.arange(R, dtype=torch.int32, device=DEV)
    act = torch.empty((R, w.I), dtype=torch.bfloat16, device=DEV)
    ro = torch.empty((R, w.H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=DEV)
    moe_grouped_fc1_swiglu(rows, T["w1"], ident, buf.slot_probs, buf.C, act)
    moe_grouped_fc2(act, T["w2"], R, buf.C, ro)
    moe_gather_combine(ro, buf.token_routes, y)
    torch.cuda.synchronize()
    assert torch.equal(act, buf.act), "act differs"
    assert torch.equal(ro, buf.route_out), "route_out differs"
    assert torch.equal(y, buf.y), "y differs"

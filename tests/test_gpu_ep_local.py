"""The grouped FFN on one expert-parallel rank's share: after the exchange a
rank holds E/ep experts with C*ep rows each, already grouped by expert, so
the route list is the identity (slot s reads row s) and the row count
exceeds the routing calls' envelope (N = E*C rows: 32768 at the
Qwen3-30B-A3B shape for any ep).  The GEMMs take any row count their 32-bit
offsets allow.

* a small layer with N > 16384 rows, every slot checked against the oracle;
* the Qwen3-30B-A3B shape at ep = 8 (16 local experts, 2048 rows each, the
  configuration `bench.py --variant ep-local` times): every row of every
  expert.

Bars: the forward's (act and route_out within 1e-2 + 2e-2|ref| and normwise
1e-2), oracle.expert_ffn / oracle.grouped_ffn on the same rows.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import assert_bf16_close, host, say
from mixture_experts_expert_amd import (moe_dispatch_rows, moe_grouped_fc1_swiglu, moe_grouped_fc2,
                                        moe_grouped_fc2_rows)

pytestmark = pytest.mark.gpu


def _run(d, stream=None):
    E, C = d["E"], d["C"]
    N = E * C
    ssi = torch.arange(N, dtype=torch.int32, device="cuda")
    act = torch.full((N, d["w2"].shape[2]), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ro = torch.full((N, d["w2"].shape[1]), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    moe_grouped_fc1_swiglu(d["x"], d["w1"], ssi, d["probs"], C, act, stream)
    moe_grouped_fc2(act, d["w2"], N, C, ro, stream)
    torch.cuda.synchronize()
    return ssi, act, ro


def test_more_rows_than_the_routing_envelope():
    w = moe_inputs.Workload("ep_local_small", 64, 128, 8, 2, 1.0, 64, 21)
    d = moe_inputs.make_ep_local(w, 2, 4608, "cuda")        # 4 experts x 4608 rows = 18432
    ssi, act, ro = _run(d)
    N = d["E"] * d["C"]
    assert N > 16384
    r_act, r_ro = oracle.grouped_ffn(host(d["x"]), host(d["w1"]), host(d["w2"]), host(ssi),
                                     host(d["probs"]), d["E"], d["C"])
    assert_bf16_close(host(act), r_act, "act")
    assert_bf16_close(host(ro), r_ro, "route_out")


def test_qwen_shape_ep8_share():
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    ep = 8
    C = oracle.source_capacity(w.N, w.K, w.E, w.F) * ep
    d = moe_inputs.make_ep_local(w, ep, C, "cuda")
    _, act, ro = _run(d)
    E = d["E"]
    say(f"  {E} local experts x {C} rows = {E * C} rows")
    x, pr, g_act, g_ro = host(d["x"]), host(d["probs"]), host(act), host(ro)
    for e in range(E):
        rows = slice(e * C, (e + 1) * C)
        r_act, r_out = oracle.expert_ffn(x[rows], host(d["w1"][e]), host(d["w2"][e]), pr[rows])
        assert_bf16_close(g_act[rows], r_act, f"act e{e}")
        assert_bf16_close(g_ro[rows], r_out, f"route_out e{e}")


def test_source_major_receive_buffer():
    """After an all-to-all the receive buffer is source-major (each source's
    chunk holds all local experts); the grouped FFN reads it in expert order
    through a fixed route list, with the same results bit for bit as on the
    expert-major copy."""
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    ep = 8
    Cs = oracle.source_capacity(w.N, w.K, w.E, w.F)
    d = moe_inputs.make_ep_local(w, ep, Cs * ep, "cuda")
    E, C = d["E"], d["C"]
    perm = torch.as_tensor(moe_inputs.ep_receive_order(E, ep, Cs), device="cuda")
    assert torch.equal(torch.sort(perm).values, torch.arange(E * C, dtype=torch.int32, device="cuda"))
    x_recv = torch.empty_like(d["x"])
    x_recv[perm.long()] = d["x"]                       # slot s's row sits at received row perm[s]
    _, act_id, ro_id = _run(d)
    act = torch.empty_like(act_id)
    ro = torch.empty_like(ro_id)
    moe_grouped_fc1_swiglu(x_recv, d["w1"], perm, d["probs"], C, act)
    moe_grouped_fc2(act, d["w2"], E * C, C, ro)
    torch.cuda.synchronize()
    assert torch.equal(act, act_id) and torch.equal(ro, ro_id)
    # the return direction: route_out back into source-major chunks is the
    # same row gather through the inverse list (received row j <- slot inv[j])
    inv = torch.empty_like(perm)
    inv[perm.long()] = torch.arange(E * C, dtype=torch.int32, device="cuda")
    back = torch.empty_like(ro)
    moe_dispatch_rows(ro, inv, back)
    torch.cuda.synchronize()
    assert torch.equal(back[perm.long()], ro)
    # or FC2 writes them there itself through the row map (no reorder pass)
    ro_map = torch.full_like(ro, float("nan"))
    moe_grouped_fc2_rows(act, d["w2"], perm, E * C, C, ro_map)
    torch.cuda.synchronize()
    assert torch.equal(ro_map, back)


def test_fc2_row_map_identity_and_drops():
    """The identity map reproduces plain FC2 bit for bit; entries outside
    the output drop their rows and leave those rows untouched."""
    w = moe_inputs.Workload("fc2_rows_small", 64, 320, 8, 2, 1.0, 192, 23)
    d = moe_inputs.make_ep_local(w, 2, 512, "cuda")         # 4 experts x 512 rows (two row tiles)
    _, act, ro = _run(d)
    E, C = d["E"], d["C"]
    R = E * C
    ident = torch.arange(R, dtype=torch.int32, device="cuda")
    out = torch.full_like(ro, float("nan"))
    moe_grouped_fc2_rows(act, d["w2"], ident, R, C, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ro)
    rng = np.random.default_rng(5)
    dropped = torch.as_tensor(np.sort(rng.choice(R, 100, replace=False)), device="cuda")
    bad = ident.clone()
    bad[dropped[:50]] = -1
    bad[dropped[50:]] = R
    out = torch.full_like(ro, 7.0)
    moe_grouped_fc2_rows(act, d["w2"], bad, R, C, out)
    torch.cuda.synchronize()
    keep = torch.ones(R, dtype=torch.bool, device="cuda")
    keep[dropped] = False
    assert torch.equal(out[keep], ro[keep])
    assert torch.all(out[~keep] == 7.0)


"""Expert parallelism emulated on one GPU: ep source ranks and ep expert
ranks in one process, the two all-to-alls replaced by device copies.

Each source routes its own N/ep tokens over all E experts (capacity from its
own N, every source selects), packs its send buffer with moe_dispatch_rows
and runs its single-GPU forward as the reference.  Rank r receives, from
every source, the segment of its E/ep experts (source-major), runs the
grouped FFN through the receive-order route list, and gets route_out back
in source-major chunks either from FC2's row map (even ranks) or by a
reorder with moe_dispatch_rows through the inverse list (odd ranks).  Each source then gathers its routes from the returned rows with
moe_gather_combine.  Its y must equal its own single-GPU forward within the
forward's bars (the ranks' launches walk K from a different starting slab,
so the float32 sums are reordered), and the pad rows and dropped routes
must behave as in the single-GPU forward.
"""

import numpy as np
import pytest
import torch

import moe_inputs
from gpu_support import assert_bf16_close, host, run_steps, say
from mixture_experts_expert_amd import (MoEBuffers, moe_dispatch_rows, moe_gather_combine,
                                        moe_grouped_fc1_swiglu, moe_grouped_fc2, moe_grouped_fc2_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("ep", [2, 8])
def test_ep_emulated_equals_single_gpu_forward(ep):
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    T = moe_inputs.make_tensors(w, DEV)
    Ns, El, H, I = w.N // ep, w.E // ep, w.H, w.I
    src = []
    for s in range(ep):
        tok = slice(s * Ns, (s + 1) * Ns)
        buf = MoEBuffers(Ns, H, I, w.E, w.K, w.F, DEV)
        x_s = T["x"][tok].contiguous()
        run_steps(buf, T["logits"][tok].contiguous(), x_s, T["w1"], T["w2"])
        send = torch.empty(w.E * buf.Cp, H, dtype=torch.bfloat16, device=DEV)
        moe_dispatch_rows(x_s, buf.sorted_slot_ids, send)
        src.append((buf, send))
    Cp = src[0][0].Cp
    seg = El * Cp                                            # rows one source sends one rank
    say(f"  ep={ep}: {Ns} tokens per source, Cp={Cp}, {ep * seg} rows per rank")
    perm = torch.as_tensor(moe_inputs.ep_receive_order(El, ep, Cp), device=DEV)
    inv = torch.empty_like(perm)
    inv[perm.long()] = torch.arange(ep * seg, dtype=torch.int32, device=DEV)
    returned = [torch.empty(w.E * Cp, H, dtype=torch.bfloat16, device=DEV) for _ in range(ep)]
    for r in range(ep):
        part = slice(r * seg, (r + 1) * seg)
        recv = torch.cat([send[part] for _, send in src])                       # all-to-all
        probs_sm = torch.cat([buf.slot_probs[part] for buf, _ in src])
        probs = probs_sm[perm.long()].contiguous()            # expert-major slot order
        w1 = T["w1"][r * El:(r + 1) * El]
        w2 = T["w2"][r * El:(r + 1) * El]
        act = torch.empty(ep * seg, I, dtype=torch.bfloat16, device=DEV)
        ro = torch.empty(ep * seg, H, dtype=torch.bfloat16, device=DEV)
        moe_grouped_fc1_swiglu(recv, w1, perm, probs, ep * Cp, act)
        back = torch.empty_like(ro)
        if r % 2 == 0:
            moe_grouped_fc2_rows(act, w2, perm, ep * seg, ep * Cp, back)   # straight to source-major
        else:
            moe_grouped_fc2(act, w2, ep * seg, ep * Cp, ro)
            moe_dispatch_rows(ro, inv, back)                  # source-major again
        for s in range(ep):                                   # the return all-to-all
            returned[s][part] = back[s * seg:(s + 1) * seg]
    torch.cuda.synchronize()
    for s, (buf, _) in enumerate(src):
        y = torch.empty(Ns, H, dtype=torch.bfloat16, device=DEV)
        moe_gather_combine(returned[s], buf.token_routes, y)
        torch.cuda.synchronize()
        pads = host(buf.sorted_slot_ids) == Ns
        assert np.all(host(returned[s])[pads] == 0), f"source {s}: pad rows must come back zero"
        assert_bf16_close(host(returned[s]), host(buf.route_out), f"source {s} route_out")
        assert_bf16_close(host(y), host(buf.y), f"source {s} y")

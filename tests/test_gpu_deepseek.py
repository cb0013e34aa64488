"""DeepSeek-style wide layer (N=8192, H=7168, E=256, K=8, F=1.0, I=2048) at full
size, hipGraph-captured with static capacity buffers.

* graph replay == eager, bitwise;
* routing, capacity selection, align and the combine are checked in full
  (step-wise, bit-exact) against the oracle;
* the FFN is checked on every slot row of every expert, pads included: the
  oracle runs one expert at a time (that expert's weights copied to the host,
  float64 products), in eight chunks of experts so that no single test runs
  long, and act and route_out must meet the forward's bars on each expert;
* y is checked on every token, end to end, against the oracle's
  gather-combine of the oracle's own route rows.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import (ATOL, NORM_TOL, RTOL, bf16_close_stats, check_capacity_and_align,
                         check_combine_stepwise, check_routing, host, say)
from mixture_experts_expert_amd import MoEBuffers

pytestmark = pytest.mark.gpu

W = moe_inputs.WORKLOADS["deepseek_wide_n8192_h7168_e256_k8"]
CHUNKS = 8                     # expert chunks of the full FFN check
_ORACLE_OUT = {}               # expert -> the oracle's route_out rows (bf16 bits)


@pytest.fixture(scope="module")
def run():
    say(f"[deepseek] generating {W.name} on the GPU")
    T = moe_inputs.make_tensors(W, "cuda")
    buf = MoEBuffers(W.N, W.H, W.I, W.E, W.K, W.F, "cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        buf.route_capacity(T["logits"])
        buf.align()
        buf.grouped_ffn(T["x"], T["w1"], T["w2"])
        buf.combine()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = {k: getattr(buf, k).clone() for k in ("sorted_slot_ids", "route_out", "y")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        buf.route_capacity(T["logits"])
        buf.align()
        buf.grouped_ffn(T["x"], T["w1"], T["w2"])
        buf.combine()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    say("[deepseek] captured and replayed")
    host_state = {"x": host(T["x"]), "ssi": host(buf.sorted_slot_ids), "sp": host(buf.slot_probs),
                  "tr": host(buf.token_routes)}
    return T, buf, eager, host_state


def test_graph_replay_equals_eager(run):
    T, buf, eager, _ = run
    for k, v in eager.items():
        assert torch.equal(getattr(buf, k), v), f"{k}: graph replay differs from eager"


def test_routing_layout_and_combine_full(run):
    T, buf, _, _ = run
    check_routing(buf, host(T["logits"]), W.K)
    C = oracle.source_capacity(W.N, W.K, W.E, W.F)
    m = check_capacity_and_align(buf, W.N, W.E, W.K, C)
    say(f"  C={C} kept={int((m['token_routes'] >= 0).sum())}/{W.N * W.K}")
    check_combine_stepwise(buf, W.N)


def _oracle_expert(T, hs, e, Cp):
    """The oracle's act and route_out rows of expert e's whole segment."""
    seg = slice(e * Cp, (e + 1) * Cp)
    rows = hs["ssi"][seg]
    a = np.zeros((Cp, W.H), np.uint16)
    real = rows < W.N
    a[real] = hs["x"][rows[real]]
    return oracle.expert_ffn(a, host(T["w1"][e]), host(T["w2"][e]), hs["sp"][seg])


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_ffn_every_slot(run, chunk):
    T, buf, _, hs = run
    Cp = buf.Cp
    per = W.E // CHUNKS
    worst = {"act": 0.0, "route_out": 0.0}
    pads = 0
    for e in range(chunk * per, (chunk + 1) * per):
        act, out = _oracle_expert(T, hs, e, Cp)
        _ORACLE_OUT[e] = out
        pads += int((hs["ssi"][e * Cp:(e + 1) * Cp] == W.N).sum())
        for name, ref in (("act", act), ("route_out", out)):
            got = host(getattr(buf, name)[e * Cp:(e + 1) * Cp])
            st = bf16_close_stats(got, ref)
            assert st["bad"] == 0, f"{name} expert {e}: {st['bad']} elements outside {ATOL} + {RTOL}|ref|"
            assert st["norm"] <= NORM_TOL, f"{name} expert {e}: normwise relative error {st['norm']:.3e}"
            worst[name] = max(worst[name], st["norm"])
    say(f"  experts {chunk * per}..{(chunk + 1) * per - 1}: {per * Cp} slot rows ({pads} pads); "
        f"worst per-expert normwise error act {worst['act']:.2e}, route_out {worst['route_out']:.2e}")


def test_y_every_token(run):
    T, buf, _, hs = run
    Cp = buf.Cp
    route_out = np.zeros((W.E * Cp, W.H), np.uint16)
    for e in range(W.E):
        out = _ORACLE_OUT.get(e)
        if out is None:                       # the chunk tests did not run (a -k selection)
            out = _oracle_expert(T, hs, e, Cp)[1]
        route_out[e * Cp:(e + 1) * Cp] = out
    y_ref = oracle.gather_combine(route_out, hs["tr"], W.N)
    st = bf16_close_stats(host(buf.y), y_ref)
    say(f"  y over all {W.N} tokens: normwise rel err {st['norm']:.2e}, max abs err "
        f"{st['max_abs']:.2e}, exact {st['exact']:.4f}")
    assert st["bad"] == 0, f"y: {st['bad']} elements outside {ATOL} + {RTOL}|ref|"
    assert st["norm"] <= NORM_TOL, f"y: normwise relative error {st['norm']:.3e}"

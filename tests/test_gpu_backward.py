"""GPU parity of the backward: the HIP path through the C ABI against the
CPU oracle (oracle.backward).

Each kernel is checked step-wise (the oracle step consumes the GPU's own
inputs to it) and the whole chain end to end from the same routing state.

Bars (derived in the design notes from the arithmetic):
* bf16 results (pre-activation, d_act, recomputed act, d_preact, per-route
  input gradients, dx, dW1, dW2): elementwise
  |gpu - ref| <= 1e-2 * rms(ref) + 2e-2 * |ref|  and normwise relative error
  <= 1e-2.  The absolute term scales with the tensor (gradients range over
  orders of magnitude between tensors); float32 accumulation in a different
  order flips about one bf16 ulp here and there, which these bounds absorb.
  End to end, each result is a sum of values rounded to bf16 along separate
  chains (dx: the token's K route gradients; dW: 256 products of rounded
  factors per element; d_logits: through dp, a sum over I of products of
  rounded d_act and pre-activation values).  A one-ulp flip (2^-8 relative)
  in any term, from a different float32 summation order upstream, reaches
  the sum unchanged in size however much the terms cancel, so the end-to-end
  bar adds 2^-7 times the sum of the terms' magnitudes.
* the dx gather-combine fed the GPU's own per-route gradients is bit-exact;
* float32 results (d_prob, d_logits): |gpu - ref| <= 1e-3 * rms(ref) +
  1e-3 * |ref| step-wise (float32 arithmetic against float64), and within the
  bf16 bars end to end (they inherit the bf16 roundings upstream).
* the FC1 forward with the pre-activation saved writes the same act, bit for
  bit, as the plain FC1.
"""

import zlib

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import (F32_TOL, assert_grad_close, check_capacity_and_align, check_routing, grad_vals,
                         host, say)
from mixture_experts_expert_amd import MoEBackwardBuffers, MoEBuffers

pytestmark = pytest.mark.gpu

DEV = "cuda"
def run_case(N, H, I, E, K, F, T, dy):
    buf = MoEBuffers(N, H, I, E, K, F, DEV)
    bw = MoEBackwardBuffers(buf)
    bw.forward(T["logits"], T["x"], T["w1"], T["w2"])
    torch.cuda.synchronize()
    act_saved = buf.act.clone()
    # the plain FC1 must write the same act
    buf.fc1_swiglu(T["x"], T["w1"])
    torch.cuda.synchronize()
    assert torch.equal(buf.act, act_saved), "FC1 with the pre-activation saved changed act"
    bw.backward(dy, T["x"], T["w1"], T["w2"])
    torch.cuda.synchronize()
    return buf, bw


def check_backward(s, T, dy):
    """s: N, H, I, E, K, F; T: device inputs; dy: device bf16 [N, H]."""
    N, H, I, E, K, F = s.N, s.H, s.I, s.E, s.K, s.F
    C = oracle.source_capacity(N, K, E, F)
    buf, bw = run_case(N, H, I, E, K, F, T, dy)
    check_routing(buf, host(T["logits"]), K)
    m = check_capacity_and_align(buf, N, E, K, C)
    Cp = buf.Cp
    ssi, sp = m["sorted_slot_ids"], m["slot_probs"]
    x, w1, w2, dyb = host(T["x"]), host(T["w1"]), host(T["w2"]), host(dy)
    say(f"  C={C} Cp={Cp} kept={int((m['token_routes'] >= 0).sum())}/{N * K}")

    # ---- step-wise: each kernel against the oracle on the GPU's own inputs
    g_pre, g_dact, g_act = host(bw.preact), host(bw.d_act), host(bw.act_re)
    g_dpre, g_dprob, g_da = host(bw.d_preact), host(bw.d_prob), host(bw.d_a)
    assert_grad_close(g_pre, oracle.fc1_preact_slots(x, w1, ssi, E, Cp), "preact")
    assert_grad_close(g_dact, oracle.fc2_dgrad(dyb, w2, ssi, E, Cp), "d_act (FC2 dgrad)")
    r_act, r_dpre, r_dprob = oracle.swiglu_backward(g_pre, g_dact, sp)
    assert_grad_close(g_act, r_act, "act recomputed")
    assert_grad_close(g_dpre, r_dpre, "d_preact (SwiGLU bwd)")
    assert_grad_close(g_dprob, r_dprob, "d_prob (SwiGLU bwd)", rtol=F32_TOL, atol_rms=F32_TOL,
                      norm_tol=F32_TOL)
    assert_grad_close(g_da, oracle.fc1_dgrad(g_dpre, w1, E, Cp), "d_a (FC1 dgrad)")
    g_dx = host(bw.dx)
    assert np.array_equal(g_dx, oracle.gather_combine(g_da, m["token_routes"], N)), \
        "dx gather-combine differs"
    assert_grad_close(host(bw.dw2), oracle.fc2_wgrad(dyb, g_act, ssi, E, Cp), "dW2 (FC2 wgrad)")
    assert_grad_close(host(bw.dw1), oracle.fc1_wgrad(g_dpre, x, ssi, E, Cp), "dW1 (FC1 wgrad)")
    r_dl = oracle.route_backward(host(buf.topk_ids), host(buf.topk_probs), m["token_routes"],
                                 g_dprob, E)
    assert_grad_close(host(bw.d_logits), r_dl, "d_logits (route bwd)", rtol=F32_TOL,
                      atol_rms=F32_TOL, norm_tol=F32_TOL)
    pads = ssi == N
    for name, v in (("d_act", g_dact), ("act", g_act), ("d_preact", g_dpre), ("d_a", g_da)):
        assert np.all(v[pads] == 0), f"{name}: pad rows must be zero"
    assert np.all(g_dprob[pads] == 0)

    # ---- end to end from the same routing state
    fwd = dict(m)
    fwd["topk_ids"] = host(buf.topk_ids)
    fwd["topk_probs"] = host(buf.topk_probs)
    R = oracle.backward(fwd, x, w1, w2, dyb)
    # Each end-to-end result sums separately rounded bf16 values; its bar
    # adds 2^-7 times the sum of those terms' magnitudes (see above).
    tr = m["token_routes"]
    da_abs = np.abs(grad_vals(R["d_a"]))
    dx_terms = np.zeros((N, H))
    for k in range(K):
        sel = tr[:, k] >= 0
        dx_terms[sel] += da_abs[tr[sel, k]]
    assert_grad_close(g_dx, R["dx"], "dx (end to end)", terms=dx_terms)
    xa, dya = np.abs(grad_vals(x)), np.abs(grad_vals(dyb))
    dpa, aca = np.abs(grad_vals(R["d_preact"])), np.abs(grad_vals(R["act"]))

    def rows(src, e):
        r = ssi[e * Cp:(e + 1) * Cp]
        out = np.zeros((Cp, src.shape[1]))
        out[r < N] = src[r[r < N]]
        return out

    dw1_terms = np.stack([dpa[e * Cp:(e + 1) * Cp].T @ rows(xa, e) for e in range(E)])
    dw2_terms = np.stack([rows(dya, e).T @ aca[e * Cp:(e + 1) * Cp] for e in range(E)])
    assert_grad_close(host(bw.dw1), R["dw1"], "dw1 (end to end)", terms=dw1_terms)
    assert_grad_close(host(bw.dw2), R["dw2"], "dw2 (end to end)", terms=dw2_terms)
    # d_logits = p_k (dp_k - sum_j p_j dp_j), dp a sum over the I columns of
    # d_act * silu(g) * u with d_act and the pre-activation rounded upstream
    pre = grad_vals(R["preact"])
    g_, u_ = pre[:, :I], pre[:, I:]
    dp_terms = (np.abs(grad_vals(R["d_act"])) * np.abs(g_ / (1 + np.exp(-g_)) * u_)).sum(axis=1)
    pk = host(buf.topk_probs).astype(np.float64)
    ak = np.where(tr >= 0, dp_terms[np.maximum(tr, 0)], 0.0)
    gk = pk * (ak + (pk * ak).sum(axis=1, keepdims=True))
    dl_terms = np.zeros((N, E))
    np.put_along_axis(dl_terms, host(buf.topk_ids).astype(np.int64), gk, axis=1)
    assert_grad_close(host(bw.d_logits), R["d_logits"], "d_logits (end to end)", terms=dl_terms)
    return buf, bw, m


class Shape:
    def __init__(self, N, H, I, E, K, F):
        self.N, self.H, self.I, self.E, self.K, self.F = N, H, I, E, K, F


def custom(s: Shape, seed: int, logits=None):
    g = torch.Generator(device=DEV).manual_seed(seed)
    lg = logits if logits is not None else moe_inputs.make_logits(s.N, s.E, seed)
    T = {
        "logits": torch.from_numpy(np.ascontiguousarray(lg, dtype=np.float32)).to(DEV),
        "x": torch.randn(s.N, s.H, generator=g, device=DEV).to(torch.bfloat16),
        "w1": (torch.randn(s.E, 2 * s.I, s.H, generator=g, device=DEV) * 0.05).to(torch.bfloat16),
        "w2": (torch.randn(s.E, s.H, s.I, generator=g, device=DEV) * 0.05).to(torch.bfloat16),
    }
    dy = torch.randn(s.N, s.H, generator=g, device=DEV).to(torch.bfloat16)
    return T, dy


@pytest.mark.parametrize("name", ["tiny_n64_h64_e4_k2", "small_qwen3moe_n1024_h512_e8_k2",
                                  "qwen3_30b_a3b_n4096_h2048_e128_k8"])
def test_backward_workload_parity(name):
    w = moe_inputs.WORKLOADS[name]
    say(f"[backward] {name}")
    T = moe_inputs.make_tensors(w, DEV)
    check_backward(w, T, moe_inputs.make_dy(w, DEV))


def test_backward_skew_parity(skew_alpha):
    w = moe_inputs.WORKLOADS["skew_zipf_n4096_e128_k8_f1.0"]
    say(f"[backward] {w.name}")
    T = moe_inputs.make_tensors(w, DEV, skew_alpha=skew_alpha)
    _, _, m = check_backward(w, T, moe_inputs.make_dy(w, DEV))
    assert (m["token_routes"] < 0).sum() > 0           # dropped routes get no gradient


EDGE = {
    "single_token": (Shape(1, 64, 64, 4, 2, 1.0), None),
    "one_expert": (Shape(100, 128, 192, 1, 1, 1.0), None),
    "ragged_n77_h192_i320": (Shape(77, 192, 320, 6, 3, 0.7), None),
    "overload_one_expert": (Shape(512, 64, 128, 8, 2, 1.0), "hot"),
    "large_factor_pads": (Shape(200, 64, 128, 8, 2, 4.0), None),
    "wide_e1000_k32": (Shape(256, 64, 64, 1000, 32, 1.0), None),
    # C = 256 and 512: whole 256-row tiles (the persistent 12-wave GEMM), one
    # with ragged column tiles (H = 320, I = 192) and a 3-slab contraction, one
    # with two row tiles per expert
    "whole_tiles_ragged_h320_i192": (Shape(512, 320, 192, 8, 4, 1.0), None),
    "two_row_tiles_c512": (Shape(1024, 256, 128, 8, 4, 1.0), None),
}


@pytest.mark.parametrize("case", list(EDGE))
def test_backward_edge_case_parity(case):
    s, mode = EDGE[case]
    say(f"[backward edge] {case}")
    lg = None
    if mode == "hot":
        rng = np.random.default_rng(zlib.crc32(case.encode()))
        lg = rng.standard_normal((s.N, s.E)).astype(np.float32)
        lg[:, 0] += 50.0
    T, dy = custom(s, 29, lg)
    buf, bw, _ = check_backward(s, T, dy)
    if case == "one_expert":
        # K = 1: the probability is constant 1, no logit gradient
        assert torch.count_nonzero(bw.d_logits).item() == 0


def test_backward_graph_replay_equals_eager():
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    T = moe_inputs.make_tensors(w, DEV)
    dy = moe_inputs.make_dy(w, DEV)
    buf = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    bw = MoEBackwardBuffers(buf)
    outs = ("preact", "d_act", "act_re", "d_preact", "d_prob", "d_a", "dx", "dw1", "dw2",
            "d_logits")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bw.forward(T["logits"], T["x"], T["w1"], T["w2"])
        bw.backward(dy, T["x"], T["w1"], T["w2"])
    s.synchronize()
    ref = {k: getattr(bw, k).clone() for k in outs}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bw.forward(T["logits"], T["x"], T["w1"], T["w2"])
        bw.backward(dy, T["x"], T["w1"], T["w2"])
    for rep in range(3):
        for k in outs:
            getattr(bw, k).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(getattr(bw, k), ref[k]), f"replay {rep}: {k} differs from eager"

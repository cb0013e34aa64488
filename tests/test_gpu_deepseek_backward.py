"""The layer's training step at the DeepSeek-style wide shape (N=8192,
H=7168, E=256, K=8, F=1.0, I=2048), full size, in the launch configuration
the benchmark times (forward keeping the pre-activation, then the backward).

The GEMM steps are checked step-wise on every expert (the oracle's step
functions over one expert's segment, fed the GPU's own inputs to each step,
that expert's weights copied to the host): the pre-activation, FC2 dgrad, the
SwiGLU backward, FC1 dgrad and both weight gradients, every element, pads
included, in eight chunks of experts so that no single test runs long.  The
dx gather-combine (bit-exact) and the router-logit gradient are checked over
every token.  Bars are the backward's (tests/test_gpu_backward.py).
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import (F32_TOL, assert_grad_close, check_capacity_and_align, host, say)
from mixture_experts_expert_amd import MoEBackwardBuffers, MoEBuffers

pytestmark = pytest.mark.gpu

W = moe_inputs.WORKLOADS["deepseek_wide_n8192_h7168_e256_k8"]


@pytest.fixture(scope="module")
def run():
    say(f"[deepseek backward] generating {W.name} on the GPU")
    T = moe_inputs.make_tensors(W, "cuda")
    dy = moe_inputs.make_dy(W, "cuda")
    buf = MoEBuffers(W.N, W.H, W.I, W.E, W.K, W.F, "cuda")
    bw = MoEBackwardBuffers(buf)
    bw.forward(T["logits"], T["x"], T["w1"], T["w2"])
    bw.backward(dy, T["x"], T["w1"], T["w2"])
    torch.cuda.synchronize()
    say("[deepseek backward] training step done")
    C = oracle.source_capacity(W.N, W.K, W.E, W.F)
    m = check_capacity_and_align(buf, W.N, W.E, W.K, C)
    return T, dy, buf, bw, m


CHUNKS = 8                     # expert chunks of the full GEMM-step check


@pytest.fixture(scope="module")
def host_state(run):
    T, dy, buf, bw, m = run
    return {"x": host(T["x"]), "dy": host(dy)}


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_gemm_steps_every_expert(run, host_state, chunk):
    T, dy, buf, bw, m = run
    Cp = buf.Cp
    ssi, sp = m["sorted_slot_ids"], m["slot_probs"]
    x, dyb = host_state["x"], host_state["dy"]
    per = W.E // CHUNKS
    experts = range(chunk * per, (chunk + 1) * per)
    worst = {}
    for e in experts:
        seg = slice(e * Cp, (e + 1) * Cp)
        ssi_e, sp_e = ssi[seg], sp[seg]
        w1_e, w2_e = host(T["w1"][e:e + 1]), host(T["w2"][e:e + 1])
        pads = ssi_e == W.N
        g_pre, g_dact, g_act = host(bw.preact[seg]), host(bw.d_act[seg]), host(bw.act_re[seg])
        g_dpre, g_dprob, g_da = host(bw.d_preact[seg]), host(bw.d_prob[seg]), host(bw.d_a[seg])
        checks = [
            (g_pre, oracle.fc1_preact_slots(x, w1_e, ssi_e, 1, Cp), "preact", {}),
            (g_dact, oracle.fc2_dgrad(dyb, w2_e, ssi_e, 1, Cp), "d_act", {}),
        ]
        r_act, r_dpre, r_dprob = oracle.swiglu_backward(g_pre, g_dact, sp_e)
        checks += [
            (g_act, r_act, "act recomputed", {}),
            (g_dpre, r_dpre, "d_preact", {}),
            (g_dprob, r_dprob, "d_prob", dict(rtol=F32_TOL, atol_rms=F32_TOL, norm_tol=F32_TOL)),
            (g_da, oracle.fc1_dgrad(g_dpre, w1_e, 1, Cp), "d_a", {}),
            (host(bw.dw2[e]), oracle.fc2_wgrad(dyb, g_act, ssi_e, 1, Cp)[0], "dW2", {}),
            (host(bw.dw1[e]), oracle.fc1_wgrad(g_dpre, x, ssi_e, 1, Cp)[0], "dW1", {}),
        ]
        for g, r, name, kw in checks:
            worst[name] = max(worst.get(name, 0.0), assert_grad_close(g, r, f"{name} e{e}", quiet=True, **kw))
        for name, v in (("d_act", g_dact), ("act", g_act), ("d_preact", g_dpre), ("d_a", g_da)):
            assert np.all(v[pads] == 0), f"{name} e{e}: pad rows must be zero"
        assert np.all(g_dprob[pads] == 0)
    say(f"  experts {experts.start}..{experts.stop - 1}: every GEMM step checked; worst normwise "
        + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))


def test_dx_and_router_gradient_all_tokens(run):
    T, dy, buf, bw, m = run
    g_dx = host(bw.dx)
    assert np.array_equal(g_dx, oracle.gather_combine(host(bw.d_a), m["token_routes"], W.N)), \
        "dx gather-combine differs"
    r_dl = oracle.route_backward(host(buf.topk_ids), host(buf.topk_probs), m["token_routes"],
                                 host(bw.d_prob), W.E)
    assert_grad_close(host(bw.d_logits), r_dl, "d_logits (route bwd)", rtol=F32_TOL,
                      atol_rms=F32_TOL, norm_tol=F32_TOL)

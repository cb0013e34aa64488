"""Pins for the oracle's backward (oracle.backward).

The backward formulas are checked against things other than themselves:

* central finite differences of a scalar loss L = sum(dy * y), with y the
  layer's forward written out here independently, token by token, in float64
  with the discrete choices (top-K ids, kept routes) frozen;
* torch autograd of the same loss in float64 (a different derivation path);
* closed forms: router-logit gradients sum to zero per token and vanish for
  K = 1; dropped routes and pad slots receive nothing;
* the recompute of the gated activation from the saved pre-activation
  reproduces the forward's activation bit for bit.

A dropped term, a wrong sign, a transposed weight or a missing probability
factor anywhere in the backward fails one of the gradient comparisons.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle


def _problem(N=6, H=8, I=4, E=3, K=2, F=0.5, seed=7):
    """Tiny float64 problem with drops (F < 1) and pad slots (Cp = 32 > C)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H))
    w1 = rng.standard_normal((E, 2 * I, H)) * 0.4
    w2 = rng.standard_normal((E, H, I)) * 0.4
    logits = rng.standard_normal((N, E)).astype(np.float32)
    dy = rng.standard_normal((N, H))
    fwd = oracle.forward(logits, oracle.f64_to_bf16_bits(x), oracle.f64_to_bf16_bits(w1),
                         oracle.f64_to_bf16_bits(w2), K, F)
    ids = fwd["topk_ids"]
    kept = fwd["token_routes"] >= 0
    return dict(x=x, w1=w1, w2=w2, logits=logits.astype(np.float64), dy=dy, ids=ids, kept=kept,
                fwd=fwd, K=K, E=E, I=I)


def _softmax_chosen(logits, ids):
    ch = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    ex = np.exp(ch - ch.max(axis=1, keepdims=True))
    return ex / ex.sum(axis=1, keepdims=True)


def _loss(x, w1, w2, logits, ids, kept, dy):
    """L = sum_t dy[t] . y[t], y[t] = sum over kept k of
    W2[e] (silu(W1g[e] x[t]) * (W1u[e] x[t]) * p[t, k]), e = ids[t, k]."""
    p = _softmax_chosen(logits, ids)
    I = w1.shape[1] // 2
    L = 0.0
    for t in range(x.shape[0]):
        for k in range(ids.shape[1]):
            if not kept[t, k]:
                continue
            e = ids[t, k]
            h = w1[e] @ x[t]
            g, u = h[:I], h[I:]
            a = g / (1.0 + np.exp(-g)) * u * p[t, k]
            L += dy[t] @ (w2[e] @ a)
    return L


def _exact_backward(P):
    """The oracle's exact-mode backward on float64 inputs, with the float64
    top-K softmax in place of the float32 forward probabilities."""
    fwd = dict(P["fwd"])
    p64 = _softmax_chosen(P["logits"], P["ids"])
    fwd["topk_probs"] = p64
    sp = np.zeros(len(fwd["slot_probs"]))
    tr = fwd["token_routes"]
    sp[tr[tr >= 0]] = p64[tr >= 0]
    fwd["slot_probs"] = sp
    return oracle.backward(fwd, P["x"], P["w1"], P["w2"], P["dy"], exact=True)


def _fd(f, v, eps=1e-6):
    g = np.zeros_like(v)
    it = np.nditer(v, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = v[i]
        v[i] = old + eps
        lp = f()
        v[i] = old - eps
        lm = f()
        v[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


def test_backward_matches_finite_differences():
    P = _problem()
    assert (~P["kept"]).any(), "the problem must drop routes"
    B = _exact_backward(P)
    f = lambda: _loss(P["x"], P["w1"], P["w2"], P["logits"], P["ids"], P["kept"], P["dy"])  # noqa: E731
    for name, key in (("x", "dx"), ("w1", "dw1"), ("w2", "dw2"), ("logits", "d_logits")):
        fd = _fd(f, P[name])
        np.testing.assert_allclose(B[key], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_backward_matches_torch_autograd():
    P = _problem(N=10, H=16, I=8, E=4, K=3, F=0.75, seed=3)
    B = _exact_backward(P)
    tx = {k: torch.tensor(P[k], dtype=torch.float64, requires_grad=True)
          for k in ("x", "w1", "w2", "logits")}
    ids = torch.tensor(P["ids"], dtype=torch.int64)
    kept = torch.tensor(P["kept"])
    p = torch.softmax(torch.gather(tx["logits"], 1, ids), dim=1)
    I = P["I"]
    y = torch.zeros(P["x"].shape, dtype=torch.float64)
    for t in range(P["x"].shape[0]):
        for k in range(P["K"]):
            if kept[t, k]:
                e = int(ids[t, k])
                h = tx["w1"][e] @ tx["x"][t]
                a = torch.nn.functional.silu(h[:I]) * h[I:] * p[t, k]
                y[t] = y[t] + tx["w2"][e] @ a
    (y * torch.tensor(P["dy"])).sum().backward()
    for name, key in (("x", "dx"), ("w1", "dw1"), ("w2", "dw2"), ("logits", "d_logits")):
        np.testing.assert_allclose(B[key], tx[name].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)


def test_pads_and_dropped_routes_receive_nothing():
    P = _problem()
    B = _exact_backward(P)
    fwd = P["fwd"]
    pad = fwd["sorted_slot_ids"] == P["x"].shape[0]
    assert pad.any()
    for k in ("preact", "d_act", "act", "d_preact", "d_a"):
        assert np.all(B[k][pad] == 0.0), k
    assert np.all(B["d_prob"][pad] == 0.0)
    # a token whose every route was dropped gets no input gradient
    none = ~P["kept"].any(axis=1)
    assert np.all(B["dx"][none] == 0.0)


def test_logit_gradient_closed_forms():
    P = _problem(N=12, E=5, K=3, F=0.6, seed=11)
    B = _exact_backward(P)
    np.testing.assert_allclose(B["d_logits"].sum(axis=1), 0.0, atol=1e-12)
    outside = np.ones_like(B["d_logits"], dtype=bool)
    np.put_along_axis(outside, P["ids"].astype(np.int64), False, axis=1)
    assert np.all(B["d_logits"][outside] == 0.0)
    # K = 1: the softmax over one logit is constant
    P1 = _problem(N=8, E=4, K=1, F=1.0, seed=5)
    assert np.all(_exact_backward(P1)["d_logits"] == 0.0)


def test_recomputed_activation_equals_forward_activation():
    w = moe_inputs.WORKLOADS["tiny_n64_h64_e4_k2"]
    T = moe_inputs.make_tensors(w, "cpu")
    x, w1, w2 = (moe_inputs.bf16_bits(T[k]) for k in ("x", "w1", "w2"))
    fwd = oracle.forward(T["logits"].numpy(), x, w1, w2, w.K, w.F)
    Cp = fwd["Cp"]
    for e in range(w.E):
        seg = slice(e * Cp, (e + 1) * Cp)
        rows = fwd["sorted_slot_ids"][seg]
        a = np.zeros((Cp, w.H), np.uint16)
        a[rows < w.N] = x[rows[rows < w.N]]
        h = oracle.fc1_preact(a, w1[e], exact=True)
        act, _, _ = oracle.swiglu_backward(h, np.zeros((Cp, w.I)), fwd["slot_probs"][seg])
        assert np.array_equal(act, fwd["act"][seg])


def test_rounded_backward_close_to_exact():
    """The bf16 rounding points move each result by about a bf16 ulp."""
    w = moe_inputs.WORKLOADS["tiny_n64_h64_e4_k2"]
    T = moe_inputs.make_tensors(w, "cpu")
    x, w1, w2 = (moe_inputs.bf16_bits(T[k]) for k in ("x", "w1", "w2"))
    fwd = oracle.forward(T["logits"].numpy(), x, w1, w2, w.K, w.F)
    dy = oracle.f64_to_bf16_bits(np.random.default_rng(0).standard_normal((w.N, w.H)))
    R = oracle.backward(fwd, x, w1, w2, dy)
    X = oracle.backward(fwd, x, w1, w2, dy, exact=True)
    for k in ("d_act", "d_preact", "d_a", "dx", "dw1", "dw2"):
        got = oracle.bf16_bits_to_f64(R[k])
        rel = np.linalg.norm(got - X[k]) / np.linalg.norm(X[k])
        assert rel < 1e-2, (k, rel)
    for k in ("d_prob", "d_logits"):
        rel = np.linalg.norm(R[k] - X[k]) / np.linalg.norm(X[k])
        assert rel < 1e-2, (k, rel)


@pytest.mark.parametrize("seed", [0, 1])
def test_swiglu_backward_finite_differences(seed):
    rng = np.random.default_rng(seed)
    M, I = 5, 7
    h = rng.standard_normal((M, 2 * I)) * 2.0
    da = rng.standard_normal((M, I))
    p = rng.uniform(0.1, 1.0, M)

    def act_sum():
        g, u = h[:, :I], h[:, I:]
        return float((da * (g / (1 + np.exp(-g)) * u * p[:, None])).sum())

    _, d_pre, d_prob = oracle.swiglu_backward(h, da, p, exact=True)
    np.testing.assert_allclose(d_pre, _fd(act_sum, h), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(d_prob, _fd(act_sum, p), rtol=1e-6, atol=1e-8)


def test_stepwise_functions_chain_to_grouped_backward():
    """The one-step-at-a-time functions, chained, give grouped_ffn_backward's
    results bit for bit (they are what the GPU parity tests feed)."""
    w = moe_inputs.WORKLOADS["tiny_n64_h64_e4_k2"]
    T = moe_inputs.make_tensors(w, "cpu")
    x, w1, w2 = (moe_inputs.bf16_bits(T[k]) for k in ("x", "w1", "w2"))
    fwd = oracle.forward(T["logits"].numpy(), x, w1, w2, w.K, w.F)
    dy = moe_inputs.bf16_bits(moe_inputs.make_dy(w, "cpu"))
    ssi, sp, E, Cp = fwd["sorted_slot_ids"], fwd["slot_probs"], w.E, fwd["Cp"]
    G = oracle.grouped_ffn_backward(x, dy, w1, w2, ssi, sp, E, Cp)
    pre = oracle.fc1_preact_slots(x, w1, ssi, E, Cp)
    assert np.array_equal(pre, G["preact"])
    d_act = oracle.fc2_dgrad(dy, w2, ssi, E, Cp)
    assert np.array_equal(d_act, G["d_act"])
    act, d_pre, d_prob = oracle.swiglu_backward(pre, d_act, sp)
    assert np.array_equal(act, G["act"]) and np.array_equal(d_pre, G["d_preact"])
    assert np.array_equal(d_prob, G["d_prob"])
    assert np.array_equal(oracle.fc1_dgrad(d_pre, w1, E, Cp), G["d_a"])
    assert np.array_equal(oracle.fc2_wgrad(dy, act, ssi, E, Cp), G["dw2"])
    assert np.array_equal(oracle.fc1_wgrad(d_pre, x, ssi, E, Cp), G["dw1"])


def test_main_grad_accumulation_is_linear_over_micro_batches():
    """Accumulating two micro-batches' weight gradients into a zero main
    gradient gives the weight gradient of both batches' slots contracted at
    once (each expert's segments of the two batches stacked into one
    contraction of 2*Cp slots); a non-zero starting main gradient is carried
    through unchanged."""
    rng = np.random.default_rng(7)
    N, H, I, E, Cp = 20, 8, 6, 3, 4

    def bf(a):
        return moe_inputs.bf16_bits(torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16))

    x = [bf(rng.standard_normal((N, H))) for _ in range(2)]
    dy = [bf(rng.standard_normal((N, H))) for _ in range(2)]
    dpre = [bf(rng.standard_normal((E * Cp, 2 * I))) for _ in range(2)]
    act = [bf(rng.standard_normal((E * Cp, I))) for _ in range(2)]
    ssi = [rng.integers(0, N + 1, E * Cp).astype(np.int32) for _ in range(2)]   # N: pad slot
    main1 = rng.standard_normal((E, 2 * I, H)).astype(np.float32)
    main2 = rng.standard_normal((E, H, I)).astype(np.float32)
    acc1 = oracle.main_grad_accumulate(np.zeros_like(main1), oracle.fc1_wgrad_sum(dpre[0], x[0], ssi[0], E, Cp))
    acc1 = oracle.main_grad_accumulate(acc1, oracle.fc1_wgrad_sum(dpre[1], x[1], ssi[1], E, Cp))
    acc2 = oracle.main_grad_accumulate(main2, oracle.fc2_wgrad_sum(dy[0], act[0], ssi[0], E, Cp))
    acc2 = oracle.main_grad_accumulate(acc2, oracle.fc2_wgrad_sum(dy[1], act[1], ssi[1], E, Cp))
    # both batches as one contraction: token rows of batch b offset by b*N
    # (pads keep pointing at a zero row, index 2N)
    xs, dys = np.concatenate(x), np.concatenate(dy)

    def stack(a):
        return np.concatenate([np.concatenate([a[0][e * Cp:(e + 1) * Cp], a[1][e * Cp:(e + 1) * Cp]])
                               for e in range(E)])

    ss = [np.where(ssi[b] == N, 2 * N, ssi[b] + b * N) for b in range(2)]
    both1 = oracle.fc1_wgrad_sum(stack(dpre), xs, stack(ss), E, 2 * Cp)
    both2 = oracle.fc2_wgrad_sum(dys, stack(act), stack(ss), E, 2 * Cp)
    np.testing.assert_allclose(acc1, both1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(acc2, main2.astype(np.float64) + both2, rtol=1e-12, atol=1e-12)
    # and the bf16 forms are these sums rounded
    assert np.array_equal(oracle.fc1_wgrad(dpre[0], x[0], ssi[0], E, Cp),
                          oracle.f64_to_bf16_bits(oracle.fc1_wgrad_sum(dpre[0], x[0], ssi[0], E, Cp)))

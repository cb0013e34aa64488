"""Plain CPU definition of the backward of the permute-free MoE FFN layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, float64
arithmetic; bf16 values are carried as uint16 bit patterns.

Page followed: [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)",
section 3 (FC1 dgrad reduces the input gradient to token rows with the
gather-combine; FC2 dgrad gathers the token-space gradient into the route
buffer), section 5 (data-gradient GEMMs against the transposed-weight view;
weight-gradient GEMMs that contract over the slot axis, one owner per dW
tile) and section 6 (only the 2I pre-activation persists across the
forward/backward boundary; the backward recomputes the gated activation from
it and differentiates it, route-probability gradient included, in one pass).

What the backward computes, for upstream gradient dy [N, H] of y:

====================  ================================================  =====================
function              what it computes                                  pinned by
====================  ================================================  =====================
fc1_preact            saved pre-activation h = x[row] @ W1[e]^T, bf16   identity with the
                                                                        forward's FC1 product
swiglu_backward       act recomputed from h; d(gate), d(up), d(prob)    finite differences,
                                                                        autograd (exact mode)
expert_backward       one expert: FC2 dgrad, SwiGLU bwd, FC1 dgrad,     finite differences,
                      both weight gradients                             autograd (exact mode)
grouped_ffn_backward  every expert over the route list                  as above
route_backward        softmax-over-top-K gradient of the router logits  finite differences,
                                                                        zero row sums, K = 1
main_grad_accumulate  a float32 main gradient plus a weight gradient    linearity over
                      (section 5: the weight-gradient GEMM can add      micro-batches
                      into a float32 main gradient inside the kernel)
backward              the whole layer: dx, dW1, dW2, d_logits           finite differences,
                                                                        autograd (exact mode)
====================  ================================================  =====================

Rounding points (``exact=False``, the form the GPU path is compared with):
the saved pre-activation, the FC2 data gradient d_act, the recomputed
activation, the pre-activation gradient, each route's input gradient and
both weight gradients are stored as bf16 (float64 -> float32 -> bf16, each
nearest-even); the probability gradient and the logit gradient as float32;
dx is the forward's gather-combine of the routes' input gradients.  With
``exact=True`` nothing is rounded and every function returns float64, which
is the form the finite-difference and autograd pins check.

The discrete choices (top-K selection, capacity selection) are piecewise
constant, so they pass no gradient: a dropped route contributes nothing,
and a logit outside its token's top K gets zero.
"""

from __future__ import annotations

import numpy as np

from .moe import bf16_bits_to_f64, f64_to_bf16_bits, gather_combine, silu


def _rnd(v, exact: bool):
    """The value a bf16 store keeps, as float64 (identity when exact)."""
    v = np.asarray(v, dtype=np.float64)
    return v if exact else bf16_bits_to_f64(f64_to_bf16_bits(v))


def _out(v, exact: bool):
    """Result form: float64 when exact, else bf16 bit patterns."""
    return np.asarray(v, dtype=np.float64) if exact else f64_to_bf16_bits(v)


def _f64(v):
    """bf16 bit patterns -> float64; float arrays pass through as float64."""
    v = np.asarray(v)
    return bf16_bits_to_f64(v) if v.dtype == np.uint16 else v.astype(np.float64)


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def fc1_preact(a, w1_e, exact: bool = False):
    """[PF] section 6: FC1 emits the raw [gate | up] pre-activation, the one
    tensor kept for the backward.  h = a @ W1[e]^T in float64, stored bf16."""
    h = _f64(a) @ _f64(w1_e).T
    return _out(h, exact)


def swiglu_backward(preact, d_act, p, exact: bool = False):
    """[PF] section 6, the gated-activation recompute and backward in one pass.

    From the saved pre-activation (gate g = h[:, :I], up u = h[:, I:]) and
    the gradient d_act of act = silu(g) * u * p:

        act    = silu(g) * u * p                           (recomputed)
        d_gate = d_act * p * u * silu'(g),  silu'(g) = s * (1 + g * (1 - s)),
                                             s = sigmoid(g)
        d_up   = d_act * p * silu(g)
        d_prob = sum over columns of d_act * silu(g) * u

    Returns (act, d_preact = [d_gate | d_up], d_prob) with act and d_preact
    bf16 (float64 when exact) and d_prob float32 (float64 when exact).
    """
    h = _f64(preact)
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    da = _f64(d_act)
    p = np.asarray(p, dtype=np.float64)[:, None]
    s = sigmoid(g)
    sg = silu(g)
    act = sg * u * p
    d_gate = da * p * u * (s * (1.0 + g * (1.0 - s)))
    d_up = da * p * sg
    d_prob = (da * sg * u).sum(axis=1)
    d_pre = np.concatenate([d_gate, d_up], axis=1)
    d_prob = d_prob if exact else d_prob.astype(np.float32)
    return _out(act, exact), _out(d_pre, exact), d_prob


def expert_backward(a, dout, w1_e, w2_e, p, exact: bool = False):
    """One expert's backward on rows already gathered ([PF] sections 3 and 5).

    a     [M, H]   the expert's gathered input rows (zeros for pads)
    dout  [M, H]   the gradient of its FC2 output rows: the token-space
                   gradient dy gathered by the same route list (zeros for pads)
    w1_e  [2I, H], w2_e [H, I], p [M]

    Steps, each a plain product:
        h       = a @ W1^T                         saved pre-activation
        d_act   = dout @ W2                        FC2 data gradient
        act, d_h, d_prob = swiglu_backward(h, d_act, p)
        d_a     = d_h @ W1                         FC1 data gradient
        dW2     = dout^T @ act                     FC2 weight gradient [H, I]
        dW1     = d_h^T @ a                        FC1 weight gradient [2I, H]
    """
    af = _f64(a)
    do = _f64(dout)
    w1 = _f64(w1_e)
    w2 = _f64(w2_e)
    h = _rnd(af @ w1.T, exact)
    d_act = _rnd(do @ w2, exact)
    act, d_h, d_prob = swiglu_backward(h, d_act, p, exact=True)
    act = _rnd(act, exact)
    d_h = _rnd(d_h, exact)
    d_a = d_h @ w1
    dw2 = do.T @ act
    dw1 = d_h.T @ af
    return dict(preact=_out(h, exact), d_act=_out(d_act, exact), act=_out(act, exact),
                d_preact=_out(d_h, exact),
                d_prob=d_prob if exact else np.asarray(d_prob).astype(np.float32),
                d_a=_out(d_a, exact), dw1=_out(dw1, exact), dw2=_out(dw2, exact))


def grouped_ffn_backward(x, dy, w1, w2, sorted_slot_ids, slot_probs, E: int, Cp: int,
                         exact: bool = False):
    """Every expert's backward over the fixed-capacity route list: slot s
    belongs to expert s // Cp and names token row sorted_slot_ids[s] (the
    sentinel N for pads, whose rows of x and dy read as zeros).  Returns the
    per-slot arrays [E*Cp, ...] and the weight gradients dw1 [E, 2I, H],
    dw2 [E, H, I]."""
    xf = _f64(x)
    dyf = _f64(dy)
    N, H = xf.shape
    I = np.asarray(w1[0]).shape[0] // 2
    R = E * Cp
    ssi = np.asarray(sorted_slot_ids)
    per_slot = {k: np.zeros((R, n)) for k, n in
                (("preact", 2 * I), ("d_act", I), ("act", I), ("d_preact", 2 * I), ("d_a", H))}
    d_prob = np.zeros(R)
    dw1 = np.zeros((E, 2 * I, H))
    dw2 = np.zeros((E, H, I))
    for e in range(E):
        seg = slice(e * Cp, (e + 1) * Cp)
        rows = ssi[seg]
        real = rows < N
        a = np.zeros((Cp, H))
        do = np.zeros((Cp, H))
        a[real] = xf[rows[real]]
        do[real] = dyf[rows[real]]
        r = expert_backward(a, do, w1[e], w2[e], np.asarray(slot_probs)[seg], exact=exact)
        for k in per_slot:
            per_slot[k][seg] = _f64(r[k])
        dw1[e] = _f64(r["dw1"])
        dw2[e] = _f64(r["dw2"])
        d_prob[seg] = r["d_prob"]
    out = {k: _out(v, exact) for k, v in per_slot.items()}
    out["d_prob"] = d_prob if exact else d_prob.astype(np.float32)
    out["dw1"] = _out(dw1, exact)
    out["dw2"] = _out(dw2, exact)
    return out


# ---------------------------------------------------------------------------
# The same steps one at a time over the whole route list, each fed whatever
# inputs the caller has (the GPU's own intermediates in the step-wise parity
# tests).  Chained in order they reproduce grouped_ffn_backward exactly.
# ---------------------------------------------------------------------------

def _gather_rows(src, sorted_slot_ids, lo, hi):
    """Rows sorted_slot_ids[lo:hi] of a token-ordered float64 array (zeros
    for the sentinel)."""
    rows = np.asarray(sorted_slot_ids)[lo:hi]
    out = np.zeros((hi - lo, src.shape[1]))
    real = rows < src.shape[0]
    out[real] = src[rows[real]]
    return out


def fc2_dgrad(dy, w2, sorted_slot_ids, E: int, Cp: int):
    """d_act[s] = bf16(dy[row(s)] @ W2[e]) for every slot (bf16 bits)."""
    dyf = _f64(dy)
    I = np.asarray(w2[0]).shape[1]
    out = np.zeros((E * Cp, I))
    for e in range(E):
        out[e * Cp:(e + 1) * Cp] = _gather_rows(dyf, sorted_slot_ids, e * Cp, (e + 1) * Cp) @ _f64(w2[e])
    return f64_to_bf16_bits(out)


def fc1_dgrad(d_preact, w1, E: int, Cp: int):
    """d_a[s] = bf16(d_preact[s] @ W1[e]) for every slot (bf16 bits)."""
    dp = _f64(d_preact)
    H = np.asarray(w1[0]).shape[1]
    out = np.zeros((E * Cp, H))
    for e in range(E):
        out[e * Cp:(e + 1) * Cp] = dp[e * Cp:(e + 1) * Cp] @ _f64(w1[e])
    return f64_to_bf16_bits(out)


def fc2_wgrad_sum(dy, act, sorted_slot_ids, E: int, Cp: int):
    """sum over e's slots of dy[row(s)]^T act[s], float64 [E, H, I], unrounded."""
    dyf = _f64(dy)
    af = _f64(act)
    return np.stack([_gather_rows(dyf, sorted_slot_ids, e * Cp, (e + 1) * Cp).T @ af[e * Cp:(e + 1) * Cp]
                     for e in range(E)])


def fc2_wgrad(dy, act, sorted_slot_ids, E: int, Cp: int):
    """dW2[e] = bf16(sum over e's slots of dy[row(s)]^T act[s]) (bf16 bits)."""
    return f64_to_bf16_bits(fc2_wgrad_sum(dy, act, sorted_slot_ids, E, Cp))


def fc1_wgrad_sum(d_preact, x, sorted_slot_ids, E: int, Cp: int):
    """sum over e's slots of d_preact[s]^T x[row(s)], float64 [E, 2I, H], unrounded."""
    dp = _f64(d_preact)
    xf = _f64(x)
    return np.stack([dp[e * Cp:(e + 1) * Cp].T @ _gather_rows(xf, sorted_slot_ids, e * Cp, (e + 1) * Cp)
                     for e in range(E)])


def fc1_wgrad(d_preact, x, sorted_slot_ids, E: int, Cp: int):
    """dW1[e] = bf16(sum over e's slots of d_preact[s]^T x[row(s)]) (bf16 bits)."""
    return f64_to_bf16_bits(fc1_wgrad_sum(d_preact, x, sorted_slot_ids, E, Cp))


def main_grad_accumulate(main, dw_sum):
    """A float32 main gradient after a weight gradient is added into it
    ([PF] section 5: the weight-gradient GEMM writes bf16 or accumulates into
    a float32 main gradient): main + dW, in float64 (main: float32 values,
    dw_sum: the unrounded sums of fc1_wgrad_sum / fc2_wgrad_sum).  Over
    micro-batches this is gradient accumulation: the sum of the batches'
    weight gradients."""
    return np.asarray(main, dtype=np.float64) + np.asarray(dw_sum, dtype=np.float64)


def fc1_preact_slots(x, w1, sorted_slot_ids, E: int, Cp: int):
    """The saved pre-activation of every slot: bf16(x[row(s)] @ W1[e]^T)."""
    xf = _f64(x)
    I2 = np.asarray(w1[0]).shape[0]
    out = np.zeros((E * Cp, I2))
    for e in range(E):
        out[e * Cp:(e + 1) * Cp] = _gather_rows(xf, sorted_slot_ids, e * Cp, (e + 1) * Cp) @ _f64(w1[e]).T
    return f64_to_bf16_bits(out)


def route_backward(ids, probs, token_routes, d_prob_slots, E: int, exact: bool = False):
    """Gradient of the router logits through the softmax over the top K.

    Route (t, k) takes dp[t, k] = d_prob_slots[token_routes[t, k]] if it was
    kept, else 0 (a dropped route does not reach y).  With p the top-K
    softmax, d logit[t, ids[t, k]] = p_k * (dp_k - sum_j p_j dp_j) (the
    softmax Jacobian, float64); every other logit gets 0.  float32 result
    (float64 when exact).
    """
    ids = np.asarray(ids, dtype=np.int64)
    p = np.asarray(probs, dtype=np.float64)
    tr = np.asarray(token_routes, dtype=np.int64)
    dps = np.asarray(d_prob_slots, dtype=np.float64)
    N, K = ids.shape
    dp = np.where(tr >= 0, dps[np.maximum(tr, 0)], 0.0)
    inner = (p * dp).sum(axis=1, keepdims=True)
    g = p * (dp - inner)
    d_logits = np.zeros((N, E))
    np.put_along_axis(d_logits, ids, g, axis=1)
    return d_logits if exact else d_logits.astype(np.float32)


def backward(fwd, x, w1, w2, dy, exact: bool = False):
    """The layer's backward given the forward's routing state ``fwd`` (the
    dict ``oracle.forward`` returns: topk_ids, topk_probs, the route list,
    its inverse and Cp).  Returns the per-slot intermediates plus

        dx        [N, H]      gather-combine of the routes' input gradients
                              ([PF] section 3: FC1 dgrad reduces to token rows
                              contention-free)
        dw1, dw2              weight gradients
        d_logits  [N, E]      router-logit gradient
    """
    E = len(w1)
    N = np.asarray(x).shape[0]
    g = grouped_ffn_backward(x, dy, w1, w2, fwd["sorted_slot_ids"], fwd["slot_probs"], E,
                             fwd["Cp"], exact=exact)
    tr = fwd["token_routes"]
    if exact:
        dx = np.zeros((N, g["d_a"].shape[1]))
        for k in range(tr.shape[1]):
            sel = tr[:, k] >= 0
            dx[sel] += g["d_a"][tr[sel, k]]
    else:
        dx = gather_combine(g["d_a"], tr, N)
    g["dx"] = dx
    g["d_logits"] = route_backward(fwd["topk_ids"], fwd["topk_probs"], tr, g["d_prob"], E,
                                   exact=exact)
    return g

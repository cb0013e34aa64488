"""Pins for the oracle's align, FFN and gather-combine steps."""

import math

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from conftest import load_golden


def bits_of(values):
    return oracle.f64_to_bf16_bits(np.asarray(values, np.float64))


# ---------------------------------------------------------------- hand-worked example

def test_worked_example_route_and_align():
    g = load_golden("worked_example_route_align.json")
    lg = np.array(g["logits"], np.float32)
    N, E, K, F, BM = g["N"], g["E"], g["K"], g["F"], g["BM"]
    C = oracle.source_capacity(N, K, E, F)
    assert C == g["C"] and oracle.padded_capacity(C, BM) == g["Cp"]
    ids, probs = oracle.route_topk(lg, K)
    assert ids.tolist() == g["topk_ids"]
    for t, gap in enumerate(g["topk_prob_gaps"]):
        p0 = 1.0 / (1.0 + math.exp(-gap))          # logistic of the logit gap
        np.testing.assert_allclose(probs[t], [p0, 1.0 - p0], rtol=2.0 ** -23, atol=0)
    slot, count = oracle.capacity_select(ids, probs, E, C)
    assert slot.tolist() == g["route_slot"]
    assert count.tolist() == g["expert_count"]
    m = oracle.align(ids, probs, slot, count, N, E, C, BM)
    assert m["sorted_slot_ids"].tolist() == g["sorted_slot_ids"]
    assert m["token_routes"].tolist() == g["token_routes"]
    assert m["token_route_count"].tolist() == g["token_route_count"]
    assert m["expert_ids"].tolist() == g["expert_ids"]
    assert m["block_start"].tolist() == g["block_start"]
    assert int(m["num_tokens_post_padded"][0]) == g["num_tokens_post_padded"]
    for s, src in enumerate(g["slot_prob_source"]):
        if src is None:
            assert m["slot_probs"][s] == 0.0 and not np.signbit(m["slot_probs"][s])
        else:
            assert m["slot_probs"][s] == probs[src[0], src[1]]


# ---------------------------------------------------------------- layout invariants

@pytest.mark.parametrize("name,BM", [("tiny_n64_h64_e4_k2", 32), ("tiny_n64_h64_e4_k2", 48),
                                     ("small_qwen3moe_n1024_h512_e8_k2", 32),
                                     ("qwen3_30b_a3b_n4096_h2048_e128_k8", 32)])
def test_align_invariants(name, BM):
    w = moe_inputs.WORKLOADS[name]
    lg = moe_inputs.make_logits(w.N, w.E, w.seed)
    C = oracle.source_capacity(w.N, w.K, w.E, w.F)
    ids, probs = oracle.route_topk(lg, w.K)
    slot, count = oracle.capacity_select(ids, probs, w.E, C)
    m = oracle.align(ids, probs, slot, count, w.N, w.E, C, BM)
    Cp = m["Cp"]
    assert Cp % BM == 0 and C <= Cp < C + BM
    ssi, sp, tr = m["sorted_slot_ids"], m["slot_probs"], m["token_routes"]
    assert len(ssi) == w.E * Cp and int(m["num_tokens_post_padded"][0]) == w.E * Cp
    for e in range(w.E):
        seg = ssi[e * Cp:(e + 1) * Cp]
        ps = sp[e * Cp:(e + 1) * Cp]
        real = seg < w.N
        # exactly count real slots first, then pads: Cp slots per expert
        assert real.sum() == count[e] and real[:count[e]].all()
        assert np.all(seg[~real] == w.N)
        assert np.all(ps[~real] == 0) and not np.signbit(ps[~real]).any()
        assert np.all(np.diff(seg[real]) > 0)          # ascending tokens
        assert np.all(ps[real] > 0)
    # inverse map
    t_idx, k_idx = np.nonzero(tr >= 0)
    assert np.array_equal(ssi[tr[t_idx, k_idx]], t_idx)
    assert np.array_equal(sp[tr[t_idx, k_idx]], probs[t_idx, k_idx])
    assert np.array_equal(tr[t_idx, k_idx] // Cp, ids[t_idx, k_idx])
    assert len(np.unique(tr[tr >= 0])) == (tr >= 0).sum() == (ssi < w.N).sum()
    assert np.array_equal(m["token_route_count"], (tr >= 0).sum(1))
    assert np.array_equal(m["expert_ids"], np.repeat(np.arange(w.E), Cp // BM))
    assert np.array_equal(m["block_start"] * BM, np.arange(w.E) * Cp)


# ---------------------------------------------------------------- bf16 helpers and SiLU

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38]])
    ours = oracle.f64_to_bf16_bits(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_silu_matches_torch():
    g = np.linspace(-30, 30, 4001)
    np.testing.assert_allclose(oracle.moe.silu(g),
                               torch.nn.functional.silu(torch.from_numpy(g)).numpy(),
                               rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- FFN pins

def _relerr(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_single_expert_equals_library_swiglu_ffn():
    """E=1, K=1: every token routes to the one expert with p=1 and C >= N, so
    y is a plain SwiGLU FFN; compare with torch's silu and float64 matmuls."""
    N, H, I = 48, 64, 96
    gen = torch.Generator().manual_seed(5)
    x = torch.randn(N, H, generator=gen).to(torch.bfloat16)
    w1 = (torch.randn(1, 2 * I, H, generator=gen) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(1, H, I, generator=gen) * 0.05).to(torch.bfloat16)
    lg = np.zeros((N, 1), np.float32)
    o = oracle.forward(lg, moe_inputs.bf16_bits(x), moe_inputs.bf16_bits(w1),
                       moe_inputs.bf16_bits(w2), K=1, F=1.0)
    assert o["C"] == N and (o["token_routes"][:, 0] == np.arange(N)).all()
    xd, wg, wu, wd = x.double(), w1[0, :I].double(), w1[0, I:].double(), w2[0].double()
    ref = ((torch.nn.functional.silu(xd @ wg.T) * (xd @ wu.T)) @ wd.T).numpy()
    y = oracle.bf16_bits_to_f64(o["y"])
    assert _relerr(y, ref) < 8e-3           # two bf16 roundings (act, out)
    assert np.max(np.abs(y - ref)) <= 2e-2 * np.max(np.abs(ref))
    # the swapped-SwiGLU mistake is far outside that bound
    swapped = ((torch.nn.functional.silu(xd @ wu.T) * (xd @ wg.T)) @ wd.T).numpy()
    assert _relerr(y, swapped) > 0.3


def _tiny_inputs(name="tiny_n64_h64_e4_k2"):
    w = moe_inputs.WORKLOADS[name]
    T = moe_inputs.make_tensors(w, "cpu")
    return w, T["logits"].numpy(), moe_inputs.bf16_bits(T["x"]), \
        moe_inputs.bf16_bits(T["w1"]), moe_inputs.bf16_bits(T["w2"])


def test_permuted_equals_permute_free_bitwise():
    w, lg, x, w1, w2 = _tiny_inputs()
    o = oracle.forward(lg, x, w1, w2, w.K, w.F)
    assert (o["token_routes"] < 0).sum() > 0             # the tiny layer drops a route
    yp = oracle.permuted_forward(x, w1, w2, o, w.E)
    assert np.array_equal(yp, o["y"])


def test_dispatch_rows_invert_the_route_list():
    """The route-ordered copy holds, for every kept route (t, k), token t's
    row at the slot the inverse map names; pads are zero rows; each token's
    row appears once per kept route and nowhere else."""
    w, lg, x, w1, w2 = _tiny_inputs()
    o = oracle.forward(lg, x, w1, w2, w.K, 1.5)
    rows = oracle.dispatch_rows(x, o["sorted_slot_ids"])
    assert rows.shape == (w.E * o["Cp"], w.H)
    tr = o["token_routes"]
    filled = np.zeros(rows.shape[0], bool)
    for t in range(w.N):
        for k in range(w.K):
            s = tr[t, k]
            if s >= 0:
                assert np.array_equal(rows[s], x[t])
                filled[s] = True
    assert filled.sum() == (tr >= 0).sum()                   # one slot per kept route
    pads = ~filled
    assert pads.sum() > 0 and np.all(rows[pads] == 0)
    # a token row with a nonzero value is found exactly where its routes went
    assert np.array_equal(np.flatnonzero(filled), np.flatnonzero(o["sorted_slot_ids"] < w.N))


def test_ffn_on_dispatched_rows_equals_permute_free():
    """An expert-parallel rank runs the grouped FFN on received rows with
    the identity route list; on the dispatched copy that must equal the
    permute-free FFN over the original route list, bit for bit."""
    w, lg, x, w1, w2 = _tiny_inputs()
    o = oracle.forward(lg, x, w1, w2, w.K, w.F)
    rows = oracle.dispatch_rows(x, o["sorted_slot_ids"])
    R = rows.shape[0]
    act, ro = oracle.grouped_ffn(rows, w1, w2, np.arange(R), o["slot_probs"], w.E, o["Cp"])
    assert np.array_equal(act, o["act"]) and np.array_equal(ro, o["route_out"])
    assert np.array_equal(oracle.gather_combine(ro, o["token_routes"], w.N), o["y"])


def test_dense_formulation_no_drops():
    """With C >= every expert's load nothing drops, and the slot machinery
    must reproduce the per-token sum of p * FFN_e(x)."""
    w, lg, x, w1, w2 = _tiny_inputs()
    F = w.E / w.K                                         # C = N
    o = oracle.forward(lg, x, w1, w2, w.K, F)
    assert (o["token_routes"] >= 0).all()
    ref = oracle.dense_forward(x, w1, w2, o["topk_ids"], o["topk_probs"])
    y = oracle.bf16_bits_to_f64(o["y"])
    assert _relerr(y, ref) < 1e-2
    # elementwise: bf16 rounding of act, of each route row and of y, where
    # route terms may cancel, so the absolute part scales with the rms
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(y - ref) <= 2e-2 * np.abs(ref) + 5e-2 * rms)
    # a forgotten probability, or a route fetched from the wrong slot, is far off
    noprob = oracle.dense_forward(x, w1, w2, o["topk_ids"], np.ones_like(o["topk_probs"]))
    assert _relerr(y, noprob) > 0.2


def test_dense_formulation_with_drops():
    """Dropped routes contribute nothing: the dense sum over kept routes only."""
    w, lg, x, w1, w2 = _tiny_inputs()
    o = oracle.forward(lg, x, w1, w2, w.K, 0.5)
    dropped = o["token_routes"] < 0
    assert dropped.sum() > 0
    p = o["topk_probs"].copy()
    p[dropped] = 0.0
    ref = oracle.dense_forward(x, w1, w2, o["topk_ids"], p)
    y = oracle.bf16_bits_to_f64(o["y"])
    assert _relerr(y, ref) < 1e-2
    allroutes = oracle.dense_forward(x, w1, w2, o["topk_ids"], o["topk_probs"])
    assert _relerr(y, allroutes) > 0.1


def test_pad_rows_are_zero():
    w, lg, x, w1, w2 = _tiny_inputs()
    o = oracle.forward(lg, x, w1, w2, w.K, 1.5)
    pads = o["sorted_slot_ids"] == w.N
    assert pads.sum() > 0
    assert np.all(o["act"][pads] == 0) and np.all(o["route_out"][pads] == 0)


# ---------------------------------------------------------------- combine

def test_combine_worked_example():
    g = load_golden("worked_example_combine.json")
    ro = bits_of(g["route_out"])
    tr = np.array(g["token_routes"], np.int32)
    y = oracle.gather_combine(ro, tr, len(tr))
    assert np.array_equal(y, bits_of(g["y"]))
    for case in g["rounding_cases"]:
        r = bits_of(np.array(case["routes"])[:, None])
        yy = oracle.gather_combine(r, np.arange(len(r), dtype=np.int32)[None, :], 1)
        v = oracle.bf16_bits_to_f64(yy)[0, 0]
        assert v == case["y"]
        if "sign_bit" in case:
            assert int(np.signbit(v)) == case["sign_bit"]


def test_all_routes_dropped_gives_zero():
    ro = bits_of(np.ones((2, 4)))
    tr = np.array([[-1, -1], [0, 1]], np.int32)
    y = oracle.bf16_bits_to_f64(oracle.gather_combine(ro, tr, 2))
    assert np.all(y[0] == 0) and not np.signbit(y[0]).any()
    assert np.all(y[1] == 2)

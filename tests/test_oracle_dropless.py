"""Pins for the oracle's dropless (dynamic-count) variant, CPU only.

* a hand-worked layout (tests/golden/worked_example_dropless_align.json) for
  two block sizes;
* the static bound in closed form;
* layout invariants on random and skewed routing;
* an independent construction by sorting routes on (expert, token) and
  laying the segments down one by one;
* the end-to-end forward equals the fixed-capacity forward bitwise whenever
  the capacity drops nothing (the same per-route arithmetic on the same
  rows, in a different slot layout).
"""

import numpy as np
import pytest

import moe_inputs
import oracle
from conftest import load_golden


def test_hand_worked_layout():
    g = load_golden("worked_example_dropless_align.json")
    ids = np.array(g["topk_ids"], np.int32)
    probs = np.array(g["topk_probs"], np.float32)
    for c in g["cases"]:
        m = oracle.dropless_align(ids, probs, g["N"], g["E"], c["BM"])
        assert m["R"] == c["R"] == oracle.dropless_bound(g["N"], g["K"], g["E"], c["BM"])
        for k in ("route_counts", "route_within", "sorted_slot_ids", "expert_ids", "block_start",
                  "token_routes", "token_route_count"):
            assert np.array_equal(m[k], np.array(c[k])), (c["BM"], k)
        assert np.array_equal(m["slot_probs"], np.array(c["slot_probs"], np.float32))
        assert int(m["num_tokens_post_padded"][0]) == c["num_tokens_post_padded"]


@pytest.mark.parametrize("N,K,E,BM,want", [(4, 2, 3, 4, 20), (4, 2, 3, 2, 12), (1, 1, 1, 32, 32),
                                           (4096, 8, 128, 32, 32768 + 128 * 31 + 0),
                                           (3, 5, 4, 32, 12 + 124)])
def test_bound_closed_form(N, K, E, BM, want):
    r = N * min(K, E) + E * (BM - 1)
    assert oracle.dropless_bound(N, K, E, BM) == -(-r // BM) * BM
    if want:
        assert oracle.dropless_bound(N, K, E, BM) == -(-want // BM) * BM


def random_routing(N, E, K, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    if skew:
        lg[:, : max(1, E // 8)] += skew
    return oracle.route_topk(lg, K)


def check_invariants(ids, probs, N, E, BM, m):
    K = ids.shape[1]
    R = m["R"]
    counts = np.bincount(ids.ravel(), minlength=E)
    assert np.array_equal(m["route_counts"], counts)
    padded = -(-counts // BM) * BM
    extent = int(m["num_tokens_post_padded"][0])
    assert extent == padded.sum() and extent <= R and R % BM == 0
    ssi, sp, tr = m["sorted_slot_ids"], m["slot_probs"], m["token_routes"]
    # every route kept, at a slot inside its expert's segment, mapping back to its token
    assert np.all(tr >= 0) and np.all(m["token_route_count"] == K)
    bs = m["block_start"].astype(np.int64) * BM
    for t in range(N):
        for k in range(K):
            e, s = ids[t, k], tr[t, k]
            assert bs[e] <= s < bs[e] + counts[e]
            assert ssi[s] == t and sp[s] == probs[t, k]
    # segments contiguous in expert order; tokens ascend inside; pads and tail are sentinels
    assert bs[0] == 0 and np.array_equal(bs[1:], np.cumsum(padded)[:-1])
    for e in range(E):
        seg = ssi[bs[e]:bs[e] + counts[e]]
        assert np.all(np.diff(seg) > 0)
        pads = slice(bs[e] + counts[e], bs[e] + padded[e])
        assert np.all(ssi[pads] == N) and np.all(sp[pads] == 0)
    assert np.all(ssi[extent:] == N) and np.all(sp[extent:] == 0)
    assert np.all(np.signbit(sp[ssi == N]) == False)  # noqa: E712  (+0.0, not -0.0)
    # block owners
    owner = np.repeat(np.arange(E), padded // BM)
    assert np.array_equal(m["expert_ids"][: extent // BM], owner)
    assert np.all(m["expert_ids"][extent // BM:] == -1)


@pytest.mark.parametrize("N,E,K,BM,skew", [(64, 4, 2, 32, 0.0), (300, 16, 4, 32, 0.0),
                                           (257, 10, 3, 8, 2.0), (1000, 100, 7, 32, 0.0),
                                           (50, 8, 8, 4, 0.0), (128, 64, 6, 32, 5.0)])
def test_layout_invariants(N, E, K, BM, skew):
    ids, probs = random_routing(N, E, K, N + E, skew)
    check_invariants(ids, probs, N, E, BM, oracle.dropless_align(ids, probs, N, E, BM))


def test_independent_sort_construction():
    """Build the layout from a (expert, token) sort and a running cursor."""
    for seed, (N, E, K, BM) in enumerate([(40, 5, 2, 4), (77, 9, 3, 8), (16, 16, 16, 2)]):
        ids, probs = random_routing(N, E, K, 100 + seed)
        m = oracle.dropless_align(ids, probs, N, E, BM)
        routes = sorted((int(ids[t, k]), t, k) for t in range(N) for k in range(K))
        ssi = [N] * m["R"]
        tr = [[-1] * K for _ in range(N)]
        cursor, prev = 0, -1
        starts = {}
        for e, t, k in routes:
            if e != prev:
                cursor = (cursor + BM - 1) // BM * BM     # close the previous segment
                for skipped in range(prev + 1, e + 1):
                    starts[skipped] = cursor             # empty experts start here too
                prev = e
            ssi[cursor] = t
            tr[t][k] = cursor
            cursor += 1
        cursor = (cursor + BM - 1) // BM * BM
        for skipped in range(prev + 1, E):
            starts[skipped] = cursor
        assert ssi == m["sorted_slot_ids"].tolist()
        assert tr == m["token_routes"].tolist()
        assert [starts[e] // BM for e in range(E)] == m["block_start"].tolist()
        assert cursor == int(m["num_tokens_post_padded"][0])


@pytest.mark.parametrize("name", ["tiny_n64_h64_e4_k2"])
def test_forward_equals_capacity_forward_without_drops(name):
    w = moe_inputs.WORKLOADS[name]
    T = moe_inputs.make_tensors(w)
    lg = T["logits"].numpy()
    x, w1, w2 = (moe_inputs.bf16_bits(T[k]) for k in ("x", "w1", "w2"))
    F = w.E / w.K                                     # C = N >= any expert's load: nothing drops
    cap = oracle.forward(lg, x, w1, w2, w.K, F)
    assert np.all(cap["token_routes"] >= 0)
    dl = oracle.dropless_forward(lg, x, w1, w2, w.K)
    assert np.array_equal(dl["y"], cap["y"])
    assert np.array_equal(dl["topk_ids"], cap["topk_ids"])
    check_invariants(dl["topk_ids"], dl["topk_probs"], w.N, w.E, oracle.BM_DEFAULT, dl)
    # the FFN rows of each route agree too, slot for slot
    for t in range(w.N):
        for k in range(w.K):
            assert np.array_equal(dl["route_out"][dl["token_routes"][t, k]],
                                  cap["route_out"][cap["token_routes"][t, k]])


def test_ffn_blocks_equals_grouped_ffn_on_fixed_layout():
    """On a fixed-capacity layout (every block owned by e = s // Cp), the
    block-driven FFN is the segment-driven one."""
    w = moe_inputs.WORKLOADS["tiny_n64_h64_e4_k2"]
    T = moe_inputs.make_tensors(w)
    x, w1, w2 = (moe_inputs.bf16_bits(T[k]) for k in ("x", "w1", "w2"))
    o = oracle.forward(T["logits"].numpy(), x, w1, w2, w.K, w.F)
    act, ro = oracle.grouped_ffn_blocks(x, w1, w2, o["sorted_slot_ids"], o["slot_probs"],
                                        o["expert_ids"])
    assert np.array_equal(act, o["act"]) and np.array_equal(ro, o["route_out"])

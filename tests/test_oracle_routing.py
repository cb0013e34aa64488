"""Pins for the oracle's capacity, routing and capacity-selection steps.

Every check here compares the oracle with something other than itself:
hand-derived values, brute-force enumeration, a library softmax, or an
invariant the pages fix.
"""

import itertools

import numpy as np
import pytest
from scipy.special import softmax

import moe_inputs
import oracle
from conftest import load_golden


# ---------------------------------------------------------------- capacity

def test_capacity_closed_form_golden():
    g = load_golden("capacity_closed_form.json")
    for c in g["cases"]:
        assert oracle.source_capacity(c["N"], c["K"], c["E"], c["F"]) == c["C"], c


@pytest.mark.parametrize("args", [(4, 0, 4, 1.0), (4, 5, 4, 1.0), (-1, 1, 4, 1.0),
                                  (4, 1, 4, 0.0), (4, 1, 4, float("nan")),
                                  (4, 1, 4, float("inf")), (4, 1, 0, 1.0)])
def test_capacity_rejects_bad_args(args):
    with pytest.raises(ValueError):
        oracle.source_capacity(*args)


def test_padded_capacity():
    assert oracle.padded_capacity(32, 32) == 32
    assert oracle.padded_capacity(33, 32) == 64
    assert oracle.padded_capacity(0, 32) == 0
    assert oracle.padded_capacity(3, 4) == 4


# ---------------------------------------------------------------- routing

def _brute_topk(row, K):
    """All K-subsets; keep those where every chosen expert beats every other
    (higher logit, or equal logit and lower index).  Exactly one survives."""
    E = len(row)
    ok = []
    for sub in itertools.combinations(range(E), K):
        s = set(sub)
        if all((row[i] > row[j]) or (row[i] == row[j] and i < j)
               for i in s for j in range(E) if j not in s):
            ok.append(sub)
    assert len(ok) == 1
    chosen = sorted(ok[0], key=lambda e: (-row[e], e))
    return chosen


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 6))
    K = int(rng.integers(1, E + 1))
    N = 8
    # integer-valued logits force many exact ties
    lg = rng.integers(-2, 3, size=(N, E)).astype(np.float32)
    ids, probs = oracle.route_topk(lg, K)
    for t in range(N):
        assert list(ids[t]) == _brute_topk(lg[t], K)


def test_topk_float_logits_brute_force():
    lg = moe_inputs.make_logits(16, 6, 11)
    ids, _ = oracle.route_topk(lg, 3)
    for t in range(16):
        assert list(ids[t]) == _brute_topk(lg[t], 3)


def test_probs_equal_renormalised_full_softmax():
    """Top-K softmax equals the library full softmax renormalised over the K."""
    lg = moe_inputs.make_logits(256, 16, 5)
    K = 4
    ids, probs = oracle.route_topk(lg, K)
    full = softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(probs, ref, rtol=2e-7, atol=0)


def test_probs_k_equals_e_is_full_softmax():
    lg = moe_inputs.make_logits(64, 5, 6)
    ids, probs = oracle.route_topk(lg, 5)
    full = softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(probs, np.take_along_axis(full, ids.astype(np.int64), 1),
                               rtol=2e-7, atol=0)


def test_probs_invariants():
    lg = moe_inputs.make_logits(512, 128, 7)
    K = 8
    ids, probs = oracle.route_topk(lg, K)
    assert ids.dtype == np.int32 and probs.dtype == np.float32
    assert np.all(np.abs(probs.astype(np.float64).sum(1) - 1.0) <= K * 2.0 ** -24)
    assert np.all(np.diff(probs, axis=1) <= 0)         # descending in k
    assert np.all(probs > 0)
    for t in range(0, 512, 37):
        assert len(set(ids[t])) == K


def test_k1_probability_is_one():
    lg = moe_inputs.make_logits(32, 4, 8)
    ids, probs = oracle.route_topk(lg, 1)
    assert np.all(probs == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))


# ---------------------------------------------------------------- capacity selection

def _brute_capacity(ids, probs, E, C):
    """Per expert: among all subsets of its candidates of size min(C, load),
    exactly one dominates (every kept (p, -t) key beats every dropped one)."""
    N, K = ids.shape
    slot = np.full((N, K), -1, np.int32)
    for e in range(E):
        cand = [(t, k) for t in range(N) for k in range(K) if ids[t, k] == e]
        m = min(C, len(cand))
        key = {c: (float(probs[c]), -c[0]) for c in cand}
        ok = []
        for sub in itertools.combinations(cand, m):
            s = set(sub)
            if all(key[a] > key[b] for a in s for b in cand if b not in s):
                ok.append(sub)
        assert len(ok) == 1
        for j, (t, k) in enumerate(sorted(ok[0])):   # token order
            slot[t, k] = j
    return slot


@pytest.mark.parametrize("seed,F", [(s, f) for s in range(8) for f in (0.5, 1.0)])
def test_capacity_select_brute_force(seed, F):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 9))
    E = int(rng.integers(2, 5))
    K = int(rng.integers(1, min(2, E) + 1))
    if seed % 2:
        lg = rng.integers(-1, 2, size=(N, E)).astype(np.float32)   # equal probabilities
    else:
        lg = rng.standard_normal((N, E)).astype(np.float32)
    C = oracle.source_capacity(N, K, E, F)
    ids, probs = oracle.route_topk(lg, K)
    slot, count = oracle.capacity_select(ids, probs, E, C)
    assert np.array_equal(slot, _brute_capacity(ids, probs, E, C))
    for e in range(E):
        assert count[e] == min(C, int((ids == e).sum()))


def _check_capacity_invariants(ids, probs, slot, count, E, C):
    N, K = ids.shape
    load = np.bincount(ids.ravel(), minlength=E)
    assert np.array_equal(count, np.minimum(C, load))
    assert (slot >= 0).sum() + (slot < 0).sum() == N * K
    assert (slot >= 0).sum() == count.sum()
    for e in range(E):
        tok, kk = np.nonzero(ids == e)
        s = slot[tok, kk]
        kept = s >= 0
        # slots 0..count-1, ascending with token
        assert np.array_equal(s[kept], np.arange(count[e]))
        if (~kept).any() and kept.any():
            kp = probs[tok[kept], kk[kept]].astype(np.float64)
            dp = probs[tok[~kept], kk[~kept]].astype(np.float64)
            kt, dt = tok[kept], tok[~kept]
            # dominance: min kept key > max dropped key under (p, -t)
            i = np.lexsort((-kt, kp))[0]
            j = np.lexsort((-dt, dp))[-1]
            assert (kp[i], -kt[i]) > (dp[j], -dt[j])


def test_capacity_invariants_qwen_shaped_logits():
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    lg = moe_inputs.make_logits(w.N, w.E, w.seed)
    C = oracle.source_capacity(w.N, w.K, w.E, w.F)
    ids, probs = oracle.route_topk(lg, w.K)
    slot, count = oracle.capacity_select(ids, probs, w.E, C)
    _check_capacity_invariants(ids, probs, slot, count, w.E, C)
    assert 0 < (slot < 0).sum() < 0.1 * w.N * w.K      # some drops, not many


def test_overload_all_tokens_one_expert():
    N, E, K, F = 40, 4, 1, 1.0
    lg = np.zeros((N, E), np.float32)
    lg[:, 2] = 5.0
    C = oracle.source_capacity(N, K, E, F)          # 10
    ids, probs = oracle.route_topk(lg, K)
    slot, count = oracle.capacity_select(ids, probs, E, C)
    assert C == 10 and count[2] == C and count.sum() == C
    assert (slot < 0).sum() == N * K - C
    # equal probabilities (all 1.0): the lowest token indices are kept
    assert np.array_equal(np.nonzero(slot[:, 0] >= 0)[0], np.arange(C))


def test_underload_large_factor_drops_nothing():
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    lg = moe_inputs.make_logits(w.N, w.E, w.seed)
    C = oracle.source_capacity(w.N, w.K, w.E, w.E / w.K)   # C = N
    ids, probs = oracle.route_topk(lg, w.K)
    slot, count = oracle.capacity_select(ids, probs, w.E, C)
    assert C == w.N and (slot >= 0).all()


def test_skew_alpha_gives_target_imbalance(skew_alpha):
    w = moe_inputs.WORKLOADS["skew_zipf_n4096_e128_k8_f1.0"]
    lg = moe_inputs.make_logits(w.N, w.E, w.seed, skew_alpha)
    ids, _ = oracle.route_topk(lg, w.K)
    load = np.bincount(ids.ravel(), minlength=w.E)
    assert abs(load.max() / (w.N * w.K / w.E) - 1.35) <= 0.02

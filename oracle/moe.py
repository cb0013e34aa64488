"""Plain CPU definition of the capacity-padded, permute-free MoE FFN forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, float64
arithmetic wherever the pages leave precision open; bf16 values are carried
as uint16 bit patterns because numpy has no bf16 type.

Pages (cited by title and section):

* [FC] "feat(cuda-graphs): capture fixed-capacity MoE execution", Design notes.
* [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)", sections 1-6.

Steps, in the order the forward runs them:

====================  =====================================  ==============
function              what it computes                       pinned by
====================  =====================================  ==============
source_capacity       C = ceil(N*K*F/E), exact               closed-form values, edge cases
route_topk            top-K experts + softmax over them      brute force, sum-to-one, order
capacity_select       per-expert keep-by-probability         brute force, dominance, counts
align                 block-padded route list + inverse map  hand-worked example, invariants
grouped_ffn           gather FC1 -> SwiGLU*prob -> FC2        library SwiGLU (E=1,K=1), dense path
gather_combine        per-token sum of its kept routes       dense path, hand-worked example
dispatch_rows         route-ordered copy of the token rows   inverse of the route list,
                      (a permute; an EP send buffer)         permuted = permute-free FFN
permuted_forward      materialised-permute formulation       cross-check only
dense_forward         per-token formulation, no capacity     cross-check only
dropless_bound        static route-list bound, dropless      closed form
dropless_align        dropless block-padded route list       hand-worked example, invariants,
                                                             independent sort-based build
grouped_ffn_blocks    FFN over a block-owned route list      = grouped_ffn on the same rows
dropless_forward      routing -> dropless align -> FFN ->    = forward when no route drops
                      combine
====================  =====================================  ==============

No function here is "parity unpinned"; the FFN values are pinned only
indirectly (a library SwiGLU FFN in the one-expert case, and the dense
per-token formulation with the probability applied after FC2), since the
pages print no worked numbers.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# Layout block: the number of slots one route-list block holds.  The pages
# leave BLOCK_SIZE_M open ([PF] section 4, "block_size_m"); 32 is one
# 32x32 MFMA M-extent and divides every workload's capacity.
BM_DEFAULT = 32


# ---------------------------------------------------------------------------
# bf16 <-> float helpers (bit-level, round-to-nearest-even)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64; exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_f32(v) -> np.ndarray:
    """Round float64 to float32, nearest-even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(f) -> np.ndarray:
    """Round finite float32 values to bf16 bit patterns, nearest-even."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def f64_to_bf16_bits(v) -> np.ndarray:
    """float64 -> float32 -> bf16, each step nearest-even."""
    return f32_to_bf16_bits(f64_to_f32(v))


# ---------------------------------------------------------------------------
# Step 0: source capacity
# ---------------------------------------------------------------------------

def source_capacity(N: int, K: int, E: int, F: float) -> int:
    """[FC] Design notes: every expert gets ceil(N*K*F/E) slots.

    Evaluated in exact rational arithmetic on the binary value of the double
    F, so no float rounding of the product decides the ceiling.
    """
    if N < 0 or K < 1 or E < 1 or K > E:
        raise ValueError("need N >= 0 and 1 <= K <= E")
    if not (isinstance(F, (int, float)) and math.isfinite(F) and F > 0):
        raise ValueError("capacity factor must be a finite positive number")
    return math.ceil(Fraction(N * K) * Fraction(F) / E)


def padded_capacity(C: int, BM: int = BM_DEFAULT) -> int:
    """Per-expert segment length: C rounded up to whole layout blocks."""
    return -(-C // BM) * BM


# ---------------------------------------------------------------------------
# Step 1: top-K softmax routing
# ---------------------------------------------------------------------------

def route_topk(logits, K: int):
    """Top-K experts per token by logit, then softmax over the K chosen.

    Selection: experts ordered by descending fp32 logit, equal logits broken
    toward the lower expert index (a stable sort of the negated logits).
    Probabilities: float64 exp of (logit - max logit), summed in k order,
    divided, and rounded once to float32.  Equal to the full softmax
    renormalised over the chosen K.

    Returns ids int32 [N, K] (descending logit) and probs float32 [N, K].
    """
    lg = np.asarray(logits, dtype=np.float32)
    N, E = lg.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :K].astype(np.int32)
    chosen = np.take_along_axis(lg, ids.astype(np.int64), axis=1).astype(np.float64)
    ex = np.exp(chosen - chosen[:, :1])
    denom = np.zeros(N, dtype=np.float64)
    for k in range(K):
        denom = denom + ex[:, k]
    probs = (ex / denom[:, None]).astype(np.float32)
    return ids, probs


# ---------------------------------------------------------------------------
# Step 2: fixed-capacity drop-and-pad slot selection
# ---------------------------------------------------------------------------

def capacity_select(ids, probs, E: int, C: int):
    """[FC] Design notes: each expert keeps exactly C slots.

    For expert e, its candidates are the routes (t, k) with ids[t, k] == e.
    The min(C, load) candidates with the largest routing probability are
    kept (equal probabilities: the lower token index wins); the rest are
    dropped.  Kept routes take slots 0 .. count-1 in ascending token order;
    slots count .. C-1 are pads, filled by ``align``.

    Returns route_slot int32 [N, K] (slot, or -1 when dropped) and
    expert_count int32 [E] (kept routes per expert).
    """
    ids = np.asarray(ids, dtype=np.int32)
    probs = np.asarray(probs, dtype=np.float32)
    N, K = ids.shape
    route_slot = np.full((N, K), -1, dtype=np.int32)
    expert_count = np.zeros(E, dtype=np.int32)
    for e in range(E):
        tok, kk = np.nonzero(ids == e)          # row-major scan: ascending token
        keys = probs[tok, kk].astype(np.float64)
        rank = np.lexsort((tok, -keys))         # by (-prob, token)
        kept = np.sort(rank[: min(C, len(rank))])
        route_slot[tok[kept], kk[kept]] = np.arange(len(kept), dtype=np.int32)
        expert_count[e] = len(kept)
    return route_slot, expert_count


# ---------------------------------------------------------------------------
# Step 3: align (route list and its inverse)
# ---------------------------------------------------------------------------

def align(ids, probs, route_slot, expert_count, N: int, E: int, C: int,
          BM: int = BM_DEFAULT):
    """[PF] section 4 "Data structures", fixed-capacity form.

    Expert e owns the Cp = roundup(C, BM) consecutive slots starting at
    e*Cp.  A kept route (t, k) with slot j lands at s = e*Cp + j:
    sorted_slot_ids[s] = t, slot_probs[s] = its probability, and
    token_routes[t, k] = s.  Every other slot is a pad: token row N (the
    sentinel whose gathered row reads as zeros) and probability +0.0.
    Dropped routes have token_routes = -1.
    """
    ids = np.asarray(ids, dtype=np.int32)
    probs = np.asarray(probs, dtype=np.float32)
    route_slot = np.asarray(route_slot, dtype=np.int32)
    K = ids.shape[1]
    Cp = padded_capacity(C, BM)
    R = E * Cp
    sorted_slot_ids = np.full(R, N, dtype=np.int32)
    slot_probs = np.zeros(R, dtype=np.float32)
    token_routes = np.full((N, K), -1, dtype=np.int32)
    for t in range(N):
        for k in range(K):
            j = int(route_slot[t, k])
            if j >= 0:
                s = int(ids[t, k]) * Cp + j
                sorted_slot_ids[s] = t
                slot_probs[s] = probs[t, k]
                token_routes[t, k] = s
    token_route_count = (token_routes >= 0).sum(axis=1).astype(np.int32)
    expert_ids = ((np.arange(R // BM, dtype=np.int64) * BM) // Cp).astype(np.int32)
    block_start = ((np.arange(E, dtype=np.int64) * Cp) // BM).astype(np.int32)
    return dict(
        Cp=Cp,
        sorted_slot_ids=sorted_slot_ids,
        slot_probs=slot_probs,
        expert_ids=expert_ids,
        block_start=block_start,
        token_routes=token_routes,
        token_route_count=token_route_count,
        num_tokens_post_padded=np.array([R], dtype=np.int32),
    )


# ---------------------------------------------------------------------------
# Step 4: grouped FC1 -> SwiGLU * prob -> FC2
# ---------------------------------------------------------------------------

def silu(g):
    """SiLU by its definition, g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def expert_ffn(a_bits, w1_e, w2_e, p):
    """One expert's FFN on rows already gathered ([PF] sections 2-3).

    a_bits  bf16 [M, H]   gathered rows (all-zero for pad slots)
    w1_e    bf16 [2I, H]  FC1 weight; output rows 0..I-1 are the gate,
                          rows I..2I-1 the up projection
    w2_e    bf16 [H, I]   FC2 weight
    p       f32  [M]      routing probability per row (0 for pads)

    h = a @ W1^T in float64; act = silu(gate) * up * p, stored as bf16;
    out = act @ W2^T, stored as bf16.  Returns (act_bits, out_bits).
    """
    a = bf16_bits_to_f64(a_bits)
    w1 = bf16_bits_to_f64(w1_e)
    w2 = bf16_bits_to_f64(w2_e)
    I = w1.shape[0] // 2
    h = a @ w1.T
    gate, up = h[:, :I], h[:, I:]
    act = f64_to_bf16_bits(silu(gate) * up * np.asarray(p, np.float64)[:, None])
    out = f64_to_bf16_bits(bf16_bits_to_f64(act) @ w2.T)
    return act, out


def grouped_ffn(x_bits, w1_bits, w2_bits, sorted_slot_ids, slot_probs, E: int,
                Cp: int, experts=None):
    """Permute-free grouped FFN over the route list ([PF] sections 2-3).

    For slot s of expert e = s // Cp, the A row is x[sorted_slot_ids[s]]
    read straight from token order (zeros for the sentinel row N); no
    permuted copy of x exists.  Returns act [E*Cp, I] and route_out
    [E*Cp, H] as bf16 bits; with ``experts`` given, only those experts'
    segments are computed (the rest stay zero).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    N, H = x_bits.shape
    I = np.asarray(w1_bits[0]).shape[0] // 2
    act = np.zeros((E * Cp, I), dtype=np.uint16)
    route_out = np.zeros((E * Cp, H), dtype=np.uint16)
    for e in (range(E) if experts is None else experts):
        seg = slice(e * Cp, (e + 1) * Cp)
        rows = np.asarray(sorted_slot_ids[seg])
        a = np.zeros((Cp, H), dtype=np.uint16)
        real = rows < N
        a[real] = x_bits[rows[real]]
        act[seg], route_out[seg] = expert_ffn(a, w1_bits[e], w2_bits[e],
                                              np.asarray(slot_probs[seg]))
    return act, route_out


# ---------------------------------------------------------------------------
# Step 5: gather-combine
# ---------------------------------------------------------------------------

def gather_combine(route_out_bits, token_routes, N: int):
    """[PF] sections 2 and 5: each token pulls its own kept routes.

    y[t] = bf16( sum over k = 0..K-1 with token_routes[t, k] >= 0 of
    float32(route_out[token_routes[t, k]]) ), a float32 running sum that
    starts at +0.0 and adds in k order.  A token whose routes were all
    dropped gets zeros.
    """
    ro = np.asarray(route_out_bits, dtype=np.uint16)
    tr = np.asarray(token_routes, dtype=np.int64)
    H = ro.shape[1]
    acc = np.zeros((N, H), dtype=np.float32)
    for k in range(tr.shape[1]):
        sel = tr[:, k] >= 0
        rows = bf16_bits_to_f64(ro[tr[sel, k]]).astype(np.float32)
        acc[sel] = acc[sel] + rows
    return f32_to_bf16_bits(acc)


# ---------------------------------------------------------------------------
# Whole forward and the two cross-check formulations
# ---------------------------------------------------------------------------

def forward(logits, x_bits, w1_bits, w2_bits, K: int, F: float, BM: int = BM_DEFAULT):
    """Steps 0-5 in order; returns every intermediate the GPU path emits."""
    lg = np.asarray(logits, dtype=np.float32)
    N, E = lg.shape
    C = source_capacity(N, K, E, F)
    ids, probs = route_topk(lg, K)
    route_slot, expert_count = capacity_select(ids, probs, E, C)
    meta = align(ids, probs, route_slot, expert_count, N, E, C, BM)
    act, route_out = grouped_ffn(x_bits, w1_bits, w2_bits, meta["sorted_slot_ids"],
                                 meta["slot_probs"], E, meta["Cp"])
    y = gather_combine(route_out, meta["token_routes"], N)
    out = dict(C=C, topk_ids=ids, topk_probs=probs, route_slot=route_slot,
               expert_count=expert_count, act=act, route_out=route_out, y=y)
    out.update(meta)
    return out


def dispatch_rows(x_bits, sorted_slot_ids):
    """Route-ordered copy of the token rows: row s is x[sorted_slot_ids[s]],
    a zero row where the entry is not a token index (the sentinel N of a pad).

    [PF] section 1 calls this the materialised permute; [FC] Design notes:
    with a fixed capacity it is also the send buffer of a uniform
    expert-parallel exchange, C rows per expert from every source.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    N, H = x_bits.shape
    ssi = np.asarray(sorted_slot_ids, dtype=np.int64)
    rows = np.zeros((ssi.shape[0], H), dtype=np.uint16)
    real = (ssi >= 0) & (ssi < N)
    rows[real] = x_bits[ssi[real]]
    return rows


def permuted_forward(x_bits, w1_bits, w2_bits, meta, E: int):
    """[PF] section 1: the conventional path with a materialised permute.

    Scatter token rows into expert-contiguous order (Xp = x[sorted_slot_ids]
    with zero rows for pads), run each expert's FFN on its contiguous block,
    then unpermute: per (t, k), fetch the block row its route landed on, and
    sum over k in float32, k order.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    N, H = x_bits.shape
    Cp = meta["Cp"]
    ssi = meta["sorted_slot_ids"]
    xp = dispatch_rows(x_bits, ssi)
    blocks = []
    for e in range(E):
        seg = slice(e * Cp, (e + 1) * Cp)
        blocks.append(expert_ffn(xp[seg], w1_bits[e], w2_bits[e], meta["slot_probs"][seg])[1])
    yp = np.concatenate(blocks, axis=0)
    tr = meta["token_routes"]
    K = tr.shape[1]
    unperm = np.zeros((N, K, H), dtype=np.float32)
    for t in range(N):
        for k in range(K):
            if tr[t, k] >= 0:
                unperm[t, k] = bf16_bits_to_f64(yp[tr[t, k]]).astype(np.float32)
    acc = np.zeros((N, H), dtype=np.float32)
    for k in range(K):
        acc = acc + unperm[:, k]
    return f32_to_bf16_bits(acc)


def dense_forward(x_bits, w1_bits, w2_bits, ids, probs):
    """No capacity: y[t] = sum_k p[t,k] * FFN_{ids[t,k]}(x[t]).

    Token by token, with the probability applied after FC2 (in float64)
    rather than inside the SwiGLU, which FC2's linearity makes equivalent.
    Equal to ``forward`` up to bf16 rounding whenever no route is dropped.
    """
    x = bf16_bits_to_f64(x_bits)
    N = x.shape[0]
    K = ids.shape[1]
    H = x.shape[1]
    y = np.zeros((N, H), dtype=np.float64)
    for t in range(N):
        for k in range(K):
            e = int(ids[t, k])
            w1 = bf16_bits_to_f64(w1_bits[e])
            w2 = bf16_bits_to_f64(w2_bits[e])
            I = w1.shape[0] // 2
            h = w1 @ x[t]
            a = silu(h[:I]) * h[I:]
            y[t] += float(probs[t, k]) * (w2 @ a)
    return y


# ---------------------------------------------------------------------------
# Dropless (dynamic-count) variant: every route kept, per-expert segments
# padded to whole blocks, the real extent a device-side number
# ---------------------------------------------------------------------------

def dropless_bound(N: int, K: int, E: int, BM: int = BM_DEFAULT) -> int:
    """Static length of the dropless route list ([PF] section 4: the route
    list is over-allocated to T*min(topk, E) slots, and block padding adds
    at most BM-1 slots per expert), rounded up to whole blocks."""
    r = N * min(K, E) + E * (BM - 1)
    return -(-r // BM) * BM


def dropless_align(ids, probs, N: int, E: int, BM: int = BM_DEFAULT):
    """[PF] sections 4-5 (route_list_scan, route_list_align), dropless form.

    Every route is kept.  Expert e's count_e routes take consecutive slots
    in ascending token order (their within-expert ranks), and its segment is
    padded to a multiple of BM; segments follow each other in expert order,
    so expert e starts at block block_start[e].  The real padded extent
    (num_tokens_post_padded) is the sum of the padded segments.  Blocks up to
    the extent name their expert in expert_ids; blocks past it hold -1.
    Pad slots and the tail past the extent hold the sentinel row N with
    probability +0.0.  token_routes[t, k] is the slot of route (t, k), and
    every token keeps all of its K routes.
    """
    ids = np.asarray(ids, dtype=np.int32)
    probs = np.asarray(probs, dtype=np.float32)
    K = ids.shape[1]
    R = dropless_bound(N, K, E, BM)
    counts = np.bincount(ids.ravel(), minlength=E).astype(np.int64)[:E]
    padded = -(-counts // BM) * BM
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    extent = int(padded.sum())
    sorted_slot_ids = np.full(R, N, dtype=np.int32)
    slot_probs = np.zeros(R, dtype=np.float32)
    token_routes = np.full((N, K), -1, dtype=np.int32)
    route_within = np.full((N, K), -1, dtype=np.int32)
    for e in range(E):
        tt, kk = np.nonzero(ids == e)          # row-major: ascending token
        s = starts[e] + np.arange(len(tt))
        sorted_slot_ids[s] = tt
        slot_probs[s] = probs[tt, kk]
        token_routes[tt, kk] = s
        route_within[tt, kk] = np.arange(len(tt))
    expert_ids = np.full(R // BM, -1, dtype=np.int32)
    for e in range(E):
        expert_ids[starts[e] // BM:(starts[e] + padded[e]) // BM] = e
    return dict(
        R=R,
        route_counts=counts.astype(np.int32),
        route_within=route_within,
        sorted_slot_ids=sorted_slot_ids,
        slot_probs=slot_probs,
        expert_ids=expert_ids,
        block_start=(starts // BM).astype(np.int32),
        token_routes=token_routes,
        token_route_count=(token_routes >= 0).sum(axis=1).astype(np.int32),
        num_tokens_post_padded=np.array([extent], dtype=np.int32),
    )


def grouped_ffn_blocks(x_bits, w1_bits, w2_bits, sorted_slot_ids, slot_probs, expert_ids,
                       BM: int = BM_DEFAULT, experts=None):
    """Grouped FFN over a route list whose blocks name their expert
    ([PF] section 5: the tile -> expert map is expert_ids).  Each slot of a
    block owned by expert e gets that expert's FFN of its gathered row
    (zeros for the sentinel); slots of -1 blocks stay zero.  With ``experts``
    given, only those experts' blocks are computed."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    N, H = x_bits.shape
    I = np.asarray(w1_bits[0]).shape[0] // 2
    R = len(sorted_slot_ids)
    act = np.zeros((R, I), dtype=np.uint16)
    route_out = np.zeros((R, H), dtype=np.uint16)
    owner = np.repeat(np.asarray(expert_ids), BM)
    todo = sorted(set(int(e) for e in np.unique(owner) if e >= 0))
    for e in (todo if experts is None else [e for e in experts if e in todo]):
        sl = np.nonzero(owner == e)[0]
        rows = np.asarray(sorted_slot_ids)[sl]
        a = np.zeros((len(sl), H), dtype=np.uint16)
        real = rows < N
        a[real] = x_bits[rows[real]]
        act[sl], route_out[sl] = expert_ffn(a, w1_bits[e], w2_bits[e], np.asarray(slot_probs)[sl])
    return act, route_out


def dropless_forward(logits, x_bits, w1_bits, w2_bits, K: int, BM: int = BM_DEFAULT):
    """Top-K routing, dropless align, grouped FFN, gather-combine."""
    lg = np.asarray(logits, dtype=np.float32)
    N, E = lg.shape
    ids, probs = route_topk(lg, K)
    meta = dropless_align(ids, probs, N, E, BM)
    act, route_out = grouped_ffn_blocks(x_bits, w1_bits, w2_bits, meta["sorted_slot_ids"],
                                        meta["slot_probs"], meta["expert_ids"], BM)
    y = gather_combine(route_out, meta["token_routes"], N)
    out = dict(topk_ids=ids, topk_probs=probs, act=act, route_out=route_out, y=y)
    out.update(meta)
    return out

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every step is checked step-wise (the oracle step consumes the GPU's previous
output) and the FFN output end to end; see gpu_support for the bars.
"""

import zlib

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import (assert_bf16_close, check_capacity_and_align, check_combine_stepwise,
                         check_routing, host, run_steps, say)
from mixture_experts_expert_amd import MoEBuffers, moe_source_capacity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def full_check(w_shape, T):
    """w_shape: object with N, H, I, E, K, F; T: device tensors."""
    N, H, I, E, K, F = w_shape.N, w_shape.H, w_shape.I, w_shape.E, w_shape.K, w_shape.F
    C = oracle.source_capacity(N, K, E, F)
    assert moe_source_capacity(N, K, E, F) == C
    buf = MoEBuffers(N, H, I, E, K, F, DEV)
    run_steps(buf, T["logits"], T["x"], T["w1"], T["w2"])
    lg = host(T["logits"])
    check_routing(buf, lg, K)
    m = check_capacity_and_align(buf, N, E, K, C)
    say(f"  C={C} Cp={buf.Cp} kept={int((m['token_routes'] >= 0).sum())}/{N * K} "
        f"pads={int((m['sorted_slot_ids'] == N).sum())}")
    x, w1, w2 = host(T["x"]), host(T["w1"]), host(T["w2"])
    act, route_out = oracle.grouped_ffn(x, w1, w2, m["sorted_slot_ids"], m["slot_probs"], E, buf.Cp)
    g_act, g_ro = host(buf.act), host(buf.route_out)
    assert_bf16_close(g_act, act, "act")
    assert_bf16_close(g_ro, route_out, "route_out")
    pads = m["sorted_slot_ids"] == N
    assert np.all(g_act[pads] == 0) and np.all(g_ro[pads] == 0), "pad rows must be zero"
    check_combine_stepwise(buf, N)
    y_ref = oracle.gather_combine(route_out, m["token_routes"], N)
    assert_bf16_close(host(buf.y), y_ref, "y (end to end)")
    return buf, m


# ------------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name", ["tiny_n64_h64_e4_k2", "small_qwen3moe_n1024_h512_e8_k2",
                                  "qwen3_30b_a3b_n4096_h2048_e128_k8"])
def test_workload_parity(name):
    w = moe_inputs.WORKLOADS[name]
    say(f"[parity] {name}")
    T = moe_inputs.make_tensors(w, DEV)
    full_check(w, T)


@pytest.mark.parametrize("name", ["skew_zipf_n4096_e128_k8_f1.0", "skew_zipf_n4096_e128_k8_f1.5"])
def test_skew_parity(name, skew_alpha):
    w = moe_inputs.WORKLOADS[name]
    say(f"[parity] {name}")
    T = moe_inputs.make_tensors(w, DEV, skew_alpha=skew_alpha)
    buf, m = full_check(w, T)
    if w.F == 1.0:
        assert (m["token_routes"] < 0).sum() > 0          # drops
    else:
        assert (m["sorted_slot_ids"] == w.N).sum() > 0    # pads


# ------------------------------------------------------------------ edge cases

class Shape:
    def __init__(self, N, H, I, E, K, F):
        self.N, self.H, self.I, self.E, self.K, self.F = N, H, I, E, K, F


def custom_tensors(s: Shape, seed: int, logits=None):
    g = torch.Generator(device=DEV).manual_seed(seed)
    lg = logits if logits is not None else moe_inputs.make_logits(s.N, s.E, seed)
    return {
        "logits": torch.from_numpy(np.ascontiguousarray(lg, dtype=np.float32)).to(DEV),
        "x": torch.randn(s.N, s.H, generator=g, device=DEV).to(torch.bfloat16),
        "w1": (torch.randn(s.E, 2 * s.I, s.H, generator=g, device=DEV) * 0.05).to(torch.bfloat16),
        "w2": (torch.randn(s.E, s.H, s.I, generator=g, device=DEV) * 0.05).to(torch.bfloat16),
    }


EDGE = {
    "single_token": (Shape(1, 64, 64, 4, 2, 1.0), None),
    "one_expert_textbook": (Shape(100, 128, 192, 1, 1, 1.0), None),
    "ragged_n77_h192_i320": (Shape(77, 192, 320, 6, 3, 0.7), None),
    "tied_integer_logits": (Shape(300, 64, 128, 16, 4, 1.0), "ties"),
    "overload_one_expert": (Shape(512, 64, 128, 8, 2, 1.0), "hot"),
    "wide_e1000_k32": (Shape(256, 64, 64, 1000, 32, 1.0), None),
    "e100_k7_f2": (Shape(1000, 128, 64, 100, 7, 2.0), None),
    "large_factor_pads": (Shape(200, 64, 128, 8, 2, 4.0), None),
    "max_tokens_all_to_one": (Shape(16384, 64, 64, 64, 6, 1.0), "hot"),
    # C = 256 and 512: whole 256-row tiles (the persistent 12-wave GEMM), one
    # with ragged column tiles (H = 320, I = 192) and a 3-slab contraction, one
    # with two row tiles per expert
    "whole_tiles_ragged_h320_i192": (Shape(512, 320, 192, 8, 4, 1.0), None),
    "two_row_tiles_c512": (Shape(1024, 256, 128, 8, 4, 1.0), None),
    # in the dropless form a mean of 125 routes per expert takes 256-row tiles
    # (the staged epilogue); "hot" puts every token on expert 0, whose
    # 1000-route segment then spans four row tiles, the last one partial
    "dyn_256_tiles_n1000_h256_i192": (Shape(1000, 256, 192, 8, 1, 1.0), None),
    "dyn_hot_rows_n1000_h256_i192": (Shape(1000, 256, 192, 8, 1, 1.0), "hot"),
}


@pytest.mark.parametrize("case", list(EDGE))
def test_edge_case_parity(case):
    s, mode = EDGE[case]
    say(f"[edge] {case}")
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    lg = None
    if mode == "ties":
        lg = rng.integers(-2, 3, size=(s.N, s.E)).astype(np.float32)
    elif mode == "hot":
        lg = rng.standard_normal((s.N, s.E)).astype(np.float32)
        lg[:, 0] += 50.0
    T = custom_tensors(s, 17, lg)
    buf, m = full_check(s, T)
    if case == "one_expert_textbook":
        # a plain SwiGLU FFN: y = (silu(x Wg^T) * (x Wu^T)) W2^T, library ops in float64
        x, w1, w2 = T["x"].double().cpu(), T["w1"][0].double().cpu(), T["w2"][0].double().cpu()
        ref = (torch.nn.functional.silu(x @ w1[:s.I].T) * (x @ w1[s.I:].T)) @ w2.T
        assert_bf16_close(host(buf.y), ref.numpy(), "y vs library SwiGLU FFN")
    if mode == "hot":
        C = buf.C
        assert host(buf.expert_count)[0] == C


# ------------------------------------------------------------------ properties

def test_determinism_bitwise():
    w = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
    T = moe_inputs.make_tensors(w, DEV)
    a = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    b = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    run_steps(a, T["logits"], T["x"], T["w1"], T["w2"])
    run_steps(b, T["logits"], T["x"], T["w1"], T["w2"])
    for k in ("topk_ids", "topk_probs", "route_slot", "sorted_slot_ids", "token_routes", "act",
              "route_out", "y"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k


def test_gather_in_gemm_equals_pregathered_rows():
    """Permute-free vs permuted on the GPU: gathering x through the route list
    inside the GEMM equals running the same kernel on a materialised,
    expert-contiguous copy of x with an identity route list."""
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    T = moe_inputs.make_tensors(w, DEV)
    buf = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    run_steps(buf, T["logits"], T["x"], T["w1"], T["w2"])
    ssi = buf.sorted_slot_ids.long()
    real = ssi < w.N
    R = buf.R
    xp = torch.zeros(R, w.H, dtype=torch.bfloat16, device=DEV)   # the permuted copy
    xp[real] = T["x"][ssi[real]]
    ident = torch.where(real, torch.arange(R, device=DEV), torch.full_like(ssi, R)).int()
    act2 = torch.empty_like(buf.act)
    ro2 = torch.empty_like(buf.route_out)
    from mixture_experts_expert_amd import moe_grouped_ffn_fwd
    # the permuted copy has R rows, so its sentinel is R; identical arithmetic otherwise
    moe_grouped_ffn_fwd(xp, T["w1"], T["w2"], ident.contiguous(), buf.slot_probs, buf.C, act2, ro2)
    torch.cuda.synchronize()
    assert torch.equal(act2, buf.act) and torch.equal(ro2, buf.route_out)


@pytest.mark.parametrize("fused", [False, True])
def test_graph_capture_replay_equals_eager(fused):
    """The whole forward captured once into a hipGraph, replayed on new inputs
    written in place, with eager work between replays (separate routing and
    align calls, or the fused routing call)."""
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    seeds = [11, 12, 13]
    inputs = [custom_tensors(w, s) for s in seeds]
    static = {k: v.clone() for k, v in inputs[0].items()}
    buf = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_steps(buf, static["logits"], static["x"], static["w1"], static["w2"])   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        if fused:
            buf.route_capacity_align(static["logits"])
        else:
            buf.route_capacity(static["logits"])
            buf.align()
        buf.grouped_ffn(static["x"], static["w1"], static["w2"])
        buf.combine()
    for rep in range(2):
        for inp in inputs:
            for k in static:
                static[k].copy_(inp[k])
            g.replay()
            torch.cuda.synchronize()
            y_graph = buf.y.clone()
            slots_graph = buf.sorted_slot_ids.clone()
            eager = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
            run_steps(eager, inp["logits"], inp["x"], inp["w1"], inp["w2"])
            assert torch.equal(y_graph, eager.y), f"replay {rep} differs from eager"
            assert torch.equal(slots_graph, eager.sorted_slot_ids)


ROUTE_OUTPUTS = ("topk_ids", "topk_probs", "route_slot", "expert_count", "sorted_slot_ids",
                 "slot_probs", "expert_ids", "block_start", "token_routes", "token_route_count",
                 "num_tokens_post_padded")


@pytest.mark.parametrize("case", ["tiny_n64_h64_e4_k2", "qwen3_30b_a3b_n4096_h2048_e128_k8",
                                  "skew_zipf_n4096_e128_k8_f1.0", "skew_zipf_n4096_e128_k8_f1.5",
                                  "tied_integer_logits", "overload_one_expert", "wide_e1000_k32",
                                  "max_tokens_all_to_one", "ragged_n77_h192_i320"])
def test_fused_route_align_equals_separate_calls(case, skew_alpha):
    """moe_route_capacity_align == moe_route_capacity then moe_align, bitwise,
    on buffers that start out filled with junk (every element is written)."""
    if case in EDGE:
        s, mode = EDGE[case]
        rng = np.random.default_rng(zlib.crc32(case.encode()))
        lg = None
        if mode == "ties":
            lg = rng.integers(-2, 3, size=(s.N, s.E)).astype(np.float32)
        elif mode == "hot":
            lg = rng.standard_normal((s.N, s.E)).astype(np.float32)
            lg[:, 0] += 50.0
        logits = custom_tensors(s, 17, lg)["logits"]
    else:
        s = moe_inputs.WORKLOADS[case]
        logits = moe_inputs.make_tensors(s, DEV, skew_alpha=skew_alpha if s.skew else None,
                                         weights=False)["logits"]
    say(f"[fused routing] {case}")
    a = MoEBuffers(s.N, s.H, s.I, s.E, s.K, s.F, DEV)
    b = MoEBuffers(s.N, s.H, s.I, s.E, s.K, s.F, DEV)
    for buf in (a, b):
        for k in ROUTE_OUTPUTS:
            getattr(buf, k).fill_(-7)
    a.route_capacity(logits)
    a.align()
    b.route_capacity_align(logits)
    torch.cuda.synchronize()
    for k in ROUTE_OUTPUTS:
        assert torch.equal(getattr(a, k), getattr(b, k)), k


def test_n_zero_is_noop():
    buf = MoEBuffers(0, 64, 64, 4, 2, 1.0, DEV)
    T = {"logits": torch.zeros(0, 4, device=DEV), "x": torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)}
    w1 = torch.zeros(4, 128, 64, dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros(4, 64, 64, dtype=torch.bfloat16, device=DEV)
    run_steps(buf, T["logits"], T["x"], w1, w2)
    assert buf.y.numel() == 0


def test_split_fc1_fc2_equals_fused_call():
    """moe_grouped_ffn_fwd == moe_grouped_fc1_swiglu then moe_grouped_fc2, bitwise."""
    w = moe_inputs.WORKLOADS["small_qwen3moe_n1024_h512_e8_k2"]
    T = moe_inputs.make_tensors(w, DEV)
    a = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    run_steps(a, T["logits"], T["x"], T["w1"], T["w2"])
    b = MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, DEV)
    b.route_capacity(T["logits"])
    b.align()
    b.fc1_swiglu(T["x"], T["w1"])
    b.fc2(T["w2"])
    b.combine()
    torch.cuda.synchronize()
    for k in ("act", "route_out", "y"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k

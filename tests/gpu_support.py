"""Shared pieces of the GPU parity tests: run the HIP path step by step and
compare each step with the oracle on the very same inputs.

Bars (the oracle is the reference):
* integer and index outputs, and the float32 routing probabilities, are
  compared bit for bit;
* the bf16 FFN outputs (act, route_out, y) must satisfy, elementwise,
  |gpu - ref| <= ATOL + RTOL * |ref| with ATOL = 1e-2, RTOL = 2e-2, and,
  because ATOL is large next to these tensors' magnitudes, also a normwise
  relative error ||gpu - ref|| / ||ref|| <= NORM_TOL = 1e-2 (one-ulp bf16
  flips from a different float32 summation order give about 2-4e-3);
* the combine, fed the GPU's own route_out, is bit-exact (same float32
  additions in the same order).
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import moe_inputs
import oracle
from mixture_experts_expert_amd import MoEBuffers

ATOL, RTOL, NORM_TOL = 1e-2, 2e-2, 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return moe_inputs.bf16_bits(t)
    return t.detach().cpu().numpy()


def run_steps(buf: MoEBuffers, logits, x, w1, w2):
    buf.route_capacity(logits)
    buf.align()
    buf.grouped_ffn(x, w1, w2)
    buf.combine()
    torch.cuda.synchronize()


def assert_bf16_close(gpu_bits, ref, what):
    """ref: bf16 bits (uint16) or float64 values."""
    g = oracle.bf16_bits_to_f64(gpu_bits)
    r = oracle.bf16_bits_to_f64(ref) if np.asarray(ref).dtype == np.uint16 else np.asarray(ref, np.float64)
    d = np.abs(g - r)
    bad = d > ATOL + RTOL * np.abs(r)
    nr = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    exact = float(np.mean(g == r))
    say(f"  {what}: normwise rel err {nr:.2e}, max abs err {d.max():.2e}, exact {exact:.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside {ATOL} + {RTOL}|ref|"
    assert nr <= NORM_TOL, f"{what}: normwise relative error {nr:.3e} > {NORM_TOL}"
    return nr


def bf16_close_stats(gpu_bits, ref_bits):
    """The forward's bars, quietly: elements outside ATOL + RTOL*|ref|, the
    normwise relative error, the largest absolute error and the share of
    bit-equal elements (both sides bf16 bit patterns)."""
    g = oracle.bf16_bits_to_f64(gpu_bits)
    r = oracle.bf16_bits_to_f64(ref_bits)
    d = np.abs(g - r)
    return {"bad": int((d > ATOL + RTOL * np.abs(r)).sum()),
            "norm": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)),
            "max_abs": float(d.max(initial=0.0)),
            "exact": float(np.mean(g == r)) if g.size else 1.0}


def check_routing(buf: MoEBuffers, lg: np.ndarray, K: int):
    """S1 bit-exact against the oracle on the same logits."""
    ids, probs = oracle.route_topk(lg, K)
    g_ids, g_probs = host(buf.topk_ids), host(buf.topk_probs)
    assert np.array_equal(g_ids, ids), f"topk_ids differ in {(g_ids != ids).sum()} entries"
    diff = g_probs.view(np.uint32).astype(np.int64) - probs.view(np.uint32).astype(np.int64)
    n = int((diff != 0).sum())
    if n:
        say(f"  topk_probs: {n} values differ (max {np.abs(diff).max()} ulp)")
    assert np.abs(diff).max(initial=0) <= 1 and n <= max(1, g_probs.size // 100000), \
        "topk_probs differ beyond a rare one-ulp near tie"
    return ids, probs


def check_capacity_and_align(buf: MoEBuffers, N, E, K, C):
    """S2 and S3 step-wise: the oracle consumes the GPU's previous outputs."""
    g_ids, g_probs = host(buf.topk_ids), host(buf.topk_probs)
    slot, count = oracle.capacity_select(g_ids, g_probs, E, C)
    assert np.array_equal(host(buf.route_slot), slot), "route_slot differs"
    assert np.array_equal(host(buf.expert_count), count), "expert_count differs"
    m = oracle.align(g_ids, g_probs, slot, count, N, E, C, buf.BM)
    assert m["Cp"] == buf.Cp
    for k in ("sorted_slot_ids", "expert_ids", "block_start", "token_routes",
              "token_route_count", "num_tokens_post_padded"):
        assert np.array_equal(host(getattr(buf, k)).reshape(m[k].shape), m[k]), f"{k} differs"
    g_sp = host(buf.slot_probs)
    assert np.array_equal(g_sp.view(np.uint32), m["slot_probs"].view(np.uint32)), "slot_probs differ"
    return m


def check_combine_stepwise(buf: MoEBuffers, N):
    y = oracle.gather_combine(host(buf.route_out), host(buf.token_routes), N)
    g = host(buf.y)
    assert np.array_equal(g, y), f"combine differs in {(g != y).sum()} elements"


# Backward bars (the derivation is in test_gpu_backward's module notes):
# elementwise |gpu - ref| <= ATOL_RMS * rms(ref) + RTOL * |ref| (+ 2^-7 times
# the summed magnitudes of separately rounded terms, end to end) and a
# normwise relative error <= NORM_TOL; float32 results step-wise at F32_TOL.
ATOL_RMS = 1e-2
F32_TOL = 1e-3


def grad_vals(v):
    v = np.asarray(v)
    return oracle.bf16_bits_to_f64(v) if v.dtype == np.uint16 else v.astype(np.float64)


def assert_grad_close(gpu, ref, what, rtol=RTOL, atol_rms=ATOL_RMS, norm_tol=NORM_TOL, terms=None,
                      quiet=False):
    """terms: for a result that sums separately rounded bf16 values, the
    elementwise sum of their magnitudes; one ulp (2^-8 relative) may flip in
    each of them, so 2^-7 * terms joins the bar.  Returns the normwise
    relative error (quiet: without printing it)."""
    g, r = grad_vals(gpu), grad_vals(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    d = np.abs(g - r)
    bar = atol_rms * rms + rtol * np.abs(r)
    if terms is not None:
        bar = bar + 2.0 ** -7 * terms
    bad = d > bar
    nr = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    if not quiet:
        say(f"  {what}: normwise rel err {nr:.2e}, max abs err {d.max(initial=0):.2e} "
            f"(rms {rms:.2e}), exact {float(np.mean(g == r)) if g.size else 1.0:.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the bar"
    assert nr <= norm_tol, f"{what}: normwise relative error {nr:.3e}"
    return nr

"""Weight gradients added into float32 main gradients
(moe_grouped_fc1_wgrad_accum, moe_grouped_fc2_wgrad_accum; [PF] "Permute-Free
Grouped GEMM for MoE (bf16, gfx950)", section 5: the weight-gradient GEMM
writes bf16 or accumulates into a float32 main gradient inside the kernel).

For each shape, on a real route list (pads included) and seeded bf16 inputs:

* into zeros, the result rounded to bf16 (nearest-even) equals the bf16
  entry point's dW bit for bit -- the same float32 sums;
* into a random main gradient G, the result is float32(G + S) bit for bit,
  S being the into-zeros result (one float32 addition per element);
* two micro-batches accumulated into G match the oracle
  (oracle.main_grad_accumulate of oracle.fc*_wgrad_sum, float64) within a
  float32 bar: |gpu - ref| <= 2^-20 * (|G| + the sum over both batches of
  the products' magnitudes) -- a float32 sum of K products in any order is
  within K * 2^-24 of the exact sum relative to that magnitude, K <= 512
  here -- plus a normwise relative error <= 1e-5;
* N == 0 leaves the main gradient untouched;
* in a captured graph replayed three times after an eager call, the main
  gradient holds float32(float32(float32(S + S) + S) + S), bit for bit.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_support import host, say
from mixture_experts_expert_amd import (MoEBuffers, moe_grouped_fc1_wgrad, moe_grouped_fc1_wgrad_accum,
                                        moe_grouped_fc2_wgrad, moe_grouped_fc2_wgrad_accum,
                                        moe_padded_capacity)

pytestmark = pytest.mark.gpu

DEV = "cuda"

SHAPES = {
    # N, H, I, E, K, F
    "tiny_n64_h64_i64_e4_k2": (64, 64, 64, 4, 2, 1.0),
    "ragged_tiles_n512_h320_i192_e8_k4": (512, 320, 192, 8, 4, 1.0),
    "two_row_tiles_n1024_h256_i128_e8_k4_c512": (1024, 256, 128, 8, 4, 1.0),
    "qwen3_30b_a3b_n4096_h2048_i768_e128_k8": (4096, 2048, 768, 128, 8, 1.0),
}


def batch(N, H, I, E, K, F, seed):
    """Routing state and seeded bf16 operands of one micro-batch."""
    buf = MoEBuffers(N, H, I, E, K, F, DEV)
    logits = torch.from_numpy(np.ascontiguousarray(moe_inputs.make_logits(N, E, seed), dtype=np.float32)).to(DEV)
    buf.route_capacity_align(logits)
    g = torch.Generator(device=DEV).manual_seed(seed)
    R = buf.R
    ops = {
        "x": torch.randn(N, H, generator=g, device=DEV).to(torch.bfloat16),
        "dy": torch.randn(N, H, generator=g, device=DEV).to(torch.bfloat16),
        "d_preact": (torch.randn(R, 2 * I, generator=g, device=DEV) * 0.1).to(torch.bfloat16),
        "act": (torch.randn(R, I, generator=g, device=DEV) * 0.1).to(torch.bfloat16),
    }
    return buf, ops


def accum(buf, ops, main1, main2):
    moe_grouped_fc1_wgrad_accum(ops["d_preact"], ops["x"], buf.sorted_slot_ids, buf.E, buf.C, main1)
    moe_grouped_fc2_wgrad_accum(ops["dy"], ops["act"], buf.sorted_slot_ids, buf.E, buf.C, main2)


@pytest.mark.parametrize("name", list(SHAPES))
def test_wgrad_accumulation(name):
    N, H, I, E, K, F = SHAPES[name]
    say(f"[wgrad accum] {name}")
    b1, o1 = batch(N, H, I, E, K, F, 11)
    b2, o2 = batch(N, H, I, E, K, F, 12)
    f32 = torch.float32
    # into zeros == the bf16 entry points' sums
    z1 = torch.zeros(E, 2 * I, H, dtype=f32, device=DEV)
    z2 = torch.zeros(E, H, I, dtype=f32, device=DEV)
    accum(b1, o1, z1, z2)
    d1 = torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=DEV)
    d2 = torch.empty(E, H, I, dtype=torch.bfloat16, device=DEV)
    moe_grouped_fc1_wgrad(o1["d_preact"], o1["x"], b1.sorted_slot_ids, E, b1.C, d1)
    moe_grouped_fc2_wgrad(o1["dy"], o1["act"], b1.sorted_slot_ids, E, b1.C, d2)
    torch.cuda.synchronize()
    assert torch.equal(z1.to(torch.bfloat16), d1), "fc1: rounded float32 sums differ from the bf16 dW"
    assert torch.equal(z2.to(torch.bfloat16), d2), "fc2: rounded float32 sums differ from the bf16 dW"
    # into a random main gradient: one float32 addition per element
    g = torch.Generator(device=DEV).manual_seed(13)
    G1 = torch.randn(E, 2 * I, H, generator=g, device=DEV)
    G2 = torch.randn(E, H, I, generator=g, device=DEV)
    m1, m2 = G1.clone(), G2.clone()
    accum(b1, o1, m1, m2)
    torch.cuda.synchronize()
    assert torch.equal(m1, G1 + z1) and torch.equal(m2, G2 + z2), "old + sum differs"
    # a second micro-batch, against the oracle
    accum(b2, o2, m1, m2)
    torch.cuda.synchronize()
    # expert by expert (bounded host memory at the full shape)
    hb = [(host(b.sorted_slot_ids), {k: host(v) for k, v in o.items()}) for b, o in ((b1, o1), (b2, o2))]
    absf = {k: [np.abs(oracle.bf16_bits_to_f64(h[k])) for _, h in hb] for k in ("x", "dy", "d_preact", "act")}
    Cp = b1.Cp
    for which, m, G in (("fc1", m1, G1), ("fc2", m2, G2)):
        got_all, G_all = host(m), host(G)
        worst, num, den = 0.0, 0.0, 0.0
        for e in range(E):
            seg = slice(e * Cp, (e + 1) * Cp)
            ref = G_all[e].astype(np.float64)
            mag = np.abs(ref)
            for bi, (ssi, h) in enumerate(hb):
                if which == "fc1":
                    S = oracle.fc1_wgrad_sum(h["d_preact"][seg], h["x"], ssi[seg], 1, Cp)[0]
                    T = oracle.fc1_wgrad_sum(absf["d_preact"][bi][seg], absf["x"][bi], ssi[seg], 1, Cp)[0]
                else:
                    S = oracle.fc2_wgrad_sum(h["dy"], h["act"][seg], ssi[seg], 1, Cp)[0]
                    T = oracle.fc2_wgrad_sum(absf["dy"][bi], absf["act"][bi][seg], ssi[seg], 1, Cp)[0]
                ref = oracle.main_grad_accumulate(ref, S)
                mag = mag + T
            got = got_all[e].astype(np.float64)
            d = np.abs(got - ref)
            bad = d > 2.0 ** -20 * mag
            assert not bad.any(), f"{which} expert {e}: {int(bad.sum())} elements outside the float32 bar"
            worst = max(worst, float((d / np.maximum(mag, 1e-30)).max()))
            num += float(np.sum((got - ref) ** 2))
            den += float(np.sum(ref ** 2))
        nr = (num / max(den, 1e-60)) ** 0.5
        say(f"  {which}: max |err| / magnitude {worst:.2e}, normwise {nr:.2e}")
        assert nr <= 1e-5, f"{which}: normwise relative error {nr:.3e}"


def test_no_tokens_leaves_main_gradient():
    E, H, I, C = 4, 64, 64, 8
    main1 = torch.full((E, 2 * I, H), 3.0, device=DEV)
    main2 = torch.full((E, H, I), -2.0, device=DEV)
    R = E * moe_padded_capacity(C)
    x = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    dp = torch.zeros(R, 2 * I, dtype=torch.bfloat16, device=DEV)
    act = torch.zeros(R, I, dtype=torch.bfloat16, device=DEV)
    ssi = torch.zeros(R, dtype=torch.int32, device=DEV)
    moe_grouped_fc1_wgrad_accum(dp, x, ssi, E, C, main1)
    moe_grouped_fc2_wgrad_accum(x, act, ssi, E, C, main2)
    torch.cuda.synchronize()
    assert torch.all(main1 == 3.0) and torch.all(main2 == -2.0)


def test_graph_replays_accumulate():
    N, H, I, E, K, F = SHAPES["ragged_tiles_n512_h320_i192_e8_k4"]
    b, o = batch(N, H, I, E, K, F, 21)
    m1 = torch.zeros(E, 2 * I, H, device=DEV)
    m2 = torch.zeros(E, H, I, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        accum(b, o, m1, m2)
    s.synchronize()
    S1, S2 = m1.clone(), m2.clone()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        accum(b, o, m1, m2)
    e1, e2 = S1.clone(), S2.clone()
    for rep in range(3):
        gr.replay()
        torch.cuda.synchronize()
        e1, e2 = e1 + S1, e2 + S2
        assert torch.equal(m1, e1) and torch.equal(m2, e2), f"replay {rep}"

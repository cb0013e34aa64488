"""Seeded synthetic inputs for the MoE FFN forward.

Shared by the CPU oracle tests, the GPU parity tests and the benchmark.  It
only draws random tensors of the workloads' shapes and distributions; it
holds no step of the method (no top-K, no capacity, no FFN arithmetic).

Distributions (every workload): router logits float32 ~ N(0, 1); token
activations bf16 ~ N(0, 1); expert weights bf16 ~ N(0, 0.02).  bf16 values
are a float32 draw rounded to nearest-even.

Streams:

* logits are drawn with numpy's PCG64 seeded by SeedSequence([seed, 0]),
  which is bit-identical on every machine (the skew workload's bias scale is
  calibrated on these exact logits);
* x, W1, W2 are drawn with torch's generator on the target device, seeded
  with seed*1000 + {1, 2, 3}.  On a GPU this is torch's counter-based
  generator, fast enough for the 22.5 GB expert weights of the widest
  workload; on the CPU it is torch's Mersenne-Twister stream.  Within one
  device type the bytes are reproducible; across device types they differ,
  which is harmless because the oracle always reads the very tensors the GPU
  path consumes (copied to the host).

Backward: the upstream gradient dy of the layer output is bf16 ~ N(0, 1),
[N, H], drawn like x with seed*1000 + 5.

Skewed routing: logits + alpha * rank_e^(-1.1), rank a seeded permutation of
1..E (numpy, SeedSequence([seed, 4])).  alpha is a parameter; the value that
makes the busiest expert carry about 1.35x its balanced share is stored
beside the tests, written by a script that uses the oracle's routing.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """Shape and seed of one MoE FFN layer workload."""
    name: str
    N: int          # tokens
    H: int          # hidden size
    E: int          # experts
    K: int          # experts per token
    F: float        # capacity factor
    I: int          # expert FFN intermediate size (SwiGLU: FC1 has 2I outputs)
    seed: int
    skew: bool = False
    note: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_n64_h64_e4_k2", 64, 64, 4, 2, 1.0, 128, 0,
                 note="oracle-seconds case"),
        Workload("small_qwen3moe_n1024_h512_e8_k2", 1024, 512, 8, 2, 1.25, 1024, 1,
                 note="batch 2 x seq 512, near-balanced routing"),
        Workload("qwen3_30b_a3b_n4096_h2048_e128_k8", 4096, 2048, 128, 8, 1.0, 768, 2,
                 note="Qwen3-30B-A3B-shaped layer"),
        Workload("skew_zipf_n4096_e128_k8_f1.0", 4096, 2048, 128, 8, 1.0, 768, 3, skew=True,
                 note="Zipf(1.1) expert bias, busiest expert ~1.35x balanced"),
        Workload("skew_zipf_n4096_e128_k8_f1.5", 4096, 2048, 128, 8, 1.5, 768, 3, skew=True,
                 note="as above with capacity factor 1.5 (pad slots)"),
        Workload("deepseek_wide_n8192_h7168_e256_k8", 8192, 7168, 256, 8, 1.0, 2048, 4,
                 note="DeepSeek-style wide layer, hipGraph-captured"),
    ]
}

HEADLINE = "qwen3_30b_a3b_n4096_h2048_e128_k8"

ZIPF_S = 1.1


def zipf_rank_profile(E: int, seed: int) -> np.ndarray:
    """rank_e^(-s) for a seeded permutation rank of 1..E (float64)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4]))
    rank = rng.permutation(E) + 1
    return rank.astype(np.float64) ** (-ZIPF_S)


def make_logits(N: int, E: int, seed: int, skew_alpha: float | None = None) -> np.ndarray:
    """Router logits float32 [N, E] ~ N(0,1), plus the Zipf bias if asked."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0]))
    lg = rng.standard_normal((N, E), dtype=np.float32)
    if skew_alpha is not None:
        lg = (lg.astype(np.float64) + skew_alpha * zipf_rank_profile(E, seed)[None, :]).astype(np.float32)
    return lg


_CHUNK = 1 << 24   # float32 staging chunk (64 MiB); fixed, so streams are reproducible


def _normal_bf16(shape, std: float, gen: torch.Generator, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for lo in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - lo)
        v = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        flat[lo:lo + n].copy_(v)
    return out


def make_tensors(w: Workload, device="cpu", skew_alpha: float | None = None,
                 weights: bool = True):
    """All inputs of workload ``w`` on ``device``.

    Returns dict(logits float32 [N,E], x bf16 [N,H], w1 bf16 [E,2I,H],
    w2 bf16 [E,H,I]) as torch tensors (weights omitted if ``weights`` is
    False).  ``skew_alpha`` is required for skewed workloads.
    """
    if w.skew and skew_alpha is None:
        raise ValueError(f"{w.name} needs skew_alpha")
    device = torch.device(device)
    lg = make_logits(w.N, w.E, w.seed, skew_alpha if w.skew else None)
    out = {"logits": torch.from_numpy(lg).to(device)}
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + 1)
    out["x"] = _normal_bf16((w.N, w.H), 1.0, g, device)
    if weights:
        g.manual_seed(w.seed * 1000 + 2)
        out["w1"] = _normal_bf16((w.E, 2 * w.I, w.H), 0.02, g, device)
        g.manual_seed(w.seed * 1000 + 3)
        out["w2"] = _normal_bf16((w.E, w.H, w.I), 0.02, g, device)
    return out


def make_dy(w: Workload, device="cpu") -> torch.Tensor:
    """Upstream gradient of the layer output for the backward: bf16 [N, H]
    ~ N(0, 1), torch's generator on ``device`` seeded with seed*1000 + 5."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + 5)
    return _normal_bf16((w.N, w.H), 1.0, g, device)


def make_ep_local(w: Workload, ep: int, rows_per_expert: int, device="cpu") -> dict:
    """What one rank's expert FFN holds after an expert-parallel exchange of
    workload ``w`` at degree ``ep``: E/ep local experts, each with
    ``rows_per_expert`` rows (the caller's capacity times ep), already grouped
    by expert -- x bf16 [E/ep * rows, H] ~ N(0, 1), w1 bf16 [E/ep, 2I, H] and
    w2 bf16 [E/ep, H, I] ~ N(0, 0.02), and the rows' routing probabilities
    float32 [E/ep * rows] ~ U(0, 1).  Torch's generator on ``device``, seeded
    with seed*1000 + 10 + {1, 2, 3, 4}."""
    if ep < 1 or w.E % ep or rows_per_expert < 1:
        raise ValueError(f"ep must divide E = {w.E}; rows_per_expert must be positive")
    device = torch.device(device)
    El = w.E // ep
    rows = rows_per_expert
    g = torch.Generator(device=device)
    out = {"E": El, "C": rows}
    g.manual_seed(w.seed * 1000 + 11)
    out["x"] = _normal_bf16((El * rows, w.H), 1.0, g, device)
    g.manual_seed(w.seed * 1000 + 12)
    out["w1"] = _normal_bf16((El, 2 * w.I, w.H), 0.02, g, device)
    g.manual_seed(w.seed * 1000 + 13)
    out["w2"] = _normal_bf16((El, w.H, w.I), 0.02, g, device)
    g.manual_seed(w.seed * 1000 + 14)
    out["probs"] = torch.rand(El * rows, generator=g, device=device, dtype=torch.float32)
    return out


def ep_receive_order(E_local: int, ep: int, C: int) -> np.ndarray:
    """Row layout of a rank's receive buffer after a uniform all-to-all:
    the ep sources' chunks follow one another, each holding the rank's
    E_local experts x C rows, so received row src*E_local*C + e*C + c is
    row c of local expert e from source src.  Returns, for the expert-major
    slot s = e*(ep*C) + src*C + c, that received row (int32 [E_local*ep*C]):
    a route list that reads the receive buffer in expert order."""
    e, src, c = np.meshgrid(np.arange(E_local), np.arange(ep), np.arange(C), indexing="ij")
    return (src * (E_local * C) + e * C + c).reshape(-1).astype(np.int32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor's bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

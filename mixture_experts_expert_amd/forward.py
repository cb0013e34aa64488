"""Static-buffer MoE FFN forward over the C-ABI calls.

MoEBuffers over-allocates every intermediate to static, shape-derived
bounds once (fixed capacity makes them exact: E*Cp slots), so the forward
never allocates, never synchronises and can be captured into a hipGraph
(torch.cuda.CUDAGraph) and replayed with new inputs written in place.
"""

from __future__ import annotations

import torch

from . import _native as nat


class MoEBuffers:
    """Device buffers for one layer shape (N tokens, hidden H, E experts,
    top-K, capacity factor F, FFN width I)."""

    def __init__(self, N: int, H: int, I: int, E: int, K: int, F: float, device="cuda"):
        self.N, self.H, self.I, self.E, self.K, self.F = N, H, I, E, K, F
        self.C = nat.moe_source_capacity(N, K, E, F)
        self.Cp = nat.moe_padded_capacity(self.C)
        self.BM = nat.moe_layout_block_m()
        self.R = E * self.Cp
        i32, f32, bf16 = torch.int32, torch.float32, torch.bfloat16
        dev = torch.device(device)

        def z(shape, dt):
            return torch.zeros(shape, dtype=dt, device=dev)

        self.topk_ids = z((N, K), i32)
        self.topk_probs = z((N, K), f32)
        self.route_slot = z((N, K), i32)
        self.expert_count = z((E,), i32)
        self.sorted_slot_ids = z((self.R,), i32)
        self.slot_probs = z((self.R,), f32)
        self.expert_ids = z((self.R // self.BM,), i32)
        self.block_start = z((E,), i32)
        self.token_routes = z((N, K), i32)
        self.token_route_count = z((N,), i32)
        self.num_tokens_post_padded = z((1,), i32)
        self.act = z((self.R, I), bf16)
        self.route_out = z((self.R, H), bf16)
        self.y = z((N, H), bf16)

    def route_capacity(self, logits, stream=None):
        nat.moe_route_capacity(logits, self.K, self.C, self.topk_ids, self.topk_probs,
                               self.route_slot, self.expert_count, stream)

    def route_capacity_align(self, logits, stream=None):
        """Steps 1-3 in two launches (the selection writes the route list)."""
        nat.moe_route_capacity_align(logits, self.K, self.C, self.topk_ids, self.topk_probs,
                                     self.route_slot, self.expert_count, self.sorted_slot_ids,
                                     self.slot_probs, self.expert_ids, self.block_start,
                                     self.token_routes, self.token_route_count,
                                     self.num_tokens_post_padded, stream)

    def align(self, stream=None):
        nat.moe_align(self.topk_ids, self.topk_probs, self.route_slot, self.expert_count,
                      self.N, self.E, self.K, self.C, self.sorted_slot_ids, self.slot_probs,
                      self.expert_ids, self.block_start, self.token_routes,
                      self.token_route_count, self.num_tokens_post_padded, stream)

    def grouped_ffn(self, x, w1, w2, stream=None):
        nat.moe_grouped_ffn_fwd(x, w1, w2, self.sorted_slot_ids, self.slot_probs, self.C,
                                self.act, self.route_out, stream)

    def fc1_swiglu(self, x, w1, stream=None):
        nat.moe_grouped_fc1_swiglu(x, w1, self.sorted_slot_ids, self.slot_probs, self.C,
                                   self.act, stream)

    def fc2(self, w2, stream=None):
        nat.moe_grouped_fc2(self.act, w2, self.N, self.C, self.route_out, stream)

    def combine(self, stream=None):
        nat.moe_gather_combine(self.route_out, self.token_routes, self.y, stream)


def forward(buf: MoEBuffers, logits, x, w1, w2, stream=None):
    """Steps 1-5 on one stream; returns buf.y (bf16 [N, H])."""
    buf.route_capacity_align(logits, stream)
    buf.grouped_ffn(x, w1, w2, stream)
    buf.combine(stream)
    return buf.y


class DroplessBuffers:
    """Device buffers for the dropless variant: every route kept, expert
    segments padded to whole blocks, the route list sized to its static bound
    Rd = moe_dropless_bound(N, K, E) and the real extent a device scalar."""

    def __init__(self, N: int, H: int, I: int, E: int, K: int, device="cuda"):
        self.N, self.H, self.I, self.E, self.K = N, H, I, E, K
        self.BM = nat.moe_layout_block_m()
        self.R = nat.moe_dropless_bound(N, K, E)
        i32, f32, bf16 = torch.int32, torch.float32, torch.bfloat16
        dev = torch.device(device)

        def z(shape, dt):
            return torch.zeros(shape, dtype=dt, device=dev)

        self.topk_ids = z((N, K), i32)
        self.topk_probs = z((N, K), f32)
        self.route_within = z((N, K), i32)
        self.route_counts = z((E,), i32)
        self.sorted_slot_ids = z((self.R,), i32)
        self.slot_probs = z((self.R,), f32)
        self.expert_ids = z((self.R // self.BM,), i32)
        self.block_start = z((E,), i32)
        self.token_routes = z((N, K), i32)
        self.token_route_count = z((N,), i32)
        self.num_tokens_post_padded = z((1,), i32)
        self.act = z((self.R, I), bf16)
        self.route_out = z((self.R, H), bf16)
        self.y = z((N, H), bf16)

    def route(self, logits, stream=None):
        nat.moe_route_dropless(logits, self.K, self.topk_ids, self.topk_probs, self.route_within,
                               self.route_counts, self.sorted_slot_ids, self.slot_probs,
                               self.expert_ids, self.block_start, self.token_routes,
                               self.token_route_count, self.num_tokens_post_padded, stream)

    def grouped_ffn(self, x, w1, w2, stream=None):
        nat.moe_grouped_ffn_fwd_dropless(x, w1, w2, self.sorted_slot_ids, self.slot_probs,
                                         self.block_start, self.num_tokens_post_padded, self.K,
                                         self.act, self.route_out, stream)

    def fc1_swiglu(self, x, w1, stream=None):
        nat.moe_grouped_fc1_swiglu_dropless(x, w1, self.sorted_slot_ids, self.slot_probs,
                                            self.block_start, self.num_tokens_post_padded,
                                            self.K, self.act, stream)

    def fc2(self, w2, stream=None):
        nat.moe_grouped_fc2_dropless(self.act, w2, self.block_start, self.num_tokens_post_padded,
                                     self.N, self.K, self.route_out, stream)

    def combine(self, stream=None):
        nat.moe_gather_combine(self.route_out, self.token_routes, self.y, stream)


def forward_dropless(buf: DroplessBuffers, logits, x, w1, w2, stream=None):
    """The dropless variant on one stream; returns buf.y (bf16 [N, H])."""
    buf.route(logits, stream)
    buf.grouped_ffn(x, w1, w2, stream)
    buf.combine(stream)
    return buf.y

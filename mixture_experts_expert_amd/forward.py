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
        self.workspace = nat.route_workspace(N, E, K, dev)   # the routing map

    def route_capacity(self, logits, stream=None):
        nat.moe_route_capacity(logits, self.K, self.C, self.topk_ids, self.topk_probs,
                               self.route_slot, self.expert_count, self.workspace, stream)

    def route_capacity_align(self, logits, stream=None):
        """Steps 1-3 in two launches (the selection writes the route list)."""
        nat.moe_route_capacity_align(logits, self.K, self.C, self.topk_ids, self.topk_probs,
                                     self.route_slot, self.expert_count, self.sorted_slot_ids,
                                     self.slot_probs, self.expert_ids, self.block_start,
                                     self.token_routes, self.token_route_count,
                                     self.num_tokens_post_padded, self.workspace, stream)

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


class MoEBackwardBuffers:
    """Device buffers for the backward of one fixed-capacity layer, next to
    the forward's MoEBuffers (whose routing state and route list it reuses).

    Training step on one stream:
        fwd_save (forward FC1 also storing the 2I pre-activation), fc2,
        combine; then backward(dy): FC2 dgrad -> SwiGLU recompute + backward
        -> FC1 dgrad -> gather-combine (dx) -> both weight gradients ->
        router-logit gradient.

    main_grad=True: the weight gradients are added into float32 main
    gradients main_dw1 / main_dw2 (gradient accumulation over micro-batches;
    zeroed here, never reset by backward) instead of being written as bf16
    dw1 / dw2.
    """

    def __init__(self, fwd: MoEBuffers, main_grad: bool = False):
        self.f = fwd
        R, N, H, I, E = fwd.R, fwd.N, fwd.H, fwd.I, fwd.E
        dev = fwd.act.device
        bf16, f32 = torch.bfloat16, torch.float32

        def z(shape, dt):
            return torch.zeros(shape, dtype=dt, device=dev)

        self.preact = z((R, 2 * I), bf16)
        self.d_act = z((R, I), bf16)
        self.act_re = z((R, I), bf16)
        self.d_preact = z((R, 2 * I), bf16)
        self.d_prob = z((R,), f32)
        self.d_a = z((R, H), bf16)
        self.dx = z((N, H), bf16)
        self.main_grad = bool(main_grad)
        if self.main_grad:
            self.main_dw1 = z((E, 2 * I, H), f32)
            self.main_dw2 = z((E, H, I), f32)
        else:
            self.dw1 = z((E, 2 * I, H), bf16)
            self.dw2 = z((E, H, I), bf16)
        self.d_logits = z((N, E), f32)

    def fc1_swiglu_save(self, x, w1, stream=None):
        f = self.f
        nat.moe_grouped_fc1_swiglu_save(x, w1, f.sorted_slot_ids, f.slot_probs, f.C, f.act,
                                        self.preact, stream)

    def forward(self, logits, x, w1, w2, stream=None):
        """The forward, keeping the pre-activation for the backward."""
        f = self.f
        f.route_capacity_align(logits, stream)
        self.fc1_swiglu_save(x, w1, stream)
        f.fc2(w2, stream)
        f.combine(stream)
        return f.y

    def fc2_dgrad(self, dy, w2, stream=None):
        nat.moe_grouped_fc2_dgrad(dy, w2, self.f.sorted_slot_ids, self.f.C, self.d_act, stream)

    def swiglu_bwd(self, stream=None):
        nat.moe_swiglu_bwd(self.preact, self.d_act, self.f.slot_probs, self.act_re,
                           self.d_preact, self.d_prob, stream)

    def fc1_dgrad(self, w1, stream=None):
        nat.moe_grouped_fc1_dgrad(self.d_preact, w1, self.f.N, self.f.C, self.d_a, stream)

    def dx_combine(self, stream=None):
        nat.moe_gather_combine(self.d_a, self.f.token_routes, self.dx, stream)

    def fc2_wgrad(self, dy, stream=None):
        if self.main_grad:
            nat.moe_grouped_fc2_wgrad_accum(dy, self.act_re, self.f.sorted_slot_ids, self.f.E,
                                            self.f.C, self.main_dw2, stream)
        else:
            nat.moe_grouped_fc2_wgrad(dy, self.act_re, self.f.sorted_slot_ids, self.f.E, self.f.C,
                                      self.dw2, stream)

    def fc1_wgrad(self, x, stream=None):
        if self.main_grad:
            nat.moe_grouped_fc1_wgrad_accum(self.d_preact, x, self.f.sorted_slot_ids, self.f.E,
                                            self.f.C, self.main_dw1, stream)
        else:
            nat.moe_grouped_fc1_wgrad(self.d_preact, x, self.f.sorted_slot_ids, self.f.E, self.f.C,
                                      self.dw1, stream)

    def route_bwd(self, stream=None):
        f = self.f
        nat.moe_route_bwd(f.topk_ids, f.topk_probs, f.token_routes, self.d_prob, self.d_logits,
                          stream)

    def backward(self, dy, x, w1, w2, stream=None):
        """All backward steps in order; results in dx, dw1, dw2 (or added into
        main_dw1, main_dw2), d_logits."""
        self.fc2_dgrad(dy, w2, stream)
        self.swiglu_bwd(stream)
        self.fc1_dgrad(w1, stream)
        self.dx_combine(stream)
        self.fc2_wgrad(dy, stream)
        self.fc1_wgrad(x, stream)
        self.route_bwd(stream)


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
        self.workspace = nat.route_workspace(N, E, K, dev)   # the routing map

    def route(self, logits, stream=None):
        nat.moe_route_dropless(logits, self.K, self.topk_ids, self.topk_probs, self.route_within,
                               self.route_counts, self.sorted_slot_ids, self.slot_probs,
                               self.expert_ids, self.block_start, self.token_routes,
                               self.token_route_count, self.num_tokens_post_padded,
                               self.workspace, stream)

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

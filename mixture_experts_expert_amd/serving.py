"""Variable-N serving of the dropless MoE FFN forward from captured graphs.

[BK] "[4/5] feat: capture the FFN experts at bucketed padded shapes",
sections "What this adds" and "Bounded by free memory, not by the token
budget": a grouped GEMM takes its grouping from device-side counts, so a
graph captured at one row count serves every smaller work item; graphs are
captured for a ladder of buckets (multiples of the expected item size,
clustered just above 1.0x and 0.5x of it, where routing scatter puts items);
an item takes the smallest bucket that holds it, or runs eagerly when that
bucket would pad it beyond a maximum padding ratio; capture runs
largest-first behind one eager call at the ceiling, and stops before the
graphs would cut into a reserve of free device memory (the remaining buckets
run eagerly).

Here the live token count is a device scalar read by moe_route_dropless_live:
tokens past it route nowhere, so the route list, the GEMM tile count and the
combine cover the live tokens only, and a replay pays for its bucket only in
the routing and combine launches, whose grids follow the bucket.  Every graph
shares one set of static buffers sized at the ceiling (replays on one stream
never overlap), so the ladder costs graph objects, not buffers.

Host orchestration only: every step of the forward runs in libmoe_native's
kernels.
"""

from __future__ import annotations

import math

import torch

from . import _native as nat

# Bucket sizes as multiples of the expected item size: dense just above 0.5x
# and 1.0x, then coarser up to the ceiling.
DEFAULT_FACTORS = (0.5, 0.53, 0.56, 0.6, 0.7, 0.8, 0.9, 1.0, 1.03, 1.06, 1.1, 1.2, 1.35, 1.5,
                   1.75, 2.0)


class BucketLadder:
    """The ladder of bucket sizes and the choice of bucket for an item.

    expected     expected tokens per item (the ladder's 1.0x)
    max_tokens   ceiling: the largest bucket, and the largest item served
    align        bucket sizes are rounded up to a multiple of this
    max_padding_ratio  an item of n tokens may take bucket b only if
                 b / n <= this; otherwise it runs eagerly
    """

    def __init__(self, expected: int, max_tokens: int, factors=DEFAULT_FACTORS, align: int = 16,
                 max_padding_ratio: float = 1.25):
        if expected < 1 or max_tokens < 1 or align < 1 or max_padding_ratio < 1.0:
            raise ValueError("need expected, max_tokens, align >= 1 and max_padding_ratio >= 1")
        sizes = {min(max_tokens, -(-math.ceil(f * expected) // align) * align) for f in factors if f > 0}
        sizes.add(max_tokens)
        self.sizes = sorted(s for s in sizes if s >= 1)
        self.max_tokens = max_tokens
        self.max_padding_ratio = max_padding_ratio

    def pick(self, n: int):
        """Smallest bucket holding n tokens, or None (run eagerly) if there is
        none or it would pad n beyond the maximum padding ratio."""
        if n < 1 or n > self.max_tokens:
            return None
        for b in self.sizes:
            if b >= n:
                return b if b <= n * self.max_padding_ratio else None
        return None

    def capture_order(self):
        """Largest first."""
        return sorted(self.sizes, reverse=True)


class ServingLadder:
    """Dropless MoE FFN forward for items of 1..max_tokens tokens, replayed
    from per-bucket graphs that share one set of static buffers."""

    def __init__(self, w1, w2, K: int, expected: int, max_tokens: int, device="cuda",
                 max_padding_ratio: float = 1.25, reserve_bytes: int = 8 << 30,
                 factors=DEFAULT_FACTORS, mem_get_info=None):
        self.E, I2, self.H = w1.shape
        self.I = I2 // 2
        self.K = K
        self.w1, self.w2 = w1, w2
        self.ladder = BucketLadder(expected, max_tokens, factors,
                                   max_padding_ratio=max_padding_ratio)
        self.reserve_bytes = reserve_bytes
        self._mem = mem_get_info or torch.cuda.mem_get_info
        dev = torch.device(device)
        self.dev = dev
        N, E, H = max_tokens, self.E, self.H
        # inputs of every replay and the live-token count, at the ceiling
        self.logits = torch.zeros((N, E), dtype=torch.float32, device=dev)
        self.x = torch.zeros((N, H), dtype=torch.bfloat16, device=dev)
        self.n_live = torch.zeros((1,), dtype=torch.int32, device=dev)
        from .forward import DroplessBuffers
        self.buf = DroplessBuffers(N, H, self.I, E, K, dev)
        self.graphs = {}
        self.stream = torch.cuda.Stream(device=dev)
        self.counts = {"eager": 0}

    # ---- one forward over the first n rows of the shared buffers
    def _forward(self, n: int, live: bool):
        b, K = self.buf, self.K
        lg = self.logits[:n]
        if live:
            nat.moe_route_dropless_live(lg, K, self.n_live, b.topk_ids[:n], b.topk_probs[:n],
                                        b.route_within[:n], b.route_counts, b.sorted_slot_ids,
                                        b.slot_probs, b.expert_ids, b.block_start,
                                        b.token_routes[:n], b.token_route_count[:n],
                                        b.num_tokens_post_padded, b.workspace)
        else:
            nat.moe_route_dropless(lg, K, b.topk_ids[:n], b.topk_probs[:n], b.route_within[:n],
                                   b.route_counts, b.sorted_slot_ids, b.slot_probs, b.expert_ids,
                                   b.block_start, b.token_routes[:n], b.token_route_count[:n],
                                   b.num_tokens_post_padded, b.workspace)
        nat.moe_grouped_ffn_fwd_dropless(self.x[:n], self.w1, self.w2, b.sorted_slot_ids,
                                         b.slot_probs, b.block_start, b.num_tokens_post_padded,
                                         K, b.act, b.route_out)
        nat.moe_gather_combine(b.route_out, b.token_routes[:n], b.y[:n])

    def graph_bytes_estimate(self, n: int) -> int:
        """A conservative allowance for one captured graph's own memory."""
        return 64 << 20

    def capture(self):
        """Capture the buckets largest-first, behind one eager forward at the
        ceiling; stop at the first bucket whose graph would cut into the
        free-memory reserve.  Returns the captured sizes."""
        top = self.ladder.max_tokens
        # the weights and buffers were written on the caller's stream
        self.stream.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(self.stream):
            self.n_live.fill_(top)
            self._forward(top, live=True)
        self.stream.synchronize()
        for n in self.ladder.capture_order():
            free, _total = self._mem()
            if free - self.graph_bytes_estimate(n) < self.reserve_bytes:
                break
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                self._forward(n, live=True)
            self.graphs[n] = g
            self.counts[n] = 0
        torch.cuda.synchronize()
        return sorted(self.graphs)

    def run(self, logits, x):
        """Forward of one item (logits [n, E] float32, x [n, H] bf16, device
        tensors).  Returns y [n, H] (a view into the shared output; valid
        until the next call)."""
        n = int(logits.shape[0])
        if n < 1 or n > self.ladder.max_tokens or x.shape[0] != n:
            raise ValueError(f"an item must have 1..{self.ladder.max_tokens} tokens")
        b = self.ladder.pick(n)
        caller = torch.cuda.current_stream(self.dev)
        self.stream.wait_stream(caller)          # the item's tensors are the caller's
        with torch.cuda.stream(self.stream):
            self.logits[:n].copy_(logits)
            self.x[:n].copy_(x)
            if b is not None and b in self.graphs:
                self.n_live.fill_(n)
                self.graphs[b].replay()
                self.counts[b] += 1
            else:
                self._forward(n, live=False)
                self.counts["eager"] += 1
        caller.wait_stream(self.stream)          # y is ready for the caller's stream
        return self.buf.y[:n]

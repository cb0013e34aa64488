"""ctypes binding of libmoe_native (the C ABI in include/moe_native.h).

Argument marshalling only: every function takes torch tensors for the
device buffers, checks dtype/device/contiguity/size on the host, passes raw
pointers and the current HIP stream to the C entry point of the same name,
and raises MoEError on a non-zero status.  All arithmetic of the forward runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_native.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_native.h")
PROBE_HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_probe.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -m mixture_experts_expert_amd.build "
        "or __graft_entry__.build()); there is no non-HIP fallback")

lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_source_capacity": (_i64, [_i64, _i32, _i32, _f64]),
    "moe_layout_block_m": (_i32, []),
    "moe_padded_capacity": (_i64, [_i64]),
    "moe_dropless_bound": (_i64, [_i64, _i32, _i32]),
    "moe_route_capacity_workspace_bytes": (ctypes.c_size_t, [_i64, _i32, _i32]),
    "moe_route_dropless": (ctypes.c_int, [_vp, _i64, _i32, _i32] + [_vp] * 11
                           + [_vp, ctypes.c_size_t, _vp]),
    "moe_route_dropless_live": (ctypes.c_int, [_vp, _i64, _i32, _i32] + [_vp] * 12
                                + [_vp, ctypes.c_size_t, _vp]),
    "moe_grouped_ffn_fwd_dropless": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32,
                                                                _vp, _vp, _vp]),
    "moe_grouped_fc1_swiglu_dropless": (ctypes.c_int, [_vp] * 6 + [_i64, _i32, _i32, _i32, _i32,
                                                                   _vp, _vp]),
    "moe_grouped_fc2_dropless": (ctypes.c_int, [_vp] * 4 + [_i64, _i32, _i32, _i32, _i32,
                                                            _vp, _vp]),
    "moe_route_capacity": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                                          _vp, ctypes.c_size_t, _vp]),
    "moe_route_capacity_align": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                                                _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _vp, ctypes.c_size_t, _vp]),
    "moe_route_capacity_align_noalloc": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i64] + [_vp] * 11
                                         + [_vp]),
    "moe_align": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i64,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_ffn_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64,
                                           _vp, _vp, _vp]),
    "moe_grouped_fc1_swiglu": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64,
                                              _vp, _vp]),
    "moe_grouped_fc2": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp, _vp]),
    "moe_grouped_fc2_rows": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp, _vp]),
    "moe_gather_combine": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i64, _vp, _vp]),
    "moe_dispatch_rows": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i64, _vp, _vp]),
    "moe_grouped_fc1_swiglu_save": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                                   _i64, _vp, _vp, _vp]),
    "moe_grouped_fc2_dgrad": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp,
                                             _vp]),
    "moe_swiglu_bwd": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _vp]),
    "moe_grouped_fc1_dgrad": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp, _vp]),
    "moe_grouped_fc2_wgrad": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp,
                                             _vp]),
    "moe_grouped_fc1_wgrad": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp,
                                             _vp]),
    "moe_grouped_fc2_wgrad_accum": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64,
                                                   _vp, _vp]),
    "moe_grouped_fc1_wgrad_accum": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64,
                                                   _vp, _vp]),
    "moe_route_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i64, _vp, _vp]),
    "moe_probe_read": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, _vp]),
    "moe_probe_write": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp]),
    "moe_probe_copy": (ctypes.c_int, [_vp, _vp, ctypes.c_size_t, _vp]),
    "moe_probe_read_pieces": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _i32, _i32, _vp, _vp]),
    "moe_probe_write_pieces": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _i32, _i32, _i32, _vp]),
    "moe_probe_write_tiles": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _i32, _i32, _i32, _vp]),
    "moe_probe_gemm_loop": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "moe_probe_lds_ring": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _vp, _vp]),
    "moe_probe_mfma_rate": (ctypes.c_int, [_i32, _i32, _vp, _vp]),
    "moe_probe_lds_read": (ctypes.c_int, [_i32, _i32, _vp, _vp]),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def header_functions(path: str = HEADER_PATH):
    """Names of the functions a header (default include/moe_native.h) declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def _bytes_ptr(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size()


def moe_probe_read(src, sink, stream=None):
    """Stream-read all of src once (an HBM rate probe); sink: int32 device tensor."""
    p, n = _bytes_ptr(src, "src")
    _check("moe_probe_read", lib.moe_probe_read(p, n, _bytes_ptr(sink, "sink")[0], _stream(stream)))


def moe_probe_write(dst, stream=None):
    """Stream-write all of dst once (an HBM rate probe)."""
    p, n = _bytes_ptr(dst, "dst")
    _check("moe_probe_write", lib.moe_probe_write(p, n, _stream(stream)))


def moe_probe_copy(src, dst, stream=None):
    """dst = src, byte for byte (an HBM rate probe); equal sizes."""
    ps, n = _bytes_ptr(src, "src")
    pd, m = _bytes_ptr(dst, "dst")
    if n != m:
        raise ValueError("moe_probe_copy: src and dst differ in size")
    _check("moe_probe_copy", lib.moe_probe_copy(ps, pd, n, _stream(stream)))


def moe_probe_read_pieces(src, row_bytes: int, rows: int, piece_bytes: int, sink, stream=None):
    """Read src as panels of rows x row_bytes, piece column by piece column
    (an access-order probe); sink: int32 device tensor."""
    p, n = _bytes_ptr(src, "src")
    _check("moe_probe_read_pieces", lib.moe_probe_read_pieces(
        p, n, row_bytes, rows, piece_bytes, _bytes_ptr(sink, "sink")[0], _stream(stream)))


def moe_probe_write_pieces(dst, row_bytes: int, rows: int, piece_bytes: int, nontemporal: bool,
                           stream=None):
    """Write dst as panels of rows x row_bytes, piece column by piece column
    (an access-order probe)."""
    p, n = _bytes_ptr(dst, "dst")
    _check("moe_probe_write_pieces", lib.moe_probe_write_pieces(
        p, n, row_bytes, rows, piece_bytes, int(bool(nontemporal)), _stream(stream)))


def moe_probe_write_tiles(dst, row_bytes: int, rows: int, piece_bytes: int, nontemporal: bool,
                          stream=None):
    """Write dst as panels of rows x row_bytes in tiles of rows x piece_bytes,
    neighbouring tiles on one XCD (an access-order probe)."""
    p, n = _bytes_ptr(dst, "dst")
    _check("moe_probe_write_tiles", lib.moe_probe_write_tiles(
        p, n, row_bytes, rows, piece_bytes, int(bool(nontemporal)), _stream(stream)))


def moe_probe_gemm_loop(a, b, E: int, Cp: int, sink, stream=None):
    """The grouped GEMMs' K loop alone over E experts: a bf16 [E*Cp, K],
    b bf16 [E, N, K] (an access-order-style probe); sink: int32 device tensor."""
    K = a.shape[-1]
    N = b.shape[-2]
    if b.shape[-1] != K or a.numel() < E * Cp * K or b.numel() < E * N * K:
        raise ValueError("moe_probe_gemm_loop: a must be [E*Cp, K] and b [E, N, K]")
    _check("moe_probe_gemm_loop", lib.moe_probe_gemm_loop(
        _ptr(a, torch.bfloat16, E * Cp * K, "a"), _ptr(b, torch.bfloat16, E * N * K, "b"), E, Cp, N, K,
        _bytes_ptr(sink, "sink")[0], _stream(stream)))


def moe_probe_lds_ring(src, stages: int, sink, stream=None):
    """Stream src (whole MiB) through an LDS-DMA ring of `stages` 32 KiB
    stages (the GEMMs' load pipeline alone); sink: int32 device tensor."""
    p, n = _bytes_ptr(src, "src")
    _check("moe_probe_lds_ring", lib.moe_probe_lds_ring(p, n, stages, _bytes_ptr(sink, "sink")[0],
                                                        _stream(stream)))


def _clocks(clocks, groups: int, fn: str):
    if (not isinstance(clocks, torch.Tensor) or not clocks.is_cuda or clocks.dtype != torch.int64
            or not clocks.is_contiguous() or clocks.numel() < 2 * groups):
        raise ValueError(f"{fn}: clocks must be a contiguous int64 device tensor of 2 * groups words")
    return ctypes.c_void_p(clocks.data_ptr())


def moe_probe_mfma_rate(groups: int, iters: int, clocks, stream=None):
    """The matrix cores alone: `groups` workgroups (one per compute unit),
    each wave issuing iters x 4 bf16 32x32x16 MFMAs; clocks: int64 device
    tensor of 2 * groups words (engine-clock, constant-clock ticks per
    workgroup)."""
    _check("moe_probe_mfma_rate", lib.moe_probe_mfma_rate(
        groups, iters, _clocks(clocks, groups, "moe_probe_mfma_rate"), _stream(stream)))


def moe_probe_lds_read(groups: int, iters: int, clocks, stream=None):
    """The LDS read path alone: `groups` workgroups (one per compute unit),
    each wave issuing iters x 8 reads of 1 KB; clocks as moe_probe_mfma_rate."""
    _check("moe_probe_lds_read", lib.moe_probe_lds_read(
        groups, iters, _clocks(clocks, groups, "moe_probe_lds_read"), _stream(stream)))


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {moe_status_string(status)} ({status})")
        self.status = status


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def moe_source_capacity(N: int, K: int, E: int, F: float) -> int:
    c = lib.moe_source_capacity(int(N), int(K), int(E), float(F))
    if c < 0:
        raise MoEError("moe_source_capacity", c)
    return int(c)


def moe_layout_block_m() -> int:
    return int(lib.moe_layout_block_m())


def moe_padded_capacity(C: int) -> int:
    c = lib.moe_padded_capacity(int(C))
    if c < 0:
        raise MoEError("moe_padded_capacity", c)
    return int(c)


def moe_dropless_bound(N: int, K: int, E: int) -> int:
    r = lib.moe_dropless_bound(N, K, E)
    if r < 0:
        raise MoEError("moe_dropless_bound", r)
    return r


def moe_route_capacity_workspace_bytes(N: int, E: int, K: int) -> int:
    b = int(lib.moe_route_capacity_workspace_bytes(int(N), int(E), int(K)))
    if b == 0 and N > 0:
        raise MoEError("moe_route_capacity_workspace_bytes", -2)
    return b


def route_workspace(N: int, E: int, K: int, device="cuda") -> torch.Tensor:
    """A device workspace for the routing calls (uint8, 16-byte aligned)."""
    return torch.empty(max(moe_route_capacity_workspace_bytes(N, E, K), 16), dtype=torch.uint8,
                       device=device)


def _ws(workspace, N: int, E: int, K: int):
    need = moe_route_capacity_workspace_bytes(N, E, K)
    return _ptr(workspace, torch.uint8, need, "workspace"), ctypes.c_size_t(workspace.numel())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: torch.Tensor, dtype: torch.dtype, numel: int, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _check(fn: str, status: int):
    if status != 0:
        raise MoEError(fn, status)


def moe_route_capacity(logits, K: int, C: int, topk_ids, topk_probs, route_slot, expert_count,
                       workspace, stream=None):
    N, E = logits.shape
    _check("moe_route_capacity", lib.moe_route_capacity(
        _ptr(logits, torch.float32, N * E, "logits"), N, E, K, C,
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(route_slot, torch.int32, N * K, "route_slot"),
        _ptr(expert_count, torch.int32, E, "expert_count"), *_ws(workspace, N, E, K),
        _stream(stream)))


def moe_route_capacity_align(logits, K: int, C: int, topk_ids, topk_probs, route_slot,
                             expert_count, sorted_slot_ids, slot_probs, expert_ids, block_start,
                             token_routes, token_route_count, num_tokens_post_padded, workspace,
                             stream=None):
    N, E = logits.shape
    R = E * moe_padded_capacity(C)
    BM = moe_layout_block_m()
    _check("moe_route_capacity_align", lib.moe_route_capacity_align(
        _ptr(logits, torch.float32, N * E, "logits"), N, E, K, C,
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(route_slot, torch.int32, N * K, "route_slot"),
        _ptr(expert_count, torch.int32, E, "expert_count"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(expert_ids, torch.int32, R // BM, "expert_ids"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"),
        _ptr(token_route_count, torch.int32, N, "token_route_count"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"),
        *_ws(workspace, N, E, K), _stream(stream)))


def moe_route_capacity_align_noalloc(logits, K: int, C: int, topk_ids, topk_probs, route_slot,
                                     expert_count, sorted_slot_ids, slot_probs, expert_ids,
                                     block_start, token_routes, token_route_count,
                                     num_tokens_post_padded, stream=None):
    """moe_route_capacity_align with the routing map in the library's own
    per-device scratch array (no workspace, nothing allocated)."""
    N, E = logits.shape
    R = E * moe_padded_capacity(C)
    BM = moe_layout_block_m()
    _check("moe_route_capacity_align_noalloc", lib.moe_route_capacity_align_noalloc(
        _ptr(logits, torch.float32, N * E, "logits"), N, E, K, C,
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(route_slot, torch.int32, N * K, "route_slot"),
        _ptr(expert_count, torch.int32, E, "expert_count"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(expert_ids, torch.int32, R // BM, "expert_ids"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"),
        _ptr(token_route_count, torch.int32, N, "token_route_count"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"), _stream(stream)))


def moe_align(topk_ids, topk_probs, route_slot, expert_count, N: int, E: int, K: int, C: int,
              sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
              token_route_count, num_tokens_post_padded, stream=None):
    R = E * moe_padded_capacity(C)
    BM = moe_layout_block_m()
    _check("moe_align", lib.moe_align(
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(route_slot, torch.int32, N * K, "route_slot"),
        _ptr(expert_count, torch.int32, E, "expert_count"), N, E, K, C,
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(expert_ids, torch.int32, R // BM, "expert_ids"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"),
        _ptr(token_route_count, torch.int32, N, "token_route_count"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"), _stream(stream)))


def moe_grouped_ffn_fwd(x, w1, w2, sorted_slot_ids, slot_probs, C: int, act, route_out,
                        stream=None):
    N, H = x.shape
    E, I2, H1 = w1.shape
    I = I2 // 2
    if H1 != H or tuple(w2.shape) != (E, H, I) or I2 != 2 * I:
        raise ValueError("weights must be w1 [E, 2I, H] and w2 [E, H, I]")
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_ffn_fwd", lib.moe_grouped_ffn_fwd(
        _ptr(x, torch.bfloat16, N * H, "x"), _ptr(w1, torch.bfloat16, E * 2 * I * H, "w1"),
        _ptr(w2, torch.bfloat16, E * H * I, "w2"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"), N, H, I, E, C,
        _ptr(act, torch.bfloat16, R * I, "act"), _ptr(route_out, torch.bfloat16, R * H, "route_out"),
        _stream(stream)))


def moe_grouped_fc1_swiglu(x, w1, sorted_slot_ids, slot_probs, C: int, act, stream=None):
    N, H = x.shape
    E, I2, H1 = w1.shape
    I = I2 // 2
    if H1 != H or I2 != 2 * I:
        raise ValueError("w1 must be [E, 2I, H]")
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc1_swiglu", lib.moe_grouped_fc1_swiglu(
        _ptr(x, torch.bfloat16, N * H, "x"), _ptr(w1, torch.bfloat16, E * 2 * I * H, "w1"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"), N, H, I, E, C,
        _ptr(act, torch.bfloat16, R * I, "act"), _stream(stream)))


def moe_grouped_fc2(act, w2, N: int, C: int, route_out, stream=None):
    E, H, I = w2.shape
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc2", lib.moe_grouped_fc2(
        _ptr(act, torch.bfloat16, R * I, "act"), _ptr(w2, torch.bfloat16, E * H * I, "w2"),
        N, H, I, E, C, _ptr(route_out, torch.bfloat16, R * H, "route_out"), _stream(stream)))


def moe_grouped_fc2_rows(act, w2, out_rows, N: int, C: int, route_out, stream=None):
    E, H, I = w2.shape
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc2_rows", lib.moe_grouped_fc2_rows(
        _ptr(act, torch.bfloat16, R * I, "act"), _ptr(w2, torch.bfloat16, E * H * I, "w2"),
        _ptr(out_rows, torch.int32, R, "out_rows"), N, H, I, E, C,
        _ptr(route_out, torch.bfloat16, R * H, "route_out"), _stream(stream)))


def moe_gather_combine(route_out, token_routes, y, stream=None):
    N, K = token_routes.shape
    R, H = route_out.shape
    _check("moe_gather_combine", lib.moe_gather_combine(
        _ptr(route_out, torch.bfloat16, R * H, "route_out"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"), N, K, H, R,
        _ptr(y, torch.bfloat16, N * H, "y"), _stream(stream)))


def moe_dispatch_rows(x, sorted_slot_ids, rows, stream=None):
    N, H = x.shape
    R = sorted_slot_ids.shape[0]
    _check("moe_dispatch_rows", lib.moe_dispatch_rows(
        _ptr(x, torch.bfloat16, N * H, "x"), _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        N, H, R, _ptr(rows, torch.bfloat16, R * H, "rows"), _stream(stream)))


def moe_route_dropless(logits, K: int, topk_ids, topk_probs, route_within, route_counts,
                       sorted_slot_ids, slot_probs, expert_ids, block_start, token_routes,
                       token_route_count, num_tokens_post_padded, workspace, stream=None):
    N, E = logits.shape
    R = moe_dropless_bound(N, K, E)
    BM = moe_layout_block_m()
    _check("moe_route_dropless", lib.moe_route_dropless(
        _ptr(logits, torch.float32, N * E, "logits"), N, E, K,
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(route_within, torch.int32, N * K, "route_within"),
        _ptr(route_counts, torch.int32, E, "route_counts"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(expert_ids, torch.int32, R // BM, "expert_ids"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"),
        _ptr(token_route_count, torch.int32, N, "token_route_count"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"),
        *_ws(workspace, N, E, K), _stream(stream)))


def moe_route_dropless_live(logits, K: int, n_live, topk_ids, topk_probs, route_within,
                            route_counts, sorted_slot_ids, slot_probs, expert_ids, block_start,
                            token_routes, token_route_count, num_tokens_post_padded, workspace,
                            stream=None):
    N, E = logits.shape
    R = moe_dropless_bound(N, K, E)
    BM = moe_layout_block_m()
    _check("moe_route_dropless_live", lib.moe_route_dropless_live(
        _ptr(logits, torch.float32, N * E, "logits"), N, E, K,
        _ptr(n_live, torch.int32, 1, "n_live"),
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(route_within, torch.int32, N * K, "route_within"),
        _ptr(route_counts, torch.int32, E, "route_counts"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(expert_ids, torch.int32, R // BM, "expert_ids"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"),
        _ptr(token_route_count, torch.int32, N, "token_route_count"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"),
        *_ws(workspace, N, E, K), _stream(stream)))


def moe_grouped_ffn_fwd_dropless(x, w1, w2, sorted_slot_ids, slot_probs, block_start,
                                 num_tokens_post_padded, K: int, act, route_out, stream=None):
    N, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    R = moe_dropless_bound(N, K, E)
    _check("moe_grouped_ffn_fwd_dropless", lib.moe_grouped_ffn_fwd_dropless(
        _ptr(x, torch.bfloat16, N * H, "x"), _ptr(w1, torch.bfloat16, E * 2 * I * H, "w1"),
        _ptr(w2, torch.bfloat16, E * H * I, "w2"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"),
        N, H, I, E, K, _ptr(act, torch.bfloat16, R * I, "act"),
        _ptr(route_out, torch.bfloat16, R * H, "route_out"), _stream(stream)))


def moe_grouped_fc1_swiglu_dropless(x, w1, sorted_slot_ids, slot_probs, block_start,
                                    num_tokens_post_padded, K: int, act, stream=None):
    N, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    R = moe_dropless_bound(N, K, E)
    _check("moe_grouped_fc1_swiglu_dropless", lib.moe_grouped_fc1_swiglu_dropless(
        _ptr(x, torch.bfloat16, N * H, "x"), _ptr(w1, torch.bfloat16, E * 2 * I * H, "w1"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"),
        N, H, I, E, K, _ptr(act, torch.bfloat16, R * I, "act"), _stream(stream)))


def moe_grouped_fc2_dropless(act, w2, block_start, num_tokens_post_padded, N: int, K: int,
                             route_out, stream=None):
    E, H, I = w2.shape
    R = moe_dropless_bound(N, K, E)
    _check("moe_grouped_fc2_dropless", lib.moe_grouped_fc2_dropless(
        _ptr(act, torch.bfloat16, R * I, "act"), _ptr(w2, torch.bfloat16, E * H * I, "w2"),
        _ptr(block_start, torch.int32, E, "block_start"),
        _ptr(num_tokens_post_padded, torch.int32, 1, "num_tokens_post_padded"),
        N, H, I, E, K, _ptr(route_out, torch.bfloat16, R * H, "route_out"), _stream(stream)))


# ---------------------------------------------------------------- backward

def _ffn_shape(x, w1):
    N, H = x.shape
    E, I2, H1 = w1.shape
    if H1 != H or I2 % 2:
        raise ValueError("w1 must be [E, 2I, H] with x [N, H]")
    return N, H, I2 // 2, E


def moe_grouped_fc1_swiglu_save(x, w1, sorted_slot_ids, slot_probs, C: int, act, preact,
                                stream=None):
    N, H, I, E = _ffn_shape(x, w1)
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc1_swiglu_save", lib.moe_grouped_fc1_swiglu_save(
        _ptr(x, torch.bfloat16, N * H, "x"), _ptr(w1, torch.bfloat16, E * 2 * I * H, "w1"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"), N, H, I, E, C,
        _ptr(act, torch.bfloat16, R * I, "act"), _ptr(preact, torch.bfloat16, R * 2 * I, "preact"),
        _stream(stream)))


def moe_grouped_fc2_dgrad(dy, w2, sorted_slot_ids, C: int, d_act, stream=None):
    N, H = dy.shape
    E, H2, I = w2.shape
    if H2 != H:
        raise ValueError("w2 must be [E, H, I] with dy [N, H]")
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc2_dgrad", lib.moe_grouped_fc2_dgrad(
        _ptr(dy, torch.bfloat16, N * H, "dy"), _ptr(w2, torch.bfloat16, E * H * I, "w2"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"), N, H, I, E, C,
        _ptr(d_act, torch.bfloat16, R * I, "d_act"), _stream(stream)))


def moe_swiglu_bwd(preact, d_act, slot_probs, act, d_preact, d_prob, stream=None):
    R, I = d_act.shape
    _check("moe_swiglu_bwd", lib.moe_swiglu_bwd(
        _ptr(preact, torch.bfloat16, R * 2 * I, "preact"),
        _ptr(d_act, torch.bfloat16, R * I, "d_act"),
        _ptr(slot_probs, torch.float32, R, "slot_probs"), R, I,
        _ptr(act, torch.bfloat16, R * I, "act"),
        _ptr(d_preact, torch.bfloat16, R * 2 * I, "d_preact"),
        _ptr(d_prob, torch.float32, R, "d_prob"), _stream(stream)))


def moe_grouped_fc1_dgrad(d_preact, w1, N: int, C: int, d_a, stream=None):
    E, I2, H = w1.shape
    I = I2 // 2
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc1_dgrad", lib.moe_grouped_fc1_dgrad(
        _ptr(d_preact, torch.bfloat16, R * 2 * I, "d_preact"),
        _ptr(w1, torch.bfloat16, E * 2 * I * H, "w1"), N, H, I, E, C,
        _ptr(d_a, torch.bfloat16, R * H, "d_a"), _stream(stream)))


def moe_grouped_fc2_wgrad(dy, act, sorted_slot_ids, E: int, C: int, dw2, stream=None):
    N, H = dy.shape
    R, I = act.shape
    if R < E * moe_padded_capacity(C):
        raise ValueError("act must hold E*Cp rows")
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc2_wgrad", lib.moe_grouped_fc2_wgrad(
        _ptr(dy, torch.bfloat16, N * H, "dy"), _ptr(act, torch.bfloat16, R * I, "act"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"), N, H, I, E, C,
        _ptr(dw2, torch.bfloat16, E * H * I, "dw2"), _stream(stream)))


def moe_grouped_fc1_wgrad(d_preact, x, sorted_slot_ids, E: int, C: int, dw1, stream=None):
    N, H = x.shape
    R2, I2 = d_preact.shape
    I = I2 // 2
    R = E * moe_padded_capacity(C)
    if R2 < R:
        raise ValueError("d_preact must hold E*Cp rows")
    _check("moe_grouped_fc1_wgrad", lib.moe_grouped_fc1_wgrad(
        _ptr(d_preact, torch.bfloat16, R * 2 * I, "d_preact"), _ptr(x, torch.bfloat16, N * H, "x"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"), N, H, I, E, C,
        _ptr(dw1, torch.bfloat16, E * 2 * I * H, "dw1"), _stream(stream)))


def moe_grouped_fc2_wgrad_accum(dy, act, sorted_slot_ids, E: int, C: int, main_dw2, stream=None):
    """main_dw2 (float32 [E, H, I]) += the FC2 weight gradient."""
    N, H = dy.shape
    R, I = act.shape
    if R < E * moe_padded_capacity(C):
        raise ValueError("act must hold E*Cp rows")
    R = E * moe_padded_capacity(C)
    _check("moe_grouped_fc2_wgrad_accum", lib.moe_grouped_fc2_wgrad_accum(
        _ptr(dy, torch.bfloat16, N * H, "dy"), _ptr(act, torch.bfloat16, R * I, "act"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"), N, H, I, E, C,
        _ptr(main_dw2, torch.float32, E * H * I, "main_dw2"), _stream(stream)))


def moe_grouped_fc1_wgrad_accum(d_preact, x, sorted_slot_ids, E: int, C: int, main_dw1, stream=None):
    """main_dw1 (float32 [E, 2I, H]) += the FC1 weight gradient."""
    N, H = x.shape
    R2, I2 = d_preact.shape
    I = I2 // 2
    R = E * moe_padded_capacity(C)
    if R2 < R:
        raise ValueError("d_preact must hold E*Cp rows")
    _check("moe_grouped_fc1_wgrad_accum", lib.moe_grouped_fc1_wgrad_accum(
        _ptr(d_preact, torch.bfloat16, R * 2 * I, "d_preact"), _ptr(x, torch.bfloat16, N * H, "x"),
        _ptr(sorted_slot_ids, torch.int32, R, "sorted_slot_ids"), N, H, I, E, C,
        _ptr(main_dw1, torch.float32, E * 2 * I * H, "main_dw1"), _stream(stream)))


def moe_route_bwd(topk_ids, topk_probs, token_routes, d_prob, d_logits, stream=None):
    N, K = topk_ids.shape
    E = d_logits.shape[1]
    R = d_prob.numel()
    _check("moe_route_bwd", lib.moe_route_bwd(
        _ptr(topk_ids, torch.int32, N * K, "topk_ids"),
        _ptr(topk_probs, torch.float32, N * K, "topk_probs"),
        _ptr(token_routes, torch.int32, N * K, "token_routes"),
        _ptr(d_prob, torch.float32, R, "d_prob"), N, E, K, R,
        _ptr(d_logits, torch.float32, N * E, "d_logits"), _stream(stream)))

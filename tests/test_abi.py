"""The C-ABI library loads, exports every declared symbol, and its host-only
logic (capacity arithmetic, argument validation) is right.  No device work."""

import ctypes
import math
import random
from fractions import Fraction

import pytest

import mixture_experts_expert_amd as moe
from conftest import load_golden

lib = moe.lib
OK, INVALID, UNSUPPORTED, MISALIGNED = 0, -1, -2, -3


def test_every_declared_symbol_is_exported():
    names = moe.header_functions()
    assert set(names) == {"moe_status_string", "moe_source_capacity", "moe_layout_block_m",
                          "moe_padded_capacity", "moe_route_capacity", "moe_route_capacity_align",
                          "moe_align", "moe_dropless_bound", "moe_route_dropless",
                          "moe_grouped_ffn_fwd_dropless", "moe_grouped_fc1_swiglu_dropless",
                          "moe_grouped_fc2_dropless",
                          "moe_grouped_ffn_fwd", "moe_grouped_fc1_swiglu", "moe_grouped_fc2",
                          "moe_gather_combine", "moe_grouped_fc1_swiglu_save",
                          "moe_grouped_fc2_dgrad", "moe_swiglu_bwd", "moe_grouped_fc1_dgrad",
                          "moe_grouped_fc2_wgrad", "moe_grouped_fc1_wgrad", "moe_route_bwd",
                          "moe_grouped_fc2_wgrad_accum", "moe_grouped_fc1_wgrad_accum",
                          "moe_route_dropless_live", "moe_dispatch_rows",
                          "moe_grouped_fc2_rows", "moe_route_capacity_workspace_bytes",
                          "moe_route_capacity_align_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_probe_header_symbols_and_validation():
    names = moe.header_functions(moe.PROBE_HEADER_PATH)
    assert set(names) == {"moe_probe_read", "moe_probe_write", "moe_probe_copy",
                          "moe_probe_read_pieces", "moe_probe_write_pieces", "moe_probe_write_tiles",
                          "moe_probe_lds_ring", "moe_probe_gemm_loop", "moe_probe_mfma_rate",
                          "moe_probe_lds_read"}
    for n in names:
        assert hasattr(lib, n), n
    big = ctypes.c_size_t(1 << 20)
    assert lib.moe_probe_read(NUL, big, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_read(ALIGNED, big, NUL, NUL) == INVALID
    assert lib.moe_probe_read(MIS, big, ALIGNED, NUL) == MISALIGNED
    assert lib.moe_probe_write(ALIGNED, ctypes.c_size_t(17), NUL) == MISALIGNED
    assert lib.moe_probe_copy(ALIGNED, MIS, big, NUL) == MISALIGNED
    assert lib.moe_probe_copy(ALIGNED, ALIGNED, ctypes.c_size_t(0), NUL) == OK
    assert lib.moe_probe_write(ALIGNED, ctypes.c_size_t(0), NUL) == OK
    # access-order probes: panel geometry, pieces, sink, stages
    panel = ctypes.c_size_t(256 * 4096)
    assert lib.moe_probe_read_pieces(NUL, panel, 4096, 256, 128, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_read_pieces(ALIGNED, panel, 4096, 256, 128, NUL, NUL) == INVALID
    assert lib.moe_probe_read_pieces(MIS, panel, 4096, 256, 128, ALIGNED, NUL) == MISALIGNED
    assert lib.moe_probe_read_pieces(ALIGNED, panel, 4096, 256, 96, ALIGNED, NUL) == MISALIGNED
    assert lib.moe_probe_read_pieces(ALIGNED, panel, 4096, 256, 8, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_read_pieces(ALIGNED, panel, 4096, 0, 128, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_read_pieces(ALIGNED, ctypes.c_size_t(4096 * 100), 4096, 256, 128, ALIGNED,
                                     NUL) == INVALID                      # not whole panels
    assert lib.moe_probe_read_pieces(ALIGNED, ctypes.c_size_t(0), 4096, 256, 128, ALIGNED, NUL) == OK
    assert lib.moe_probe_write_pieces(ALIGNED, panel, 4008, 256, 16, 0, NUL) == MISALIGNED
    assert lib.moe_probe_write_pieces(ALIGNED, ctypes.c_size_t(0), 4096, 256, 512, 1, NUL) == OK
    assert lib.moe_probe_write_tiles(NUL, panel, 4096, 256, 512, 1, NUL) == INVALID
    assert lib.moe_probe_write_tiles(MIS, panel, 4096, 256, 512, 1, NUL) == MISALIGNED
    assert lib.moe_probe_write_tiles(ALIGNED, panel, 4096, 256, 96, 1, NUL) == MISALIGNED
    assert lib.moe_probe_write_tiles(ALIGNED, panel, 4096, 0, 512, 0, NUL) == INVALID
    assert lib.moe_probe_write_tiles(ALIGNED, ctypes.c_size_t(4096 * 100), 4096, 256, 512, 0,
                                     NUL) == INVALID                      # not whole panels
    assert lib.moe_probe_write_tiles(ALIGNED, ctypes.c_size_t(0), 4096, 256, 512, 0, NUL) == OK
    assert lib.moe_probe_lds_ring(ALIGNED, big, 1, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_lds_ring(ALIGNED, big, 6, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_lds_ring(ALIGNED, ctypes.c_size_t(4096), 3, ALIGNED, NUL) == INVALID
    assert lib.moe_probe_lds_ring(ALIGNED, big, 3, NUL, NUL) == INVALID
    assert lib.moe_probe_lds_ring(ALIGNED, ctypes.c_size_t(0), 3, ALIGNED, NUL) == OK
    g = lib.moe_probe_gemm_loop
    assert g(NUL, ALIGNED, 4, 256, 256, 128, ALIGNED, NUL) == INVALID
    assert g(ALIGNED, ALIGNED, 4, 256, 256, 128, NUL, NUL) == INVALID
    assert g(MIS, ALIGNED, 4, 256, 256, 128, ALIGNED, NUL) == MISALIGNED
    assert g(ALIGNED, ALIGNED, -1, 256, 256, 128, ALIGNED, NUL) == INVALID
    assert g(ALIGNED, ALIGNED, 4, 200, 256, 128, ALIGNED, NUL) == UNSUPPORTED   # Cp % 256
    assert g(ALIGNED, ALIGNED, 4, 256, 256, 100, ALIGNED, NUL) == UNSUPPORTED   # K % 64
    assert g(ALIGNED, ALIGNED, 4, 256, 1 << 20, 1 << 10, ALIGNED, NUL) == UNSUPPORTED   # 2 GiB
    assert g(ALIGNED, ALIGNED, 0, 256, 256, 128, ALIGNED, NUL) == OK
    for f in (lib.moe_probe_mfma_rate, lib.moe_probe_lds_read):
        assert f(256, 100, NUL, NUL) == INVALID       # no clocks buffer
        assert f(-1, 100, ALIGNED, NUL) == INVALID
        assert f(256, 0, ALIGNED, NUL) == INVALID     # iters < 1
        assert f(0, 100, ALIGNED, NUL) == OK          # no workgroups: nothing to do


def test_capacity_golden_values():
    for c in load_golden("capacity_closed_form.json")["cases"]:
        assert moe.moe_source_capacity(c["N"], c["K"], c["E"], c["F"]) == c["C"], c


def test_capacity_matches_exact_rationals_random():
    rng = random.Random(7)
    for _ in range(3000):
        E = rng.randint(1, 1024)
        K = rng.randint(1, min(E, 32))
        N = rng.randint(0, 1 << 20)
        F = rng.choice([rng.uniform(0.01, 4.0), rng.randint(1, 8) / rng.randint(1, 8),
                        1.0 + rng.randint(-4, 4) * 2.0 ** -52, 2.0 ** rng.randint(-30, 3)])
        want = math.ceil(Fraction(N * K) * Fraction(F) / E)
        assert moe.moe_source_capacity(N, K, E, F) == want, (N, K, E, F)


@pytest.mark.parametrize("args,status", [((4, 0, 4, 1.0), INVALID), ((4, 5, 4, 1.0), INVALID),
                                         ((-1, 1, 4, 1.0), INVALID), ((4, 1, 4, 0.0), INVALID),
                                         ((4, 1, 4, -1.0), INVALID), ((4, 1, 4, float("nan")), INVALID),
                                         ((4, 1, 4, float("inf")), INVALID), ((4, 1, 0, 1.0), INVALID),
                                         ((1 << 30, 32, 32, 1e6), UNSUPPORTED)])
def test_capacity_bad_args(args, status):
    assert lib.moe_source_capacity(*args) == status


def test_layout_block_and_padding():
    assert moe.moe_layout_block_m() == 32
    assert [moe.moe_padded_capacity(c) for c in (0, 1, 32, 33, 320)] == [0, 32, 32, 64, 320]
    assert lib.moe_padded_capacity(-5) == INVALID


def test_status_strings():
    assert moe.moe_status_string(0) == "MOE_OK"
    assert moe.moe_status_string(-2) == "MOE_ERR_UNSUPPORTED"
    assert moe.moe_status_string(123) == "MOE_ERR_UNKNOWN"


# Host-side validation returns before any device call, so these run without a GPU.
P = ctypes.c_void_p
NUL = P(0)
ALIGNED = P(0x10000)        # never dereferenced: rejected or no-op before any launch
MIS = P(0x10004)


WSB = ctypes.c_size_t(1 << 30)   # a workspace size that always suffices
WS = (ALIGNED, WSB)


def test_route_workspace_bytes():
    f = lib.moe_route_capacity_workspace_bytes
    for N, E, K in [(64, 4, 2), (1024, 8, 2), (4096, 128, 8), (8192, 256, 8), (1, 1, 1),
                    (17, 3, 2), (16384, 1024, 32), (0, 4, 2)]:
        assert f(N, E, K) == 5 * E * (-(-N // 16) * 16), (N, E, K)
        assert moe.moe_route_capacity_workspace_bytes(N, E, K) == 5 * E * (-(-N // 16) * 16)
    for bad in [(16, 4, 5), (16, 4, 0), (-1, 4, 2), (20000, 8, 2), (16, 2048, 8), (16, 64, 33)]:
        assert f(*bad) == 0, bad


def test_route_capacity_validation():
    f = lib.moe_route_capacity
    a = [ALIGNED] * 4
    assert f(ALIGNED, 16, 4, 5, 20, *a, *WS, NUL) == INVALID                 # K > E
    assert f(ALIGNED, 16, 4, 0, 8, *a, *WS, NUL) == INVALID                  # K < 1
    assert f(ALIGNED, 16, 2048, 8, 64, *a, *WS, NUL) == UNSUPPORTED          # E
    assert f(ALIGNED, 16, 64, 33, 64, *a, *WS, NUL) == UNSUPPORTED           # K
    assert f(ALIGNED, 20000, 8, 2, 5000, *a, *WS, NUL) == UNSUPPORTED        # N
    assert f(NUL, 16, 4, 2, 8, *a, *WS, NUL) == INVALID
    assert f(MIS, 16, 4, 2, 8, *a, *WS, NUL) == MISALIGNED
    assert f(ALIGNED, 16, 4, 2, 8, *a, NUL, WSB, NUL) == INVALID             # no workspace
    assert f(ALIGNED, 16, 4, 2, 8, *a, MIS, WSB, NUL) == MISALIGNED
    # the workspace must hold 5 bytes per expert and token, tokens rounded up
    # to 16: 5 * 4 * 32 here
    assert f(ALIGNED, 17, 4, 2, 9, *a, ALIGNED, ctypes.c_size_t(639), NUL) == INVALID
    assert f(NUL, 0, 4, 2, 0, NUL, NUL, NUL, NUL, NUL, ctypes.c_size_t(0), NUL) == OK   # N = 0


def test_route_capacity_align_validation():
    f = lib.moe_route_capacity_align
    o = [ALIGNED] * 7
    assert f(ALIGNED, 16, 4, 5, 20, *([ALIGNED] * 4), *o, *WS, NUL) == INVALID          # K > E
    assert f(ALIGNED, 16, 2048, 8, 64, *([ALIGNED] * 4), *o, *WS, NUL) == UNSUPPORTED   # E
    assert f(ALIGNED, 16, 4, 2, 8, *([ALIGNED] * 4), *o[:6], MIS, *WS, NUL) == MISALIGNED
    assert f(ALIGNED, 16, 4, 2, 8, *([ALIGNED] * 4), *o[:2], NUL, *o[3:], *WS, NUL) == INVALID
    assert f(ALIGNED, 16, 4, 2, 8, *([ALIGNED] * 4), *o, ALIGNED, ctypes.c_size_t(319), NUL) == INVALID
    assert f(NUL, 0, 4, 2, 0, *([NUL] * 4), *([NUL] * 7), NUL, ctypes.c_size_t(0), NUL) == OK   # N = 0


def test_route_noalloc_validation():
    f = lib.moe_route_capacity_align_noalloc
    o = [ALIGNED] * 7
    assert f(ALIGNED, 16, 4, 5, 20, *([ALIGNED] * 4), *o, NUL) == INVALID                 # K > E
    assert f(ALIGNED, 16, 4, 2, 8, *([ALIGNED] * 4), *o[:6], MIS, NUL) == MISALIGNED
    # the map must fit the 16 MiB scratch array: 5 * 1024 * 16384 bytes does not
    assert f(ALIGNED, 16384, 1024, 8, 128, *([ALIGNED] * 4), *o, NUL) == UNSUPPORTED
    assert f(NUL, 0, 4, 2, 0, *([NUL] * 4), *([NUL] * 7), NUL) == OK                       # N = 0


def test_dropless_bound_and_validation():
    for N, K, E in [(4, 2, 3), (4096, 8, 128), (1, 1, 1), (16384, 32, 1000), (0, 2, 4)]:
        r = N * min(K, E) + E * 31
        assert moe.moe_dropless_bound(N, K, E) == -(-r // 32) * 32
    assert lib.moe_dropless_bound(4, 5, 4) == INVALID and lib.moe_dropless_bound(20000, 2, 8) == UNSUPPORTED
    f = lib.moe_route_dropless
    o = [ALIGNED] * 11
    assert f(ALIGNED, 16, 4, 5, *o, *WS, NUL) == INVALID                      # K > E
    assert f(ALIGNED, 16, 4, 2, *o[:10], MIS, *WS, NUL) == MISALIGNED
    assert f(ALIGNED, 16, 4, 2, *o[:3], NUL, *o[4:], *WS, NUL) == INVALID
    assert f(ALIGNED, 16, 4, 2, *o, NUL, WSB, NUL) == INVALID                # no workspace
    assert f(NUL, 0, 4, 2, *([NUL] * 11), NUL, ctypes.c_size_t(0), NUL) == OK  # N = 0
    v = lib.moe_route_dropless_live
    assert v(ALIGNED, 16, 4, 2, NUL, *o, *WS, NUL) == INVALID                  # no live count
    assert v(ALIGNED, 16, 4, 2, MIS, *o, *WS, NUL) == MISALIGNED
    assert v(ALIGNED, 16, 4, 5, ALIGNED, *o, *WS, NUL) == INVALID              # K > E
    assert v(ALIGNED, 16, 4, 2, ALIGNED, *o, ALIGNED, ctypes.c_size_t(8), NUL) == INVALID
    g = lib.moe_grouped_ffn_fwd_dropless
    p7 = [ALIGNED] * 7
    assert g(*p7, 16, 100, 64, 4, 2, ALIGNED, ALIGNED, NUL) == UNSUPPORTED     # H % 64
    assert g(*p7, 16, 64, 64, 4, 5, ALIGNED, ALIGNED, NUL) == INVALID          # K > E
    assert g(*p7, 16, 64, 64, 4, 2, ALIGNED, MIS, NUL) == MISALIGNED
    assert g(*([NUL] * 7), 0, 64, 64, 4, 2, NUL, NUL, NUL) == OK


def test_align_validation():
    f = lib.moe_align
    a = [ALIGNED] * 4
    o = [ALIGNED] * 7
    assert f(*a, 16, 4, 2, -1, *o, NUL) == INVALID
    assert f(*a, 16, 4, 2, 8, *o[:6], MIS, NUL) == MISALIGNED
    assert f(*a, 16, 4, 2, 8, *o[:3], NUL, *o[4:], NUL) == INVALID
    assert f(*([NUL] * 4), 0, 4, 2, 0, *([NUL] * 7), NUL) == OK


def test_grouped_ffn_validation():
    f = lib.moe_grouped_ffn_fwd
    p5 = [ALIGNED] * 5
    assert f(*p5, 16, 100, 64, 4, 8, ALIGNED, ALIGNED, NUL) == UNSUPPORTED     # H % 64
    assert f(*p5, 16, 64, 96, 4, 8, ALIGNED, ALIGNED, NUL) == UNSUPPORTED      # I % 64
    assert f(*p5, 16, 64, 64, 4, 8, ALIGNED, MIS, NUL) == MISALIGNED
    assert f(*p5, 16, 64, 64, 4, 8, NUL, ALIGNED, NUL) == INVALID
    assert f(*([NUL] * 5), 0, 64, 64, 4, 0, NUL, NUL, NUL) == OK


def test_split_ffn_validation():
    f1, f2 = lib.moe_grouped_fc1_swiglu, lib.moe_grouped_fc2
    p4 = [ALIGNED] * 4
    assert f1(*p4, 16, 100, 64, 4, 8, ALIGNED, NUL) == UNSUPPORTED
    assert f1(*p4, 16, 64, 64, 4, 8, MIS, NUL) == MISALIGNED
    assert f1(*([NUL] * 4), 0, 64, 64, 4, 0, NUL, NUL) == OK
    assert f2(ALIGNED, ALIGNED, 16, 64, 96, 4, 8, ALIGNED, NUL) == UNSUPPORTED
    assert f2(ALIGNED, NUL, 16, 64, 64, 4, 8, ALIGNED, NUL) == INVALID
    assert f2(NUL, NUL, 0, 64, 64, 4, 0, NUL, NUL) == OK


def test_combine_validation():
    f = lib.moe_gather_combine
    assert f(ALIGNED, ALIGNED, 16, 0, 64, 128, ALIGNED, NUL) == INVALID
    assert f(ALIGNED, ALIGNED, 16, 2, 72, 128, ALIGNED, NUL) == UNSUPPORTED
    assert f(ALIGNED, MIS, 16, 2, 64, 128, ALIGNED, NUL) == MISALIGNED
    assert f(NUL, NUL, 0, 2, 64, 0, NUL, NUL) == OK


def test_fc2_rows_validation():
    f = lib.moe_grouped_fc2_rows
    A = ALIGNED
    assert f(A, A, A, -1, 64, 64, 4, 8, A, NUL) == INVALID
    assert f(A, A, A, 16, 72, 64, 4, 8, A, NUL) == UNSUPPORTED
    assert f(A, A, NUL, 16, 64, 64, 4, 8, A, NUL) == INVALID
    assert f(A, A, MIS, 16, 64, 64, 4, 8, A, NUL) == MISALIGNED
    # the whole output past 2^31 bytes: 1024 experts x 128 slots x 8192 x 2
    assert f(A, A, A, 16, 8192, 64, 1024, 128, A, NUL) == UNSUPPORTED
    assert f(NUL, NUL, NUL, 0, 64, 64, 4, 8, NUL, NUL) == OK   # no tokens


def test_dispatch_rows_validation():
    f = lib.moe_dispatch_rows
    assert f(ALIGNED, ALIGNED, -1, 64, 128, ALIGNED, NUL) == INVALID
    assert f(ALIGNED, ALIGNED, 16, 0, 128, ALIGNED, NUL) == INVALID
    assert f(ALIGNED, ALIGNED, 16, 64, -1, ALIGNED, NUL) == INVALID
    assert f(ALIGNED, ALIGNED, 16, 72, 128, ALIGNED, NUL) == UNSUPPORTED
    assert f(ALIGNED, ALIGNED, 16, 64, 2**31, ALIGNED, NUL) == UNSUPPORTED
    assert f(NUL, ALIGNED, 16, 64, 128, ALIGNED, NUL) == INVALID
    assert f(ALIGNED, MIS, 16, 64, 128, ALIGNED, NUL) == MISALIGNED
    assert f(NUL, NUL, 16, 64, 0, NUL, NUL) == OK          # no slots: nothing to write


def test_backward_validation():
    A = ALIGNED
    f = lib.moe_grouped_fc1_swiglu_save
    assert f(A, A, A, A, 16, 100, 64, 4, 8, A, A, NUL) == UNSUPPORTED               # H % 64
    assert f(A, A, A, A, 16, 64, 64, 4, 8, A, MIS, NUL) == MISALIGNED
    assert f(A, A, A, A, 16, 64, 64, 4, 8, A, NUL, NUL) == INVALID
    assert f(*([NUL] * 4), 0, 64, 64, 4, 0, NUL, NUL, NUL) == OK
    for g in (lib.moe_grouped_fc2_dgrad, lib.moe_grouped_fc2_wgrad, lib.moe_grouped_fc1_wgrad,
              lib.moe_grouped_fc2_wgrad_accum, lib.moe_grouped_fc1_wgrad_accum):
        assert g(A, A, A, 16, 64, 96, 4, 8, A, NUL) == UNSUPPORTED                   # I % 64
        assert g(A, A, A, -1, 64, 64, 4, 8, A, NUL) == INVALID                        # N < 0
        assert g(A, A, NUL, 16, 64, 64, 4, 8, A, NUL) == INVALID
        assert g(A, A, A, 16, 64, 64, 4, 8, MIS, NUL) == MISALIGNED
        assert g(NUL, NUL, NUL, 0, 64, 64, 4, 0, NUL, NUL) == OK
    for g in (lib.moe_grouped_fc2_wgrad_accum, lib.moe_grouped_fc1_wgrad_accum):
        # one expert's float32 gradient (2*I*H*4 bytes) reaches 2 GiB; its bf16 one does not
        assert g(A, A, A, 16, 16384, 16384, 4, 8, A, NUL) == UNSUPPORTED
        assert g(A, A, A, 16, 16384, 8192, 4, 8, NUL, NUL) == INVALID
    assert lib.moe_grouped_fc1_wgrad(A, A, A, 16, 16384, 16384, 4, 8, NUL, NUL) == INVALID
    g = lib.moe_grouped_fc1_dgrad
    assert g(A, A, 16, 64, 64, 2048, 8, A, NUL) == UNSUPPORTED                         # E > 1024
    assert g(A, NUL, 16, 64, 64, 4, 8, A, NUL) == INVALID
    assert g(NUL, NUL, 0, 64, 64, 4, 0, NUL, NUL) == OK
    h = lib.moe_swiglu_bwd
    assert h(A, A, A, 128, 100, A, A, A, NUL) == UNSUPPORTED                           # I % 64
    assert h(A, A, A, -1, 64, A, A, A, NUL) == INVALID
    assert h(A, A, A, 128, 64, A, A, MIS, NUL) == MISALIGNED
    assert h(NUL, NUL, NUL, 0, 64, NUL, NUL, NUL, NUL) == OK
    r = lib.moe_route_bwd
    assert r(A, A, A, A, 16, 4, 5, 128, A, NUL) == INVALID                             # K > E
    assert r(A, A, A, A, 16, 4, 2, 128, NUL, NUL) == INVALID
    assert r(A, A, A, A, 16, 2048, 2, 128, A, NUL) == UNSUPPORTED
    assert r(NUL, NUL, NUL, NUL, 0, 4, 2, 0, NUL, NUL) == OK

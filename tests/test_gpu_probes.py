"""The HBM rate probes do what their rates assume: the copy reproduces its
source byte for byte and the write fills every 16-byte word of its buffer,
for sizes that leave partial chunks; the access-order writes (piece columns
per workgroup, and tiles dealt over the XCDs) fill every word in each piece
order and policy (the reads, and the LDS ring, are checked for running
through the buffer)."""

import pytest
import torch

import mixture_experts_expert_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 777, (64 << 20) + 48])
def test_probe_copy_write_read(nbytes):
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    moe.moe_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    moe.moe_probe_write(dst)
    torch.cuda.synchronize()
    words = dst.view(torch.int32).view(-1, 4)
    expect = torch.tensor([0x5A5A0000, 0x5A5A0001, 0x5A5A0002, 0x5A5A0003], dtype=torch.int32,
                          device="cuda")
    assert torch.equal(words, expect.expand_as(words))
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    moe.moe_probe_read(src, sink)
    torch.cuda.synchronize()


@pytest.mark.parametrize("piece,nt", [(128, True), (512, False), (4096, True), (48, False)])
def test_access_order_write_covers_every_word(piece, nt):
    row_bytes = 4096 if piece != 48 else 96 * 16
    rows, panels = 256, 3
    dst = torch.zeros(panels * rows * row_bytes, dtype=torch.uint8, device="cuda")
    moe.moe_probe_write_pieces(dst, row_bytes, rows, piece, nt)
    torch.cuda.synchronize()
    words = dst.view(torch.int32).view(-1, 4)
    expect = torch.tensor([0x3C3C0000, 0x3C3C0001, 0x3C3C0002, 0x3C3C0003], dtype=torch.int32,
                          device="cuda")
    assert torch.equal(words, expect.expand_as(words))
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    moe.moe_probe_read_pieces(dst, row_bytes, rows, piece, sink)
    torch.cuda.synchronize()


@pytest.mark.parametrize("piece,nt,panels", [(512, True, 3), (1024, False, 5), (4096, True, 2), (48, False, 7)])
def test_tile_order_write_covers_every_word(piece, nt, panels):
    row_bytes = 4096 if piece != 48 else 96 * 16
    rows = 256
    dst = torch.zeros(panels * rows * row_bytes, dtype=torch.uint8, device="cuda")
    moe.moe_probe_write_tiles(dst, row_bytes, rows, piece, nt)
    torch.cuda.synchronize()
    words = dst.view(torch.int32).view(-1, 4)
    expect = torch.tensor([0x3C3C0000, 0x3C3C0001, 0x3C3C0002, 0x3C3C0003], dtype=torch.int32,
                          device="cuda")
    assert torch.equal(words, expect.expand_as(words))


@pytest.mark.parametrize("stages", [2, 3, 4, 5])
def test_lds_ring_runs(stages):
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    moe.moe_probe_lds_ring(src, stages, sink)
    torch.cuda.synchronize()


def test_gemm_loop_runs():
    """The GEMM-loop probe runs over several tiles per workgroup and experts
    (two row tiles, ragged tile count against the CUs)."""
    E, Cp, N, K = 3, 512, 768, 192
    a = torch.randn(E * Cp, K, device="cuda").to(torch.bfloat16)
    b = torch.randn(E, N, K, device="cuda").to(torch.bfloat16)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    moe.moe_probe_gemm_loop(a, b, E, Cp, sink)
    torch.cuda.synchronize()


@pytest.mark.parametrize("probe", ["mfma", "lds"])
def test_compute_probes_record_their_clocks(probe):
    """Every workgroup of the matrix-core and LDS-read probes records its
    engine-clock and constant-clock ticks; the ratio is a clock in the range a
    GPU engine runs at, and the MFMA probe's issue rate per SIMD stays at or
    below one 32x32x16 MFMA per 32 engine clocks (a pipe's full rate: 512
    bf16 multiply-adds per clock)."""
    groups = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    clocks = torch.zeros(2 * groups, dtype=torch.int64, device="cuda")
    f = moe.moe_probe_mfma_rate if probe == "mfma" else moe.moe_probe_lds_read
    f(groups, iters, clocks)
    torch.cuda.synchronize()
    c = clocks.view(groups, 2).cpu()
    assert bool((c > 0).all())
    ghz = c[:, 0].double() / c[:, 1].double() * 0.1
    assert 0.3 < float(ghz.min()) and float(ghz.max()) < 4.0
    if probe == "mfma":
        # each SIMD hosts two of the eight waves: 2 * 4 * iters MFMAs per SIMD
        ticks_per_mfma = c[:, 0].double() / (2 * 4 * iters)
        assert float(ticks_per_mfma.min()) >= 32 * 0.97
    with pytest.raises(ValueError):
        f(groups, iters, clocks[:-1])

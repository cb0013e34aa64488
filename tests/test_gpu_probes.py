"""The HBM rate probes do what their rates assume: the copy reproduces its
source byte for byte and the write fills every 16-byte word of its buffer,
for sizes that leave partial chunks (the read is checked only for running
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

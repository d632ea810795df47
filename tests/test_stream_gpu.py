"""GPU: the reference streams (rr_test_stream) move exactly the bytes asked
for -- a copy reproduces its source, a write covers its range and nothing
beyond it -- including sizes with a ragged tail past the last whole tile."""
import pytest
import torch

import split_deterministic_combine_amd as rr

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 2048 * 3 + 48, (64 << 20) + 16 * 999])
def test_copy_reproduces_its_source(nbytes):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(nbytes)
    x = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    y = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    rr._test_stream("copy", x, y[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(y[:nbytes], x)
    assert int(y[nbytes:].count_nonzero()) == 0


@pytest.mark.parametrize("nbytes", [16, 16 * 2048 * 5 + 32])
def test_write_covers_exactly_its_range(nbytes):
    y = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    rr._test_stream("write", None, y[:nbytes])
    torch.cuda.synchronize()
    words = y[:nbytes].view(torch.int32).view(-1, 4)
    assert bool((words[:, 2] == 0x5EED).all())   # every 16-byte chunk holds the pattern
    assert int(y[nbytes:].count_nonzero()) == 0


def test_read_runs_and_leaves_its_input_unchanged():
    x = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    ref = x.clone()
    for bpc in (1, 2, 4):
        rr._test_stream("read", x, blocks_per_cu=bpc)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)

"""The HBM probes that give the measured bandwidth denominators: the copy
probe copies exactly (whole 1,024-element chunks and the ragged tail), and
the read probe runs without touching its sink for ordinary data."""
import pytest

from tests.gpu_helpers import say, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 1023, 16 * 1024, 16 * 1025, (1 << 20) + 48, (64 << 20) + 16 * 777])
def test_copy_probe_copies_exactly(nbytes):
    from bit_block_scaled_vq_amd import ops
    torch, dev = torch_dev()
    say(f"case: copy probe {nbytes} B")
    g = torch.Generator(device=dev)
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8, device=dev)
    pad = torch.full((nbytes + 4096,), 0xA5, dtype=torch.uint8, device=dev)
    dst = pad[:nbytes]
    ops.vq_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.all(pad[nbytes:] == 0xA5)


def test_read_probe_leaves_sink():
    from bit_block_scaled_vq_amd import ops
    torch, dev = torch_dev()
    src = torch.ones((16 << 20,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    ops.vq_probe_read(src, sink)
    torch.cuda.synchronize()
    assert not sink.any()

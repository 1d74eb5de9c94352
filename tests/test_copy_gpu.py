"""The stream-copy reference kernel (monarch_stream_copy) copies exactly,
including a ragged tail of fewer than 16 bytes."""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("nbytes", [16, 1000, 4096 * 16 + 7, (1 << 24) + 13, 3 << 26])
def test_stream_copy_is_exact(nbytes):
    from monarch_block_diagonal_amd import binding as B
    g = torch.Generator(device="cuda:0")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, device="cuda:0", dtype=torch.uint8)
    dst = torch.zeros(nbytes + 64, device="cuda:0", dtype=torch.uint8)
    B.monarch_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert torch.count_nonzero(dst[nbytes:]).item() == 0     # nothing past the end

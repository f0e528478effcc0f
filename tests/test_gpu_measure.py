"""The measuring sticks of the bench, through the C ABI: the plain copy (ecf8_hbm_copy) and the plain
stream of a decode's byte mix (ecf8_hbm_stream) write exactly what they define."""
import pytest
import torch

from lossless_entropy_coded_ecf8_amd import binding as B

pytestmark = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("n", [16, 4096 * 16 + 7, 3 * (1 << 20) + 5, 64 << 20])
def test_copy_writes_the_source(n):
    d = dev()
    g = torch.Generator(device=d).manual_seed(n)
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, device=d, generator=g)
    b = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device=d)
    B.hbm_copy(a, b[:n])
    torch.cuda.synchronize()
    assert torch.equal(b[:n], a)
    assert (b[n:] == 0xA5).all()


@pytest.mark.parametrize("read_units,write_units", [(1, 1), (1, 1000), (999, 1000), (1000, 1000), (4096, 5123),
                                                    (675_799, 855_638), (3_000_001, 3_800_017)])
def test_stream_writes_the_defined_gather(read_units, write_units):
    """Output unit i = input unit (i * m) >> 32 with m = floor(2^32 * read_units / write_units)."""
    d = dev()
    g = torch.Generator(device=d).manual_seed(read_units)
    src = torch.randint(0, 256, (read_units * 16,), dtype=torch.uint8, device=d, generator=g)
    dst = torch.full((write_units * 16 + 64,), 0xA5, dtype=torch.uint8, device=d)
    B.hbm_stream(src, read_units * 16, dst, write_units * 16)
    torch.cuda.synchronize()
    m = (read_units << 32) // write_units
    i = torch.arange(write_units, dtype=torch.int64, device=d)
    j = (i * m) >> 32
    assert int(j.max()) < read_units
    want = src.view(-1, 16)[j]
    assert torch.equal(dst[:write_units * 16].view(-1, 16), want)
    assert (dst[write_units * 16:] == 0xA5).all()

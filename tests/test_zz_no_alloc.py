"""The no-allocation decode entry point (ecf8_decode_batched_noalloc) against ecf8_decode_batched.

Both are called through the C ABI on the same encoded tensors; outputs must
be identical byte for byte (and equal the original bytes).  Two calls in a
row, the second with a smaller batch, check that the shared device scratch is
rewritten correctly; the block-check counter lands in a caller's device word.
"""
import numpy as np
import pytest
import torch

import synth
import lossless_entropy_coded_ecf8_amd as E
from lossless_entropy_coded_ecf8_amd import binding as B

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def batch(d, sizes, seed):
    xs, encs = [], []
    for i, n in enumerate(sizes):
        x = synth.small_stable(n, 1.6 + 0.05 * i, seed + i) if i % 3 else synth.random_bytes(n, seed + i)
        xs.append(x)
        encs.append(E.encode(x).to(d))
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 15) // 16 * 16 + 16
    return xs, encs, offs, off


def run_both(d, xs, encs, offs, total):
    ref = torch.full((total + 64,), CANARY, dtype=torch.uint8, device=d)
    ws = torch.empty(E.workspace_bytes(len(encs)), dtype=torch.uint8, device=d)
    B.decode_batched(encs, out=ref, offsets=offs, workspace=ws)
    got = torch.full((total + 64,), CANARY, dtype=torch.uint8, device=d)
    bad = torch.full((1,), 12345, dtype=torch.int64, device=d)
    B.decode_batched_noalloc(encs, got, offs, bad_blocks=bad)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    g = got.cpu().numpy()
    for x, o in zip(xs, offs):
        assert np.array_equal(g[o:o + x.size], x)
    return int(bad.item())


def test_noalloc_matches_batched_twice_then_smaller():
    d = dev()
    xs, encs, offs, total = batch(d, [300_001, 70_000, 1 << 20, 5, 123_457, 8192 * 3, 999_999], 40)
    assert run_both(d, xs, encs, offs, total) == 0
    assert run_both(d, xs, encs, offs, total) == 0
    xs2, encs2, offs2, total2 = batch(d, [4097, 65_537], 90)
    assert run_both(d, xs2, encs2, offs2, total2) == 0


def test_noalloc_limit_and_block_check():
    d = dev()
    xs, encs, offs, total = batch(d, [20_000] * 17, 7)
    out = torch.empty(total, dtype=torch.uint8, device=d)
    with pytest.raises(E.Ecf8Error) as ei:
        B.decode_batched_noalloc(encs, out, offs)
    assert ei.value.code == -7
    # a corrupt block offset is counted in the caller's word; the next clean call reports 0
    x = synth.small_stable(400_000, 1.7, 3)
    enc = E.encode(x).to(d)
    enc.blk_off[1] += 3
    buf = torch.full((x.size + 64,), CANARY, dtype=torch.uint8, device=d)
    bad = torch.zeros(1, dtype=torch.int64, device=d)
    B.decode_batched_noalloc([enc], buf[16:16 + x.size], [0], bad_blocks=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) >= 1
    b = buf.cpu().numpy()
    assert (b[:16] == CANARY).all() and (b[16 + x.size:] == CANARY).all()
    enc.blk_off[1] -= 3
    B.decode_batched_noalloc([enc], buf[16:16 + x.size], [0], bad_blocks=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert np.array_equal(buf.cpu().numpy()[16:16 + x.size], x)
    # an empty batch only clears the word
    bad.fill_(7)
    B.decode_batched_noalloc([], buf, [], bad_blocks=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0

"""GPU checks of the measurement probes (libssa_peaks): the streaming read and
copy that give the bench its measured HBM rates must touch exactly the bytes
asked for, whatever the split over workgroups."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_attention_kv_amd import peaks as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.load_library()  # raises if the library is missing
    return torch.device("cuda:0")


# sizes in bytes (multiples of 16): one 4 KB step, a ragged tail, more blocks than words
SIZES = [16, 4096, 4096 * 37 + 16 * 5, 1 << 20]


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("blocks", [1, 7, 256])
def test_read_xors_every_word_once(dev, nbytes, blocks):
    print(f"\n[case] peak read {nbytes} bytes, {blocks} blocks", flush=True)
    rng = np.random.default_rng(nbytes + blocks)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(dev)
    out = torch.zeros(blocks, dtype=torch.int32, device=dev)
    P.read(src, out, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("blocks", [1, 7, 256])
def test_copy_is_exact(dev, nbytes, blocks):
    print(f"\n[case] peak copy {nbytes} bytes, {blocks} blocks", flush=True)
    rng = np.random.default_rng(nbytes * 3 + blocks)
    host = rng.integers(-2**31, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).to(dev)
    dst = torch.full((nbytes // 4 + 8,), 7, dtype=torch.int32, device=dev)  # 32 guard bytes past the end
    P.copy(src, dst[: nbytes // 4], blocks)
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    assert np.array_equal(d[: nbytes // 4], host)
    assert (d[nbytes // 4:] == 7).all()

"""The streaming bandwidth reference (pqb_stream_reference): output tile j of
each chunk of T tiles of 1 KiB is the XOR of its source tiles R j .. R j + R - 1,
checked byte for byte against numpy on a buffer of several thousand chunks."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tiles", [4, 8])
@pytest.mark.parametrize("r", [1, 2, 4])
def test_stream_reference_xor_pattern(r, tiles):
    import precision_quantization_block_amd as p
    rng = np.random.default_rng(41 + r + tiles)
    nbytes = 3001 * 8192
    src = rng.integers(0, 256, nbytes, dtype=np.uint8)
    got = p.stream_reference(torch.from_numpy(src).cuda(), r, tiles_per_wave=tiles).cpu().numpy()
    t = src.reshape(nbytes // (1024 * tiles), tiles // r, r, 1024)
    want = np.bitwise_xor.reduce(t, axis=2).reshape(-1)
    assert got.shape == want.shape and np.array_equal(got, want)

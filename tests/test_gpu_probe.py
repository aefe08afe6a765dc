"""The measurement read (dflash_probe_read) reads every 16-byte word of its buffer once, in
both load forms: each of its 1024 workgroups writes the xor of the words it read (word w
belongs to workgroup (w // 256) % 1024, the grid-stride split over 256 threads), checked
against the same xor on the host."""
import ctypes

import numpy as np
import pytest
import torch

from block_diffusion_drafter_03_amd import _lib
from block_diffusion_drafter_03_amd import runtime as rt

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("words", [1, 1000, 262144 + 4097])
def test_probe_read_reads_every_word_once(nontemporal, words):
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**32, size=(words, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.zeros(1024, 4, dtype=torch.int32, device="cuda")
    _lib.probe_read(ctypes.c_void_p(src.data_ptr()), words * 16, nontemporal,
                    ctypes.c_void_p(sink.data_ptr()), rt._stream())
    torch.cuda.synchronize()
    want = np.zeros((1024, 4), dtype=np.uint32)
    wg = (np.arange(words) // 256) % 1024
    for b in np.unique(wg):
        want[b] = np.bitwise_xor.reduce(host[wg == b], axis=0)
    np.testing.assert_array_equal(sink.cpu().numpy().view(np.uint32), want)

"""Host-side weight packing: the B-fragment order documented in include/dflash.h."""
import torch

from block_diffusion_drafter_03_amd.runtime import frag_pack, pack_gate_up, rotary_interleave


def _offset(n, k, K):
    # element (n, k) of W [N, K] as the header states it
    return ((n // 16 * (K // 32) + k // 32) * 64 + (k % 32) // 8 * 16 + n % 16) * 8 + k % 8


def test_frag_pack_follows_the_documented_offsets():
    for N, K in ((16, 32), (40, 96), (3000 % 97 + 16, 64)):
        w = torch.randn(N, K)
        f = frag_pack(w).reshape(-1)
        NT = (N + 15) // 16
        assert f.numel() == NT * 16 * K
        idx = torch.tensor([[_offset(n, k, K) for k in range(K)] for n in range(N)])
        assert torch.equal(f[idx], w)
        # padded rows are zero and every element lands exactly once
        mask = torch.ones(f.numel(), dtype=torch.bool)
        mask[idx.reshape(-1)] = False
        assert torch.all(f[mask] == 0) and int(mask.sum()) == (NT * 16 - N) * K


def test_row_interleaves():
    w = torch.arange(2 * 8 * 3, dtype=torch.float32).reshape(16, 3)     # 2 heads of d = 8
    r = rotary_interleave(w, 2, 8)
    for h in range(2):
        for i in range(4):
            assert torch.equal(r[h * 8 + 2 * i], w[h * 8 + i])
            assert torch.equal(r[h * 8 + 2 * i + 1], w[h * 8 + i + 4])
    g, u = torch.randn(5, 3), torch.randn(5, 3)
    gu = pack_gate_up(g, u)
    assert torch.equal(gu[0::2], g) and torch.equal(gu[1::2], u)

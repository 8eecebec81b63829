"""Bit-exact device index math (G, f, band, tile classes) and RoPE parity."""
import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import jetlong as jl

from _parity import say

pytestmark = pytest.mark.gpu


def _oracle_band(n, w_local, bifocal, G):
    bif = bifocal and G > 1
    return np.array([[oracle.band(i, j, w_local, bif) for j in range(n)] for i in range(n)],
                    dtype=np.uint8)


@pytest.mark.parametrize("L,w_pre,w_local,bifocal,bm,bn", [
    (300, 64, 20, True, 32, 64), (300, 64, 20, False, 32, 64), (257, 300, 10, True, 16, 16),
    (250, 50, 0, True, 64, 32), (199, 10, 199, True, 7, 13), (64, 16, 7, True, 1, 1),
])
def test_index_math_bit_exact(L, w_pre, w_local, bifocal, bm, bn):
    G, f, band, tile = jl.debug_index_math(L, w_pre, w_local, bifocal, bm, bn)
    assert G == oracle.group_size(L, w_pre)
    assert [int(x) for x in f] == [oracle.remap(x, G) for x in range(L)]
    ref = _oracle_band(L, w_local, bifocal, G)
    assert np.array_equal(band, ref)
    # a tile's class bits are the union of its pairs' bands
    for a in range(tile.shape[0]):
        for b in range(tile.shape[1]):
            blk = ref[a * bm:(a + 1) * bm, b * bn:(b + 1) * bn]
            bits = (1 if (blk == 1).any() else 0) | (2 if (blk == 2).any() else 0) | \
                   (4 if (blk == 0).any() else 0)
            if not ((blk == 1).any() or (blk == 2).any()):
                bits = 0
            assert tile[a, b] == bits, (a, b)


def test_index_math_long_sequence():
    L, w_pre = 131072, 32768
    G, f, band, _ = jl.debug_index_math(L, w_pre, 2048, True, 256, 64)
    assert G == 4
    x = np.arange(L)
    assert np.array_equal(f, x // 4)
    assert oracle.remap(L - 1, 4) == int(f[-1])
    ref = _oracle_band(64, 2048, True, G)
    assert np.array_equal(band[:64, :64], ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("G,d,base", [(1, 128, 1e6), (3, 64, 1e4), (4, 128, 1e6)])
def test_rope_apply_parity(dtype, G, d, base):
    g = torch.Generator().manual_seed(G + d)
    T, H = 300, 3
    x = torch.randn(T, H, d, generator=g).to(dtype)
    pos = torch.randint(0, 131072, (T,), generator=g)
    pos[:4] = torch.tensor([0, 1, 131071, 65536])
    say("rope", dtype, G, d)
    y = jl.rope_apply(x.cuda(), pos, base, G=G)
    torch.cuda.synchronize()
    ref = oracle.rope(x, (pos // G).numpy(), base)
    got = y.float().cpu().double().numpy()
    if dtype == torch.float32:
        assert np.abs(got - ref).max() <= 2e-6 * max(1.0, np.abs(ref).max())
    else:
        # one bf16 rounding of the fp32 result
        assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6).all()


def test_rope_apply_in_place():
    x = torch.randn(50, 2, 64).cuda()
    pos = torch.arange(50)
    y = jl.rope_apply(x.clone(), pos, 1e4)
    x2 = x.clone()
    jl.rope_apply(x2, pos, 1e4, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(y, x2)

"""The read-stream measurement entry point reads every byte once: the wrapping
sum of its per-workgroup word sums equals the buffer's (checked on the host)."""
import numpy as np
import pytest
import torch

from long_context_attention_jl_amd import jetlong as jl

from _parity import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (10 << 20) + 16 * 37, 3 * 256 * 512 * 64])
def test_stream_read_sums_every_word(nbytes):
    g = torch.Generator("cpu").manual_seed(nbytes % 1000)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64)
    host = host.to(torch.int32)
    say("stream read", nbytes, "bytes")
    part = jl.stream_read(host.cuda())
    torch.cuda.synchronize()
    got = int(part.cpu().numpy().astype(np.uint32).astype(np.uint64).sum()) & 0xFFFFFFFF
    want = int(host.numpy().astype(np.uint32).astype(np.uint64).sum()) & 0xFFFFFFFF
    assert got == want


def _wave_totals(ops16, iters):
    """Expected sum of every accumulator element of each wave of the
    matrix-core stream, from the definition of a 32 x 32 x 16 MFMA: lane l
    holds A[l % 32][8 (l // 32) + j] and B[8 (l // 32) + j][l % 32] for
    j < 8, so the sum of all elements of A B is
    sum_{h, j} (sum of A-vector component j over lane half h) x (the same for B)."""
    v = ops16.astype(np.float64).reshape(-1, 64, 16, 8)  # waves, lanes, vectors, components
    a, b = v[:, :, :8, :], v[:, :, 8:, :]
    halves = lambda x: x.reshape(x.shape[0], 2, 32, 8, 8).sum(axis=2)  # waves, half, vector, comp

    ah, bh = halves(a), halves(b)

    def t(x, y, i, k):
        return (x[:, :, i, :] * y[:, :, k, :]).sum(axis=(1, 2))

    tot = np.zeros(v.shape[0])
    for k in range(8):
        tot += t(ah, bh, k, k) + t(bh, ah, (k + 3) & 7, (k + 5) & 7)
        tot += t(ah, bh, (k + 1) & 7, (k + 6) & 7) + t(bh, ah, (k + 2) & 7, (k + 4) & 7)
    return tot * iters


def test_mfma_stream_counts_every_product():
    """Operands of 1: each of the 4 x 16 accumulator elements a thread holds
    gains 16 per MFMA, 8 MFMAs per chain per iteration (exact in fp32)."""
    iters = 5
    ops = torch.ones(jl.MFMA_STREAM_OPERAND_BYTES // 2, dtype=torch.float16, device="cuda")
    say("mfma stream ones, iters", iters)
    out = jl.mfma_stream(ops, iters)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.full((256 * 512,), 64.0 * 16 * 8 * iters))


def test_mfma_stream_matches_its_definition_on_random_operands():
    """N(0,1)/4 operands: the sum of every wave's accumulators equals the
    fp64 sum of the products its 32 MFMAs per iteration define."""
    iters = 3
    g = torch.Generator("cpu").manual_seed(7)
    host = (torch.randn(jl.MFMA_STREAM_OPERAND_BYTES // 2, generator=g) / 4).to(torch.float16)
    say("mfma stream randn, iters", iters)
    out = jl.mfma_stream(host.cuda(), iters)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(-1, 64).sum(axis=1)
    want = _wave_totals(host.numpy(), iters)
    scale = np.abs(want).max()
    assert np.abs(got - want).max() <= 1e-4 * scale + 1e-3, np.abs(got - want).max()

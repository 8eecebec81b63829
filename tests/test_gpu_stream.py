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

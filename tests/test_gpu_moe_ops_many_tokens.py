"""Permute and combine over more tokens than one wave each could address in a single dispatch:
T = 2^26 + 5 tokens (a grid of one 64-lane wave per token would hold 2^32 + 320 work-items, past
the 32-bit work-item count of a dispatch), with short rows (d = 8, 16 bytes in bf16) and K = 2.
The permutation is a rotation of the flat assignments, so every expected value has a closed form
checked on the GPU in chunks: row p of the permuted buffer is token ((p - r) mod T K) // K, and
with gates 0.25 and 0.75 the combine returns every token row exactly (both products and their
sum are exact in fp32 for bf16 inputs)."""

import pytest
import torch

import expert_load_balancing_amd as elb
from gpu_util import log

pytestmark = pytest.mark.gpu

T, D, K, ROT = (1 << 26) + 5, 8, 2, 12_345
CHUNK = 1 << 24


def test_permute_and_combine_past_the_dispatch_work_item_limit():
    n = T * K
    assert 64 * T > 2 ** 32
    log(f"permute/combine: T={T} d={D} K={K}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    x = torch.randn((T, D), generator=gen, device="cuda").to(torch.bfloat16)
    inv = torch.remainder(torch.arange(n, device="cuda", dtype=torch.int64) + ROT, n).to(torch.int32)
    xp = elb.permute_rows(x, inv, K)
    torch.cuda.synchronize()
    for lo in range(0, n, CHUNK):
        p = torch.arange(lo, min(lo + CHUNK, n), device="cuda", dtype=torch.int64)
        src = torch.div(torch.remainder(p - ROT, n), K, rounding_mode="floor")
        assert torch.equal(xp[p].view(torch.int16), x[src].view(torch.int16)), f"permuted rows differ near {lo}"
    gates = torch.tensor([0.25, 0.75], device="cuda").repeat(T, 1).contiguous()
    y = elb.unpermute_combine(xp, gates, inv)
    torch.cuda.synchronize()
    for lo in range(0, T, CHUNK):
        hi = min(lo + CHUNK, T)
        assert torch.equal(y[lo:hi], x[lo:hi].float()), f"combined rows differ near {lo}"
    log(f"  {n} permuted rows and {T} combined rows hold their closed forms")

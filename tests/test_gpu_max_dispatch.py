"""The dispatch at the largest size its int32 positions allow: T = 268,435,455 tokens with K = 8
(T K = 2,147,483,640 assignments, one tile short of 2^31), random expert ids over 256 experts
(repeats inside a token included; the sort is defined for any ids).  At this size the oracle's
loops are out of reach, so the test checks on the GPU, in chunks, the properties that define the
stable counting sort uniquely: the bucket sizes are the id histogram, perm is a permutation
with inv its inverse, ids read through perm never decrease, and inside a bucket the flat
positions ascend.  Those four together leave exactly one valid perm."""

import pytest
import torch

import expert_load_balancing_amd as elb
from gpu_util import log

pytestmark = pytest.mark.gpu

T, K, N_E = (1 << 31) // 8 - 1, 8, 256
CHUNK = 1 << 27


def test_dispatch_at_the_int32_position_limit():
    n = T * K
    assert n < 2 ** 31 and n + 2048 > 2 ** 31 - 1
    log(f"max dispatch: T={T} K={K} ({n} assignments)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2718)
    idx = torch.randint(0, N_E, (T, K), generator=gen, device="cuda", dtype=torch.int32)
    offs, perm, inv = elb.router_dispatch(idx, N_E)
    torch.cuda.synchronize()
    flat = idx.view(-1)

    # Bucket sizes are the histogram of the ids; the buckets tile [0, T K).
    hist = torch.zeros(N_E, dtype=torch.int64, device="cuda")
    for lo in range(0, n, CHUNK):
        hist += torch.bincount(flat[lo:lo + CHUNK].long(), minlength=N_E)
    o = offs.long()
    assert o[0].item() == 0 and o[-1].item() == n
    assert torch.equal(o[1:] - o[:-1], hist)

    # perm is a permutation with inverse inv: perm[inv[j]] == j for every j.
    for lo in range(0, n, CHUNK):
        hi = min(lo + CHUNK, n)
        back = perm[inv[lo:hi].long()]
        assert torch.equal(back.long(), torch.arange(lo, hi, device="cuda")), f"perm[inv] at {lo}"
    del back

    # Ids along perm never decrease, and equal ids keep ascending flat positions (stability);
    # each chunk is checked together with the first entry of the next.
    for lo in range(0, n, CHUNK):
        hi = min(lo + CHUNK + 1, n)
        p = perm[lo:hi].long()
        e = flat[p]
        de = e[1:] - e[:-1]
        assert bool((de >= 0).all()), f"ids decrease along perm near {lo}"
        same = de == 0
        assert bool((p[1:][same] > p[:-1][same]).all()), f"unstable bucket near {lo}"
    log(f"  {n} assignments: histogram, permutation, order and stability hold")

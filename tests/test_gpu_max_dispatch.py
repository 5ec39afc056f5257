"""The dispatch at the largest size its int32 positions allow: T = 268,435,455 tokens with K = 8
(T K = 2,147,483,640 assignments, one tile short of 2^31), random expert ids over 256 experts
(repeats inside a token included; the sort is defined for any ids).  At this size the oracle's
loops are out of reach, so the test checks on the GPU, in chunks, the properties that define the
stable counting sort uniquely (gpu_util.check_dispatch_device)."""

import pytest
import torch

import expert_load_balancing_amd as elb
from gpu_util import check_dispatch_device, log

pytestmark = pytest.mark.gpu

T, K, N_E = (1 << 31) // 8 - 1, 8, 256


def test_dispatch_at_the_int32_position_limit():
    n = T * K
    assert n < 2 ** 31 and n + 2048 > 2 ** 31 - 1
    log(f"max dispatch: T={T} K={K} ({n} assignments)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2718)
    idx = torch.randint(0, N_E, (T, K), generator=gen, device="cuda", dtype=torch.int32)
    offs, perm, inv = elb.router_dispatch(idx, N_E)
    torch.cuda.synchronize()
    check_dispatch_device(offs, perm, inv, idx.view(-1), N_E)
    log(f"  {n} assignments: histogram, permutation, order and stability hold")

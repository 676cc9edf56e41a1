"""moe_permute_noalloc -- the permutation with the library's static histogram
memory instead of a caller workspace -- called through the C ABI and
compared bit for bit with moe_permute (index arrays and gathered rows) and
with the oracle's counting sort, on two calls in a row, the second smaller:
the static memory keeps the first call's contents, which must not matter.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_dispatch_amd as moe
import oracle
from gpu_common import announce, device

pytestmark = pytest.mark.gpu


def _inputs(T, K, S, H, dt, frac_in, seed):
    g = torch.Generator().manual_seed(seed)
    slot = torch.randint(0, S, (T, K), generator=g, dtype=torch.int32)
    mask = (torch.rand(T, K, generator=g) < frac_in).to(torch.uint8)
    x = (torch.randn(T, H, generator=g) * 4).to(dt)
    return x, slot, mask


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("gather", [True, False])
def test_noalloc_permute_matches_workspace_permute(gather):
    dev = device()
    so = moe.lib()
    cases = [(5000, 8, 80, 256, torch.bfloat16, 0.9, 1),   # larger first
             (333, 4, 12, 64, torch.float32, 0.6, 2)]      # then a smaller call
    for T, K, S, H, dt, frac, seed in cases:
        announce(f"permute_noalloc T={T} K={K} S={S} H={H} {dt} gather={gather}")
        x, slot, mask = _inputs(T, K, S, H, dt, frac, seed)
        x, slot, mask = x.to(dev), slot.to(dev), mask.to(dev)
        off = torch.full((S + 1,), -7, dtype=torch.int32, device=dev)
        sp = torch.full((T * K,), -7, dtype=torch.int32, device=dev)
        pr = torch.full((T * K,), -7, dtype=torch.int32, device=dev)
        xp = torch.zeros(T * K, H, dtype=dt, device=dev) if gather else None
        dcode = moe.MOE_DTYPE_BF16 if dt == torch.bfloat16 else moe.MOE_DTYPE_F32
        st = so.moe_permute_noalloc(x.data_ptr(), dcode, T, H, K, slot.data_ptr(),
                                    mask.data_ptr(), S, off.data_ptr(), sp.data_ptr(),
                                    pr.data_ptr(), xp.data_ptr() if gather else None,
                                    torch.cuda.current_stream().cuda_stream)
        assert st == 0, moe.status_str(st)
        r_off, r_sp, r_pr, r_xp = moe.permute(x, slot, mask, S, gather=gather)
        torch.cuda.synchronize()
        P_in = int(r_off[-1])
        assert torch.equal(off, r_off)
        assert torch.equal(sp[:P_in], r_sp[:P_in])
        assert torch.equal(pr, r_pr)
        if gather:
            assert torch.equal(_bits(xp[:P_in]), _bits(r_xp[:P_in]))
        o_off, o_sp, o_pr = oracle.permute_indices(slot.cpu().numpy(), mask.cpu().numpy(), S)
        assert np.array_equal(off.cpu().numpy(), o_off)
        assert np.array_equal(sp[:P_in].cpu().numpy(), o_sp)
        assert np.array_equal(pr.cpu().numpy(), o_pr)


def test_noalloc_permute_binding_and_validation():
    dev = device()
    so = moe.lib()
    x, slot, mask = _inputs(100, 3, 7, 72, torch.bfloat16, 0.8, 3)
    x, slot, mask = x.to(dev), slot.to(dev), mask.to(dev)
    got = moe.permute_noalloc(x, slot, mask, 7)
    want = moe.permute(x, slot, mask, 7)
    torch.cuda.synchronize()
    P_in = int(want[0][-1])
    assert torch.equal(got[0], want[0]) and torch.equal(got[2], want[2])
    assert torch.equal(got[1][:P_in], want[1][:P_in])
    assert torch.equal(_bits(got[3][:P_in]), _bits(want[3][:P_in]))
    # host validation as moe_permute, before any launch
    fake = ctypes.c_void_p(256)
    assert so.moe_permute_noalloc(None, 1, 4, 12, 2, fake, fake, 4, fake, fake, fake, None,
                                  None) == 2   # H % 8
    assert so.moe_permute_noalloc(None, 1, 4, 16, 0, fake, fake, 4, fake, fake, fake, None,
                                  None) == 1   # K < 1

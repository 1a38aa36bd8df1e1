"""GPU parity of pa_copy_blocks against the oracle (bit-exact): device to
device, eviction to a pinned host pool and restore, out-of-pool pairs."""
import pytest
import torch

import oracle
import paged_varlen_attention_amd as pa

pytestmark = pytest.mark.gpu


def caches(n, shape, dt, seed, nan=False):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((n,) + shape, generator=g).to(dt)
    v = torch.randn((n,) + shape, generator=g).to(dt)
    if nan:
        k[1, 0, 0, :3] = float("nan")
    return k, v


def same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("dt,shape", [(torch.bfloat16, (16, 8, 128)), (torch.float32, (8, 2, 64)),
                                      (torch.bfloat16, (32, 4, 256))])
def test_device_to_device(dt, shape):
    sk, sv = caches(40, shape, dt, 1, nan=True)
    dk, dv = caches(30, shape, dt, 2)
    pairs = torch.tensor([[1, 0], [39, 29], [7, 3], [0, 11], [50, 4], [5, -2], [12, 12]])
    ek, ev = dk.clone(), dv.clone()
    oracle.copy_blocks(ek, ev, sk, sv, pairs)
    gk, gv = dk.cuda(), dv.cuda()
    pa.copy_blocks(gk, gv, sk.cuda(), sv.cuda(), pairs.cuda())
    torch.cuda.synchronize()
    assert same_bytes(gk.cpu(), ek) and same_bytes(gv.cpu(), ev)


def test_evict_to_pinned_host_and_restore():
    """Blocks of a device cache go to a pinned host pool (pairs in pinned
    memory), are wiped on the device, and come back bit for bit."""
    shape = (16, 8, 128)
    sk, sv = caches(64, shape, torch.bfloat16, 3, nan=True)
    gk, gv = sk.cuda(), sv.cuda()
    hk = torch.zeros((20,) + shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    ids = [5, 17, 1, 63, 40, 22, 9, 30]
    out = torch.tensor([[b, i] for i, b in enumerate(ids)], dtype=torch.int64).pin_memory()
    pa.copy_blocks(hk, hv, gk, gv, out)
    torch.cuda.synchronize()
    ek, ev = torch.zeros_like(hk), torch.zeros_like(hv)
    oracle.copy_blocks(ek, ev, sk, sv, out)
    assert same_bytes(hk, ek) and same_bytes(hv, ev)
    gk[ids] = 0
    gv[ids] = 0
    back = out.flip(1).contiguous().cuda()
    pa.copy_blocks(gk, gv, hk, hv, back)
    torch.cuda.synchronize()
    assert same_bytes(gk.cpu(), sk) and same_bytes(gv.cpu(), sv)


def test_pageable_host_memory_is_refused():
    shape = (16, 2, 64)
    sk, sv = caches(4, shape, torch.bfloat16, 4)
    hk = torch.zeros((4,) + shape, dtype=torch.bfloat16)  # pageable
    pairs = torch.tensor([[0, 0]]).cuda()
    with pytest.raises(ValueError):
        pa.copy_blocks(hk, hk.clone(), sk.cuda(), sv.cuda(), pairs)
    import ctypes
    gk, gv = sk.cuda(), sv.cuda()
    st = pa.lib.pa_copy_blocks(ctypes.c_void_p(hk.data_ptr()), ctypes.c_void_p(hk.data_ptr()),
                               ctypes.c_void_p(gk.data_ptr()), ctypes.c_void_p(gv.data_ptr()),
                               ctypes.c_void_p(pairs.data_ptr()), 1, 16 * 2 * 64 * 2, 4, 4, None)
    assert st == pa.PA_EINVAL
    torch.cuda.synchronize()

"""GPU parity of pa_reshape_and_cache and pa_expand_block_tables: bit-exact
against the oracle on the same seeded inputs, untouched slots unchanged."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _poisoned_cache(rng, nb, bs, hkv, d, dtype):
    if dtype == torch.bfloat16:
        bits = rng.integers(-2 ** 15, 2 ** 15 - 1, size=(nb, bs, hkv, d), dtype=np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16)
    bits = rng.integers(-2 ** 31, 2 ** 31 - 1, size=(nb, bs, hkv, d), dtype=np.int32)
    return torch.from_numpy(bits).view(torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("hkv,d,bs,nb,T", [(2, 128, 16, 40, 300), (1, 64, 8, 9, 50),
                                          (4, 256, 144, 6, 700), (8, 128, 32, 70, 1)])
def test_reshape_and_cache_bit_exact(dtype, hkv, d, bs, nb, T):
    import paged_varlen_attention_amd as pa
    rng = np.random.default_rng(hkv * 1000 + d + bs + T)
    T = min(T, nb * bs)
    key = torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32)).to(dtype)
    value = torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32)).to(dtype)
    slots = torch.from_numpy(rng.choice(nb * bs, size=T, replace=False).astype(np.int64))
    if T > 4:
        slots[rng.choice(T, size=T // 4, replace=False)] = -1
    kc = _poisoned_cache(rng, nb, bs, hkv, d, dtype)
    vc = _poisoned_cache(rng, nb, bs, hkv, d, dtype)
    ref_k, ref_v = kc.clone(), vc.clone()
    oracle.reshape_and_cache(key, value, ref_k, ref_v, slots)
    gk, gv = kc.cuda(), vc.cuda()
    pa.reshape_and_cache(key.cuda(), value.cuda(), gk, gv, slots.cuda())
    torch.cuda.synchronize()
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(gk.cpu().view(iv), ref_k.view(iv))
    assert torch.equal(gv.cpu().view(iv), ref_v.view(iv))


def test_reshape_and_cache_spec_verify_workload():
    """The 144-token-block cache write of the speculative-verify batch, whole cache compared."""
    import paged_varlen_attention_amd as pa
    w = W.spec_verify_bf16()
    ref_k, ref_v = w.key_cache.clone(), w.value_cache.clone()
    oracle.reshape_and_cache(w.new_key, w.new_value, ref_k, ref_v, w.slot_mapping)
    gk, gv = w.key_cache.cuda(), w.value_cache.cuda()
    pa.reshape_and_cache(w.new_key.cuda(), w.new_value.cuda(), gk, gv, w.slot_mapping.cuda())
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu().view(torch.int16), ref_k.view(torch.int16))
    assert torch.equal(gv.cpu().view(torch.int16), ref_v.view(torch.int16))


def test_reshape_and_cache_empty_is_noop():
    import paged_varlen_attention_amd as pa
    kc = torch.zeros((2, 16, 1, 64), device="cuda")
    pa.reshape_and_cache(torch.empty((0, 1, 64), device="cuda"), torch.empty((0, 1, 64), device="cuda"),
                         kc, kc.clone(), torch.empty((0,), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert kc.abs().sum().item() == 0


@pytest.mark.parametrize("ratio", [1, 2, 9])
def test_expand_block_tables_bit_exact(ratio):
    import paged_varlen_attention_amd as pa
    rng = np.random.default_rng(ratio)
    bt = torch.from_numpy(rng.integers(-1, 500, size=(37, 23)).astype(np.int32))
    ref = oracle.expand_block_tables(bt, ratio)
    got = pa.expand_block_tables(bt.cuda(), ratio)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), ref)

"""GPU parity of attention sinks (one extra softmax term per query head that
carries no value) against the fp64 oracle: the VALU decode path, the MFMA
tile path and the split-KV reduce, including -inf sinks (no sink) and sinks
that dominate the scores."""
import dataclasses

import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu


def with_sinks(w, seed, scale):
    g = torch.Generator().manual_seed(seed)
    return dataclasses.replace(w, sinks=(torch.randn(w.num_q_heads, generator=g) * scale).float())


CASES = [  # (max_q, hq, hkv, d, bs, dtype)
    (1, 32, 8, 128, 16, torch.bfloat16),
    (1, 24, 4, 256, 16, torch.bfloat16),
    (1, 4, 1, 64, 8, torch.float32),
    (40, 16, 2, 128, 16, torch.bfloat16),
    (40, 16, 2, 256, 32, torch.bfloat16),
    (7, 8, 2, 64, 16, torch.float32),
]


@pytest.mark.parametrize("max_q,hq,hkv,d,bs,dt", CASES,
                         ids=[f"q{c[0]}-{c[1]}-{c[2]}-{c[3]}-bs{c[4]}-{str(c[5])[6:]}" for c in CASES])
@pytest.mark.parametrize("sink_scale", [1.0, 8.0])
def test_sinks(max_q, hq, hkv, d, bs, dt, sink_scale):
    """Random sinks (std 1 and 8: the latter dominates many rows), every
    partition size, against the oracle."""
    w = W.random_case(hq + d + bs + max_q, num_seqs=5, max_q=max_q, max_ctx=900, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dt)
    w = with_sinks(w, 11 + hq, sink_scale)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, dt, f"sinks P={P}")


@pytest.mark.parametrize("max_q", [1, 30])
def test_neg_inf_sink_is_no_sink(max_q):
    """A -inf sink leaves every output bit unchanged."""
    w = W.random_case(71 + max_q, num_seqs=4, max_q=max_q, max_ctx=700, num_q_heads=16,
                      num_kv_heads=2, head_dim=128, block_size=16, dtype=torch.bfloat16)
    b = to_device(w)
    bs = dataclasses.replace(b, sinks=torch.full((16,), float("-inf"), device="cuda"))
    for P in (0, 256):
        a = run_gpu(b, P).clone()
        c = run_gpu(bs, P).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), c.view(torch.int16)), P

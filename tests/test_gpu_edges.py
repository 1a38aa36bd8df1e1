"""GPU parity on degenerate and extreme batches: requests with no new tokens
(with and without a cached prefix) inside prefill batches, thousands of
requests in one call, the largest group size with many heads, and rows whose
key ranges end exactly on page and partition boundaries, on every path (VALU
decode, per-token fp32, bf16 tiles, 8-bit tiles)."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_close, run_gpu, sample_rows, to_device

pytestmark = pytest.mark.gpu


def _check_all(w, dtype, Ps, what):
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in Ps:
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, dtype, f"{what} P={P}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kind", ["bf16", "f32", "fp8"])
def test_zero_length_requests(d, kind):
    """Requests with q_len 0 (one with an empty cache, one with a prefix)
    between prefill, decode and verify requests; keys ending on page (16) and
    partition (256) boundaries."""
    q_lens = [0, 20, 0, 1, 0, 33, 256, 3]
    seq_lens = [0, 20, 17, 256, 0, 100, 512, 272]
    dt = torch.float32 if kind == "f32" else torch.bfloat16
    w = W.build(f"zero_{kind}_{d}", seed=61 + d, q_lens=q_lens, seq_lens=seq_lens,
                num_q_heads=8, num_kv_heads=2, head_dim=d, block_size=16, num_blocks=90, dtype=dt)
    if kind == "fp8":
        w = pins.fp8_case(w, seed=d)
    _check_all(w, dt, (0, 256, 512), f"zero-length {kind} D={d}")


def test_many_decode_requests():
    """8,192 decode requests (contexts 1..64) in one call, 32/8/128 bf16: the
    grid's request dimension far beyond the CU count; every row."""
    rng = np.random.default_rng(5)
    n = 8192
    seq = rng.integers(1, 65, size=n)
    w = W.build("many_decode", seed=62, q_lens=[1] * n, seq_lens=seq, num_q_heads=32,
                num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=int(sum((s + 15) // 16 for s in seq)) + 8, dtype=torch.bfloat16)
    _check_all(w, torch.bfloat16, (0, 256), "8192 decode requests")


def test_many_ragged_requests_tiled():
    """2,000 requests of 1..3 new tokens over 0..200 cached keys on the tiled
    path (the tile-to-request search over a long cu_seqlens), 16/2/128."""
    rng = np.random.default_rng(6)
    n = 2000
    ql = rng.integers(1, 4, size=n)
    seq = ql + rng.integers(0, 201, size=n)
    w = W.build("many_tiled", seed=63, q_lens=ql, seq_lens=seq, num_q_heads=16, num_kv_heads=2,
                head_dim=128, block_size=16,
                num_blocks=int(sum((s + 15) // 16 for s in seq)) + 8, dtype=torch.bfloat16)
    rows = sample_rows(w, 400, seed=7)
    ref = oracle.run_workload(w, rows=rows)
    b = to_device(w)
    for P in (0, 256):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        got = torch.stack([out[t, h] for t, h in rows])
        assert_close(got, ref, torch.bfloat16, f"2000 tiled requests P={P}")


@pytest.mark.parametrize("max_q", [1, 40])
def test_largest_group_many_heads(max_q):
    """Group size 8 with 64 query heads (8 KV heads), D=256: decode and tiles."""
    w = W.random_case(64 + max_q, num_seqs=5, max_q=max_q, max_ctx=700, num_q_heads=64,
                      num_kv_heads=8, head_dim=256, block_size=32, dtype=torch.bfloat16)
    _check_all(w, torch.bfloat16, (0, 512), f"group 8, 64 heads, max_q={max_q}")

"""GPU parity of the decode path (one query token per request), unsplit and
split-KV with the reduce, against the fp64 oracle on the same seeded inputs."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, errors, run_gpu, sample_rows, to_device

pytestmark = pytest.mark.gpu


def test_tiny_decode_f32():
    """Two requests, 37 and 50 keys, Hq=4 Hkv=1 D=64, fp32: max-abs <= 1e-5."""
    w = W.tiny_decode_f32()
    ref = oracle.run_workload(w)
    out = run_gpu(to_device(w))
    torch.cuda.synchronize()
    assert_close(out, ref, torch.float32, "tiny fp32 decode")


GEOMS = [(4, 1, 64), (32, 8, 128), (24, 4, 256), (16, 2, 128), (16, 2, 256), (8, 8, 128),
         (6, 2, 64), (10, 2, 128), (14, 2, 256)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv,d", GEOMS, ids=[f"{a}-{b}-{c}" for a, b, c in GEOMS])
def test_decode_geometries(hq, hkv, d, bs, dtype):
    """Ragged contexts (including lengths that are not a multiple of the page
    size or the partition), every partition size, against the oracle."""
    w = W.random_case(hq * 100 + d + bs, num_seqs=5, max_q=1, max_ctx=1400, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, dtype, f"P={P}")


@pytest.mark.parametrize("form", ["1", "0"], ids=["auto-whole-row", "per-head"])
def test_gqa_decode_batch_split512(form, monkeypatch):
    """32 requests, ctx U[512,4096], 32/8/128 bf16, split 512 + reduce; every row;
    the launch bench.py times (whole-row kernel) and the per-KV-head kernel."""
    monkeypatch.setenv("PA_DECODE_ROWS", form)
    w = W.gqa_decode_bf16()
    ref = oracle.run_workload(w)
    b = to_device(w)
    out = run_gpu(b, 512)
    torch.cuda.synchronize()
    assert_close(out, ref, torch.bfloat16, "gqa decode P=512")
    out0 = run_gpu(b, 0)
    torch.cuda.synchronize()
    assert_close(out0, ref, torch.bfloat16, "gqa decode P=0")


@pytest.mark.parametrize("P", [256, 512])
def test_long_context_decode(P):
    """4 requests of 32,768 keys, 24/4/256 bf16, split + reduce; every row."""
    w = W.long_decode_bf16()
    ref = oracle.run_workload(w)
    out = run_gpu(to_device(w), P)
    torch.cuda.synchronize()
    assert_close(out, ref, torch.bfloat16, f"long decode P={P}")


@pytest.mark.parametrize("form", ["0", "2"], ids=["per-head", "whole-row"])
def test_split_partials_match_oracle(form, monkeypatch):
    """The partials themselves (log2-space max, exp-sum, normalised output),
    from both bf16 decode kernels."""
    import paged_varlen_attention_amd as pa
    monkeypatch.setenv("PA_DECODE_ROWS", form)
    w = W.random_case(77, num_seqs=4, max_q=1, max_ctx=1500, num_q_heads=16, num_kv_heads=2,
                      head_dim=128, block_size=16, dtype=torch.bfloat16)
    P = 256
    o, m, l = oracle.attention_partials(w.q, w.key_cache, w.value_cache, w.cu_seqlens_q,
                                        w.seq_lens, w.block_tables, w.scale, P)
    b = to_device(w)
    parts = pa.alloc_partials(w.total_q, w.num_q_heads, w.head_dim, m.shape[2], "cuda")
    for t in parts:
        t.fill_(float("nan"))
    run_gpu(b, P, partials=parts, reduce=False)
    torch.cuda.synchronize()
    valid = torch.isfinite(m)
    # rows with a single partition are finalised directly and write no partials
    multi = (w.seq_lens.long() > P)[:, None, None].expand_as(m) & valid
    gm, gl, go = parts.max_logits.cpu().double(), parts.exp_sums.cpu().double(), parts.tmp_out.cpu().double()
    assert (gm[multi] - m[multi]).abs().max() < 1e-3
    assert ((gl[multi] - l[multi]).abs() / l[multi]).max() < 1e-2
    assert_close(go[multi], o[multi], torch.bfloat16, "partial outputs")


def test_decode_edge_cases():
    """seq_len 1, lengths at partition and page boundaries, an empty request."""
    q_lens = [1, 1, 1, 1, 0, 1, 1]
    seq_lens = [1, 256, 257, 512, 40, 513, 16]
    w = W.build("edges", seed=9, q_lens=q_lens, seq_lens=seq_lens, num_q_heads=8, num_kv_heads=2,
                head_dim=128, block_size=16, num_blocks=120, dtype=torch.bfloat16)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"edges P={P}")


def test_decode_deterministic():
    w = W.random_case(5, num_seqs=6, max_q=1, max_ctx=3000, num_q_heads=24, num_kv_heads=4,
                      head_dim=256, block_size=16, dtype=torch.bfloat16)
    b = to_device(w)
    a = run_gpu(b, 512).clone()
    c = run_gpu(b, 512).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_empty_batch_noop():
    w = W.tiny_decode_f32()
    b = to_device(w)
    import paged_varlen_attention_amd as pa
    out = torch.full((0, 4, 64), 1.0, device="cuda")
    pa.varlen_attention(b.q[:0], b.key_cache, b.value_cache,
                        torch.zeros(1, dtype=torch.int32, device="cuda"),
                        torch.zeros(0, dtype=torch.int32, device="cuda"),
                        torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                        max_q_len=1, max_seq_len=1, scale=0.125, out=out)
    torch.cuda.synchronize()

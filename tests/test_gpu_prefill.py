"""GPU parity of the tiled MFMA path (prefill and mixed batches, bf16) against
the fp64 oracle on the same seeded inputs: ragged batches over the GQA
geometries and page sizes, every partition size, the chunked-prefill and
speculative-verify workloads, and edge cases of the causal alignment."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu

GEOMS = [(32, 8, 128), (24, 4, 256), (16, 2, 128), (16, 2, 256), (4, 1, 64), (8, 8, 64),
         (12, 4, 128), (14, 2, 64)]


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv,d", GEOMS, ids=[f"{a}-{b}-{c}" for a, b, c in GEOMS])
def test_mixed_geometries(hq, hkv, d, bs):
    """Ragged q_len 1..45 with cached prefixes 0..300 (spans several q-tiles
    and key tiles with ragged tails), every partition size."""
    w = W.random_case(hq * 7 + d + bs, num_seqs=6, max_q=45, max_ctx=300, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=torch.bfloat16)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"P={P}")


@pytest.mark.parametrize("variant", ["A", "B"])
def test_mixed_chunked_prefill(variant):
    """8 prompts packed to 6,000 tokens plus 8 decode tokens, 16/2/256; every row."""
    w = W.mixed_prefill_bf16(variant=variant)
    ref = oracle.run_workload(w)
    b = to_device(w)
    out = run_gpu(b, 0)
    torch.cuda.synchronize()
    assert_close(out, ref, torch.bfloat16, f"mixed {variant}")
    out = run_gpu(b, 512)
    torch.cuda.synchronize()
    assert_close(out, ref, torch.bfloat16, f"mixed {variant} P=512")


def test_spec_verify_with_cache_write():
    """Verify windows of 1..5 tokens and two 512-token chunks over 1k..8k
    contexts, 144-token blocks seen as 9x16-token pages, new K/V written by
    pa_reshape_and_cache first; every row, unsplit and split (1,024 is the
    partition the benchmark times this batch at)."""
    import paged_varlen_attention_amd as pa
    w = W.spec_verify_bf16()
    ref = oracle.run_workload(w)  # oracle: cache write then attention on 144-token blocks
    b = to_device(w)              # GPU: cache write, 9x16 view, expanded block table
    assert b.block_tables.shape[1] == w.block_tables.shape[1] * 9
    for P in (0, 512, 1024):
        out = run_gpu(b, P, reduce=False)
        rec = pa.last_dispatch()
        assert rec["path"] == "tiled" and rec["partition_size"] == P, rec
        if P:
            out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"spec verify P={P}")


def test_uniform_prefill_workload():
    """The benchmark's uniform prefill batch itself (8 x 4,096 new tokens over
    4,096 cached ones, 16/2/256): it takes the 8-wave, 3-stage form of the
    tiled kernel, and sampled rows -- every request's first and last tokens
    among them -- match the oracle."""
    import paged_varlen_attention_amd as pa
    from gpu_helpers import sample_rows
    w = W.prefill_uniform_bf16()
    rows = sample_rows(w, 96, seed=7)
    ends = w.cu_seqlens_q[1:].tolist()
    rows = sorted(set(rows) | {(t - 1, h) for t in ends for h in (0, 9, 15)})
    ref = oracle.run_workload(w, rows=rows)
    b = to_device(w)
    out = run_gpu(b, 0)
    rec = pa.last_dispatch()
    assert rec["path"] == "tiled" and rec["block"] == 512 and rec["tile"][1] == 3, rec
    torch.cuda.synchronize()
    got = torch.stack([out[t, h] for t, h in rows])
    assert_close(got, ref, torch.bfloat16, "uniform prefill (sampled rows)")


def test_causal_edges():
    """No prefix, prefix of exactly one key tile, q_len equal to the q-tile,
    one decode token, a single key."""
    q_lens = [16, 17, 1, 32, 5, 1, 64]
    seq_lens = [16, 49, 1, 64, 5, 300, 64 + 31]
    w = W.build("edges", seed=31, q_lens=q_lens, seq_lens=seq_lens, num_q_heads=16,
                num_kv_heads=2, head_dim=128, block_size=16, num_blocks=40, dtype=torch.bfloat16)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"edges P={P}")


def test_prefill_deterministic():
    w = W.random_case(12, num_seqs=4, max_q=200, max_ctx=500, num_q_heads=16, num_kv_heads=2,
                      head_dim=256, block_size=16, dtype=torch.bfloat16)
    b = to_device(w)
    a = run_gpu(b, 0).clone()
    c = run_gpu(b, 0).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("hq,hkv,d,bs", [(4, 1, 64, 16), (16, 2, 128, 8), (24, 4, 256, 32)])
def test_mixed_fp32_per_token(hq, hkv, d, bs):
    """fp32 batches with multi-token windows (one workgroup per query token on
    the VALU path): max-abs 1e-5 against the oracle, every partition size."""
    w = W.random_case(hq + d + bs + 5, num_seqs=5, max_q=12, max_ctx=700, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=torch.float32)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.float32, f"fp32 mixed P={P}")


@pytest.mark.parametrize("scale", [-0.11, 0.0, 0.9])
def test_scale_values(scale):
    """A negative scale, a zero scale (uniform weights over the visible keys)
    and a large one (scores spread over tens of log2 units, so the running max
    jumps far between tiles), on the MFMA path (multi-token windows) and the
    VALU decode path, unsplit and split."""
    for max_q, seed in ((40, 51), (1, 52)):
        w = W.random_case(seed, num_seqs=5, max_q=max_q, max_ctx=700, num_q_heads=16,
                          num_kv_heads=2, head_dim=128, block_size=16, dtype=torch.bfloat16)
        w = dataclasses.replace(w, scale=scale)
        ref = oracle.run_workload(w)
        b = to_device(w)
        for P in (0, 256):
            out = run_gpu(b, P)
            torch.cuda.synchronize()
            assert_close(out, ref, torch.bfloat16, f"scale={scale} max_q={max_q} P={P}")


@pytest.mark.parametrize("max_q", [1, 60])
def test_large_partitions(max_q):
    """Partition sizes beyond the pages' 256/512 (any multiple of 256): rows
    cut into 1..4 partitions, on the decode path (max_q 1) and the MFMA path."""
    w = W.random_case(61 + max_q, num_seqs=6, max_q=max_q, max_ctx=2900, num_q_heads=16,
                      num_kv_heads=2, head_dim=128, block_size=16, dtype=torch.bfloat16)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (768, 1024, 2048):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"max_q={max_q} P={P}")


@pytest.mark.parametrize("d", [256, 128])
@pytest.mark.parametrize("kv8", [False, True], ids=["bf16", "fp8"])
def test_wide_workgroups(kv8, d):
    """A batch large enough for 8-wave workgroups (64/8 heads, ten 450..500-
    token prompts over short prefixes, D = 256 and 128): the launch takes the
    8-wave kernel over bf16 caches and the 4-wave kernel over 8-bit caches
    (which keep 4 waves), and sampled rows match the oracle."""
    import paged_varlen_attention_amd as pa
    import oracle_pins as pins
    from gpu_helpers import sample_rows
    w = W.random_case(4242 + d, num_seqs=10, min_q=450, max_q=500, max_ctx=200, num_q_heads=64,
                      num_kv_heads=8, head_dim=d, block_size=16, dtype=torch.bfloat16)
    if kv8:
        w = pins.fp8_case(w, seed=42)
    rows = sample_rows(w, 160, seed=3)
    ref = oracle.run_workload(w, rows=rows)
    b = to_device(w)
    for P in (0, 256):
        parts = (pa.alloc_partials(w.total_q, 64, d, pa.max_partitions(w.max_seq_len, P), "cuda")
                 if P else None)
        out = run_gpu(b, P, partials=parts, reduce=False)
        assert pa.last_dispatch()["block"] == (256 if kv8 else 512)  # waves x 64
        if P:
            pa.split_kv_reduce(out, parts, b.cu_seqlens_q, b.seq_lens, P, sinks=b.sinks)
        torch.cuda.synchronize()
        got = torch.stack([out[t, h] for t, h in rows])
        assert_close(got, ref, torch.bfloat16, f"wide P={P}")


def test_wide_workgroups_many_short():
    """8-wave workgroups over 80 short requests (1..40 new tokens on 0..400
    cached, 64/8 heads, D=256): more than 64 requests, so q-tiles are found by
    the search over cu_seqlens_q; workgroups walk from one to fourteen key
    tiles, so first and last tiles (prefetch start, masking, the sequence
    end) weigh in.  The whole output is compared, unsplit and split at 256
    keys."""
    import paged_varlen_attention_amd as pa
    w = W.random_case(8080, num_seqs=80, max_q=40, max_ctx=400, num_q_heads=64,
                      num_kv_heads=8, head_dim=256, block_size=16, dtype=torch.bfloat16)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256):
        parts = (pa.alloc_partials(w.total_q, 64, 256, pa.max_partitions(w.max_seq_len, P), "cuda")
                 if P else None)
        out = run_gpu(b, P, partials=parts, reduce=False)
        assert pa.last_dispatch()["block"] == 512  # 8 waves
        if P:
            pa.split_kv_reduce(out, parts, b.cu_seqlens_q, b.seq_lens, P, sinks=b.sinks)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"wide many short P={P}")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_wide_workgroups_long_prompts(bs):
    """8-wave workgroups (64/8 heads, D=256) over prompts of 1,500..2,000
    tokens on short cached prefixes: each workgroup walks dozens of key tiles,
    the last one cut by the sequence end (V rows past it zeroed); sampled rows
    include every request's last tokens."""
    import paged_varlen_attention_amd as pa
    from gpu_helpers import sample_rows
    w = W.random_case(5150 + bs, num_seqs=3, min_q=1500, max_q=2000, max_ctx=300, num_q_heads=64,
                      num_kv_heads=8, head_dim=256, block_size=bs, dtype=torch.bfloat16)
    rows = sample_rows(w, 160, seed=bs)
    ends = w.cu_seqlens_q[1:].tolist()
    rows += [(t - 1, h) for t in ends for h in (0, 7, 63)]
    ref = oracle.run_workload(w, rows=rows)
    b = to_device(w)
    for P in (0, 512):
        parts = (pa.alloc_partials(w.total_q, 64, 256, pa.max_partitions(w.max_seq_len, P), "cuda")
                 if P else None)
        out = run_gpu(b, P, partials=parts, reduce=False)
        assert pa.last_dispatch()["block"] == 512  # 8 waves
        if P:
            pa.split_kv_reduce(out, parts, b.cu_seqlens_q, b.seq_lens, P, sinks=b.sinks)
        torch.cuda.synchronize()
        got = torch.stack([out[t, h] for t, h in rows])
        assert_close(got, ref, torch.bfloat16, f"wide long bs={bs} P={P}")

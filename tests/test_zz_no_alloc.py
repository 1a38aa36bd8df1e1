"""GPU check of pa_varlen_attention_noalloc, the entry point for callers that
cannot allocate (split-KV partials in the library's static device scratch):
through the C ABI its output equals that of pa_varlen_attention +
pa_split_kv_reduce with caller-allocated partials on the same inputs, on two
calls in a row (the second smaller, so it runs over what the first left in
the scratch), and both meet the oracle bar.  A call whose partials would
overflow the scratch is refused before anything is enqueued."""
import pytest
import torch

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _noalloc(b, P, out):
    import paged_varlen_attention_amd as pa
    return pa.varlen_attention_noalloc(b.q, b.key_cache, b.value_cache, b.cu_seqlens_q,
                                       b.seq_lens, b.block_tables, out, max_q_len=b.max_q_len,
                                       max_seq_len=b.max_seq_len, scale=b.scale,
                                       partition_size=P, sinks=b.sinks, k_scale=b.k_scale,
                                       v_scale=b.v_scale)


CASES = [
    # (what, workload factory, partition sizes): decode batches on the MFMA
    # decode kernels and mixed batches on the tiles, the larger first
    ("gqa decode", lambda: W.gqa_decode_bf16(), (512, 256)),
    ("small decode", lambda: W.random_case(71, num_seqs=5, max_q=1, max_ctx=1500, num_q_heads=16,
                                           num_kv_heads=2, head_dim=128, block_size=16,
                                           dtype=torch.bfloat16), (256, 512)),
    ("mixed", lambda: W.random_case(72, num_seqs=6, max_q=90, max_ctx=900, num_q_heads=16,
                                    num_kv_heads=2, head_dim=256, block_size=16,
                                    dtype=torch.bfloat16), (512, 0)),
    ("fp32 decode", lambda: W.random_case(73, num_seqs=3, max_q=1, max_ctx=700, num_q_heads=8,
                                          num_kv_heads=2, head_dim=64, block_size=16,
                                          dtype=torch.float32), (256,)),
    # 8-bit caches: the whole-row 8-bit decode (256 and 512 launch items) and the tiles
    ("gqa decode fp8kv", lambda: pins.fp8_case(W.gqa_decode_bf16(), 2), (512, 256)),
    ("mixed fp8kv", lambda: pins.fp8_case(W.random_case(75, num_seqs=6, max_q=90, max_ctx=900,
                                                         num_q_heads=16, num_kv_heads=2, head_dim=256,
                                                         block_size=16, dtype=torch.bfloat16), 3),
     (512, 0)),
]


@pytest.mark.parametrize("what,make,Ps", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_allocating_entry_point(what, make, Ps):
    w = make()
    dt = w.dtype
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in Ps:
        want = run_gpu(b, P)  # pa_varlen_attention (+ pa_split_kv_reduce)
        got = _noalloc(b, P, torch.empty_like(b.q))
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{what} P={P}: differs from the allocating entry point"
        assert_close(got, ref, dt, f"{what} P={P} (no-alloc)")


def test_noalloc_two_calls_second_smaller():
    """Two calls in a row on one stream, the second over a smaller batch that
    reuses a prefix of the scratch the first one filled."""
    big, small = W.gqa_decode_bf16(), W.random_case(74, num_seqs=3, max_q=1, max_ctx=1300,
                                                    num_q_heads=32, num_kv_heads=8,
                                                    head_dim=128, block_size=16,
                                                    dtype=torch.bfloat16)
    bb, bsm = to_device(big), to_device(small)
    o1 = _noalloc(bb, 256, torch.empty_like(bb.q))
    o2 = _noalloc(bsm, 256, torch.empty_like(bsm.q))
    w1, w2 = run_gpu(bb, 256), run_gpu(bsm, 256)
    torch.cuda.synchronize()
    assert torch.equal(o1, w1) and torch.equal(o2, w2)
    assert_close(o2, oracle.run_workload(small), torch.bfloat16, "second, smaller call")


def test_noalloc_refuses_overflow():
    import paged_varlen_attention_amd as pa
    w = W.random_case(75, num_seqs=2, max_q=1, max_ctx=600, num_q_heads=8, num_kv_heads=2,
                      head_dim=128, block_size=16, dtype=torch.bfloat16)
    b = to_device(w)
    out = torch.full_like(b.q, 7.0)
    # 8192 query rows x 8 heads x 32 partitions x 130 floats > 32 MiB: refused
    # by the size check before any launch; out stays untouched
    big_q = torch.zeros(8192, 8, 128, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 8192], dtype=torch.int32, device="cuda")
    sl = torch.tensor([8192], dtype=torch.int32, device="cuda")
    bt = torch.zeros(1, 8192 // 16, dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.varlen_attention_noalloc(big_q, b.key_cache, b.value_cache, cu, sl, bt,
                                    torch.empty_like(big_q), max_q_len=8192, max_seq_len=8192,
                                    scale=0.1, partition_size=256)
    assert e.value.status == pa.PA_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

"""The dispatch record on real launches, and the PA_NO_SPLIT switch: results
stay at parity with the oracle while the split is skipped."""
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu


def test_record_paths():
    import paged_varlen_attention_amd as pa
    w = W.random_case(81, num_seqs=3, max_q=1, max_ctx=600, num_q_heads=8, num_kv_heads=2,
                      head_dim=128, block_size=16, dtype=torch.bfloat16)
    b = to_device(w)
    run_gpu(b, 256, reduce=False)
    rec = pa.last_dispatch()
    assert rec["path"] == "decode" and rec["status"] == 0 and rec["partition_size"] == 256
    assert rec["grid"][0] == 2 and rec["block"] == rec["tile"][1] * 64
    w = W.random_case(82, num_seqs=3, max_q=40, max_ctx=300, num_q_heads=8, num_kv_heads=2,
                      head_dim=128, block_size=16, dtype=torch.bfloat16)
    run_gpu(to_device(w), 0)
    rec = pa.last_dispatch()
    assert rec["path"] == "tiled" and rec["tile"][0] in (32, 64) and rec["block"] == 256
    w = W.random_case(83, num_seqs=3, max_q=5, max_ctx=300, num_q_heads=4, num_kv_heads=1,
                      head_dim=64, block_size=16, dtype=torch.float32)
    run_gpu(to_device(w), 0)
    assert pa.last_dispatch()["path"] == "decode_per_token"
    torch.cuda.synchronize()


@pytest.mark.parametrize("max_q", [1, 40])
def test_no_split_switch(monkeypatch, max_q):
    import paged_varlen_attention_amd as pa
    w = W.random_case(84 + max_q, num_seqs=4, max_q=max_q, max_ctx=1500, num_q_heads=16,
                      num_kv_heads=2, head_dim=128, block_size=16, dtype=torch.bfloat16)
    ref = oracle.run_workload(w)
    b = to_device(w)
    monkeypatch.setenv("PA_NO_SPLIT", "1")
    out = run_gpu(b, 512, reduce=False)
    assert pa.last_dispatch()["split_disabled"] and pa.last_dispatch()["partition_size"] == 0
    parts = pa.alloc_partials(w.total_q, w.num_q_heads, w.head_dim, 4, "cuda")
    pa.split_kv_reduce(out, parts, b.cu_seqlens_q, b.seq_lens, 512)  # a no-op
    assert pa.last_dispatch()["path"] == "reduce_skipped"
    torch.cuda.synchronize()
    assert_close(out, ref, torch.bfloat16, "PA_NO_SPLIT")


@pytest.mark.parametrize("name,expect,kv8", [("gqa_decode_bf16", 512, False), ("long_decode_bf16", 2048, False),
                                             ("gqa_decode_bf16", 512, True), ("long_decode_bf16", 2048, True)],
                         ids=["gqa", "long", "gqa-fp8kv", "long-fp8kv"])
def test_policy_pick_on_the_device(name, expect, kv8):
    """pa_pick_partition_size with the device's own CU count (num_cus = 0) on
    the two benchmark decode batches, over bf16 and over 8-bit caches: it
    picks the partition size measured fastest for them on MI355X (256 CUs;
    8-bit GQA batch: 34 us at 512 against 40 / 42 at 256 / 1024; 8-bit long
    decode: step 69.3-69.6 us at 2048 against 70.3-70.9 at 1024), and
    attention + reduce at that size match the oracle on every row."""
    import paged_varlen_attention_amd as pa
    import oracle_pins as pins
    w = W.CONFIGS[name]()
    if kv8:
        w = pins.fp8_case(w, 7)
    P = pa.pick_partition_size(w.seq_lens.tolist(), w.num_q_heads, w.num_kv_heads, w.head_dim,
                               w.block_size, w.dtype, kv8=kv8)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert P == expect, P
    ref = oracle.run_workload(w)
    out = run_gpu(to_device(w), P)
    torch.cuda.synchronize()
    assert_close(out, ref, torch.bfloat16, f"{name} at the policy's P={P}")

"""The whole step (cache write, block-table view, attention, split-KV reduce)
captured in a HIP graph: every replay, with other eager work and
synchronizations in between, equals the eager result bit for bit."""
import pytest
import torch

import workloads as W
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _step_fn(w, b, P, new_rows, out, partials):
    import paged_varlen_attention_amd as pa

    def step():
        nk, nv, sm = new_rows
        pa.reshape_and_cache(nk, nv, b.key_cache, b.value_cache, sm, k_scale=b.k_scale,
                             v_scale=b.v_scale)
        pa.varlen_attention(b.q, b.key_cache, b.value_cache, b.cu_seqlens_q, b.seq_lens,
                            b.block_tables, max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                            scale=b.scale, partition_size=P, out=out, partials=partials,
                            k_scale=b.k_scale, v_scale=b.v_scale)
    return step


# (workload, partition size, 8-bit caches): the 8-bit GQA step runs the
# quantising cache write and the whole-row 8-bit decode, the 8-bit mixed B
# step the raw 8-bit tiles
@pytest.mark.parametrize("name,P,kv8", [("gqa_decode_bf16", 512, False), ("spec_verify_bf16", 0, False),
                                        ("tiny_decode_f32", 0, False), ("gqa_decode_bf16", 512, True),
                                        ("mixed_prefill_bf16_B", 0, True)],
                         ids=["gqa", "verify", "tiny-f32", "gqa-fp8kv", "mixed-B-fp8kv"])
def test_graph_replays_match_eager(name, P, kv8):
    import paged_varlen_attention_amd as pa
    import oracle_pins as pins
    w0 = W.CONFIGS[name]()
    w = pins.fp8_case(w0, 11) if kv8 else w0
    b = to_device(w, write_cache=False)
    if w.slot_mapping is not None:
        # a slot addresses the same bytes in the 144-token and the 16-token page view
        rows = (w.new_key.cuda(), w.new_value.cuda(), w.slot_mapping.cuda())
    else:
        # (8-bit caches: the bf16 rows, quantised again by the cache write)
        k, v, s = W.last_token_rows(w0)
        rows = (k.cuda(), v.cuda(), s.cuda())
    out = torch.empty_like(b.q)
    partials = (pa.alloc_partials(w.total_q, w.num_q_heads, w.head_dim,
                                  pa.max_partitions(w.max_seq_len, P), "cuda") if P else None)
    step = _step_fn(w, b, P, rows, out, partials)
    step()
    torch.cuda.synchronize()
    eager = out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = to_device(W.random_case(3, num_seqs=3, max_q=1, max_ctx=700, num_q_heads=8,
                                    num_kv_heads=2, head_dim=128, block_size=16,
                                    dtype=torch.bfloat16))
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        # eager work of the program between replays
        pa.varlen_attention(other.q, other.key_cache, other.value_cache, other.cu_seqlens_q,
                            other.seq_lens, other.block_tables, max_q_len=1,
                            max_seq_len=other.max_seq_len, scale=other.scale, partition_size=256)
        torch.cuda.synchronize()
        iv = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(iv), eager.view(iv)), f"replay {i} differs"

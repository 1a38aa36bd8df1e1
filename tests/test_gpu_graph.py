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
        pa.reshape_and_cache(nk, nv, b.key_cache, b.value_cache, sm)
        pa.varlen_attention(b.q, b.key_cache, b.value_cache, b.cu_seqlens_q, b.seq_lens,
                            b.block_tables, max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                            scale=b.scale, partition_size=P, out=out, partials=partials)
    return step


@pytest.mark.parametrize("name,P", [("gqa_decode_bf16", 512), ("spec_verify_bf16", 0),
                                    ("tiny_decode_f32", 0)])
def test_graph_replays_match_eager(name, P):
    import paged_varlen_attention_amd as pa
    w = W.CONFIGS[name]()
    b = to_device(w, write_cache=False)
    if w.slot_mapping is not None:
        # a slot addresses the same bytes in the 144-token and the 16-token page view
        rows = (w.new_key.cuda(), w.new_value.cuda(), w.slot_mapping.cuda())
    else:
        k, v, s = W.last_token_rows(w)
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

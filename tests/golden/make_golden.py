"""Writes the hand-derived golden cases in this folder.

Each case is a tiny input whose exact result follows from a closed form
(stated in its ``derivation`` field) and the passage of the pages it pins
(``source``).  Nothing here calls the oracle or the HIP library: the expected
values are the arithmetic written out.  Run: ``python tests/golden/make_golden.py``.
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def cases():
    c = {}
    c["two_keys_weights"] = dict(
        source="vllm-metal kernel walkthrough, 'What is Paged Attention': attention over a request's cached keys; softmax(q.k*scale) weights the values",
        derivation="scores 0 and ln3 (scale = ln 3, q.k = 0, 1) -> softmax weights 1/4, 3/4 -> out = 1/4*[1,0] + 3/4*[0,1]",
        dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=2, block_size=16, num_blocks=1,
        cu_seqlens_q=[0, 1], seq_lens=[2], block_tables=[[0]], scale=math.log(3.0),
        q=[[[1, 0]]],
        cache_rows={"0": {"k": [[[0, 0]]], "v": [[[1, 0]]]}, "1": {"k": [[[1, 0]]], "v": [[[0, 1]]]}},
        expected_out=[[[0.25, 0.75]]])
    c["causal_bottom_right"] = dict(
        source="v0.28.0 release post, 'Packed queries and paged KV': a chunked-prefill step packs a request's new tokens after its cached prefix; query j sits at position ctx+j and sees keys 0..ctx+j",
        derivation="q_len 2, seq_len 3 (ctx 1), all scores equal -> uniform weights over visible keys; v_i=[i,1]; query 0 (pos 1) sees keys 0,1 -> [0.5,1]; query 1 (pos 2) sees keys 0..2 -> [1,1]",
        dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=2, block_size=16, num_blocks=1,
        cu_seqlens_q=[0, 2], seq_lens=[3], block_tables=[[0]], scale=0.125,
        q=[[[1, 0]], [[1, 0]]],
        cache_rows={str(i): {"k": [[[0, 0]]], "v": [[[i, 1]]]} for i in range(3)},
        expected_out=[[[0.5, 1.0]], [[1.0, 1.0]]])
    c["gqa_head_map"] = dict(
        source="vllm-metal kernel walkthrough, GQA decode section: several query heads share one KV head (grouped-query attention)",
        derivation="Hq=4, Hkv=2 -> heads 0,1 read KV head 0 and heads 2,3 read KV head 1; one visible key -> out = v_0 of that KV head",
        dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=2, block_size=16, num_blocks=1,
        cu_seqlens_q=[0, 1], seq_lens=[1], block_tables=[[0]], scale=0.5,
        q=[[[1, 2], [3, 4], [5, 6], [7, 8]]],
        cache_rows={"0": {"k": [[[1, 1], [2, 2]]], "v": [[[10, 11], [20, 21]]]}},
        expected_out=[[[10, 11], [10, 11], [20, 21], [20, 21]]])
    c["paged_walk"] = dict(
        source="vllm-metal kernel walkthrough, 'What is Paged Attention': block_tables map a logical position to a physical page; unified-memory article section three: slots past seq_len never reach the output",
        derivation="bs 2, block table [2,0]: logical keys 0,1 in block 2, key 2 in block 0 slot 0; other slots NaN. k_i=[i,0], q=[1,0], scale=ln2 -> weights 1,2,4 (/7); v_i=[1,i] -> out=[1, 10/7]",
        dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=2, block_size=2, num_blocks=3,
        cu_seqlens_q=[0, 1], seq_lens=[3], block_tables=[[2, 0]], scale=math.log(2.0),
        q=[[[1, 0]]],
        cache_rows={str(i): {"k": [[[i, 0]]], "v": [[[1, i]]]} for i in range(3)},
        expected_out=[[[1.0, 10.0 / 7.0]]])
    c["split_partials_log2"] = dict(
        source="vllm-metal kernel walkthrough, GQA decode tip 4 'Split-KV partitions': partials are log2-space (max, exp-sum) plus the normalised partial output, merged by a shared reduce",
        derivation="paged_walk with partition 2: log2 scores 0,1,2. part 0 (keys 0,1): m=1, l=2^-1+2^0=1.5, o=(0.5*v0+v1)/1.5=[1,2/3]. part 1 (key 2): m=2, l=1, o=v2=[1,2]. merge: M=2, w=(0.75,1) -> [1,10/7]",
        dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=2, block_size=2, num_blocks=3,
        cu_seqlens_q=[0, 1], seq_lens=[3], block_tables=[[2, 0]], scale=math.log(2.0), partition_size=2,
        q=[[[1, 0]]],
        cache_rows={str(i): {"k": [[[i, 0]]], "v": [[[1, i]]]} for i in range(3)},
        expected_m=[[[1.0, 2.0]]], expected_l=[[[1.5, 1.0]]],
        expected_o=[[[[1.0, 2.0 / 3.0], [1.0, 2.0]]]],
        expected_out=[[[1.0, 10.0 / 7.0]]])
    c["attention_sink"] = dict(
        source="vllm-metal kernel walkthrough, 'three Metal kernels': the decode kernel carries online softmax with attention-sink support (read as one more softmax term per query head that carries no value)",
        derivation="paged_walk's keys (e^s = 1, 2, 4; v_i = [1, i]) plus a sink logit ln 8 (e^sink = 8): out = (1*v0 + 2*v1 + 4*v2) / (7 + 8) = [7/15, 10/15]. Split at 2 keys: partials as in split_partials_log2; merge with sigma = log2(8) = 3: M = 3, w = (1.5/4, 1/2), sink weight 1 -> (0.375*[1,2/3] + 0.5*[1,2]) / 1.875 = [7/15, 2/3]",
        dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=2, block_size=2, num_blocks=3,
        cu_seqlens_q=[0, 1], seq_lens=[3], block_tables=[[2, 0]], scale=math.log(2.0), partition_size=2,
        sinks=[math.log(8.0)],
        q=[[[1, 0]]],
        cache_rows={str(i): {"k": [[[i, 0]]], "v": [[[1, i]]]} for i in range(3)},
        expected_out=[[[7.0 / 15.0, 10.0 / 15.0]]])
    c["copy_blocks_pairs"] = dict(
        source="KV-offloading article: blocks move between the GPU cache and a host tier by block-id lists (evict and restore); a block is one page of every KV head",
        derivation="src blocks s_b filled with b*10 + slot (K) and b*10 + slot + 100 (V); pairs (2,0), (0,1), (5,1): dst[0] = s_2, dst[1] = s_0, the pair naming src block 5 of a 3-block pool is skipped",
        dtype="f32", block_shape=[2, 1, 1], num_src_blocks=3, num_dst_blocks=2,
        pairs=[[2, 0], [0, 1], [5, 1]],
        expected_dst_key=[[[[20.0]], [[21.0]]], [[[0.0]], [[1.0]]]],
        expected_dst_value=[[[[120.0]], [[121.0]]], [[[100.0]], [[101.0]]]])
    c["reshape_and_cache_scatter"] = dict(
        source="vllm-metal kernel walkthrough, 'three Metal kernels': reshape_and_cache scatters projected K/V into the paged cache; a slot is block*block_size + offset",
        derivation="bs 2, 3 blocks, slots [5,-1,0]: token 0 -> block 2 offset 1, token 1 skipped, token 2 -> block 0 offset 0; every other slot keeps its previous content (0 here)",
        block_size=2, num_blocks=3, slot_mapping=[5, -1, 0],
        key=[[[1, 2]], [[3, 4]], [[5, 6]]], value=[[[-1, -2]], [[-3, -4]], [[-5, -6]]],
        expected_key_cache=[[[[5, 6]], [[0, 0]]], [[[0, 0]], [[0, 0]]], [[[0, 0]], [[1, 2]]]],
        expected_value_cache=[[[[-5, -6]], [[0, 0]]], [[[0, 0]], [[0, 0]]], [[[0, 0]], [[-1, -2]]]])
    c["expand_block_tables_9x16"] = dict(
        source="unified-memory article, section six: a 144-token vLLM block is viewed as nine 16-token kernel blocks, [nb,144,...] -> [nb*9,16,...] with no byte moved",
        derivation="kernel page 9*b+j of a 144-block b is page 9*phys(b)+j; -1 padding stays -1",
        ratio=9, src=[[3, -1], [0, 1]],
        expected=[list(range(27, 36)) + [-1] * 9, list(range(0, 18))])
    return c


if __name__ == "__main__":
    for name, case in cases().items():
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(case, f, indent=1)

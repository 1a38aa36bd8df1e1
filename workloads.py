"""Seeded synthetic inputs for paged variable-length attention.

This module only draws random numbers and lays them out: request lengths,
page permutations, block tables, slot mappings and N(0,1) Q/K/V values.  It
holds none of the attention arithmetic, so both the fp64 oracle (``oracle/``)
and the HIP library (``paged_varlen_attention_amd``) can be fed from it
without sharing any of the method.

Shapes follow the pages' workloads (vllm-metal, "Packed queries and paged KV"
in the v0.28.0 release post; "What is Paged Attention" and the GQA decode
section of the kernel walkthrough; section six of the unified-memory article
for the 144-token block viewed as nine 16-token pages):

* packed queries ``q[total_q, Hq, D]`` with request boundaries in
  ``cu_seqlens_q[B+1]``;
* a paged cache ``key_cache/value_cache[num_blocks, block_size, Hkv, D]``
  addressed through ``block_tables[B, max_blocks]`` (unused entries = -1);
* ``seq_lens[B]``: the number of keys each request sees after this step,
  including the step's own query tokens (their K/V are already in the cache,
  or are written by ``reshape_and_cache`` just before attention).

Every slot that no request owns -- page tails past ``seq_len`` and all unused
pages -- holds NaN, so any read of it shows up in the result.

Recipe (all draws from ``numpy.random.default_rng(seed)``, in this order):
request lengths, the page permutation of the pool, then Q, then K, then V
(only for the slots that hold valid tokens), then the new K/V rows and their
slot order for the cache-write workload.  Values are float32 N(0,1), cast to
bfloat16 with round-to-nearest-even where the workload is bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

NAN_BF16 = 0x7FC0


@dataclasses.dataclass
class Workload:
    name: str
    dtype: torch.dtype
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int            # page size of ``key_cache`` as stored
    num_blocks: int
    q: torch.Tensor            # [total_q, Hq, D]
    key_cache: torch.Tensor    # [num_blocks, block_size, Hkv, D]
    value_cache: torch.Tensor
    cu_seqlens_q: torch.Tensor  # int32 [B+1]
    seq_lens: torch.Tensor      # int32 [B]
    block_tables: torch.Tensor  # int32 [B, max_blocks], -1 = unused
    scale: float
    partition_sizes: List[int]
    # cache-write workloads: rows written by reshape_and_cache before attention
    new_key: Optional[torch.Tensor] = None     # [T, Hkv, D]
    new_value: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None  # int64 [T]
    # page size the attention kernel walks (block_size / kernel_page_ratio)
    kernel_page_ratio: int = 1
    description: str = ""
    sinks: Optional[torch.Tensor] = None  # float32 [Hq] attention-sink logits, or None
    # 8-bit caches: float32 [Hkv] per-head scales of K and V (None for bf16/fp32 caches)
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        cu = self.cu_seqlens_q.numpy()
        return cu[1:] - cu[:-1]

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == torch.float32 else 2

    def algorithmic_bytes(self, kv_elt_bytes: Optional[int] = None) -> int:
        """Each visible KV row once per KV head (shared by its query-head group),
        plus Q in and O out, plus the integer metadata.  kv_elt_bytes: bytes per
        cached element when the cache type differs from the queries' (1 for
        8-bit caches)."""
        ke = self.elt_bytes if kv_elt_bytes is None else kv_elt_bytes
        kv = int(self.seq_lens.to(torch.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * ke
        qo = 2 * self.total_q * self.num_q_heads * self.head_dim * self.elt_bytes
        meta = 4 * (self.cu_seqlens_q.numel() + self.seq_lens.numel() + self.block_tables.numel())
        return kv + qo + meta

    def algorithmic_flops(self) -> int:
        """4*Hq*D per unmasked (query, key) pair: QK^T and PV."""
        ql = self.q_lens.astype(np.int64)
        sl = self.seq_lens.numpy().astype(np.int64)
        ctx = sl - ql
        pairs = int((ql * ctx + ql * (ql + 1) // 2).sum())
        return 4 * self.num_q_heads * self.head_dim * pairs


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal(int(np.prod(shape)), dtype=np.float32)).reshape(shape)
    return x.to(dtype)


def _nan_pool(num_blocks: int, bs: int, hkv: int, d: int, dtype: torch.dtype) -> torch.Tensor:
    return torch.full((num_blocks, bs, hkv, d), float("nan"), dtype=dtype)


def build(name: str, *, seed: int, q_lens, seq_lens, num_q_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int, num_blocks: int, dtype: torch.dtype,
          partition_sizes=(0,), scale: Optional[float] = None, write_new_kv: bool = False,
          kernel_page_ratio: int = 1, description: str = "",
          rng: Optional[np.random.Generator] = None) -> Workload:
    """Lay out one batch.  ``q_lens``/``seq_lens`` are given; the pool pages
    are a uniform random permutation of the pool, handed out to the requests in
    order.  With ``write_new_kv`` the query tokens' K/V rows are returned as
    ``new_key/new_value`` plus their ``slot_mapping`` and are NOT in the cache;
    otherwise every visible row is already in the cache."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    assert q_lens.shape == seq_lens.shape and (seq_lens >= q_lens).all() and (q_lens >= 0).all()
    B = len(q_lens)
    pages = [(int(s) + block_size - 1) // block_size for s in seq_lens]
    assert sum(pages) <= num_blocks, "pool too small"
    perm = rng.permutation(num_blocks).astype(np.int64)
    max_blocks = max(1, max(pages) if pages else 1)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for r in range(B):
        bt[r, :pages[r]] = perm[off:off + pages[r]]
        off += pages[r]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    total_q = int(cu[-1])

    q = _normal(rng, (total_q, num_q_heads, head_dim), dtype)
    kc = _nan_pool(num_blocks, block_size, num_kv_heads, head_dim, dtype)
    vc = _nan_pool(num_blocks, block_size, num_kv_heads, head_dim, dtype)

    # which logical positions are already cached
    cached = [int(s - (q if write_new_kv else 0)) for s, q in zip(seq_lens, q_lens)]
    n_cached = sum(cached)
    kvals = _normal(rng, (n_cached, num_kv_heads, head_dim), dtype)
    vvals = _normal(rng, (n_cached, num_kv_heads, head_dim), dtype)
    blk_idx = np.empty(n_cached, dtype=np.int64)
    slot_idx = np.empty(n_cached, dtype=np.int64)
    o = 0
    for r in range(B):
        pos = np.arange(cached[r], dtype=np.int64)
        blk_idx[o:o + cached[r]] = bt[r, pos // block_size]
        slot_idx[o:o + cached[r]] = pos % block_size
        o += cached[r]
    bi = torch.from_numpy(blk_idx)
    si = torch.from_numpy(slot_idx)
    kc[bi, si] = kvals
    vc[bi, si] = vvals

    new_key = new_value = slot_mapping = None
    if write_new_kv:
        new_key = _normal(rng, (total_q, num_kv_heads, head_dim), dtype)
        new_value = _normal(rng, (total_q, num_kv_heads, head_dim), dtype)
        sm = np.empty(total_q, dtype=np.int64)
        for r in range(B):
            ctx = int(seq_lens[r] - q_lens[r])
            pos = ctx + np.arange(int(q_lens[r]), dtype=np.int64)
            sm[cu[r]:cu[r + 1]] = bt[r, pos // block_size].astype(np.int64) * block_size + pos % block_size
        slot_mapping = torch.from_numpy(sm)

    return Workload(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks, q=q,
        key_cache=kc, value_cache=vc, cu_seqlens_q=torch.from_numpy(cu),
        seq_lens=torch.from_numpy(seq_lens.astype(np.int32)), block_tables=torch.from_numpy(bt),
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
        partition_sizes=list(partition_sizes), new_key=new_key, new_value=new_value,
        slot_mapping=slot_mapping, kernel_page_ratio=kernel_page_ratio, description=description)


# --------------------------------------------------------------------------
# The five workloads.  Seeds 1-5.
# --------------------------------------------------------------------------

def tiny_decode_f32(seed: int = 1) -> Workload:
    """2 decode requests, 37 and 50 keys, Hq=4 Hkv=1 D=64, 16-token pages
    drawn from a shuffled 8-block pool, fp32, scale 1/8, no split."""
    return build("tiny_decode_f32", seed=seed, q_lens=[1, 1], seq_lens=[37, 50], num_q_heads=4,
                 num_kv_heads=1, head_dim=64, block_size=16, num_blocks=8, dtype=torch.float32,
                 partition_sizes=[0], description="2 req, ctx 37/50, 4/1/64, bs16, pool 8, fp32")


def gqa_decode_bf16(seed: int = 2, num_seqs: int = 32, lo: int = 512, hi: int = 4096,
                    num_blocks: int = 16384) -> Workload:
    """32 decode requests, seq_len U[512,4096], Hq=32 Hkv=8 D=128, 16-token
    pages shuffled across a 16,384-block pool, bf16, split 512 + reduce."""
    rng = np.random.default_rng(seed)
    sl = rng.integers(lo, hi + 1, size=num_seqs)
    return build("gqa_decode_bf16", seed=seed, q_lens=[1] * num_seqs, seq_lens=sl, num_q_heads=32,
                 num_kv_heads=8, head_dim=128, block_size=16, num_blocks=num_blocks,
                 dtype=torch.bfloat16, partition_sizes=[512], rng=rng,
                 description=f"{num_seqs} req x 1 tok, ctx U[{lo},{hi}], 32/8/128, bs16, pool {num_blocks}")


def mixed_prefill_bf16(seed: int = 3, variant: str = "A", num_blocks: int = 4096) -> Workload:
    """8 prefill prompts packed to 6,000 tokens (A: ~750 each; B: one 3,000
    among seven ~429) plus 8 decode tokens, Hq=16 Hkv=2 D=256, bf16.
    Prefill prompts have no cached prefix; each decode request already holds
    its ~750-token prompt plus 1..20 generated tokens.  Decode requests come
    first in the batch."""
    rng = np.random.default_rng(seed)
    if variant == "A":
        pl = 750 + rng.integers(-50, 51, size=8)
        pl[-1] = 6000 - int(pl[:-1].sum())
    elif variant == "B":
        pl = np.array([3000, 429, 429, 429, 429, 428, 428, 428], dtype=np.int64)
        pl = pl[rng.permutation(8)]
    else:
        raise ValueError(variant)
    dec_prompt = 750 + rng.integers(-50, 51, size=8)
    dec_gen = rng.integers(1, 21, size=8)
    q_lens = np.concatenate([np.ones(8, dtype=np.int64), pl])
    seq_lens = np.concatenate([dec_prompt + dec_gen, pl])
    return build(f"mixed_prefill_bf16_{variant}", seed=seed, q_lens=q_lens, seq_lens=seq_lens,
                 num_q_heads=16, num_kv_heads=2, head_dim=256, block_size=16, num_blocks=num_blocks,
                 dtype=torch.bfloat16, partition_sizes=[0], rng=rng,
                 description=f"8 prefill ({variant}) ~6000 tok + 8 decode, 16/2/256, bs16")


def long_decode_bf16(seed: int = 4, num_seqs: int = 4, ctx: int = 32768,
                     num_blocks: int = 16384) -> Workload:
    """4 decode requests of 32,768 keys, Hq=24 Hkv=4 D=256, pages randomly
    permuted, split 256 and 512 + reduce."""
    return build("long_decode_bf16", seed=seed, q_lens=[1] * num_seqs, seq_lens=[ctx] * num_seqs,
                 num_q_heads=24, num_kv_heads=4, head_dim=256, block_size=16, num_blocks=num_blocks,
                 dtype=torch.bfloat16, partition_sizes=[256, 512],
                 description=f"{num_seqs} req x 1 tok, ctx {ctx}, 24/4/256, bs16, pool {num_blocks}")


def spec_verify_bf16(seed: int = 5, lo: int = 1024, hi: int = 8192, num_blocks: int = 1024,
                     chunk: int = 512) -> Workload:
    """16 requests: 14 verify windows of 1..5 tokens (decode token + drafts)
    and two 512-token prefill chunks, seq_len U[1k,8k], Hq=16 Hkv=2 D=128,
    bf16.  The cache is stored in 144-token blocks (a 1,024-block pool) and
    walked as nine 16-token pages per block.  The query tokens' K/V are
    written by reshape_and_cache through slot_mapping before attention."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, 6, size=16)
    chunk_pos = rng.choice(16, size=2, replace=False)
    q_lens[chunk_pos] = chunk
    seq_lens = rng.integers(lo, hi + 1, size=16)
    seq_lens = np.maximum(seq_lens, q_lens)
    return build("spec_verify_bf16", seed=seed, q_lens=q_lens, seq_lens=seq_lens, num_q_heads=16,
                 num_kv_heads=2, head_dim=128, block_size=144, num_blocks=num_blocks,
                 dtype=torch.bfloat16, partition_sizes=[0], write_new_kv=True,
                 kernel_page_ratio=9, rng=rng,
                 description="16 req: 14 x 1-5 tok + 2 x 512 chunk, ctx U[1k,8k], 16/2/128, 144->9x16")


def prefill_uniform_bf16(seed: int = 7, num_seqs: int = 8, q_len: int = 4096,
                         ctx: int = 4096) -> Workload:
    """8 prompt chunks of 4,096 new tokens over 4,096 cached ones each, the
    mixed batches' head shape (Hq=16 Hkv=2 D=256, 16-token pages), bf16: a
    long uniform batch that shows the tiled kernel's steady state apart from
    the load imbalance of short ragged batches."""
    seq = q_len + ctx
    return build("prefill_uniform_bf16", seed=seed, q_lens=[q_len] * num_seqs,
                 seq_lens=[seq] * num_seqs, num_q_heads=16, num_kv_heads=2, head_dim=256,
                 block_size=16, num_blocks=num_seqs * seq // 16 + 8, dtype=torch.bfloat16,
                 partition_sizes=[0],
                 description=f"{num_seqs} x {q_len}-token prompt chunks over {ctx} cached tokens, 16/2/256")


def last_token_rows(w: Workload):
    """(key, value, slot_mapping) of each request's newest token, read back
    from the cache: writing them again with reshape_and_cache is the cache
    write of a decode step that leaves the cache's content unchanged."""
    cu = w.cu_seqlens_q.numpy()
    sl = w.seq_lens.numpy().astype(np.int64)
    bt = w.block_tables.numpy().astype(np.int64)
    slots = []
    for r in range(w.num_seqs):
        for j in range(int(cu[r + 1] - cu[r])):
            pos = int(sl[r]) - int(cu[r + 1] - cu[r]) + j
            slots.append(bt[r, pos // w.block_size] * w.block_size + pos % w.block_size)
    slots = torch.tensor(slots, dtype=torch.int64)
    flat_k = w.key_cache.reshape(-1, w.num_kv_heads, w.head_dim)
    flat_v = w.value_cache.reshape(-1, w.num_kv_heads, w.head_dim)
    return flat_k[slots].clone(), flat_v[slots].clone(), slots


CONFIGS = {
    "tiny_decode_f32": tiny_decode_f32,
    "gqa_decode_bf16": gqa_decode_bf16,
    "mixed_prefill_bf16_A": lambda seed=3: mixed_prefill_bf16(seed, "A"),
    "mixed_prefill_bf16_B": lambda seed=3: mixed_prefill_bf16(seed, "B"),
    "long_decode_bf16": long_decode_bf16,
    "spec_verify_bf16": spec_verify_bf16,
    "prefill_uniform_bf16": prefill_uniform_bf16,
}


def kv_scales(seed: int, num_kv_heads: int):
    """Per-KV-head scales for an 8-bit E4M3 cache holding N(0,1) data: K and V
    scales drawn U[0.008, 0.016] (so |x| / scale reaches the format's largest
    magnitude, 448, for |x| between 3.6 and 7.2: the tails saturate, as with a
    scale calibrated to the bulk of the data).  Returns (k_scale, v_scale)."""
    rng = np.random.default_rng(seed)
    ks = rng.uniform(0.008, 0.016, size=num_kv_heads).astype(np.float32)
    vs = rng.uniform(0.008, 0.016, size=num_kv_heads).astype(np.float32)
    return torch.from_numpy(ks), torch.from_numpy(vs)


def random_fp8_codes(seed: int, shape) -> torch.Tensor:
    """Uniform draws over the 254 finite E4M3 codes (NaN codes 0x7F, 0xFF
    excluded), as raw uint8."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 254, size=int(np.prod(shape)), dtype=np.int64)
    c = c + (c >= 0x7F)  # 0..126 and 128..254: skips 0x7F, never reaches 0xFF
    return torch.from_numpy(c.astype(np.uint8)).reshape(shape)


def random_case(seed: int, *, num_seqs: int, max_q: int, max_ctx: int, num_q_heads: int,
                num_kv_heads: int, head_dim: int, block_size: int, dtype: torch.dtype,
                min_q: int = 1, spare_blocks: int = 3, write_new_kv: bool = False) -> Workload:
    """Small ragged batch for parity sweeps: q_len U{min_q..max_q},
    cached prefix U{0..max_ctx}."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(min_q, max_q + 1, size=num_seqs)
    ctx = rng.integers(0, max_ctx + 1, size=num_seqs)
    seq_lens = q_lens + ctx
    pages = int(sum((int(s) + block_size - 1) // block_size for s in seq_lens))
    return build(f"random_{seed}", seed=seed, q_lens=q_lens, seq_lens=seq_lens,
                 num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                 block_size=block_size, num_blocks=pages + spare_blocks, dtype=dtype,
                 write_new_kv=write_new_kv, rng=rng)

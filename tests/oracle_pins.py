"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each ``pin_*`` takes an oracle library handle so the same checks can run
against a deliberately broken build of the oracle (see
``test_oracle.py::test_pins_catch_planted_mistakes``).  They use:

* hand-derived closed-form cases in ``tests/golden/`` (each cites its passage);
* independent dense computations -- numpy fp64 with an explicit mask, and
  torch's scaled_dot_product_attention in fp64 on the CPU -- over K/V gathered
  contiguously through the block table;
* invariances the pages imply: physical page order, page size (including a
  144-token block seen as nine 16-token pages), the split-KV partition size,
  and running a request alone in a contiguous cache;
* closed forms of softmax attention (single key, equal keys, constant V,
  zero query, a dominant key, repeated KV heads, plain top-left causal).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers

def golden(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        return json.load(f)


def golden_inputs(c):
    dt = torch.float32
    hkv, d, bs, nb = c["num_kv_heads"], c["head_dim"], c["block_size"], c["num_blocks"]
    kc = torch.full((nb, bs, hkv, d), float("nan"), dtype=dt)
    vc = torch.full((nb, bs, hkv, d), float("nan"), dtype=dt)
    bt = torch.tensor(c["block_tables"], dtype=torch.int32)
    for pos, rows in c["cache_rows"].items():
        i = int(pos)
        blk = int(bt[0, i // bs])
        kc[blk, i % bs] = torch.tensor(rows["k"], dtype=dt)[0]
        vc[blk, i % bs] = torch.tensor(rows["v"], dtype=dt)[0]
    q = torch.tensor(c["q"], dtype=dt)
    cu = torch.tensor(c["cu_seqlens_q"], dtype=torch.int32)
    sl = torch.tensor(c["seq_lens"], dtype=torch.int32)
    return q, kc, vc, cu, sl, bt, float(c["scale"])


def run(w, lib, rows=None):
    return oracle.run_workload(w, rows=rows, lib=lib)


def gather_request(w, r):
    """Contiguous K/V [L, Hkv, D] (fp64) of request r, read through its block table."""
    L = int(w.seq_lens[r])
    pos = np.arange(L)
    blocks = w.block_tables[r].numpy()[pos // w.block_size]
    offs = pos % w.block_size
    K = w.key_cache.double().numpy()[blocks, offs]
    V = w.value_cache.double().numpy()[blocks, offs]
    return K, V


def dense_numpy(w):
    """softmax(QK^T*scale + mask)V per request on contiguous K/V, numpy fp64."""
    q = w.q.double().numpy()
    out = np.zeros(q.shape)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_seqlens_q.numpy()
    for r in range(w.num_seqs):
        K, V = gather_request(w, r)
        L, ql = K.shape[0], cu[r + 1] - cu[r]
        if ql == 0:
            continue
        ctx = L - ql
        Kx, Vx = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
        Q = q[cu[r]:cu[r + 1]]
        S = np.einsum("jhd,ihd->hji", Q, Kx) * w.scale
        mask = np.arange(L)[None, :] <= (ctx + np.arange(ql))[:, None]
        S = np.where(mask[None], S, -np.inf)
        S = S - S.max(axis=-1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=-1, keepdims=True)
        out[cu[r]:cu[r + 1]] = np.einsum("hji,ihd->jhd", P, Vx)
    return torch.from_numpy(out)


def dense_sdpa(w):
    """torch scaled_dot_product_attention in fp64 on the CPU, KV heads repeated."""
    q = w.q.double()
    out = torch.zeros_like(q)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_seqlens_q.numpy()
    for r in range(w.num_seqs):
        K, V = gather_request(w, r)
        L, ql = K.shape[0], int(cu[r + 1] - cu[r])
        if ql == 0:
            continue
        ctx = L - ql
        Kt = torch.from_numpy(K).repeat_interleave(G, dim=1).permute(1, 0, 2)
        Vt = torch.from_numpy(V).repeat_interleave(G, dim=1).permute(1, 0, 2)
        Qt = q[cu[r]:cu[r + 1]].permute(1, 0, 2)
        mask = torch.arange(L)[None, :] <= (ctx + torch.arange(ql))[:, None]
        o = F.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mask, scale=w.scale)
        out[cu[r]:cu[r + 1]] = o.permute(1, 0, 2)
    return out


def micro_cases():
    """Small ragged batches spanning the geometries, page sizes and dtypes."""
    specs = [
        dict(num_seqs=3, max_q=1, max_ctx=39, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16),
        dict(num_seqs=2, max_q=5, max_ctx=35, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=8),
        dict(num_seqs=3, max_q=4, max_ctx=30, num_q_heads=6, num_kv_heads=1, head_dim=256, block_size=32),
        dict(num_seqs=2, max_q=9, max_ctx=20, num_q_heads=2, num_kv_heads=2, head_dim=64, block_size=16),
    ]
    out = []
    for i, s in enumerate(specs):
        for dt in (torch.float32, torch.bfloat16):
            out.append(W.random_case(100 + 2 * i + (dt == torch.bfloat16), dtype=dt, **s))
    return out


def with_cache(w, key_cache, value_cache, block_tables, block_size):
    import dataclasses
    return dataclasses.replace(w, key_cache=key_cache, value_cache=value_cache,
                               block_tables=block_tables, block_size=block_size,
                               num_blocks=key_cache.shape[0])


def relayout(w, block_size, seed, ratio=1):
    """Same logical K/V stored with another page size, pages in a random order.
    With ratio > 1 the pool holds blocks of block_size*ratio tokens."""
    rng = np.random.default_rng(seed)
    bsz = block_size * ratio
    pages = [(int(s) + bsz - 1) // bsz for s in w.seq_lens]
    nb = sum(pages) + 2
    perm = rng.permutation(nb)
    kc = torch.full((nb, bsz, w.num_kv_heads, w.head_dim), float("nan"), dtype=w.dtype)
    vc = kc.clone()
    bt = torch.full((w.num_seqs, max(pages)), -1, dtype=torch.int32)
    o = 0
    for r in range(w.num_seqs):
        bt[r, :pages[r]] = torch.from_numpy(perm[o:o + pages[r]].astype(np.int32))
        o += pages[r]
        L = int(w.seq_lens[r])
        pos = np.arange(L)
        src_b = w.block_tables[r].numpy()[pos // w.block_size]
        src_o = pos % w.block_size
        dst_b = bt[r].numpy()[pos // bsz]
        dst_o = pos % bsz
        kc[dst_b, dst_o] = w.key_cache[src_b, src_o]
        vc[dst_b, dst_o] = w.value_cache[src_b, src_o]
    return with_cache(w, kc, vc, bt, bsz)


def bitwise_equal(a, b):
    return a.shape == b.shape and torch.equal(a.view(torch.int64), b.view(torch.int64))


# ------------------------------------------------------------------- pins

def pin_golden_attention(lib):
    for name in ("two_keys_weights", "causal_bottom_right", "gqa_head_map", "paged_walk"):
        c = golden(name)
        q, kc, vc, cu, sl, bt, scale = golden_inputs(c)
        out = oracle.attention(q, kc, vc, cu, sl, bt, scale, lib=lib)
        exp = torch.tensor(c["expected_out"], dtype=torch.float64)
        assert torch.allclose(out, exp, rtol=1e-13, atol=1e-13), (name, out, exp)


def pin_golden_split(lib):
    c = golden("split_partials_log2")
    q, kc, vc, cu, sl, bt, scale = golden_inputs(c)
    P = c["partition_size"]
    o, m, l = oracle.attention_partials(q, kc, vc, cu, sl, bt, scale, P, lib=lib)
    assert torch.allclose(m, torch.tensor(c["expected_m"], dtype=torch.float64), rtol=1e-13, atol=1e-13), m
    assert torch.allclose(l, torch.tensor(c["expected_l"], dtype=torch.float64), rtol=1e-13, atol=1e-13), l
    assert torch.allclose(o, torch.tensor(c["expected_o"], dtype=torch.float64), rtol=1e-13, atol=1e-13), o
    out = oracle.split_reduce(o, m, l, cu, sl, P, lib=lib)
    assert torch.allclose(out, torch.tensor(c["expected_out"], dtype=torch.float64), rtol=1e-13, atol=1e-13)


def pin_golden_cache_write(lib):
    c = golden("reshape_and_cache_scatter")
    key = torch.tensor(c["key"], dtype=torch.float32)
    value = torch.tensor(c["value"], dtype=torch.float32)
    nb, bs = c["num_blocks"], c["block_size"]
    kc = torch.zeros((nb, bs) + tuple(key.shape[1:]), dtype=torch.float32)
    vc = torch.zeros_like(kc)
    oracle.reshape_and_cache(key, value, kc, vc, torch.tensor(c["slot_mapping"], dtype=torch.int64), lib=lib)
    assert torch.equal(kc, torch.tensor(c["expected_key_cache"], dtype=torch.float32)), kc
    assert torch.equal(vc, torch.tensor(c["expected_value_cache"], dtype=torch.float32)), vc
    g = golden("expand_block_tables_9x16")
    dst = oracle.expand_block_tables(torch.tensor(g["src"], dtype=torch.int32), g["ratio"], lib=lib)
    assert torch.equal(dst, torch.tensor(g["expected"], dtype=torch.int32)), dst


def pin_dense(lib):
    for w in micro_cases() + [W.tiny_decode_f32()]:
        out = run(w, lib)
        ref_np = dense_numpy(w)
        ref_t = dense_sdpa(w)
        assert torch.isfinite(out).all()
        assert (out - ref_np).abs().max() <= 1e-12, (w.name, (out - ref_np).abs().max())
        assert (out - ref_t).abs().max() <= 1e-12, (w.name, (out - ref_t).abs().max())


def pin_cache_write_vs_index_copy(lib):
    rng = np.random.default_rng(7)
    for dt, hkv, d, bs, nb, T in ((torch.bfloat16, 2, 128, 16, 9, 40), (torch.float32, 1, 64, 8, 5, 30)):
        key = torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32)).to(dt)
        value = torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32)).to(dt)
        slots = torch.from_numpy(rng.choice(nb * bs, size=T, replace=False).astype(np.int64))
        slots[rng.choice(T, size=T // 5, replace=False)] = -1
        # poison: random bit patterns in every slot
        bits = torch.from_numpy(rng.integers(0, 2 ** 15, size=(nb, bs, hkv, d), dtype=np.int16))
        if dt == torch.float32:
            bits = torch.from_numpy(rng.integers(-2 ** 31, 2 ** 31 - 1, size=(nb, bs, hkv, d),
                                                 dtype=np.int32))
        kc = bits.clone().view(dt)
        vc = (bits.clone() ^ 0x55).view(dt)
        ref_k, ref_v = kc.clone(), vc.clone()
        valid = slots >= 0
        ref_k.view(-1, hkv, d).index_copy_(0, slots[valid], key[valid])
        ref_v.view(-1, hkv, d).index_copy_(0, slots[valid], value[valid])
        oracle.reshape_and_cache(key, value, kc, vc, slots, lib=lib)
        iv = torch.int16 if dt == torch.bfloat16 else torch.int32
        assert torch.equal(kc.view(iv), ref_k.view(iv))
        assert torch.equal(vc.view(iv), ref_v.view(iv))


def pin_page_permutation(lib):
    for w in micro_cases()[:4]:
        base = run(w, lib)
        w2 = relayout(w, w.block_size, seed=11)
        assert bitwise_equal(base, run(w2, lib)), w.name


def pin_page_size(lib):
    for w in micro_cases()[:4]:
        base = run(w, lib)
        for bs in (8, 16, 32):
            assert bitwise_equal(base, run(relayout(w, bs, seed=bs), lib)), (w.name, bs)
        # 144-token blocks, then the same bytes seen as nine 16-token pages
        w144 = relayout(w, 16, seed=5, ratio=9)
        out144 = run(w144, lib)
        assert bitwise_equal(base, out144), w.name
        kbt = oracle.expand_block_tables(w144.block_tables, 9, lib=lib)
        nb = w144.key_cache.shape[0]
        kview = w144.key_cache.view(nb * 9, 16, w.num_kv_heads, w.head_dim)
        vview = w144.value_cache.view(nb * 9, 16, w.num_kv_heads, w.head_dim)
        assert bitwise_equal(base, run(with_cache(w, kview, vview, kbt, 16), lib)), w.name


def pin_split_invariance(lib):
    for w in micro_cases()[:6] + [W.tiny_decode_f32()]:
        base = run(w, lib)
        for P in (8, 16, 32):
            o, m, l = oracle.attention_partials(w.q, w.key_cache, w.value_cache, w.cu_seqlens_q,
                                                w.seq_lens, w.block_tables, w.scale, P, lib=lib)
            out = oracle.split_reduce(o, m, l, w.cu_seqlens_q, w.seq_lens, P, lib=lib)
            err = ((out - base).abs() / base.abs().clamp_min(1e-3)).max()
            assert err <= 1e-12, (w.name, P, err)


def pin_single_request(lib):
    import dataclasses
    for w in micro_cases()[:4]:
        base = run(w, lib)
        cu = w.cu_seqlens_q.numpy()
        for r in range(w.num_seqs):
            L = int(w.seq_lens[r])
            n = (L + w.block_size - 1) // w.block_size
            pos = np.arange(L)
            src_b = w.block_tables[r].numpy()[pos // w.block_size]
            kc = torch.full((n, w.block_size, w.num_kv_heads, w.head_dim), float("nan"), dtype=w.dtype)
            vc = kc.clone()
            kc.view(-1, w.num_kv_heads, w.head_dim)[:L] = w.key_cache[src_b, pos % w.block_size]
            vc.view(-1, w.num_kv_heads, w.head_dim)[:L] = w.value_cache[src_b, pos % w.block_size]
            ql = int(cu[r + 1] - cu[r])
            wr = dataclasses.replace(
                w, q=w.q[cu[r]:cu[r + 1]].contiguous(), key_cache=kc, value_cache=vc,
                cu_seqlens_q=torch.tensor([0, ql], dtype=torch.int32),
                seq_lens=w.seq_lens[r:r + 1].contiguous(),
                block_tables=torch.arange(n, dtype=torch.int32)[None], num_blocks=n)
            assert bitwise_equal(base[cu[r]:cu[r + 1]], run(wr, lib)), (w.name, r)


def _single(L, ql, hq, hkv, d, seed, dt=torch.float32, bs=16):
    return W.build("cf", seed=seed, q_lens=[ql], seq_lens=[L], num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=d, block_size=bs, num_blocks=(L + bs - 1) // bs + 1, dtype=dt)


def pin_closed_forms(lib):
    import dataclasses
    # (i) one visible key -> its V row, exactly
    w = _single(1, 1, 4, 2, 64, 21)
    out = run(w, lib)
    K, V = gather_request(w, 0)
    assert torch.equal(out[0], torch.from_numpy(np.repeat(V[0], 2, axis=0)))
    # (ii) all keys equal -> uniform mean of the visible V rows (per query)
    w = _single(30, 3, 2, 1, 64, 22)
    blk = w.block_tables[0, 0]
    w.key_cache[w.block_tables[0, :2].long()] = w.key_cache[blk, 0].clone()
    out = run(w, lib)
    K, V = gather_request(w, 0)
    for j in range(3):
        exp = V[:28 + j, 0].mean(axis=0)
        assert np.abs(out[j, :, :].numpy() - exp[None]).max() <= 1e-13
    # (iii) V constant -> that constant
    w = _single(45, 2, 4, 1, 128, 23)
    w.value_cache[w.block_tables[0, :3].long()] = 0.375
    out = run(w, lib)
    assert (out - 0.375).abs().max() <= 1e-14
    # (iv) q = 0 -> mean of visible V
    w = _single(20, 4, 2, 2, 64, 24)
    w.q.zero_()
    out = run(w, lib)
    K, V = gather_request(w, 0)
    for j in range(4):
        assert np.abs(out[j].numpy() - V[:17 + j].mean(axis=0)).max() <= 1e-13
    # (v) a dominant key: huge scale, distinct scores -> V of the argmax key
    w = _single(33, 1, 2, 1, 64, 25)
    w = dataclasses.replace(w, scale=1e6)
    out = run(w, lib)
    K, V = gather_request(w, 0)
    qv = w.q.double().numpy()[0]
    for h in range(2):
        i = int(np.argmax(K[:, 0] @ qv[h]))
        assert torch.equal(out[0, h], torch.from_numpy(V[i, 0]))
    # (vi) GQA == MHA with every KV head repeated for its query heads, exactly
    w = W.random_case(26, num_seqs=2, max_q=3, max_ctx=30, num_q_heads=8, num_kv_heads=2,
                      head_dim=64, block_size=16, dtype=torch.bfloat16)
    rep_k = w.key_cache.repeat_interleave(4, dim=2).contiguous()
    rep_v = w.value_cache.repeat_interleave(4, dim=2).contiguous()
    w_mha = dataclasses.replace(w, num_kv_heads=8, key_cache=rep_k, value_cache=rep_v)
    assert bitwise_equal(run(w, lib), run(w_mha, lib))
    # (vii) no cached prefix -> standard top-left causal attention
    w = _single(37, 37, 4, 4, 64, 27)
    out = run(w, lib)
    K, V = gather_request(w, 0)
    ref = F.scaled_dot_product_attention(w.q.double().permute(1, 0, 2), torch.from_numpy(K).permute(1, 0, 2),
                                         torch.from_numpy(V).permute(1, 0, 2), is_causal=True,
                                         scale=w.scale).permute(1, 0, 2)
    assert (out - ref).abs().max() <= 1e-12


def _with_sinks(w, seed, scale=2.0):
    import dataclasses
    g = torch.Generator().manual_seed(seed)
    return dataclasses.replace(w, sinks=(torch.randn(w.num_q_heads, generator=g) * scale).float())


def dense_numpy_sinks(w):
    """The dense numpy reference with each head's sink as one more key whose
    logit is the sink and whose value is zero."""
    q = w.q.double().numpy()
    out = np.zeros(q.shape)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_seqlens_q.numpy()
    sk = w.sinks.double().numpy()
    for r in range(w.num_seqs):
        K, V = gather_request(w, r)
        L, ql = K.shape[0], cu[r + 1] - cu[r]
        if ql == 0:
            continue
        ctx = L - ql
        Kx, Vx = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
        Q = q[cu[r]:cu[r + 1]]
        S = np.einsum("jhd,ihd->hji", Q, Kx) * w.scale
        mask = np.arange(L)[None, :] <= (ctx + np.arange(ql))[:, None]
        S = np.where(mask[None], S, -np.inf)
        S = np.concatenate([S, np.broadcast_to(sk[:, None, None], S.shape[:2] + (1,))], axis=-1)
        Vz = np.concatenate([Vx, np.zeros((1,) + Vx.shape[1:])], axis=0)
        S = S - S.max(axis=-1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=-1, keepdims=True)
        out[cu[r]:cu[r + 1]] = np.einsum("hji,ihd->jhd", P, Vz)
    return torch.from_numpy(out)


def pin_golden_sink(lib):
    c = golden("attention_sink")
    q, kc, vc, cu, sl, bt, scale = golden_inputs(c)
    sinks = torch.tensor(c["sinks"], dtype=torch.float32)
    exp = torch.tensor(c["expected_out"], dtype=torch.float64)
    out = oracle.attention(q, kc, vc, cu, sl, bt, scale, sinks=sinks, lib=lib)
    assert torch.allclose(out, exp, rtol=1e-7, atol=1e-7), out  # the sink is stored as float32
    o, m, l = oracle.attention_partials(q, kc, vc, cu, sl, bt, scale, c["partition_size"], lib=lib)
    out = oracle.split_reduce(o, m, l, cu, sl, c["partition_size"], sinks=sinks, lib=lib)
    assert torch.allclose(out, exp, rtol=1e-7, atol=1e-7), out


def pin_sinks(lib):
    """Sinks against the dense reference with a zero-value key, against the
    closed form of one key, -inf against no sink, and split invariance."""
    import dataclasses
    for i, w in enumerate(micro_cases()[:6]):
        ws = _with_sinks(w, 7 + i)
        out = run(ws, lib)
        ref = dense_numpy_sinks(ws)
        assert (out - ref).abs().max() <= 1e-12, (w.name, (out - ref).abs().max())
        none = dataclasses.replace(w, sinks=torch.full((w.num_q_heads,), float("-inf")))
        assert bitwise_equal(run(none, lib), run(w, lib)), w.name
        for P in (8, 32):
            o, m, l = oracle.attention_partials(w.q, w.key_cache, w.value_cache, w.cu_seqlens_q,
                                                w.seq_lens, w.block_tables, w.scale, P, lib=lib)
            red = oracle.split_reduce(o, m, l, w.cu_seqlens_q, w.seq_lens, P, sinks=ws.sinks, lib=lib)
            err = ((red - out).abs() / out.abs().clamp_min(1e-3)).max()
            assert err <= 1e-12, (w.name, P, err)
    # one key of logit x and a sink sigma: out = v * e^x / (e^x + e^sigma)
    w = _single(1, 1, 2, 1, 64, seed=41)
    x = (w.q.double()[0] @ w.key_cache.double()[int(w.block_tables[0, 0]), 0, 0]) * w.scale
    for sig in (-3.0, 0.0, 2.5):
        ws = dataclasses.replace(w, sinks=torch.tensor([sig, -sig], dtype=torch.float32))
        out = run(ws, lib)
        v = w.value_cache.double()[int(w.block_tables[0, 0]), 0, 0]
        for h in range(2):
            s = float(ws.sinks[h])
            expect = v / (1.0 + math.exp(s - float(x[h])))
            assert (out[0, h] - expect).abs().max() <= 1e-13, (sig, h)


def pin_golden_copy_blocks(lib):
    c = golden("copy_blocks_pairs")
    shp = tuple(c["block_shape"])
    nbs, nbd = c["num_src_blocks"], c["num_dst_blocks"]
    sk = torch.zeros((nbs,) + shp, dtype=torch.float32)
    for b in range(nbs):
        sk[b] = (b * 10 + torch.arange(shp[0], dtype=torch.float32)).view(shp[0], 1, 1)
    sv = sk + 100
    dk = torch.full((nbd,) + shp, -1.0)
    dv = dk.clone()
    oracle.copy_blocks(dk, dv, sk, sv, c["pairs"], lib=lib)
    assert torch.equal(dk, torch.tensor(c["expected_dst_key"])), dk
    assert torch.equal(dv, torch.tensor(c["expected_dst_value"])), dv


def pin_copy_blocks(lib):
    """Against torch indexing (bitwise, NaN payloads kept), pair order for
    repeated destinations, out-of-pool pairs skipped, and evict + restore
    giving back the cache bit for bit."""
    g = torch.Generator().manual_seed(5)
    for dt, shape in ((torch.bfloat16, (16, 2, 64)), (torch.float32, (8, 4, 128))):
        nbs, nbd = 12, 9
        sk = torch.randn((nbs,) + shape, generator=g).to(dt)
        sv = torch.randn((nbs,) + shape, generator=g).to(dt)
        sk[3, 0, 0, :4] = float("nan")
        dk = torch.randn((nbd,) + shape, generator=g).to(dt)
        dv = torch.randn((nbd,) + shape, generator=g).to(dt)
        pairs = torch.tensor([[3, 0], [7, 8], [0, 4], [11, 2], [20, 1], [5, -1], [6, 4]])
        ek, ev = dk.clone(), dv.clone()
        for s_, d_ in pairs.tolist():  # later pairs win
            if 0 <= s_ < nbs and 0 <= d_ < nbd:
                ek[d_] = sk[s_]
                ev[d_] = sv[s_]
        oracle.copy_blocks(dk, dv, sk, sv, pairs, lib=lib)
        assert torch.equal(dk.view(torch.uint8), ek.view(torch.uint8))
        assert torch.equal(dv.view(torch.uint8), ev.view(torch.uint8))
        # evict three blocks to a host pool, wipe them, restore: bitwise round trip
        hk = torch.zeros((4,) + shape, dtype=dt)
        hv = torch.zeros_like(hk)
        keep_k, keep_v = sk.clone(), sv.clone()
        out = torch.tensor([[3, 0], [9, 1], [1, 2]])
        oracle.copy_blocks(hk, hv, sk, sv, out, lib=lib)
        sk[[3, 9, 1]] = 0
        sv[[3, 9, 1]] = 0
        oracle.copy_blocks(sk, sv, hk, hv, out.flip(1), lib=lib)
        assert torch.equal(sk.view(torch.uint8), keep_k.view(torch.uint8))
        assert torch.equal(sv.view(torch.uint8), keep_v.view(torch.uint8))


# ------------------------------------------------------------ 8-bit KV cache

# Values of E4M3 codes worked out by hand from the format (sign, 4-bit exponent
# with bias 7, 3-bit mantissa; exponent 0 = subnormals m/8 * 2^-6).
E4M3_BY_HAND = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6, 0x08: 2.0 ** -6,
                0x38: 1.0, 0xB8: -1.0, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0,
                0xFE: -448.0}


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.int64).to(torch.uint8).view(torch.float8_e4m3fn).double()


def pin_e4m3_format(lib):
    """All 256 code values against torch's float8_e4m3fn (a library decode),
    hand-worked values, the sign of zero, NaN codes and monotonic order."""
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    v = oracle.e4m3_values(codes, lib=lib)
    ref = _torch_e4m3_values()
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(v), nan) and nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert torch.equal(v[~nan], ref[~nan])
    for c, x in E4M3_BY_HAND.items():
        assert float(v[c]) == x, (hex(c), float(v[c]), x)
    assert math.copysign(1.0, float(v[0x80])) == -1.0 and float(v[0x80]) == 0.0
    assert bool((v[1:127] > v[0:126]).all()) and bool((v[0x81:0xFF] < v[0x80:0xFE]).all())


def pin_e4m3_encode(lib):
    """The encoder: code -> value -> code round trip, every midpoint between
    neighbouring codes going to the even mantissa, points just off each
    midpoint, saturation and NaN, and torch's own float32 -> float8_e4m3fn
    rounding on random in-range values across all binades."""
    vals = _torch_e4m3_values()
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    back = oracle.e4m3_encode(vals[finite].float(), lib=lib)
    assert back.tolist() == finite
    mids, expect, above, below = [], [], [], []
    for c in range(0, 0x7E):
        a, b = float(vals[c]), float(vals[c + 1])
        m = (a + b) / 2  # exact in float32 (one more mantissa bit)
        mids.append(m)
        expect.append(c if c % 2 == 0 else c + 1)
        above.append(np.nextafter(np.float32(m), np.float32(np.inf)))
        below.append(np.nextafter(np.float32(m), np.float32(-np.inf)))
    mids_t = torch.tensor(mids, dtype=torch.float32)
    assert oracle.e4m3_encode(mids_t, lib=lib).tolist() == expect
    assert oracle.e4m3_encode(-mids_t, lib=lib).tolist() == [e | 0x80 for e in expect]
    up = oracle.e4m3_encode(torch.tensor(np.array(above, dtype=np.float32)), lib=lib).tolist()
    dn = oracle.e4m3_encode(torch.tensor(np.array(below, dtype=np.float32)), lib=lib).tolist()
    assert up == list(range(1, 0x7F)) and dn == list(range(0, 0x7E))
    special = torch.tensor([448.0, 449.0, 464.0, 480.0, 1e30, float("inf"), -500.0,
                            float("-inf"), float("nan"), -0.0, 1e-30, -1e-30, 2.0 ** -10,
                            1.5 * 2.0 ** -10, 2.0 ** -149], dtype=torch.float32)
    assert oracle.e4m3_encode(special, lib=lib).tolist() == [
        0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x00, 0x80, 0x00, 0x01, 0x00]
    g = torch.Generator().manual_seed(11)
    mag = torch.pow(10.0, torch.empty(200000).uniform_(-5.0, 2.66, generator=g))
    sign = torch.where(torch.rand(200000, generator=g) < 0.5, -1.0, 1.0)
    y = (mag * sign).clamp(-448.0, 448.0).float()
    ours = oracle.e4m3_encode(y, lib=lib)
    theirs = y.to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(ours, theirs), int((ours != theirs).sum())


def pin_golden_fp8_cache_write(lib):
    c = golden("fp8_cache_write")
    hkv, d, nb, bs = c["num_kv_heads"], c["head_dim"], c["num_blocks"], c["block_size"]
    f = lambda x: [[[float(e) for e in h] for h in t] for t in x]  # noqa: E731  ("inf", "nan")
    key = torch.tensor(f(c["key"]), dtype=torch.float32)
    value = torch.tensor(f(c["value"]), dtype=torch.float32)
    kc = torch.zeros((nb, bs, hkv, d), dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    oracle.reshape_and_cache_fp8(key, value, kc, vc, torch.tensor(c["slot_mapping"]),
                                 torch.tensor(c["k_scale"]), torch.tensor(c["v_scale"]), lib=lib)
    assert kc.reshape(nb * bs, hkv * d).tolist() == c["expected_key_codes"], kc
    assert vc.reshape(nb * bs, hkv * d).tolist() == c["expected_value_codes"], vc


def fp8_case(w, seed):
    """Workload ``w`` with its caches quantised to E4M3 (per-head scales drawn
    by workloads.kv_scales); NaN slots stay NaN codes."""
    import dataclasses
    ks, vs = W.kv_scales(seed, w.num_kv_heads)
    return dataclasses.replace(w, key_cache=oracle.quantize_cache(w.key_cache, ks),
                               value_cache=oracle.quantize_cache(w.value_cache, vs),
                               k_scale=ks, v_scale=vs)


def dequantised(w):
    """float64 caches value(code) * scale, decoded by torch (not the oracle)."""
    import dataclasses
    kc = w.key_cache.double() * w.k_scale.double()[None, None, :, None]
    vc = w.value_cache.double() * w.v_scale.double()[None, None, :, None]
    return dataclasses.replace(w, key_cache=kc, value_cache=vc, k_scale=None, v_scale=None)


def pin_fp8_cache_write(lib):
    """The quantising write against torch: fp32 division, clamp to +-448,
    torch's float32 -> float8_e4m3fn rounding; bf16 and fp32 rows."""
    g = torch.Generator().manual_seed(13)
    for dt in (torch.bfloat16, torch.float32):
        T, hkv, d, nb, bs = 37, 3, 64, 6, 8
        key = (torch.randn(T, hkv, d, generator=g) * 3).to(dt)
        value = (torch.randn(T, hkv, d, generator=g) * 3).to(dt)
        ks = torch.tensor([0.004, 0.01, 0.37], dtype=torch.float32)
        vs = torch.tensor([0.0123, 1.0, 0.005], dtype=torch.float32)
        slots = torch.randperm(nb * bs, generator=g)[:T]
        slots[5] = -1
        kc = torch.zeros((nb, bs, hkv, d), dtype=torch.uint8)
        vc = torch.zeros_like(kc)
        oracle.reshape_and_cache_fp8(key, value, kc, vc, slots, ks, vs, lib=lib)
        for x, sc, cache in ((key, ks, kc), (value, vs, vc)):
            y = (x.float() / sc[None, :, None]).clamp(-448.0, 448.0)
            ref = torch.zeros_like(cache).view(nb * bs, hkv, d)
            keep = slots >= 0
            ref[slots[keep]] = y[keep].to(torch.float8_e4m3fn).view(torch.uint8)
            assert torch.equal(cache.view(nb * bs, hkv, d), ref), dt


def pin_fp8_attention(lib):
    """Attention over 8-bit caches: against the dense numpy reference on
    torch-decoded, scaled caches; with power-of-two scales bit-identical to
    the oracle on an fp32 cache holding the decoded values; split partials
    merged back to the same rows."""
    import dataclasses
    for i, w in enumerate(micro_cases()):
        wq = fp8_case(w, 50 + i)
        out = run(wq, lib)
        ref = dense_numpy(dequantised(wq))
        err = (out - ref).abs().max()
        assert err <= 1e-12, (w.name, float(err))
        for P in (8, 16):
            o, m, l = oracle.attention_partials(wq.q, wq.key_cache, wq.value_cache,
                                                wq.cu_seqlens_q, wq.seq_lens, wq.block_tables,
                                                wq.scale, P, k_scale=wq.k_scale,
                                                v_scale=wq.v_scale, lib=lib)
            red = oracle.split_reduce(o, m, l, wq.cu_seqlens_q, wq.seq_lens, P, lib=lib)
            rel = ((red - out).abs() / out.abs().clamp_min(1e-3)).max()
            assert rel <= 1e-12, (w.name, P, float(rel))
    for i, w in enumerate(micro_cases()):
        if w.dtype != torch.float32:
            continue
        hkv = w.num_kv_heads
        ks = torch.tensor([2.0 ** -(6 + h) for h in range(hkv)], dtype=torch.float32)
        vs = torch.tensor([2.0 ** -(5 - h) for h in range(hkv)], dtype=torch.float32)
        wq = dataclasses.replace(w, key_cache=oracle.quantize_cache(w.key_cache, ks),
                                 value_cache=oracle.quantize_cache(w.value_cache, vs),
                                 k_scale=ks, v_scale=vs)
        d = dequantised(wq)
        plain = dataclasses.replace(d, key_cache=d.key_cache.float(), value_cache=d.value_cache.float())
        assert bitwise_equal(run(wq, lib), run(plain, lib)), w.name


ALL_PINS = [pin_golden_attention, pin_golden_split, pin_golden_cache_write, pin_dense,
            pin_cache_write_vs_index_copy, pin_page_permutation, pin_page_size,
            pin_split_invariance, pin_single_request, pin_closed_forms, pin_golden_sink, pin_sinks,
            pin_golden_copy_blocks, pin_copy_blocks, pin_e4m3_format, pin_e4m3_encode,
            pin_golden_fp8_cache_write, pin_fp8_cache_write, pin_fp8_attention]

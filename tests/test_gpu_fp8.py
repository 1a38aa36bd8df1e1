"""GPU parity of the 8-bit (E4M3) KV cache: the quantising cache write
bit-exact against the oracle's codes, and attention over 8-bit caches against
the fp64 oracle reading the same codes (decode, split-KV with the reduce,
multi-token windows, sinks, every finite code)."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_close, run_gpu, sample_rows, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gpu_write(key, value, nb, bs, slots, ks, vs, fill=0):
    import paged_varlen_attention_amd as pa
    T, hkv, d = key.shape
    kc = torch.full((nb, bs, hkv, d), fill, dtype=torch.uint8, device="cuda")
    vc = kc.clone()
    pa.reshape_and_cache(key.cuda(), value.cuda(), kc, vc, slots.cuda(), k_scale=ks.cuda(),
                         v_scale=vs.cuda())
    torch.cuda.synchronize()
    return kc.cpu(), vc.cpu()


def _oracle_write(key, value, nb, bs, slots, ks, vs, fill=0):
    T, hkv, d = key.shape
    kc = torch.full((nb, bs, hkv, d), fill, dtype=torch.uint8)
    vc = kc.clone()
    oracle.reshape_and_cache_fp8(key, value, kc, vc, slots, ks, vs)
    return kc, vc


def test_fp8_cache_write_golden():
    """The hand-derived golden write (saturation, NaN, ties, subnormals, the
    sign of zero, a non-power-of-two scale) on the GPU."""
    with open(os.path.join(GOLDEN, "fp8_cache_write.json")) as f:
        c = json.load(f)
    conv = lambda x: [[[float(e) for e in h] for h in t] for t in x]  # noqa: E731
    key = torch.tensor(conv(c["key"]), dtype=torch.float32)
    value = torch.tensor(conv(c["value"]), dtype=torch.float32)
    # rows of 8 elements are below the 16-element piece the kernel writes:
    # pad D to 16 with zeros and compare the first 4 elements of each head
    hkv, d = c["num_kv_heads"], c["head_dim"]
    kp = torch.zeros(1, hkv, 16)
    vp = torch.zeros(1, hkv, 16)
    kp[:, :, :d] = key
    vp[:, :, :d] = value
    kc, vc = _gpu_write(kp, vp, c["num_blocks"], c["block_size"], torch.tensor(c["slot_mapping"]),
                        torch.tensor(c["k_scale"]), torch.tensor(c["v_scale"]))
    nslots = c["num_blocks"] * c["block_size"]
    got_k = kc.view(nslots, hkv, 16)[:, :, :d].reshape(nslots, hkv * d)
    got_v = vc.view(nslots, hkv, 16)[:, :, :d].reshape(nslots, hkv * d)
    assert got_k.tolist() == c["expected_key_codes"]
    assert got_v.tolist() == c["expected_value_codes"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("hkv,d", [(1, 64), (8, 128), (4, 256), (3, 64)])
def test_fp8_cache_write_bit_exact(dtype, hkv, d):
    """Random rows spanning 12 binades around the scale (so codes saturate and
    reach the subnormals), specials (NaN, +-inf, +-0, tiny), skipped slots:
    every code equal to the oracle's."""
    _bit_exact_write(dtype, hkv, d, 300, 40)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_fp8_cache_write_bit_exact_large(dtype):
    """A write large enough (4,500 rows of 8 x 128) for the kernel's
    16-elements-a-thread form; the smaller writes above take 4 a thread."""
    _bit_exact_write(dtype, 8, 128, 4500, 300)


def _bit_exact_write(dtype, hkv, d, T, nb):
    g = torch.Generator().manual_seed(hkv * 1000 + d + (dtype == torch.float32) + (T if T != 300 else 0))
    bs = 16
    mag = torch.pow(2.0, torch.empty(T, hkv, d).uniform_(-14.0, 10.0, generator=g))
    sign = torch.where(torch.rand(T, hkv, d, generator=g) < 0.5, -1.0, 1.0)
    key = (mag * sign * 0.01).to(dtype)
    value = (torch.randn(T, hkv, d, generator=g) * 2).to(dtype)
    key[0, 0, :6] = torch.tensor([float("nan"), float("inf"), float("-inf"), 0.0, -0.0, 1e-30])
    ks = torch.empty(hkv).uniform_(0.004, 0.05, generator=g).float()
    vs = torch.empty(hkv).uniform_(0.004, 0.05, generator=g).float()
    slots = torch.randperm(nb * bs, generator=g)[:T]
    slots[[3, 77, 150]] = -1
    gk, gv = _gpu_write(key, value, nb, bs, slots, ks, vs, fill=0x5A)
    ok, ov = _oracle_write(key, value, nb, bs, slots, ks, vs, fill=0x5A)
    assert torch.equal(gk, ok), int((gk != ok).sum())
    assert torch.equal(gv, ov), int((gv != ov).sum())


def test_fp8_cache_write_midpoints():
    """Every midpoint between neighbouring E4M3 values (and its float32
    neighbours), both signs, through the kernel with scale 1: ties to even."""
    vals = torch.arange(256, dtype=torch.int64).to(torch.uint8).view(torch.float8_e4m3fn).float()
    mids = [(float(vals[c]) + float(vals[c + 1])) / 2 for c in range(0x7E)]
    m = np.array(mids, dtype=np.float32)
    xs = np.concatenate([m, np.nextafter(m, np.float32(np.inf)), np.nextafter(m, np.float32(-np.inf))])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    n = (len(xs) + 63) // 64 * 64
    row = np.zeros(n, dtype=np.float32)
    row[:len(xs)] = xs
    key = torch.from_numpy(row).view(n // 64, 1, 64)
    ones = torch.ones(1)
    slots = torch.arange(n // 64)
    gk, _ = _gpu_write(key, key, n // 64, 1, slots, ones, ones)
    ok, _ = _oracle_write(key, key, n // 64, 1, slots, ones, ones)
    assert torch.equal(gk, ok), int((gk != ok).sum())


def _fp8(w, seed):
    return pins.fp8_case(w, seed)


GEOMS = [(4, 1, 64), (32, 8, 128), (24, 4, 256), (16, 2, 128), (8, 8, 64), (14, 2, 256),
         (6, 2, 128)]


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv,d", GEOMS, ids=[f"{a}-{b}-{c}" for a, b, c in GEOMS])
def test_fp8_decode_geometries(hq, hkv, d, bs):
    """Ragged decode batches over 8-bit caches, every partition size."""
    w = _fp8(W.random_case(7000 + hq * 10 + d + bs, num_seqs=5, max_q=1, max_ctx=1300,
                           num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                           dtype=torch.bfloat16), seed=hq + d + bs)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 P={P}")


@pytest.mark.parametrize("bs", [8, 16])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (16, 4, 128), (8, 1, 256)])
def test_fp8_multi_token_windows(hq, hkv, d, bs):
    """Prefill chunks and verify windows over 8-bit caches, with the new
    tokens' K/V written by the quantising cache write first."""
    w = W.random_case(7100 + hq + d + bs, num_seqs=4, max_q=37, max_ctx=700, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=torch.bfloat16,
                      write_new_kv=True)
    w = _fp8(w, seed=d + bs)
    ref = oracle.run_workload(w)
    b = to_device(w)
    import paged_varlen_attention_amd as pa
    for P in (0, 256):
        parts = (pa.alloc_partials(w.total_q, hq, d, pa.max_partitions(w.max_seq_len, P), "cuda")
                 if P else None)
        out = run_gpu(b, P, partials=parts, reduce=False)
        # windows over 8-bit pages run on the MFMA tiles
        assert pa.last_dispatch()["path"] == "tiled"
        if P:
            pa.split_kv_reduce(out, parts, b.cu_seqlens_q, b.seq_lens, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 windows P={P}")


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (24, 4, 256), (16, 2, 256), (12, 4, 128),
                                      (8, 8, 128), (4, 1, 64), (14, 2, 64)])
def test_fp8_tiled_geometries(hq, hkv, d, bs):
    """Ragged q_len 1..45 over cached prefixes 0..300 (several q-tiles and key
    tiles with ragged tails) on 8-bit pages, every partition size."""
    w = _fp8(W.random_case(7300 + hq * 7 + d + bs, num_seqs=6, max_q=45, max_ctx=300,
                           num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                           dtype=torch.bfloat16), seed=hq + bs)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 tiles P={P}")


def test_fp8_mixed_chunked_prefill():
    """The mixed chunked-prefill batch A (6,000 prompt tokens + 8 decode
    tokens, 16/2/256) over 8-bit pages; every row, unsplit and split."""
    w = _fp8(W.mixed_prefill_bf16(variant="A"), seed=3)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 mixed P={P}")


def test_fp8_spec_verify_with_cache_write():
    """Verify windows and two 512-token chunks over 1k..8k contexts, 144-token
    blocks seen as 9x16 pages, the new K/V quantised by the cache write first;
    every row, split at 1024."""
    w = _fp8(W.spec_verify_bf16(), seed=5)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 1024):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 verify P={P}")


def test_fp8_every_code_and_sinks():
    """Caches of uniformly drawn finite codes (all 254 of them, small scales)
    and per-head sinks, split and unsplit."""
    w = W.random_case(7200, num_seqs=6, max_q=1, max_ctx=2000, num_q_heads=16, num_kv_heads=4,
                      head_dim=128, block_size=16, dtype=torch.bfloat16)
    shape = tuple(w.key_cache.shape)
    kc = W.random_fp8_codes(1, shape).view(torch.float8_e4m3fn)
    vc = W.random_fp8_codes(2, shape).view(torch.float8_e4m3fn)
    ks = torch.tensor([2.0 ** -8, 0.003, 0.0017, 2.0 ** -9])
    vs = torch.tensor([0.01, 2.0 ** -6, 0.002, 0.0041])
    g = torch.Generator().manual_seed(3)
    w = dataclasses.replace(w, key_cache=kc, value_cache=vc, k_scale=ks, v_scale=vs,
                            sinks=(torch.randn(16, generator=g) * 2).float())
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (0, 256, 512):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 all codes + sinks P={P}")


def test_fp8_gqa_decode_batch():
    """The GQA decode batch (32 requests, ctx U[512,4096], 32/8/128) over an
    8-bit cache: every row, split 512 and unsplit."""
    w = _fp8(W.gqa_decode_bf16(), seed=2)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in (512, 0):
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"fp8 gqa decode P={P}")


def test_fp8_long_context_sampled():
    """4 requests of 32,768 keys, 24/4/256, 8-bit cache, split 512: sampled
    rows against the oracle."""
    w = _fp8(W.long_decode_bf16(), seed=4)
    rows = sample_rows(w, 24, seed=9)
    ref = oracle.run_workload(w, rows=rows)
    b = to_device(w)
    out = run_gpu(b, 512)
    torch.cuda.synchronize()
    got = torch.stack([out[t, h] for t, h in rows])
    assert_close(got, ref, torch.bfloat16, "fp8 long decode")

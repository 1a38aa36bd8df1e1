"""GPU parity of the 8-bit whole-row decode kernel (one workgroup per request
and partition serving every KV head over E4M3 caches), forced on with
PA_DECODE_ROWS=2 so small batches take it too: head groups of 4 heads (group
4) and of 2 heads (group 8), one, two and four head groups per row, pages of
16 and 32 tokens, key counts on and next to chunk (16 keys), page and
partition edges, unsplit ranges whose chunks outrun one block-table window,
sinks, requests without a query token, caches of every finite code with NaN
codes in the page tails, and the dispatch record.  Shapes it does not serve
(other groups, other head sizes, 8-token pages) keep the per-head kernel."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _rows_on(monkeypatch):
    monkeypatch.setenv("PA_DECODE_ROWS", "2")


def _pool(seq_lens, bs):
    return int(sum((int(s) + bs - 1) // bs for s in seq_lens)) + 8


def _case(name, seed, seq_lens, hq, hkv, d, bs, q_lens=None):
    w = W.build(name, seed=seed, q_lens=q_lens or [1] * len(seq_lens), seq_lens=seq_lens,
                num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                num_blocks=_pool(seq_lens, bs), dtype=torch.bfloat16)
    return pins.fp8_case(w, seed)


def _rows8_form(hq, hkv, d, bs):
    """Whether the 8-bit whole-row kernel serves the shape (mirrors the
    library's rule): D = 128, group 4 or 8 (head groups of 16 / group heads),
    1, 2 or 4 head groups, pages of a multiple of 16 tokens."""
    g = hq // hkv
    if d != 128 or g not in (4, 8) or bs % 16:
        return False
    hg = 16 // g
    return hkv % hg == 0 and hkv // hg in (1, 2, 4)


def _check(w, Ps, what):
    import paged_varlen_attention_amd as pa
    expect = _rows8_form(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in Ps:
        out = run_gpu(b, P, reduce=True)
        rec = pa.last_dispatch()
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"{what} P={P}")
        if P:  # the attention launch is the one before the reduce: check it alone
            run_gpu(b, P, reduce=False)
            rec = pa.last_dispatch()
        assert rec["path"] == "decode"
        # grid x: requests (whole rows) or KV heads (per-head kernel)
        assert (rec["grid"][0] == w.num_seqs) == expect or w.num_seqs == w.num_kv_heads, rec


# (hq, hkv): group 4 with 1, 2 and 4 head groups of 4 heads; group 8 with 1, 2
# and 4 head groups of 2 heads; group 2 and group 6 stay on the per-head kernel
SHAPES = [(16, 4), (32, 8), (64, 16), (16, 2), (32, 4), (64, 8), (16, 8), (24, 4)]


@pytest.mark.parametrize("hq,hkv", SHAPES)
def test_block_shapes(hq, hkv):
    rng = np.random.default_rng(hq * 5 + hkv)
    seq = rng.integers(1, 2500, size=5)
    w = _case(f"rows8_{hq}_{hkv}", 1600 + hq + hkv, seq, hq, hkv, 128, 16)
    _check(w, (0, 256, 512), f"rows8 hq={hq} hkv={hkv}")


def test_other_head_sizes_stay_per_head():
    """D = 64 and D = 256 batches over 8-bit caches keep the per-head kernel."""
    for d in (64, 256):
        w = _case(f"rows8_d{d}", 1700 + d, [700, 1300, 5], 32, 8, d, 16)
        _check(w, (0, 512), f"rows8 D={d}")


EDGES = [1, 2, 3, 15, 16, 17, 31, 32, 33, 47, 48, 49, 255, 256, 257, 511, 512, 513]


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 2), (64, 16)])
def test_chunk_and_page_edges(hq, hkv, bs):
    """Key counts on and next to chunk (16 keys), page and partition edges;
    8-token pages go to the per-head kernel."""
    w = _case(f"rows8_edges_{hq}_{hkv}_{bs}", 1800 + hq + hkv + bs, EDGES, hq, hkv, 128, bs)
    _check(w, (0, 256, 512), f"rows8 edges hq={hq} hkv={hkv} bs={bs}")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 2), (64, 16)])
def test_sliding_window(hq, hkv):
    """Unsplit ranges of 9,000 and 5,000 keys and 8,192-key partitions: each
    wave's chunks outrun one 64-entry block-table window."""
    w = _case(f"rows8_slide_{hq}_{hkv}", 1900 + hq + hkv, [9000, 5000, 37], hq, hkv, 128, 16)
    _check(w, (0, 8192), f"rows8 sliding window hq={hq} hkv={hkv}")


@pytest.mark.parametrize("scale", [1.0, 8.0])
def test_sinks(scale):
    """Sinks in the kernel's own finish (unsplit) and in the reduce (split)."""
    rng = np.random.default_rng(41)
    w = _case("rows8_sinks", 1951, rng.integers(1, 3000, size=6), 32, 8, 128, 16)
    g = torch.Generator().manual_seed(6)
    w = dataclasses.replace(w, sinks=(torch.randn(w.num_q_heads, generator=g) * scale).float())
    _check(w, (0, 512), f"rows8 sinks x{scale}")


def test_empty_and_mixed_rows():
    """Requests with no query token next to decode rows: only rows with a
    token are written."""
    seq = [300, 50, 1, 700, 9, 1024]
    w = _case("rows8_mixed", 1977, seq, 32, 8, 128, 16, q_lens=[1, 0, 1, 1, 0, 1])
    _check(w, (0, 256), "rows8 with empty requests")


@pytest.mark.parametrize("hq,hkv", [(16, 4), (32, 4)])
def test_every_code_nan_tails(hq, hkv):
    """Caches of uniformly drawn finite codes (all 254 of them) with NaN codes
    in every slot past each request's keys, per-head scales of both kinds
    (powers of two and not)."""
    seq = [1, 17, 250, 1500, 2000, 33]
    w = _case(f"rows8_codes_{hq}_{hkv}", 1990 + hq, seq, hq, hkv, 128, 16)
    shape = tuple(w.key_cache.shape)
    kc = W.random_fp8_codes(11, shape)
    vc = W.random_fp8_codes(12, shape)
    # NaN codes (0x7F / 0xFF) in every page slot past the request's last key
    bt = w.block_tables
    for r, L in enumerate(seq):
        nblk = (L + 15) // 16
        last = int(bt[r, nblk - 1])
        kc[last, L - (nblk - 1) * 16:] = 0x7F
        vc[last, L - (nblk - 1) * 16:] = 0xFF
    ks = torch.tensor([2.0 ** -8, 0.003, 0.0017, 2.0 ** -9][:hkv])
    vs = torch.tensor([0.01, 2.0 ** -6, 0.002, 0.0041][:hkv])
    w = dataclasses.replace(w, key_cache=kc.view(torch.float8_e4m3fn),
                            value_cache=vc.view(torch.float8_e4m3fn), k_scale=ks, v_scale=vs)
    _check(w, (0, 256, 512), f"rows8 every code hq={hq} hkv={hkv}")


def test_auto_choice(monkeypatch):
    """Default mode on the GQA decode batch over 8-bit caches: split 512 (256
    items) takes the whole-row kernel, split 1024 (128 items) and unsplit (32
    items) the per-head one; all against the oracle."""
    import paged_varlen_attention_amd as pa
    monkeypatch.setenv("PA_DECODE_ROWS", "1")
    w = pins.fp8_case(W.gqa_decode_bf16(), 2)
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P, rows in ((512, True), (1024, False), (0, False)):
        run_gpu(b, P, reduce=False)
        rec = pa.last_dispatch()
        assert (rec["grid"][0] == w.num_seqs) == rows, rec
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"auto rows8 P={P}")

"""GPU parity of the whole-row decode kernel (one workgroup per request and
partition serving every KV head), forced on with PA_DECODE_ROWS=2 so small
batches take it too: every block shape it has (heads per MFMA block 2, 4 and
8, one or two blocks per row, head sizes 128 and 256), key counts on and next
to chunk, page and partition edges, unsplit ranges whose chunks outrun one
block-table window, sinks, and the dispatch record.  Batches it does not
serve (8-bit caches, one KV head) keep the per-head kernel."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _rows_on(monkeypatch):
    monkeypatch.setenv("PA_DECODE_ROWS", "2")


def _pool(seq_lens, bs):
    return int(sum((int(s) + bs - 1) // bs for s in seq_lens)) + 8


def _case(name, seed, seq_lens, hq, hkv, d, bs):
    return W.build(name, seed=seed, q_lens=[1] * len(seq_lens), seq_lens=seq_lens, num_q_heads=hq,
                   num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=_pool(seq_lens, bs),
                   dtype=torch.bfloat16)


def _rows_form(hq, hkv, d, bs):
    """Whether the whole-row kernel serves the shape (mirrors the library's
    rule): heads per block = the largest power of two <= 8 and <= hkv whose
    groups fit 16 columns; one or two blocks per cache row (one at D = 256);
    chunks of 16 / heads-per-block keys inside one page."""
    g = hq // hkv
    h = 8
    while h > 1 and (h * g > 16 or h > hkv):
        h //= 2
    if h < 2 or hkv not in (h, 2 * h) or 16 // h > bs or g > 8:
        return False
    return not (d == 256 and hkv == 2 * h)


def _check(w, Ps, what):
    expect_rows = _rows_form(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size)
    import paged_varlen_attention_amd as pa
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
        assert (rec["grid"][0] == w.num_seqs) == expect_rows or w.num_seqs == w.num_kv_heads, rec


# (hq, hkv): heads per block 4 x 2 blocks, 2 x 2, 8 x 1, 8 x 1 (group 1),
# 4 x 1, 2 x 1 (group 5), 2 x 1 (group 4 over 2 heads), 2 x 2 (group 8);
# two blocks at D = 256 stay on the per-head kernel (checked as such)
SHAPES = [(32, 8), (24, 4), (16, 8), (8, 8), (12, 4), (10, 2), (8, 2), (32, 4)]


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("hq,hkv", SHAPES)
def test_block_shapes(hq, hkv, d):
    rng = np.random.default_rng(hq * 7 + hkv + d)
    seq = rng.integers(1, 2500, size=5)
    w = _case(f"rows_{hq}_{hkv}_{d}", 600 + hq + hkv + d, seq, hq, hkv, d, 16)
    _check(w, (0, 256, 512), f"rows hq={hq} hkv={hkv} D={d}")


EDGES = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513]


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (12, 4, 256), (16, 8, 128), (8, 2, 256)])
def test_chunk_and_page_edges(hq, hkv, d, bs):
    """Key counts on and next to chunk (2/4/8 keys), page and partition edges."""
    w = _case(f"rows_edges_{hq}_{hkv}_{d}_{bs}", 700 + hq + d + bs, EDGES, hq, hkv, d, bs)
    _check(w, (0, 256, 512), f"rows edges hq={hq} hkv={hkv} D={d} bs={bs}")


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (12, 4, 256), (16, 8, 128)])
def test_sliding_window(hq, hkv, d):
    """Unsplit ranges of 9,000 and 5,000 keys and 8,192-key partitions: each
    wave's chunks outrun one 64-entry block-table window."""
    w = _case(f"rows_slide_{hq}_{hkv}_{d}", 800 + hq + d, [9000, 5000, 37], hq, hkv, d, 16)
    _check(w, (0, 8192), f"rows sliding window hq={hq} hkv={hkv} D={d}")


@pytest.mark.parametrize("scale", [1.0, 8.0])
def test_sinks(scale):
    """Sinks in the kernel's own finish (unsplit) and in the reduce (split)."""
    rng = np.random.default_rng(31)
    w = _case("rows_sinks", 901, rng.integers(1, 3000, size=6), 32, 8, 128, 16)
    g = torch.Generator().manual_seed(5)
    w = dataclasses.replace(w, sinks=(torch.randn(w.num_q_heads, generator=g) * scale).float())
    _check(w, (0, 512), f"rows sinks x{scale}")


def test_empty_and_mixed_rows():
    """Requests with no query token next to decode rows: only rows with a
    token are written, the others keep their (absent) output."""
    seq = [300, 50, 1, 700, 9, 1024]
    w = W.build("rows_mixed", seed=77, q_lens=[1, 0, 1, 1, 0, 1], seq_lens=seq, num_q_heads=32,
                num_kv_heads=8, head_dim=128, block_size=16, num_blocks=_pool(seq, 16),
                dtype=torch.bfloat16)
    _check(w, (0, 256), "rows with empty requests")


def test_auto_choice(monkeypatch):
    """Default mode: the whole-row kernel for a launch of at least 128
    (request, partition) items, the per-head kernel below that."""
    import paged_varlen_attention_amd as pa
    monkeypatch.setenv("PA_DECODE_ROWS", "1")
    rng = np.random.default_rng(3)
    big = _case("rows_auto_big", 41, rng.integers(1500, 2048, size=32), 32, 8, 128, 16)
    small = _case("rows_auto_small", 42, rng.integers(100, 600, size=4), 32, 8, 128, 16)
    for w, rows in ((big, True), (small, False)):
        ref = oracle.run_workload(w)
        b = to_device(w)
        out = run_gpu(b, 512, reduce=False)
        rec = pa.last_dispatch()
        assert (rec["grid"][0] == w.num_seqs) == rows, rec
        out = run_gpu(b, 512)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"auto rows={rows}")
    monkeypatch.setenv("PA_DECODE_ROWS", "0")
    b = to_device(big)
    run_gpu(b, 512, reduce=False)
    assert pa.last_dispatch()["grid"][0] == big.num_kv_heads
    torch.cuda.synchronize()

"""GPU parity of the MFMA decode kernel's own cases: every group size (the
group's heads are the columns of a 16-wide MFMA block, zero past the group),
key ranges ending on and next to the 16- and 32-key chunk and page edges
(8-bit chunks span up to four 8-token pages), and unsplit or long partitions
whose chunks outrun one block-table window, so the window slides -- over bf16
and 8-bit caches, every head size and page size."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_close, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _pool(seq_lens, bs):
    return int(sum((int(s) + bs - 1) // bs for s in seq_lens)) + 8


def _case(name, seed, seq_lens, hq, hkv, d, bs, kv):
    w = W.build(name, seed=seed, q_lens=[1] * len(seq_lens), seq_lens=seq_lens, num_q_heads=hq,
                num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=_pool(seq_lens, bs),
                dtype=torch.bfloat16)
    return pins.fp8_case(w, seed=seed) if kv == "fp8" else w


def _check(w, Ps, what):
    ref = oracle.run_workload(w)
    b = to_device(w)
    for P in Ps:
        out = run_gpu(b, P)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, f"{what} P={P}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_group(group, kv):
    """Groups 1..8 with 2 KV heads, D=128, 16-token pages, ragged contexts."""
    rng = np.random.default_rng(100 + group)
    seq = rng.integers(1, 1500, size=6)
    w = _case(f"group{group}_{kv}", 300 + group, seq, 2 * group, 2, 128, 16, kv)
    _check(w, (0, 256, 512), f"group {group} {kv}")


EDGES = [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_chunk_and_page_edges(d, bs, kv):
    """Key counts on and next to chunk (16/32), page (8/16/32) and partition
    (256/512) edges; 8/2 heads."""
    w = _case(f"edges_{d}_{bs}_{kv}", 400 + d + bs, EDGES, 8, 2, d, bs, kv)
    _check(w, (0, 256, 512), f"edges D={d} bs={bs} {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_sliding_window(d, bs, kv):
    """Unsplit ranges of 9,000 and 5,000 keys and 8,192-key partitions: a wave's
    chunks outrun one 64-entry block-table window and the window slides."""
    w = _case(f"slide_{d}_{bs}_{kv}", 500 + d + bs, [9000, 5000, 37], 8, 2, d, bs, kv)
    _check(w, (0, 8192), f"sliding window D={d} bs={bs} {kv}")

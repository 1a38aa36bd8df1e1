"""Shared helpers of the GPU parity tests: move a workload to the GPU, run the
HIP path through the C ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# Tolerances of the parity bar: fp32 max-abs 1e-5; bf16 max-abs 2e-2 and
# relative RMS 5e-3 over the whole tensor (GPU values widened exactly to fp64
# and compared with the unrounded fp64 oracle).
TOL_F32_MAXABS = 1e-5
TOL_BF16_MAXABS = 2e-2
TOL_BF16_RELRMS = 5e-3


@dataclasses.dataclass
class DeviceBatch:
    q: torch.Tensor
    key_cache: torch.Tensor       # kernel-page view
    value_cache: torch.Tensor
    cu_seqlens_q: torch.Tensor
    seq_lens: torch.Tensor
    block_tables: torch.Tensor    # kernel-page view
    max_q_len: int
    max_seq_len: int
    scale: float
    sinks: Optional[torch.Tensor] = None   # float32 [Hq] on the device, or None
    k_scale: Optional[torch.Tensor] = None  # 8-bit caches: float32 [Hkv] on the device
    v_scale: Optional[torch.Tensor] = None


def _cache_to(c: torch.Tensor, device) -> torch.Tensor:
    """8-bit caches travel as their raw uint8 codes (the binding reads uint8
    caches as E4M3)."""
    if c.dtype == torch.float8_e4m3fn:
        c = c.view(torch.uint8)
    return c.to(device)


def to_device(w, device="cuda", write_cache=True) -> DeviceBatch:
    """Copy a workload to the GPU.  A cache-write workload runs
    pa_reshape_and_cache first; a workload with a page ratio > 1 is then viewed
    as kernel pages (cache reshape + pa_expand_block_tables)."""
    import paged_varlen_attention_amd as pa
    kc = _cache_to(w.key_cache, device)
    vc = _cache_to(w.value_cache, device)
    bt = w.block_tables.to(device)
    ks = None if w.k_scale is None else w.k_scale.to(device).float().contiguous()
    vs = None if w.v_scale is None else w.v_scale.to(device).float().contiguous()
    if w.slot_mapping is not None and write_cache:
        pa.reshape_and_cache(w.new_key.to(device), w.new_value.to(device), kc, vc,
                             w.slot_mapping.to(device), k_scale=ks, v_scale=vs)
    if w.kernel_page_ratio > 1:
        r = w.kernel_page_ratio
        nb, bs, hkv, d = kc.shape
        kc = kc.view(nb * r, bs // r, hkv, d)
        vc = vc.view(nb * r, bs // r, hkv, d)
        bt = pa.expand_block_tables(bt, r)
    return DeviceBatch(q=w.q.to(device), key_cache=kc, value_cache=vc,
                       cu_seqlens_q=w.cu_seqlens_q.to(device), seq_lens=w.seq_lens.to(device),
                       block_tables=bt, max_q_len=w.max_q_len, max_seq_len=w.max_seq_len,
                       scale=w.scale,
                       sinks=None if w.sinks is None else w.sinks.to(device).float().contiguous(),
                       k_scale=ks, v_scale=vs)


def run_gpu(b: DeviceBatch, partition_size=0, out=None, partials=None, reduce=True):
    import paged_varlen_attention_amd as pa
    return pa.varlen_attention(b.q, b.key_cache, b.value_cache, b.cu_seqlens_q, b.seq_lens,
                               b.block_tables, max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                               scale=b.scale, partition_size=partition_size, out=out,
                               partials=partials, reduce=reduce, sinks=b.sinks,
                               k_scale=b.k_scale, v_scale=b.v_scale)


def errors(gpu: torch.Tensor, ref: torch.Tensor):
    g = gpu.detach().to("cpu").double()
    ref = ref.double()
    diff = g - ref
    max_abs = float(diff.abs().max()) if diff.numel() else 0.0
    rel_rms = float(diff.norm() / ref.norm().clamp_min(1e-300)) if diff.numel() else 0.0
    finite = bool(torch.isfinite(g).all())
    return max_abs, rel_rms, finite


def assert_close(gpu: torch.Tensor, ref: torch.Tensor, dtype: torch.dtype, what: str = ""):
    max_abs, rel_rms, finite = errors(gpu, ref)
    assert finite, f"{what}: non-finite values in the GPU result"
    if dtype == torch.float32:
        assert max_abs <= TOL_F32_MAXABS, f"{what}: max-abs {max_abs:.3e} > {TOL_F32_MAXABS}"
    else:
        assert max_abs <= TOL_BF16_MAXABS, f"{what}: max-abs {max_abs:.3e} > {TOL_BF16_MAXABS}"
        assert rel_rms <= TOL_BF16_RELRMS, f"{what}: rel-RMS {rel_rms:.3e} > {TOL_BF16_RELRMS}"
    return max_abs, rel_rms


def sample_rows(w, n, seed):
    """(token, head) pairs: every request's last token, plus random rows."""
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens_q.numpy()
    rows = set()
    for r in range(w.num_seqs):
        if cu[r + 1] > cu[r]:
            rows.add((int(cu[r + 1] - 1), int(rng.integers(w.num_q_heads))))
            rows.add((int(cu[r]), int(rng.integers(w.num_q_heads))))
    while len(rows) < n:
        rows.add((int(rng.integers(w.total_q)), int(rng.integers(w.num_q_heads))))
    return sorted(rows)

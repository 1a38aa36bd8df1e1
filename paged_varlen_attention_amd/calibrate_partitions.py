"""Calibrate the decode partition policy on this GPU.

    python -m paged_varlen_attention_amd.calibrate_partitions

Times pa_varlen_attention + pa_split_kv_reduce captured as one HIP graph per
KV-pool copy (replays bracketed by HIP events; two copies alternate so pages
are not reused from the last-level cache) for every
partition size on synthetic decode batches generated on the device -- 1 to
256 requests, 1K to 64K keys (uniform in [L/2, L]), two head shapes -- and
prints one JSON line per batch with the time of each partition size, the
policy's pick and the fastest size.  Nothing here is used by the library.
"""
import itertools
import json

import torch

import paged_varlen_attention_amd as pa

dev = 'cuda'


def make(B, L, hq, hkv, d, jitter=True):
    bs = 16
    g = torch.Generator(device='cpu').manual_seed(B * 7 + L)
    if jitter:
        sl = torch.randint(max(1, L // 2), L + 1, (B,), generator=g).to(torch.int32)
    else:
        sl = torch.full((B,), L, dtype=torch.int32)
    pages = ((sl + bs - 1) // bs)
    nb = int(pages.sum()) + 8
    perm = torch.randperm(nb, generator=g).to(torch.int32)
    mb = int(pages.max())
    bt = torch.full((B, mb), -1, dtype=torch.int32)
    o = 0
    for r in range(B):
        n = int(pages[r]); bt[r, :n] = perm[o:o + n]; o += n
    q = torch.randn(B, hq, d, device=dev).to(torch.bfloat16)
    pools = []
    for _ in range(2):
        kc = torch.randn(nb, bs, hkv, d, device=dev).to(torch.bfloat16)
        vc = torch.randn(nb, bs, hkv, d, device=dev).to(torch.bfloat16)
        pools.append((kc, vc))
    cu = torch.arange(B + 1, dtype=torch.int32)
    return q, pools, cu.to(dev), sl.to(dev), bt.to(dev), int(sl.max()), sl


def timed(q, pools, cu, sl, bt, msl, P, reps=20):
    """Median time (us) of one graph replay of attention (+ reduce when P > 0)."""
    out = torch.empty_like(q)
    parts = pa.alloc_partials(q.shape[0], q.shape[1], q.shape[2], pa.max_partitions(msl, P), dev) if P else None

    def step(i):
        kc, vc = pools[i % 2]
        pa.varlen_attention(q, kc, vc, cu, sl, bt, max_q_len=1, max_seq_len=msl, scale=0.1,
                            partition_size=P, out=out, partials=parts)
    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(3):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    evs = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graphs[i % 2].replay()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2] * 1e3


def main():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (hq, hkv, d) in ((32, 8, 128), (24, 4, 256)):
        for B, L in itertools.product((1, 4, 16, 64, 256), (1024, 4096, 16384, 65536)):
            if B * L * hkv * d * 2 * 2 * 2 > 24e9:
                continue
            q, pools, cu, sl, bt, msl, slh = make(B, L, hq, hkv, d)
            row = dict(hq=hq, hkv=hkv, d=d, B=B, L=L)
            for P in (0, 256, 512, 1024, 2048, 4096, 8192):
                row[f"P{P}"] = round(timed(q, pools, cu, sl, bt, msl, P), 1)
            row["pick"] = pa.pick_partition_size(slh.tolist(), hkv, cus)
            row["best"] = min((k for k in row if k.startswith("P")), key=lambda k: row[k])
            print(json.dumps(row), flush=True)
            del q, pools
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()

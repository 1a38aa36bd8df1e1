"""CPU tests of the C ABI: the library loads, exports every function that
include/pa.h declares, and rejects bad arguments with the documented status
before anything is enqueued.  Every call below carries at least one invalid
argument, so none of them reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def _lib():
    import paged_varlen_attention_amd as pa
    return pa.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("pa_reshape_and_cache", "pa_varlen_attention", "pa_split_kv_reduce",
              "pa_expand_block_tables", "pa_pick_partition_size", "pa_status_string"):
        assert f in names


def test_library_exports_every_declared_symbol():
    import paged_varlen_attention_amd as pa
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pa_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        getattr(pa.lib, f)  # resolvable through ctypes


def test_status_strings_and_version():
    lib = _lib()
    for s in range(5):
        assert lib.pa_status_string(s)
    assert lib.pa_abi_version() == 300


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: every call below is rejected


def attn_args(**over):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, cu=FAKE, sl=FAKE, bt=FAKE, num_seqs=2,
             total_q=2, max_q_len=1, max_seq_len=50, max_blocks=4, hq=4, hkv=1, d=64, nb=8,
             bs=16, scale=0.125, sinks=None, dtype=0, kv_dtype=None, ks=None, vs=None, P=0,
             tmp=None, ml=None, es=None, mp=0, stream=None)
    a.update(over)
    if a["kv_dtype"] is None:
        a["kv_dtype"] = a["dtype"]
    return [a[k] for k in ("out", "q", "kc", "vc", "cu", "sl", "bt", "num_seqs", "total_q",
                           "max_q_len", "max_seq_len", "max_blocks", "hq", "hkv", "d", "nb", "bs",
                           "scale", "sinks", "dtype", "kv_dtype", "ks", "vs", "P", "tmp", "ml",
                           "es", "mp", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), 2), (dict(d=96), 2), (dict(bs=12), 2), (dict(bs=64), 2),
    (dict(hq=5, hkv=2), 1), (dict(hq=32, hkv=2), 2), (dict(P=128), 2), (dict(P=384), 2),
    (dict(P=8192 + 256), 2), (dict(num_seqs=-1), 1),
    (dict(hq=0), 1), (dict(nb=0), 1), (dict(out=None), 1), (dict(q=None), 1), (dict(bt=None), 1),
    (dict(cu=None), 1), (dict(max_q_len=0), 1), (dict(max_seq_len=0), 1),
    (dict(max_blocks=3), 1), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(q=ctypes.c_void_p(0x100004)), 1), (dict(kc=ctypes.c_void_p(0x100008)), 1),
    (dict(P=512), 3), (dict(P=256, tmp=FAKE, ml=FAKE, es=FAKE, mp=0), 3),
    (dict(P=256, max_seq_len=600, max_blocks=40, tmp=FAKE, ml=FAKE, es=FAKE, mp=2), 3),
    (dict(P=256, tmp=FAKE, ml=None, es=FAKE, mp=4), 3),
    (dict(num_seqs=70000), 2), (dict(sinks=ctypes.c_void_p(0x100002)), 1),
    # 8-bit caches: bf16 queries only, both scales required and 4-byte aligned,
    # scales refused for caches of the query dtype, unknown cache types refused
    (dict(kv_dtype=2, ks=FAKE, vs=FAKE), 2), (dict(dtype=1, kv_dtype=2, ks=FAKE), 1),
    (dict(dtype=1, kv_dtype=2, vs=FAKE), 1),
    (dict(dtype=1, kv_dtype=2, ks=ctypes.c_void_p(0x100002), vs=FAKE), 1),
    (dict(dtype=1, ks=FAKE, vs=FAKE), 1), (dict(dtype=1, kv_dtype=0), 2),
    (dict(dtype=1, kv_dtype=5), 2), (dict(dtype=1, kv_dtype=2, ks=FAKE, vs=FAKE, d=96), 2),
    (dict(dtype=1, kv_dtype=2, ks=FAKE, vs=FAKE, hq=36, hkv=4), 2),
    (dict(dtype=1, kv_dtype=2, ks=FAKE, vs=FAKE, P=512), 3),
])
def test_varlen_attention_rejects(over, status):
    assert _lib().pa_varlen_attention(*attn_args(**over)) == status


def test_varlen_attention_empty_batch_is_ok_without_pointers():
    args = attn_args(total_q=0, out=None, q=None)
    assert _lib().pa_varlen_attention(*args) == 0


@pytest.mark.parametrize("over,status", [
    (dict(dtype=3), 2), (dict(T=-1), 1), (dict(hkv=0), 1), (dict(key=None), 1),
    (dict(slots=None), 1), (dict(d=3), 2), (dict(bs=0), 1), (dict(nb=0), 1),
    (dict(kc=ctypes.c_void_p(0x100002)), 1),
    # 8-bit caches: scales required, refused for plain caches; rows of 16-byte
    # multiples with head_dim a multiple of 16
    (dict(kv_dtype=2), 1), (dict(kv_dtype=2, ks=FAKE), 1), (dict(ks=FAKE, vs=FAKE), 1),
    (dict(kv_dtype=0), 2), (dict(kv_dtype=2, ks=FAKE, vs=FAKE, d=8), 2),
    (dict(kv_dtype=2, ks=FAKE, vs=FAKE, d=24, hkv=2), 2),
    (dict(kv_dtype=2, ks=FAKE, vs=FAKE, key=None), 1),
    (dict(kv_dtype=2, ks=ctypes.c_void_p(0x100001), vs=FAKE), 1),
])
def test_reshape_and_cache_rejects(over, status):
    a = dict(key=FAKE, value=FAKE, kc=FAKE, vc=FAKE, slots=FAKE, T=4, hkv=1, d=64, nb=2, bs=16,
             dtype=1, kv_dtype=None, ks=None, vs=None, stream=None)
    a.update(over)
    if a["kv_dtype"] is None:
        a["kv_dtype"] = a["dtype"]
    args = [a[k] for k in ("key", "value", "kc", "vc", "slots", "T", "hkv", "d", "nb", "bs",
                           "dtype", "kv_dtype", "ks", "vs", "stream")]
    assert _lib().pa_reshape_and_cache(*args) == status


def test_reshape_and_cache_zero_tokens_ok():
    lib = _lib()
    assert lib.pa_reshape_and_cache(None, None, None, None, None, 0, 1, 64, 2, 16, 1, 1, None,
                                    None, None) == 0
    assert lib.pa_reshape_and_cache(None, None, None, None, None, 0, 1, 64, 2, 16, 1, 2, FAKE,
                                    FAKE, None) == 0


@pytest.mark.parametrize("over,status", [
    (dict(dtype=9), 2), (dict(d=48), 2), (dict(P=0), 2), (dict(P=300), 2), (dict(P=8448), 2),
    (dict(out=None), 1),
    (dict(tmp=None), 3), (dict(mp=0), 3), (dict(hq=0), 1), (dict(out=ctypes.c_void_p(0x100006)), 1),
    (dict(sinks=ctypes.c_void_p(0x100001)), 1),
])
def test_split_kv_reduce_rejects(over, status):
    a = dict(out=FAKE, tmp=FAKE, ml=FAKE, es=FAKE, cu=FAKE, sl=FAKE, B=2, TQ=2, hq=4, d=64,
             sinks=None, P=256, mp=2, dtype=1, stream=None)
    a.update(over)
    args = [a[k] for k in ("out", "tmp", "ml", "es", "cu", "sl", "B", "TQ", "hq", "d", "sinks", "P",
                           "mp", "dtype", "stream")]
    assert _lib().pa_split_kv_reduce(*args) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 2, 3, 3, 26, 9), 1),   # dst_stride < src_blocks * ratio
    ((FAKE, FAKE, 2, 3, 3, 27, 0), 1),   # ratio 0
    ((None, FAKE, 2, 3, 3, 27, 9), 1),
    ((FAKE, FAKE, -1, 3, 3, 27, 9), 1),
    ((FAKE, FAKE, 2, 2, 3, 27, 9), 1),   # src_stride < src_blocks
])
def test_expand_block_tables_rejects(args, status):
    assert _lib().pa_expand_block_tables(*args, None) == status


def test_partials_bytes():
    lib = _lib()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.pa_partials_bytes(32, 32, 128, 8, ctypes.byref(a), ctypes.byref(b)) == 0
    assert a.value == 32 * 32 * 8 * 128 * 4 and b.value == 32 * 32 * 8 * 4
    assert lib.pa_partials_bytes(-1, 32, 128, 8, ctypes.byref(a), ctypes.byref(b)) == 1


def test_partition_policy():
    """Host-only policy with an explicit CU count (no device query): budget
    256 * 9/16 = 144 workgroups, items no longer than 3/2 of the mean; the
    whole-row kernel takes 32/8/128 bf16 batches with >= 128 (request,
    partition) items, the per-head kernel the rest (workgroups x Hkv)."""
    import workloads as W
    import paged_varlen_attention_amd as pa
    cus = 256
    pick = lambda sl, hq, hkv, d, **kw: pa.pick_partition_size(sl, hq, hkv, d, num_cus=cus, **kw)  # noqa: E731
    assert pick([100] * 4, 32, 8, 128) == 0                  # nothing longer than 256
    # the GQA decode batch: 512 routes 32 x 8 items to the whole-row kernel,
    # 156 of them non-empty (>= 144), the longest 512 <= 1.5 x 463 (mean);
    # 1024 gives 86 and larger sizes route to the per-head kernel (tried later)
    sl2 = W.gqa_decode_bf16().seq_lens.tolist()
    assert sum(-(-s // 512) for s in sl2) == 156 and sum(-(-s // 1024) for s in sl2) == 86
    assert pick(sl2, 32, 8, 128) == 512
    # the 32K-token decode (24/4/256: per-head kernel only): 2048 gives
    # 4 x 16 x 4 = 256 workgroups; 4096 gives 128 < 144
    assert pick([32768] * 4, 24, 4, 256) == 2048
    # 256 requests of 4096 keys: unsplit is 256 whole-row workgroups, balanced
    assert pick([4096] * 256, 32, 8, 128) == 0
    # one long request among short ones: no size both fills and balances
    assert pick([512] * 31 + [8000], 32, 8, 128) == 256
    # 8-bit caches: 16 x 4000 keys -> the whole-row 8-bit kernel needs 256 items (512 gives
    # 16 x 8 = 128), so the per-head kernel at 2048 (16 x 2 x 8 = 256 workgroups)
    assert pick([4000] * 16, 32, 8, 128, kv8=True) == 2048
    # the GQA batch over 8-bit caches: 512 routes 32 x 8 = 256 items to the whole-row 8-bit
    # kernel (156 non-empty >= 144)
    assert pick(sl2, 32, 8, 128, kv8=True) == 512
    # 24/4/256 (group 6) has no 8-bit whole-row form: per-head, as over bf16 caches
    assert pick([32768] * 4, 24, 4, 256, kv8=True) == 2048
    with pytest.raises(ValueError):
        pick([-5], 8, 1, 128)
    with pytest.raises(ValueError):
        pick([1000], 12, 8, 128)                             # 12 % 8 != 0


def test_dispatch_record_and_no_split_switch(monkeypatch):
    """The record of the last call on this thread, and PA_NO_SPLIT (checked on
    calls that enqueue nothing: an empty batch and a rejected call)."""
    import paged_varlen_attention_amd as pa
    lib = _lib()
    assert lib.pa_last_dispatch(None) == 1
    monkeypatch.delenv("PA_NO_SPLIT", raising=False)
    assert lib.pa_varlen_attention(*attn_args(total_q=0, out=None, q=None, P=512)) == 0
    rec = pa.last_dispatch()
    assert rec["path"] == "none" and rec["status"] == 0 and rec["partition_size"] == 512
    assert not rec["split_disabled"] and rec["grid"] == (0, 0, 0)
    monkeypatch.setenv("PA_NO_SPLIT", "1")
    assert lib.pa_varlen_attention(*attn_args(total_q=0, out=None, q=None, P=512)) == 0
    rec = pa.last_dispatch()
    assert rec["partition_size"] == 0 and rec["split_disabled"]
    # with the split off, the partials are not required
    assert lib.pa_varlen_attention(*attn_args(total_q=0, out=None, q=None, P=512, tmp=None)) == 0
    a = dict(out=FAKE, tmp=FAKE, ml=FAKE, es=FAKE, cu=FAKE, sl=FAKE, B=2, TQ=2, hq=4, d=64,
             sinks=None, P=256, mp=2, dtype=1, stream=None)
    args = [a[k] for k in ("out", "tmp", "ml", "es", "cu", "sl", "B", "TQ", "hq", "d", "sinks", "P",
                           "mp", "dtype", "stream")]
    assert lib.pa_split_kv_reduce(*args) == 0       # skipped: nothing is enqueued
    assert pa.last_dispatch()["path"] == "reduce_skipped"
    monkeypatch.setenv("PA_NO_SPLIT", "0")
    assert lib.pa_varlen_attention(*attn_args(dtype=7)) == 2
    rec = pa.last_dispatch()
    assert rec["path"] == "none" and rec["status"] == 2


@pytest.mark.parametrize("over,status", [
    (dict(n=-1), 1), (dict(bb=0), 1), (dict(bb=24), 1), (dict(ns=-1), 1), (dict(nd=-1), 1),
    (dict(n=0), 0), (dict(dk=None), 1), (dict(pairs=None), 1), (dict(sk=ctypes.c_void_p(0x100008)), 1),
])
def test_copy_blocks_rejects(over, status):
    """Checks that return before any pointer is looked at or work enqueued."""
    a = dict(dk=FAKE, dv=FAKE, sk=FAKE, sv=FAKE, pairs=FAKE, n=2, bb=32768, ns=4, nd=4, stream=None)
    a.update(over)
    args = [a[k] for k in ("dk", "dv", "sk", "sv", "pairs", "n", "bb", "ns", "nd", "stream")]
    assert _lib().pa_copy_blocks(*args) == status

"""fp64 CPU oracle for paged variable-length attention -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does: it
shares no code with the HIP path, and a product call that reached this code
would be a CPU fallback.

The arithmetic lives in ``pa_oracle.c`` (plain C, fp64, compiled with gcc -O2,
no fast-math).  This wrapper only marshals host tensors into it.  Every
function cites, in the C header, the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_lib = None

F32, BF16, FP8_E4M3 = 0, 1, 2


def build(force: bool = False, out_path: Optional[str] = None, src_path: Optional[str] = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE).  Returns the .so path."""
    out_path = out_path or _LIB_PATH
    src_path = src_path or _SRC
    if force or not os.path.exists(out_path) or os.path.getmtime(out_path) < os.path.getmtime(src_path):
        tmp = out_path + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-I", _HERE, src_path, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out_path)
    return out_path


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        _lib = _declare(ctypes.CDLL(build()))
    return _lib


def _declare(lib):
    P, I, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    lib.pa_ref_num_threads.restype = ctypes.c_int
    lib.pa_ref_set_num_threads.argtypes = [ctypes.c_int]
    lib.pa_ref_set_num_threads.restype = None
    lib.pa_ref_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
    lib.pa_ref_expand_block_tables.argtypes = [P, P, I, I, I, I, I]
    lib.pa_ref_copy_blocks.argtypes = [P, P, P, P, P, I, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.pa_ref_attention.argtypes = [P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, D, I,
                                     I, P, P, P]
    lib.pa_ref_attention_partials.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                              D, I, I, P, P, I, I]
    lib.pa_ref_reshape_and_cache_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P]
    lib.pa_ref_e4m3_values.argtypes = [P, P, ctypes.c_int64]
    lib.pa_ref_e4m3_encode_f32.argtypes = [P, P, ctypes.c_int64]
    lib.pa_ref_copy_blocks.restype = ctypes.c_int
    lib.pa_ref_split_reduce.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
    for f in ("pa_ref_reshape_and_cache", "pa_ref_expand_block_tables", "pa_ref_attention",
              "pa_ref_attention_partials", "pa_ref_split_reduce", "pa_ref_reshape_and_cache_fp8",
              "pa_ref_e4m3_values", "pa_ref_e4m3_encode_f32"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return ctypes.c_void_p(t.ctypes.data)
    assert t.device.type == "cpu" and t.is_contiguous()
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"oracle supports float32 and bfloat16, not {dt}")


def _kv_code(cache: torch.Tensor, q_dtype: torch.dtype) -> int:
    """Element type of a cache: 8-bit caches (float8_e4m3fn or raw uint8 codes)
    are E4M3; otherwise the cache shares the query dtype."""
    if cache.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3
    if cache.dtype != q_dtype:
        raise TypeError(f"cache dtype {cache.dtype} differs from query dtype {q_dtype}")
    return _dtype_code(cache.dtype)


def _scales(k_scale, v_scale, hkv, kv_code):
    if kv_code != FP8_E4M3:
        if k_scale is not None or v_scale is not None:
            raise ValueError("k_scale/v_scale apply to 8-bit caches only")
        return None, None
    if k_scale is None or v_scale is None:
        raise ValueError("8-bit caches need k_scale and v_scale")
    ks = torch.as_tensor(k_scale, dtype=torch.float32).contiguous()
    vs = torch.as_tensor(v_scale, dtype=torch.float32).contiguous()
    if ks.shape != (hkv,) or vs.shape != (hkv,):
        raise ValueError("k_scale and v_scale must be float32 [num_kv_heads]")
    return ks, vs


def e4m3_values(codes, lib=None) -> torch.Tensor:
    """float64 values of E4M3 codes (uint8 or float8_e4m3fn tensor of any shape)."""
    lib = lib or _load()
    c = torch.as_tensor(codes)
    c = (c.view(torch.uint8) if c.dtype == torch.float8_e4m3fn else c.to(torch.uint8)).contiguous()
    out = torch.empty(c.shape, dtype=torch.float64)
    if lib.pa_ref_e4m3_values(_ptr(out), _ptr(c), c.numel()):
        raise ValueError("oracle e4m3_values: bad arguments")
    return out


def e4m3_encode(y, lib=None) -> torch.Tensor:
    """E4M3 codes (uint8) of float32 values: nearest, ties to even, saturating."""
    lib = lib or _load()
    y = torch.as_tensor(y, dtype=torch.float32).contiguous()
    out = torch.empty(y.shape, dtype=torch.uint8)
    if lib.pa_ref_e4m3_encode_f32(_ptr(out), _ptr(y), y.numel()):
        raise ValueError("oracle e4m3_encode: bad arguments")
    return out


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                          lib=None) -> None:
    """In place on host tensors: 8-bit caches (uint8 or float8_e4m3fn) receive
    the E4M3 codes of key / k_scale[g] and value / v_scale[g]."""
    lib = lib or _load()
    T, hkv, d = key.shape
    nb, bs = key_cache.shape[:2]
    ks, vs = _scales(k_scale, v_scale, hkv, FP8_E4M3)
    kc = key_cache.view(torch.uint8) if key_cache.dtype == torch.float8_e4m3fn else key_cache
    vc = value_cache.view(torch.uint8) if value_cache.dtype == torch.float8_e4m3fn else value_cache
    if kc.dtype != torch.uint8 or vc.dtype != torch.uint8:
        raise TypeError("8-bit caches must be uint8 or float8_e4m3fn")
    rc = lib.pa_ref_reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(kc), _ptr(vc),
                                          _ptr(slot_mapping), T, hkv, d, nb, bs,
                                          _dtype_code(key.dtype), _ptr(ks), _ptr(vs))
    if rc:
        raise ValueError("oracle reshape_and_cache_fp8: bad arguments")


def quantize_cache(cache: torch.Tensor, scale, lib=None) -> torch.Tensor:
    """A whole [num_blocks, block_size, Hkv, D] cache quantised slot by slot with
    the cache write above (NaN slots stay NaN codes); returns float8_e4m3fn."""
    nb, bs, hkv, d = cache.shape
    rows = cache.reshape(nb * bs, hkv, d)
    # slots that are NaN throughout (unused pool slots) store the NaN code the
    # write gives NaN; only the others go through the write
    used = ~torch.isnan(rows.float()).all(dim=2).all(dim=1)
    slots = torch.nonzero(used).flatten().to(torch.int64).contiguous()
    src = rows[slots].contiguous()
    out = torch.full((nb, bs, hkv, d), 0x7F, dtype=torch.uint8)
    spare = torch.empty_like(out)
    reshape_and_cache_fp8(src, src, out, spare, slots, scale, scale, lib=lib)
    return out.view(torch.float8_e4m3fn)


def num_threads(lib=None) -> int:
    return int((lib or _load()).pa_ref_num_threads())


def set_num_threads(n: int, lib=None) -> None:
    """Threads of the oracle's row loop (timing only: each row's arithmetic is
    the same whatever the count)."""
    (lib or _load()).pa_ref_set_num_threads(int(n))


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, lib=None) -> None:
    """In place on host tensors: caches[slot // bs, slot % bs] = rows; slot < 0 skipped."""
    lib = lib or _load()
    T, hkv, d = key.shape
    nb, bs = key_cache.shape[:2]
    rc = lib.pa_ref_reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                      _ptr(slot_mapping), T, hkv, d, nb, bs, _dtype_code(key.dtype))
    if rc:
        raise ValueError("oracle reshape_and_cache: bad arguments")


def copy_blocks(dst_key, dst_value, src_key, src_value, pairs, lib=None) -> None:
    """In place on host tensors: dst[pairs[i,1]] = src[pairs[i,0]] for K and V
    (whole blocks), pairs int64 [n, 2]; out-of-pool pairs skipped."""
    lib = lib or _load()
    pairs = torch.as_tensor(pairs, dtype=torch.int64).contiguous()
    nbs, nbd = src_key.shape[0], dst_key.shape[0]
    block_bytes = src_key[0].numel() * src_key.element_size() if nbs else 0
    if dst_key[0].numel() * dst_key.element_size() != block_bytes:
        raise ValueError("block sizes differ")
    rc = lib.pa_ref_copy_blocks(_ptr(dst_key), _ptr(dst_value), _ptr(src_key), _ptr(src_value),
                                _ptr(pairs), int(pairs.shape[0]), block_bytes, nbs, nbd)
    if rc:
        raise ValueError("oracle copy_blocks: bad arguments")


def expand_block_tables(block_tables: torch.Tensor, ratio: int, lib=None) -> torch.Tensor:
    lib = lib or _load()
    B, nb = block_tables.shape
    dst = torch.empty((B, nb * ratio), dtype=torch.int32)
    rc = lib.pa_ref_expand_block_tables(_ptr(dst), _ptr(block_tables), B, nb, nb, nb * ratio, ratio)
    if rc:
        raise ValueError("oracle expand_block_tables: bad arguments")
    return dst


def _raw(cache: torch.Tensor) -> torch.Tensor:
    return cache.view(torch.uint8) if cache.dtype == torch.float8_e4m3fn else cache


def _common(w_q, key_cache, cu, seq_lens, block_tables):
    TQ, hq, d = w_q.shape
    nb, bs, hkv, _ = key_cache.shape
    return TQ, hq, d, nb, bs, hkv, int(seq_lens.numel()), int(block_tables.shape[1])


def _sinks(sinks, hq):
    if sinks is None:
        return None
    sinks = torch.as_tensor(sinks, dtype=torch.float32).contiguous()
    if sinks.shape != (hq,):
        raise ValueError("sinks must be float32 [num_q_heads]")
    return sinks


def attention(q, key_cache, value_cache, cu_seqlens_q, seq_lens, block_tables, scale: float,
              rows: Optional[Sequence[Sequence[int]]] = None, sinks=None, k_scale=None,
              v_scale=None, lib=None) -> torch.Tensor:
    """fp64 masked softmax(QK^T*scale)V through the block tables.
    rows=None -> [total_q, Hq, D]; rows=[(t, h), ...] -> [n, D].
    sinks: optional float32 [Hq] sink logits (one more softmax term, no value).
    8-bit caches (float8_e4m3fn / uint8) need k_scale and v_scale [Hkv]."""
    lib = lib or _load()
    TQ, hq, d, nb, bs, hkv, B, mb = _common(q, key_cache, cu_seqlens_q, seq_lens, block_tables)
    if rows is None:
        out = torch.empty((TQ, hq, d), dtype=torch.float64)
        tok = head = None
        n = 0
    else:
        rows = np.asarray(rows, dtype=np.int32).reshape(-1, 2)
        tok = np.ascontiguousarray(rows[:, 0])
        head = np.ascontiguousarray(rows[:, 1])
        n = len(rows)
        out = torch.empty((n, d), dtype=torch.float64)
    sk = _sinks(sinks, hq)  # kept alive across the call
    kv = _kv_code(key_cache, q.dtype)
    ks, vs = _scales(k_scale, v_scale, hkv, kv)
    rc = lib.pa_ref_attention(_ptr(out), _ptr(tok), _ptr(head), n, _ptr(q), _ptr(_raw(key_cache)),
                              _ptr(_raw(value_cache)), _ptr(cu_seqlens_q), _ptr(seq_lens),
                              _ptr(block_tables), B, TQ, mb, hq, hkv, d, nb, bs, float(scale),
                              _dtype_code(q.dtype), kv, _ptr(ks), _ptr(vs), _ptr(sk))
    if rc:
        raise ValueError("oracle attention: bad arguments")
    return out


def max_partitions(max_seq_len: int, partition_size: int) -> int:
    return (max_seq_len + partition_size - 1) // partition_size


def attention_partials(q, key_cache, value_cache, cu_seqlens_q, seq_lens, block_tables,
                       scale: float, partition_size: int, max_parts: Optional[int] = None,
                       k_scale=None, v_scale=None, lib=None):
    """Split-KV partials (o, m, l) in the log2-space contract; untouched entries are NaN."""
    lib = lib or _load()
    TQ, hq, d, nb, bs, hkv, B, mb = _common(q, key_cache, cu_seqlens_q, seq_lens, block_tables)
    mp = max_parts or max_partitions(int(seq_lens.max()), partition_size)
    o = torch.full((TQ, hq, mp, d), float("nan"), dtype=torch.float64)
    m = torch.full((TQ, hq, mp), float("nan"), dtype=torch.float64)
    l = torch.full((TQ, hq, mp), float("nan"), dtype=torch.float64)
    kv = _kv_code(key_cache, q.dtype)
    ks, vs = _scales(k_scale, v_scale, hkv, kv)
    rc = lib.pa_ref_attention_partials(_ptr(o), _ptr(m), _ptr(l), _ptr(q), _ptr(_raw(key_cache)),
                                       _ptr(_raw(value_cache)), _ptr(cu_seqlens_q), _ptr(seq_lens),
                                       _ptr(block_tables), B, TQ, mb, hq, hkv, d, nb, bs,
                                       float(scale), _dtype_code(q.dtype), kv, _ptr(ks), _ptr(vs),
                                       partition_size, mp)
    if rc:
        raise ValueError("oracle attention_partials: bad arguments")
    return o, m, l


def split_reduce(o, m, l, cu_seqlens_q, seq_lens, partition_size: int, sinks=None,
                 lib=None) -> torch.Tensor:
    lib = lib or _load()
    TQ, hq, mp, d = o.shape
    out = torch.empty((TQ, hq, d), dtype=torch.float64)
    sk = _sinks(sinks, hq)  # kept alive across the call
    rc = lib.pa_ref_split_reduce(_ptr(out), _ptr(o), _ptr(m), _ptr(l), _ptr(cu_seqlens_q),
                                 _ptr(seq_lens), int(seq_lens.numel()), TQ, hq, d, partition_size, mp,
                                 _ptr(sk))
    if rc:
        raise ValueError("oracle split_reduce: bad arguments")
    return out


def run_workload(w, rows=None, lib=None) -> torch.Tensor:
    """Oracle result for a ``workloads.Workload``: applies its cache write first
    (on copies of the caches) when it has one, then attention on the stored
    block size."""
    kc, vc = w.key_cache, w.value_cache
    ks, vs = getattr(w, "k_scale", None), getattr(w, "v_scale", None)
    if w.slot_mapping is not None:
        kc, vc = kc.clone(), vc.clone()
        if ks is not None:
            reshape_and_cache_fp8(w.new_key, w.new_value, kc, vc, w.slot_mapping, ks, vs, lib=lib)
        else:
            reshape_and_cache(w.new_key, w.new_value, kc, vc, w.slot_mapping, lib=lib)
    return attention(w.q, kc, vc, w.cu_seqlens_q, w.seq_lens, w.block_tables, w.scale, rows=rows,
                     sinks=getattr(w, "sinks", None), k_scale=ks, v_scale=vs, lib=lib)

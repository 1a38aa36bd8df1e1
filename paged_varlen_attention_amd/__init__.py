"""paged_varlen_attention_amd -- paged variable-length attention on AMD MI355X.

A thin ctypes binding over ``libpa.so`` (C ABI in ``include/pa.h``).  This
layer only checks tensors and marshals pointers: every step of the path runs
in the HIP kernels of the library.  PyTorch supplies device memory and the
current HIP stream.  If the library is missing, importing this package fails
loudly; there is no CPU fallback.

Entry points (same names as the C ABI, without the ``pa_`` prefix):
``reshape_and_cache``, ``expand_block_tables``, ``varlen_attention``,
``split_kv_reduce``, plus ``pick_partition_size`` and ``alloc_partials``.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP = 0, 1, 2, 3, 4


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python paged_varlen_attention_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.pa_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, P, P]
    lib.pa_expand_block_tables.argtypes = [P, P, I, I, I, I, I, P]
    lib.pa_varlen_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, P,
                                        I, I, P, P, I, P, P, P, I, P]
    lib.pa_split_kv_reduce.argtypes = [P, P, P, P, P, P, I, I, I, I, P, I, I, I, P]
    lib.pa_varlen_attention_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I,
                                                F, P, I, I, P, P, I, P]
    lib.pa_pick_partition_size.argtypes = [P, I, I, I, I, I, I, I, I]
    lib.pa_pick_partition_size.restype = ctypes.c_int32
    lib.pa_partials_bytes.argtypes = [I, I, I, I, ctypes.POINTER(ctypes.c_size_t),
                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_last_dispatch.argtypes = [P]
    lib.pa_copy_blocks.argtypes = [P, P, P, P, P, I, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    for f in ("pa_reshape_and_cache", "pa_expand_block_tables", "pa_varlen_attention",
              "pa_varlen_attention_noalloc",
              "pa_split_kv_reduce", "pa_partials_bytes", "pa_abi_version", "pa_last_dispatch",
              "pa_copy_blocks"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


lib = _load()


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(fn, status, lib.pa_status_string(status).decode())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return PA_F32
    if dt == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def _kv_code(cache: torch.Tensor, row_dtype: torch.dtype) -> int:
    """Cache element type: 8-bit caches (float8_e4m3fn, or raw uint8 codes) are
    E4M3; any other cache must have the row dtype."""
    if cache.dtype in (torch.float8_e4m3fn, torch.uint8):
        return PA_FP8_E4M3
    if cache.dtype != row_dtype:
        raise TypeError(f"cache dtype {cache.dtype} differs from {row_dtype}")
    return _dtype_code(cache.dtype)


def _scales(k_scale, v_scale, kv_code: int, hkv: int, dev):
    if kv_code != PA_FP8_E4M3:
        if k_scale is not None or v_scale is not None:
            raise ValueError("k_scale/v_scale apply to 8-bit caches only")
        return ctypes.c_void_p(0), ctypes.c_void_p(0)
    if k_scale is None or v_scale is None:
        raise ValueError("8-bit caches need k_scale and v_scale (float32 [num_kv_heads])")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.shape != (hkv,):
            raise ValueError(f"{n} must be [num_kv_heads]")
    return (_dev(k_scale, "k_scale", torch.float32, dev),
            _dev(v_scale, "v_scale", torch.float32, dev))


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, device=None) -> ctypes.c_void_p:
    """Pointer of a dense device tensor (non-contiguous or negative strides refused)."""
    if t is None:
        return ctypes.c_void_p(0)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (no strides, no negative strides)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Partials(NamedTuple):
    tmp_out: torch.Tensor     # float32 [total_q, Hq, max_parts, D]
    max_logits: torch.Tensor  # float32 [total_q, Hq, max_parts]
    exp_sums: torch.Tensor    # float32 [total_q, Hq, max_parts]

    @property
    def max_parts(self) -> int:
        return int(self.max_logits.shape[2])


def max_partitions(max_seq_len: int, partition_size: int) -> int:
    return max(1, (max_seq_len + partition_size - 1) // partition_size) if partition_size else 0


def alloc_partials(total_q: int, num_q_heads: int, head_dim: int, max_parts: int,
                   device) -> Partials:
    return Partials(
        torch.empty((total_q, num_q_heads, max_parts, head_dim), dtype=torch.float32, device=device),
        torch.empty((total_q, num_q_heads, max_parts), dtype=torch.float32, device=device),
        torch.empty((total_q, num_q_heads, max_parts), dtype=torch.float32, device=device))


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                      k_scale: Optional[torch.Tensor] = None,
                      v_scale: Optional[torch.Tensor] = None) -> None:
    """key/value [T, Hkv, D]; caches [num_blocks, block_size, Hkv, D]; slot_mapping int64 [T].
    8-bit caches (float8_e4m3fn or uint8) store E4M3 codes of row / scale and
    need k_scale and v_scale (float32 [Hkv] on the GPU)."""
    T, hkv, d = key.shape
    nb, bs, chkv, cd = key_cache.shape
    if (chkv, cd) != (hkv, d) or value.shape != key.shape or value_cache.shape != key_cache.shape:
        raise ValueError("reshape_and_cache: shape mismatch")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    if value_cache.dtype != key_cache.dtype:
        raise TypeError("key_cache and value_cache differ in dtype")
    dev = key.device
    kv = _kv_code(key_cache, key.dtype)
    ks, vs = _scales(k_scale, v_scale, kv, hkv, dev)
    st = lib.pa_reshape_and_cache(
        _dev(key, "key", device=dev), _dev(value, "value", key.dtype, dev),
        _dev(key_cache, "key_cache", device=dev), _dev(value_cache, "value_cache", device=dev),
        _dev(slot_mapping, "slot_mapping", torch.int64, dev), T, hkv, d, nb, bs,
        _dtype_code(key.dtype), kv, ks, vs, _stream(dev))
    _check("pa_reshape_and_cache", st)


def _gpu_visible(t: torch.Tensor, name: str) -> ctypes.c_void_p:
    """Pointer of a dense tensor the GPU can address: on the GPU, or pinned host."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type == "cpu" and not t.is_pinned():
        raise ValueError(f"{name} is in pageable host memory: allocate it pinned (pin_memory=True)")
    if t.device.type not in ("cpu", "cuda"):
        raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def copy_blocks(dst_key: torch.Tensor, dst_value: torch.Tensor, src_key: torch.Tensor,
                src_value: torch.Tensor, pairs: torch.Tensor) -> None:
    """dst[pairs[i, 1]] = src[pairs[i, 0]] for K and V (whole blocks, caches
    [num_blocks, ...]); each tensor on the GPU or in pinned host memory.
    pairs: int64 [n, 2] (GPU or pinned).  Out-of-pool pairs are skipped;
    destination ids must be distinct."""
    if src_key.shape[1:] != dst_key.shape[1:] or src_key.dtype != dst_key.dtype:
        raise ValueError("caches differ in block shape or dtype")
    if src_value.shape != src_key.shape or dst_value.shape != dst_key.shape:
        raise ValueError("K and V caches differ")
    if pairs.dtype != torch.int64 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int64 [n, 2]")
    dev = next((t.device for t in (dst_key, src_key, pairs) if t.device.type == "cuda"),
               torch.device("cuda", torch.cuda.current_device()))
    block_bytes = src_key[0].numel() * src_key.element_size() if src_key.shape[0] else 16
    st = lib.pa_copy_blocks(_gpu_visible(dst_key, "dst_key"), _gpu_visible(dst_value, "dst_value"),
                            _gpu_visible(src_key, "src_key"), _gpu_visible(src_value, "src_value"),
                            _gpu_visible(pairs, "pairs"), pairs.shape[0], block_bytes,
                            src_key.shape[0], dst_key.shape[0], _stream(dev))
    _check("pa_copy_blocks", st)


def expand_block_tables(block_tables: torch.Tensor, ratio: int,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Kernel-page view of a block table of ``ratio``-page blocks (int32 on the GPU)."""
    B, nb = block_tables.shape
    if out is None:
        out = torch.empty((B, nb * ratio), dtype=torch.int32, device=block_tables.device)
    st = lib.pa_expand_block_tables(_dev(out, "out", torch.int32),
                                    _dev(block_tables, "block_tables", torch.int32), B, nb, nb,
                                    out.shape[1], ratio, _stream(block_tables.device))
    _check("pa_expand_block_tables", st)
    return out


def varlen_attention(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                     cu_seqlens_q: torch.Tensor, seq_lens: torch.Tensor, block_tables: torch.Tensor,
                     *, max_q_len: int, max_seq_len: int, scale: float, partition_size: int = 0,
                     out: Optional[torch.Tensor] = None, partials: Optional[Partials] = None,
                     reduce: bool = True, sinks: Optional[torch.Tensor] = None,
                     k_scale: Optional[torch.Tensor] = None,
                     v_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged varlen attention; with partition_size > 0 and reduce=True the split
    partials are merged by pa_split_kv_reduce on the same stream.  sinks:
    optional float32 [Hq] attention-sink logits on the same device.  8-bit
    caches (float8_e4m3fn / uint8 E4M3 codes) need k_scale and v_scale
    (float32 [Hkv]) and bf16 queries."""
    TQ, hq, d = q.shape
    nb, bs, hkv, cd = key_cache.shape
    if cd != d or value_cache.shape != key_cache.shape:
        raise ValueError("cache shape mismatch")
    B = seq_lens.shape[0]
    if cu_seqlens_q.shape != (B + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("metadata shape mismatch")
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if partition_size and partials is None:
        partials = alloc_partials(TQ, hq, d, max_partitions(max_seq_len, partition_size), dev)
    tmp = ml = es = None
    mp = 0
    if partials is not None and partition_size:
        tmp, ml, es = partials
        mp = partials.max_parts
    if sinks is not None and sinks.shape != (hq,):
        raise ValueError("sinks must be [num_q_heads]")
    if value_cache.dtype != key_cache.dtype:
        raise TypeError("key_cache and value_cache differ in dtype")
    kv = _kv_code(key_cache, q.dtype)
    ks, vs = _scales(k_scale, v_scale, kv, hkv, dev)
    s = _stream(dev)
    st = lib.pa_varlen_attention(
        _dev(out, "out", q.dtype, dev), _dev(q, "q", device=dev),
        _dev(key_cache, "key_cache", device=dev), _dev(value_cache, "value_cache", device=dev),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev), _dev(seq_lens, "seq_lens", torch.int32, dev),
        _dev(block_tables, "block_tables", torch.int32, dev), B, TQ, int(max_q_len),
        int(max_seq_len), block_tables.shape[1], hq, hkv, d, nb, bs, float(scale),
        _dev(sinks, "sinks", torch.float32, dev),
        _dtype_code(q.dtype), kv, ks, vs, int(partition_size), _dev(tmp, "tmp_out", torch.float32, dev),
        _dev(ml, "max_logits", torch.float32, dev), _dev(es, "exp_sums", torch.float32, dev), mp, s)
    _check("pa_varlen_attention", st)
    if partition_size and reduce:
        split_kv_reduce(out, partials, cu_seqlens_q, seq_lens, partition_size, sinks=sinks)
    return out


# Bytes of device scratch behind varlen_attention_noalloc (one copy per GPU).
NOALLOC_SCRATCH_BYTES = 32 << 20


def varlen_attention_noalloc(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                             cu_seqlens_q: torch.Tensor, seq_lens: torch.Tensor,
                             block_tables: torch.Tensor, out: torch.Tensor, *, max_q_len: int,
                             max_seq_len: int, scale: float, partition_size: int = 0,
                             sinks: Optional[torch.Tensor] = None,
                             k_scale: Optional[torch.Tensor] = None,
                             v_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_varlen_attention_noalloc: attention and (partition_size > 0) the
    split-KV reduce in one call, the partials in the library's static device
    scratch; nothing is allocated, ``out`` (same shape and dtype as q) is the
    caller's.  Calls that overlap on one GPU share that scratch and race."""
    TQ, hq, d = q.shape
    nb, bs, hkv, cd = key_cache.shape
    if cd != d or value_cache.shape != key_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch")
    B = seq_lens.shape[0]
    if cu_seqlens_q.shape != (B + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("metadata shape mismatch")
    if sinks is not None and sinks.shape != (hq,):
        raise ValueError("sinks must be [num_q_heads]")
    if value_cache.dtype != key_cache.dtype:
        raise TypeError("key_cache and value_cache differ in dtype")
    dev = q.device
    kv = _kv_code(key_cache, q.dtype)
    ks, vs = _scales(k_scale, v_scale, kv, hkv, dev)
    st = lib.pa_varlen_attention_noalloc(
        _dev(out, "out", q.dtype, dev), _dev(q, "q", device=dev),
        _dev(key_cache, "key_cache", device=dev), _dev(value_cache, "value_cache", device=dev),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev), _dev(seq_lens, "seq_lens", torch.int32, dev),
        _dev(block_tables, "block_tables", torch.int32, dev), B, TQ, int(max_q_len),
        int(max_seq_len), block_tables.shape[1], hq, hkv, d, nb, bs, float(scale),
        _dev(sinks, "sinks", torch.float32, dev), _dtype_code(q.dtype), kv, ks, vs,
        int(partition_size), _stream(dev))
    _check("pa_varlen_attention_noalloc", st)
    return out


def split_kv_reduce(out: torch.Tensor, partials: Partials, cu_seqlens_q: torch.Tensor,
                    seq_lens: torch.Tensor, partition_size: int,
                    sinks: Optional[torch.Tensor] = None) -> torch.Tensor:
    TQ, hq, d = out.shape
    dev = out.device
    tmp, ml, es = partials
    if tmp.shape[:2] != (TQ, hq) or tmp.shape[3] != d:
        raise ValueError("partials shape mismatch")
    if sinks is not None and sinks.shape != (hq,):
        raise ValueError("sinks must be [num_q_heads]")
    st = lib.pa_split_kv_reduce(
        _dev(out, "out", device=dev), _dev(tmp, "tmp_out", torch.float32, dev),
        _dev(ml, "max_logits", torch.float32, dev), _dev(es, "exp_sums", torch.float32, dev),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev), _dev(seq_lens, "seq_lens", torch.int32, dev),
        seq_lens.shape[0], TQ, hq, d, _dev(sinks, "sinks", torch.float32, dev),
        int(partition_size), partials.max_parts,
        _dtype_code(out.dtype), _stream(dev))
    _check("pa_split_kv_reduce", st)
    return out


class _DispatchInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("status", ctypes.c_int32),
                ("partition_size", ctypes.c_int32), ("split_disabled", ctypes.c_int32),
                ("grid", ctypes.c_int32 * 3), ("block", ctypes.c_int32),
                ("tile", ctypes.c_int32 * 3)]


PATHS = {0: "none", 1: "decode", 2: "decode_per_token", 3: "tiled", 4: "reduce_rows",
         5: "reduce_slices", 6: "reduce_skipped"}


def last_dispatch() -> dict:
    """The calling thread's last pa_varlen_attention / pa_split_kv_reduce decision."""
    info = _DispatchInfo()
    _check("pa_last_dispatch", lib.pa_last_dispatch(ctypes.byref(info)))
    return {"path": PATHS.get(info.path, str(info.path)), "status": info.status,
            "partition_size": info.partition_size, "split_disabled": bool(info.split_disabled),
            "grid": tuple(info.grid), "block": info.block, "tile": tuple(info.tile)}


def pick_partition_size(seq_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                        head_dim: int, block_size: int = 16, dtype: torch.dtype = torch.bfloat16,
                        kv8: bool = False, num_cus: int = 0) -> int:
    """Host-side partition policy for a decode batch (0 or a power of two from
    256 to 8192), for the kernel the launch routes to; seq_lens is a host
    sequence, kv8 selects 8-bit E4M3 caches."""
    arr = (ctypes.c_int32 * len(seq_lens))(*[int(s) for s in seq_lens])
    dt = _dtype_code(dtype)
    r = lib.pa_pick_partition_size(ctypes.cast(arr, ctypes.c_void_p), len(seq_lens), num_q_heads,
                                   num_kv_heads, head_dim, block_size, dt,
                                   PA_FP8_E4M3 if kv8 else dt, num_cus)
    if r < 0:
        raise ValueError("pick_partition_size: bad arguments")
    return int(r)

"""attention_sdpa_amd -- Python binding of libattn.so (include/attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of libattn.so.  Tensors are torch tensors on the GPU (torch supplies
device memory and streams); calls are enqueued on the current torch stream.
If libattn.so is missing the import of a function raises -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(6)
ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2

# exported C symbols (kept in sync with include/attn.h by the CPU tests)
SYMBOLS = ("attn_status_str", "attn_version", "kv_store_slots", "attn_prefill_varlen",
           "attn_decode_workspace_bytes", "attn_decode_paged", "attn_unfused_workspace_bytes",
           "attn_prefill_unfused", "attn_prefill_padded", "attn_decode_paged_noalloc")


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m attention_sdpa_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    vp, i32p = ctypes.c_void_p, ctypes.c_void_p
    ci, cf, csz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_status_str.argtypes = [ci]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ci
    lib.kv_store_slots.argtypes = [vp, vp, vp, vp, i32p, ci, ci, ci, ci, ci, ci, vp]
    lib.kv_store_slots.restype = ci
    lib.attn_prefill_varlen.argtypes = [vp, vp, vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci, ci, ci,
                                        cf, ci, i32p, ci, ci, ci, ci, ci, vp]
    lib.attn_prefill_varlen.restype = ci
    lib.attn_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    lib.attn_decode_workspace_bytes.restype = csz
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci, ci, cf,
                                      ci, ci, ci, vp, csz, vp]
    lib.attn_decode_paged.restype = ci
    lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci, ci,
                                              cf, ci, ci, ci, vp]
    lib.attn_decode_paged_noalloc.restype = ci
    lib.attn_prefill_padded.argtypes = [vp, vp, vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci, cf, ci, ci,
                                        ci, vp]
    lib.attn_prefill_padded.restype = ci
    lib.attn_unfused_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.attn_unfused_workspace_bytes.restype = csz
    lib.attn_prefill_unfused.argtypes = [vp, vp, vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci, ci, ci,
                                         cf, ci, ci, ci, vp, csz, vp]
    lib.attn_prefill_unfused.restype = ci
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != ATTN_OK:
        msg = load_library().attn_status_str(status).decode()
        raise AttnError(fn, status, msg)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.float16:
        return ATTN_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError("index tensors must be int32")
    return _ptr(t)


def _same_device(what: str, ref: torch.Tensor, *ts: Optional[torch.Tensor]):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{what}: every tensor must be on {ref.device}, got {t.device}")


def _need(cond: bool, what: str, msg: str):
    if not cond:
        raise ValueError(f"{what}: {msg}")


def _index(t: torch.Tensor, n: int, what: str, name: str):
    """A 1-D-like int32 index tensor with exactly n entries."""
    if t.dtype != torch.int32:
        raise TypeError(f"{what}: {name} must be int32")
    _need(t.numel() == n, what, f"{name} has {t.numel()} entries, expected {n}")


def _kv_pair(k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, what: str):
    """K and V agree with each other and with Q in dtype and head_dim."""
    _need(k.dtype == v.dtype == q.dtype, what,
          f"q, k and v must share a dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    _need(k.shape == v.shape, what, f"k {tuple(k.shape)} and v {tuple(v.shape)} differ in shape")
    _need(k.shape[-1] == q.shape[-1], what,
          f"head_dim of k ({k.shape[-1]}) differs from q ({q.shape[-1]})")


def _stream(dev: torch.device, stream=None):
    """The stream to enqueue on: the given one, which must belong to the
    tensors' device, or that device's current torch stream."""
    s = torch.cuda.current_stream(dev) if stream is None else stream
    if s.device != dev:
        raise ValueError(f"the stream is on {s.device}, the tensors on {dev}")
    return ctypes.c_void_p(s.cuda_stream)


def _run(dev: torch.device, fn, *args):
    """Call into the library with the tensors' device current: the library
    launches on the current device and reads its properties there."""
    with torch.cuda.device(dev):
        return fn(*args)


def kv_store_slots(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   slot_mapping: torch.Tensor, stream=None) -> None:
    """Scatter k/v [T, Hkv, d] into caches [num_blocks, block_size, Hkv, d]."""
    T, hkv, d = k.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    if k_cache.shape != v_cache.shape or k.shape != v.shape or tuple(k_cache.shape[2:]) != (hkv, d):
        raise ValueError("shape mismatch")
    if slot_mapping.numel() != T or k.dtype != k_cache.dtype or v.dtype != k.dtype or v_cache.dtype != k.dtype:
        raise ValueError("slot_mapping/dtype mismatch")
    if slot_mapping.dtype != torch.int32:
        raise TypeError("kv_store_slots: slot_mapping must be int32")
    _same_device("kv_store_slots", k, v, k_cache, v_cache, slot_mapping)
    lib = load_library()
    _check("kv_store_slots", _run(k.device, lib.kv_store_slots,
        _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _i32(slot_mapping), T, hkv, d, nb, bs,
        _dt(k), _stream(k.device, stream)))


def attn_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                        max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                        causal: bool = True, block_table: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, out_dtype=None, stream=None) -> torch.Tensor:
    """Varlen prefill.  block_table=None: k/v packed [total_k, Hkv, d];
    otherwise k/v are the paged caches [num_blocks, block_size, Hkv, d]."""
    what = "attn_prefill_varlen"
    _need(q.dim() == 3, what, f"q must be [total_q, Hq, d], got {tuple(q.shape)}")
    total_q, hq, d = q.shape
    _kv_pair(k, v, q, what)
    batch = cu_seqlens_q.numel() - 1
    _need(batch >= 1, what, "cu_seqlens_q needs at least 2 entries")
    _index(cu_seqlens_q, batch + 1, what, "cu_seqlens_q")
    _index(cu_seqlens_k, batch + 1, what, "cu_seqlens_k")
    if block_table is None:
        _need(k.dim() == 3, what, f"k must be [total_k, Hkv, d], got {tuple(k.shape)}")
        total_k, hkv = k.shape[0], k.shape[1]
        mbs = nb = bs = 0
    else:
        _need(k.dim() == 4, what, f"paged k must be [num_blocks, block_size, Hkv, d], got {tuple(k.shape)}")
        _need(block_table.dim() == 2 and block_table.shape[0] >= batch, what,
              f"block_table must be [>= {batch}, max_blocks_per_seq], got {tuple(block_table.shape)}")
        if block_table.dtype != torch.int32:
            raise TypeError(f"{what}: block_table must be int32")
        total_k = 0
        nb, bs, hkv = k.shape[0], k.shape[1], k.shape[2]
        mbs = block_table.shape[1]
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(tuple(out.shape) == (total_q, hq, d), what, f"out must be {(total_q, hq, d)}, got {tuple(out.shape)}")
    _same_device(what, q, k, v, out, cu_seqlens_q, cu_seqlens_k, block_table)
    lib = load_library()
    _check("attn_prefill_varlen", _run(q.device, lib.attn_prefill_varlen,
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _i32(cu_seqlens_q), _i32(cu_seqlens_k), batch,
        int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, hq, hkv, d, float(softmax_scale),
        int(bool(causal)), _i32(block_table), mbs, nb, bs, _dt(q), _dt(out), _stream(q.device, stream)))
    return out


def attn_decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                max_blocks_per_seq: int, block_size: int, split_tokens: int = 0) -> int:
    return int(load_library().attn_decode_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size, split_tokens))


def attn_decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      cache_seqlens: torch.Tensor, block_table: torch.Tensor, softmax_scale: float,
                      split_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, out_dtype=None, stream=None) -> torch.Tensor:
    """Single-token decode; q [B, Hq, d], caches [num_blocks, block_size, Hkv, d]."""
    what = "attn_decode_paged"
    _need(q.dim() == 3, what, f"q must be [batch, Hq, d], got {tuple(q.shape)}")
    B, hq, d = q.shape
    _kv_pair(k_cache, v_cache, q, what)
    _need(k_cache.dim() == 4, what, f"caches must be [num_blocks, block_size, Hkv, d], got {tuple(k_cache.shape)}")
    nb, bs, hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    _index(cache_seqlens, B, what, "cache_seqlens")
    _need(block_table.dim() == 2 and block_table.shape[0] >= B, what,
          f"block_table must be [>= {B}, max_blocks_per_seq], got {tuple(block_table.shape)}")
    if block_table.dtype != torch.int32:
        raise TypeError(f"{what}: block_table must be int32")
    mbs = block_table.shape[1]
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(tuple(out.shape) == (B, hq, d), what, f"out must be {(B, hq, d)}, got {tuple(out.shape)}")
    need = attn_decode_workspace_bytes(B, hq, hkv, d, mbs, bs, split_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _same_device(what, q, k_cache, v_cache, out, cache_seqlens, block_table, workspace)
    lib = load_library()
    _check("attn_decode_paged", _run(q.device, lib.attn_decode_paged,
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _i32(cache_seqlens), _i32(block_table),
        B, hq, hkv, d, mbs, nb, bs, float(softmax_scale), int(split_tokens), _dt(q), _dt(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device, stream)))
    return out


def attn_decode_paged_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              cache_seqlens: torch.Tensor, block_table: torch.Tensor, softmax_scale: float,
                              split_tokens: int = 0, out: Optional[torch.Tensor] = None, out_dtype=None,
                              stream=None) -> torch.Tensor:
    """attn_decode_paged on the library's built-in scratch (no workspace;
    the library call allocates nothing -- pass `out` to allocate nothing
    here either).  Calls that overlap on one GPU race on that scratch."""
    what = "attn_decode_paged_noalloc"
    _need(q.dim() == 3, what, f"q must be [batch, Hq, d], got {tuple(q.shape)}")
    B, hq, d = q.shape
    _kv_pair(k_cache, v_cache, q, what)
    _need(k_cache.dim() == 4, what, f"caches must be [num_blocks, block_size, Hkv, d], got {tuple(k_cache.shape)}")
    nb, bs, hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    _index(cache_seqlens, B, what, "cache_seqlens")
    _need(block_table.dim() == 2 and block_table.shape[0] >= B, what,
          f"block_table must be [>= {B}, max_blocks_per_seq], got {tuple(block_table.shape)}")
    if block_table.dtype != torch.int32:
        raise TypeError(f"{what}: block_table must be int32")
    mbs = block_table.shape[1]
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(tuple(out.shape) == (B, hq, d), what, f"out must be {(B, hq, d)}, got {tuple(out.shape)}")
    _same_device(what, q, k_cache, v_cache, out, cache_seqlens, block_table)
    lib = load_library()
    _check(what, _run(q.device, lib.attn_decode_paged_noalloc,
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _i32(cache_seqlens), _i32(block_table),
        B, hq, hkv, d, mbs, nb, bs, float(softmax_scale), int(split_tokens), _dt(q), _dt(out),
        _stream(q.device, stream)))
    return out


def attn_unfused_workspace_bytes(batch: int, num_q_heads: int, max_seqlen_q: int, max_seqlen_k: int) -> int:
    return int(load_library().attn_unfused_workspace_bytes(batch, num_q_heads, max_seqlen_q, max_seqlen_k))


def attn_prefill_unfused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                         max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                         causal: bool = True, workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, out_dtype=None, stream=None) -> torch.Tensor:
    """The unfused three-kernel baseline (X and A through HBM); arguments as
    attn_prefill_varlen with contiguous K/V."""
    what = "attn_prefill_unfused"
    _need(q.dim() == 3, what, f"q must be [total_q, Hq, d], got {tuple(q.shape)}")
    total_q, hq, d = q.shape
    _kv_pair(k, v, q, what)
    _need(k.dim() == 3, what, f"k must be [total_k, Hkv, d], got {tuple(k.shape)}")
    total_k, hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    _need(B >= 1, what, "cu_seqlens_q needs at least 2 entries")
    _index(cu_seqlens_q, B + 1, what, "cu_seqlens_q")
    _index(cu_seqlens_k, B + 1, what, "cu_seqlens_k")
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(tuple(out.shape) == (total_q, hq, d), what, f"out must be {(total_q, hq, d)}, got {tuple(out.shape)}")
    need = attn_unfused_workspace_bytes(B, hq, max_seqlen_q, max_seqlen_k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _same_device(what, q, k, v, out, cu_seqlens_q, cu_seqlens_k, workspace)
    lib = load_library()
    _check("attn_prefill_unfused", _run(q.device, lib.attn_prefill_unfused,
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _i32(cu_seqlens_q), _i32(cu_seqlens_k), B,
        int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, hq, hkv, d, float(softmax_scale),
        int(bool(causal)), _dt(q), _dt(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device, stream)))
    return out


def attn_prefill_padded(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqlens_q: torch.Tensor,
                        seqlens_k: torch.Tensor, softmax_scale: float, causal: bool = True,
                        out: Optional[torch.Tensor] = None, out_dtype=None, stream=None) -> torch.Tensor:
    """Prefill on a padded batch: q [B, Lq_max, Hq, d], k/v [B, Lk_max, Hkv, d],
    seqlens_q/seqlens_k [B] int32.  Output rows at or past seqlens_q[b] are
    left as they are in `out` (zeros when `out` is omitted)."""
    what = "attn_prefill_padded"
    _need(q.dim() == 4, what, f"q must be [B, Lq_max, Hq, d], got {tuple(q.shape)}")
    B, mq, hq, d = q.shape
    _kv_pair(k, v, q, what)
    _need(k.dim() == 4 and k.shape[0] == B, what, f"k must be [{B}, Lk_max, Hkv, d], got {tuple(k.shape)}")
    mk, hkv = k.shape[1], k.shape[2]
    _index(seqlens_q, B, what, "seqlens_q")
    _index(seqlens_k, B, what, "seqlens_k")
    if out is None:
        out = torch.zeros((B, mq, hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(tuple(out.shape) == (B, mq, hq, d), what, f"out must be {(B, mq, hq, d)}, got {tuple(out.shape)}")
    _same_device(what, q, k, v, out, seqlens_q, seqlens_k)
    lib = load_library()
    _check("attn_prefill_padded", _run(q.device, lib.attn_prefill_padded,
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _i32(seqlens_q), _i32(seqlens_k), B, mq, mk, hq, hkv, d,
        float(softmax_scale), int(bool(causal)), _dt(q), _dt(out), _stream(q.device, stream)))
    return out

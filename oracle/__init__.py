"""CPU oracle for fused scaled-dot-product attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it,
and it shares no code with the HIP path.

What it computes follows the blog post "从零实现 vLLM (1.3)：如何加速
Attention 计算":

* ``softmax_naive`` / ``softmax_safe3`` / ``softmax_online2`` -- the three
  softmax formulations of the sections "安全 Softmax"的提出, 解决方法 and
  在线 Softmax (2-Pass), in fp64 (C, ``oracle.c``).
* ``attn_varlen`` -- O = softmax(s * Q K^T) V per query row, the standard
  three-step method (section 标准实现方法) with the three-pass safe softmax,
  over the varlen layout of the Prefill section, with causal alignment to the
  end of the sequence when Lq < Lk, in fp64 (C, ``oracle.c``).
* ``attn_decode`` -- the single-query form of the Decode section (C).
* ``kv_store`` -- the slot scatter performed by ``store_kvcache`` (Attention
  源码分析 section), written as a plain numpy loop.

Readings of points the pages leave open (stated once here, used throughout):
scale is an explicit argument; GQA maps query head h to KV head
h // (hq // hkv); a flat slot is block_id * block_size + offset and a negative
slot means "skip"; a row with no visible key is all zeros.

Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, invariants and brute force; none is pinned only against itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC_PATH = os.path.join(_HERE, "oracle.c")

__all__ = [
    "build", "default", "build_variant", "source_text", "OracleLib",
    "softmax_naive", "softmax_safe3", "softmax_online2",
    "attn_varlen", "attn_decode", "kv_store",
]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-shared", "-fPIC", _SRC_PATH, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class OracleLib:
    """ctypes view of one compiled oracle library (the default one, or a
    variant built by a test that plants a mistake in a copy of oracle.c)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        ip = ctypes.POINTER(ctypes.c_int32)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        for name in ("oracle_softmax_naive", "oracle_softmax_safe3"):
            fn = getattr(lib, name)
            fn.argtypes = [dp, i64, dp]
            fn.restype = None
        lib.oracle_softmax_online2.argtypes = [dp, i64, dp, dp, dp]
        lib.oracle_softmax_online2.restype = None
        lib.oracle_attn_varlen.argtypes = [
            fp, fp, fp, dp, ip, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_double, ctypes.c_int, lp, i64, ctypes.c_int]
        lib.oracle_attn_varlen.restype = ctypes.c_int
        lib.oracle_attn_decode.argtypes = [
            fp, fp, fp, dp, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_decode.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def softmax_naive(self, x) -> np.ndarray:
        x = _f64(x)
        out = np.empty_like(x)
        self.lib.oracle_softmax_naive(_ptr(x, ctypes.c_double), x.size, _ptr(out, ctypes.c_double))
        return out

    def softmax_safe3(self, x) -> np.ndarray:
        x = _f64(x)
        out = np.empty_like(x)
        self.lib.oracle_softmax_safe3(_ptr(x, ctypes.c_double), x.size, _ptr(out, ctypes.c_double))
        return out

    def softmax_online2(self, x):
        """Returns (softmax, running maxima m_i, running proxy denominators d'_i)."""
        x = _f64(x)
        out = np.empty_like(x)
        m = np.empty_like(x)
        d = np.empty_like(x)
        self.lib.oracle_softmax_online2(_ptr(x, ctypes.c_double), x.size,
                                        _ptr(m, ctypes.c_double), _ptr(d, ctypes.c_double),
                                        _ptr(out, ctypes.c_double))
        return out, m, d

    def attn_varlen(self, q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale,
                    causal=True, rows=None, threads: int = 0) -> np.ndarray:
        """fp64 attention over the varlen layout.

        q [total_q, hq, d], k/v [total_k, hkv, d] float32; cu_seqlens_* int
        [batch+1].  rows=None returns [total_q, hq, d]; otherwise rows is an
        int array of flat (token * hq + head) indices and the result is
        [len(rows), d].
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        cu_q, cu_k = _i32(cu_seqlens_q), _i32(cu_seqlens_k)
        total_q, hq, d = q.shape
        hkv = k.shape[1]
        batch = cu_q.size - 1
        if cu_k.size != batch + 1 or k.shape != v.shape or k.shape[2] != d:
            raise ValueError("inconsistent shapes")
        if int(cu_q[-1]) != total_q or int(cu_k[-1]) > k.shape[0]:
            raise ValueError("cu_seqlens do not match the packed arrays")
        if rows is None:
            out = np.full((total_q, hq, d), np.nan, dtype=np.float64)
            rp, nrows = None, 0
        else:
            rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            out = np.full((rows.size, d), np.nan, dtype=np.float64)
            rp, nrows = _ptr(rows, ctypes.c_int64), rows.size
        rc = self.lib.oracle_attn_varlen(
            _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
            _ptr(out, ctypes.c_double), _ptr(cu_q, ctypes.c_int32), _ptr(cu_k, ctypes.c_int32),
            batch, hq, hkv, d, float(softmax_scale), int(bool(causal)), rp, nrows, int(threads))
        if rc != 0:
            raise ValueError("oracle_attn_varlen rejected its arguments")
        return out

    def attn_decode(self, q, k, v, cu_seqlens_k, softmax_scale, threads: int = 0) -> np.ndarray:
        """fp64 single-query decode; q [batch, hq, d], logical k/v [total_k, hkv, d]."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        cu_k = _i32(cu_seqlens_k)
        batch, hq, d = q.shape
        if cu_k.size != batch + 1 or int(cu_k[-1]) > k.shape[0]:
            raise ValueError("cu_seqlens_k does not match k")
        out = np.full((batch, hq, d), np.nan, dtype=np.float64)
        rc = self.lib.oracle_attn_decode(
            _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
            _ptr(out, ctypes.c_double), _ptr(cu_k, ctypes.c_int32), batch, hq,
            k.shape[1], d, float(softmax_scale), int(threads))
        if rc != 0:
            raise ValueError("oracle_attn_decode rejected its arguments")
        return out


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _f32(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float32:
        raise TypeError("oracle attention inputs must be float32 arrays "
                        "(bf16 values are passed upcast, exactly, to float32)")
    return np.ascontiguousarray(a)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


_default = None


def default() -> OracleLib:
    """The oracle built from oracle.c next to this file (rebuilt if stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH)):
            build(force=True)
        _default = OracleLib(_LIB_PATH)
    return _default


def build_variant(src_text: str, out_dir: str) -> OracleLib:
    """Compile a modified copy of oracle.c (tests plant mistakes this way, to
    show that the pins catch them) and load it."""
    src = os.path.join(out_dir, "oracle_variant.c")
    lib = os.path.join(out_dir, "liboracle_variant.so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-shared", "-fPIC", src, "-o", lib, "-lm"],
                   check=True)
    return OracleLib(lib)


def source_text() -> str:
    with open(_SRC_PATH) as f:
        return f.read()


def softmax_naive(x):
    return default().softmax_naive(x)


def softmax_safe3(x):
    return default().softmax_safe3(x)


def softmax_online2(x):
    return default().softmax_online2(x)


def attn_varlen(*args, **kwargs):
    return default().attn_varlen(*args, **kwargs)


def attn_decode(*args, **kwargs):
    return default().attn_decode(*args, **kwargs)


def kv_store(k_new, v_new, k_cache, v_cache, slot_mapping) -> None:
    """store_kvcache: write row t of k_new/v_new ([T, hkv, d]) into cache slot
    slot_mapping[t] of k_cache/v_cache ([num_blocks, block_size, hkv, d]);
    slot = block_id * block_size + offset; a negative slot skips the token.
    Works on any dtype (use integer views for bit-exact comparisons)."""
    block_size = k_cache.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        k_cache[blk, off] = k_new[t]
        v_cache[blk, off] = v_new[t]

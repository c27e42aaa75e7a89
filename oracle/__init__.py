"""CPU oracle for one paged-attention step -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper over ``oracle/_build/liboracle.so`` (plain C, double
precision, built by ``oracle/build.py``).  Only ``tests/``, the package's
``smoke()`` check and the benchmark's CPU-baseline leg may import this
module; the HIP library and its Python binding never do.

The oracle keeps its own KV pool in the layout the pages print,
``[num_blocks][block_size][num_kv_heads][head_dim]`` per K and V
("vLLM 推理流程分析" §6.2), so any comparison with the HIP pool goes through
logical (block, offset, head, dim) indexing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("PA_ORACLE_LIB") or os.path.join(_HERE, "_build", "liboracle.so")

F32, BF16, FP8 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8}
_NP = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}
# Canary written into every pool element that no step has written: the
# all-ones bit pattern, a NaN in each element type (fp32, bf16, and E4M3FN
# S.1111.111).
_CANARY = {F32: np.uint32(0xFFFFFFFF).view(np.float32), BF16: np.uint16(0xFFFF), FP8: np.uint8(0xFF)}


class _Pool(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("num_blocks", C.c_int32),
                ("block_size", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("dtype", C.c_int32), ("k_scale", C.c_float),
                ("v_scale", C.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b  # noqa: F401  (build on first use)
            _b.build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.oracle_num_threads.restype = C.c_int
        L.oracle_e4m3_decode.restype = C.c_double
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_encode.argtypes = [C.c_float]
        L.oracle_e4m3_encode_array.argtypes = [P, P, i64]
        L.oracle_e4m3_decode_array.argtypes = [P, P, i64]
        L.oracle_query_start_loc.argtypes = [i32, P, P]
        L.oracle_seq_lens.argtypes = [i32, P, P, P]
        L.oracle_validate.argtypes = [i32, i32, P, P, P, i32, i32, i32]
        L.oracle_slot_mapping.argtypes = [i32, P, P, P, i32, i32, P]
        L.oracle_write_kv.argtypes = [C.POINTER(_Pool), P, P, i32, P, i32]
        L.oracle_attention.argtypes = [C.POINTER(_Pool), i32, P, P, P, i32, P, i32, i32, C.c_float,
                                       i32, P, P, i32]
        L.oracle_attention_probs.restype = i32
        L.oracle_attention_probs.argtypes = [C.POINTER(_Pool), i32, P, P, P, i32, P, i32, i32,
                                             C.c_float, i32, i32, i32, P]
        L.oracle_attention_partitioned.argtypes = [C.POINTER(_Pool), i32, P, P, P, i32, P, i32, i32,
                                                   C.c_float, i32, i32, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ----------------------------------------------------------------- codecs --

def e4m3_encode(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(y), _p(out), y.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_e4m3_decode_array(_p(c), _p(out), c.size)
    return out


# --------------------------------------------------------------- metadata --

def query_start_loc(num_scheduled) -> np.ndarray:
    ns = _c(num_scheduled, np.int32)
    out = np.empty(ns.size + 1, dtype=np.int32)
    rc = lib().oracle_query_start_loc(ns.size, _p(ns), _p(out))
    if rc:
        raise ValueError("oracle_query_start_loc failed")
    return out


def seq_lens(num_computed, num_scheduled) -> np.ndarray:
    nc, ns = _c(num_computed, np.int32), _c(num_scheduled, np.int32)
    out = np.empty(nc.size, dtype=np.int32)
    if lib().oracle_seq_lens(nc.size, _p(nc), _p(ns), _p(out)):
        raise ValueError("oracle_seq_lens failed")
    return out


def validate(qsl, sl, bt, block_size, num_blocks, num_tokens=None) -> int:
    qsl, sl, bt = _c(qsl, np.int32), _c(sl, np.int32), _c(bt, np.int32)
    n = sl.size
    T = int(qsl[-1]) if num_tokens is None else int(num_tokens)
    stride = bt.shape[1] if bt.ndim == 2 else 0
    return int(lib().oracle_validate(n, T, _p(qsl), _p(sl), _p(bt), stride, block_size, num_blocks))


def slot_mapping(qsl, sl, bt, block_size) -> np.ndarray:
    qsl, sl, bt = _c(qsl, np.int32), _c(sl, np.int32), _c(bt, np.int32)
    out = np.empty(int(qsl[-1]), dtype=np.int64)
    if lib().oracle_slot_mapping(sl.size, _p(qsl), _p(sl), _p(bt), bt.shape[1], block_size, _p(out)):
        raise ValueError("oracle_slot_mapping failed")
    return out


# ------------------------------------------------------------------ pool ---

class Pool:
    """K and V pools in the pages' layout, NaN canaries in unwritten slots."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype: str, k_scale: float = 1.0, v_scale: float = 1.0):
        self.dtype = _DT[dtype]
        shape = (num_blocks, block_size, num_kv_heads, head_dim)
        self.k = np.full(shape, _CANARY[self.dtype], dtype=_NP[self.dtype])
        self.v = np.full(shape, _CANARY[self.dtype], dtype=_NP[self.dtype])
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)

    def _struct(self) -> _Pool:
        return _Pool(self.k.ctypes.data, self.v.ctypes.data, self.num_blocks, self.block_size,
                     self.num_kv_heads, self.head_dim, self.dtype, self.k_scale, self.v_scale)

    def decoded(self, which: str) -> np.ndarray:
        """Pool contents as float64 (fp8 dequantised with its scale)."""
        a = self.k if which == "k" else self.v
        if self.dtype == F32:
            return a.astype(np.float64)
        if self.dtype == BF16:
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        s = self.k_scale if which == "k" else self.v_scale
        return e4m3_decode(a) * s


def write_kv(pool: Pool, key, value, in_dtype: str, slots) -> None:
    dt = _DT[in_dtype]
    key, value = _c(key, _NP[dt]), _c(value, _NP[dt])
    slots = _c(slots, np.int64)
    st = pool._struct()
    rc = lib().oracle_write_kv(C.byref(st), _p(key), _p(value), dt, _p(slots), slots.size)
    if rc:
        raise ValueError(f"oracle_write_kv failed ({rc})")


def attention(pool: Pool, qsl, sl, bt, q, q_dtype: str, num_q_heads: int, scale: float,
              causal: bool = True, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    qsl, sl, bt = _c(qsl, np.int32), _c(sl, np.int32), _c(bt, np.int32)
    q = _c(q, _NP[_DT[q_dtype]])
    sub = None if tokens is None else _c(tokens, np.int32)
    rows = int(qsl[-1]) if sub is None else sub.size
    out = np.empty((rows, num_q_heads, pool.head_dim), dtype=np.float64)
    st = pool._struct()
    rc = lib().oracle_attention(C.byref(st), sl.size, _p(qsl), _p(sl), _p(bt), bt.shape[1], _p(q),
                                _DT[q_dtype], num_q_heads, scale, int(causal), _p(out),
                                None if sub is None else _p(sub), 0 if sub is None else sub.size)
    if rc:
        raise ValueError(f"oracle_attention failed ({rc})")
    return out


def attention_probs(pool: Pool, qsl, sl, bt, q, q_dtype: str, num_q_heads: int, scale: float,
                    token: int, head: int, causal: bool = True) -> np.ndarray:
    qsl, sl, bt = _c(qsl, np.int32), _c(sl, np.int32), _c(bt, np.int32)
    q = _c(q, _NP[_DT[q_dtype]])
    buf = np.empty(max(1, int(sl.max())), dtype=np.float64)
    st = pool._struct()
    n = lib().oracle_attention_probs(C.byref(st), sl.size, _p(qsl), _p(sl), _p(bt), bt.shape[1],
                                     _p(q), _DT[q_dtype], num_q_heads, scale, int(causal), token,
                                     head, _p(buf))
    if n < 0:
        raise ValueError("oracle_attention_probs failed")
    return buf[:n].copy()


def attention_partitioned(pool: Pool, qsl, sl, bt, q, q_dtype: str, num_q_heads: int, scale: float,
                          part: int, causal: bool = True) -> np.ndarray:
    qsl, sl, bt = _c(qsl, np.int32), _c(sl, np.int32), _c(bt, np.int32)
    q = _c(q, _NP[_DT[q_dtype]])
    out = np.empty((int(qsl[-1]), num_q_heads, pool.head_dim), dtype=np.float64)
    st = pool._struct()
    rc = lib().oracle_attention_partitioned(C.byref(st), sl.size, _p(qsl), _p(sl), _p(bt),
                                            bt.shape[1], _p(q), _DT[q_dtype], num_q_heads, scale,
                                            int(causal), part, _p(out))
    if rc:
        raise ValueError("oracle_attention_partitioned failed")
    return out


# ------------------------------------------------------- whole workloads ---

class StepResult:
    def __init__(self, pool, qsl, seq_lens, slots, out, tokens):
        self.pool, self.qsl, self.seq_lens = pool, qsl, seq_lens
        self.slots, self.out, self.tokens = slots, out, tokens


def build_pool(w) -> Pool:
    """Pool after the workload's earlier steps, each applied with the oracle's
    own metadata, slot derivation and write."""
    pool = Pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype,
                w.k_scale, w.v_scale)
    for h in w.history:
        bt = w.block_table[h.requests]
        hq = query_start_loc(h.count)
        hs = slot_mapping(hq, h.total, bt, w.block_size)
        write_kv(pool, h.key, h.value, w.io_dtype, hs)
    return pool


def run_step(w, tokens: Optional[Sequence[int]] = None, pool: Optional[Pool] = None,
             causal: bool = True) -> StepResult:
    """Metadata -> slots -> write -> attention for the workload's step."""
    pool = build_pool(w) if pool is None else pool
    qsl = query_start_loc(w.num_scheduled)
    sl = seq_lens(w.num_computed, w.num_scheduled)
    rc = validate(qsl, sl, w.block_table, w.block_size, w.num_blocks, w.num_tokens)
    if rc:
        raise ValueError(f"workload fails the metadata checks ({rc})")
    slots = slot_mapping(qsl, sl, w.block_table, w.block_size)
    write_kv(pool, w.key, w.value, w.io_dtype, slots)
    out = attention(pool, qsl, sl, w.block_table, w.query, w.io_dtype, w.num_q_heads,
                    w.softmax_scale, causal, tokens)
    return StepResult(pool, qsl, sl, slots, out, tokens)

"""Thin ctypes binding over libpa.so (declared in include/pa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpa.so.  PyTorch supplies device memory and the stream.  The
names mirror the C ABI: ``prepare_metadata``, ``slot_mapping``, ``write_kv``,
``attention_workspace_bytes``, ``attention``.

If libpa.so is missing this module raises on import: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIB") or os.path.join(_HERE, "_build", "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": PA_F32, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}
STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_WORKSPACE",
          4: "PA_ERR_VALIDATION", 5: "PA_ERR_HIP", 6: "PA_ERR_CAPACITY"}

# Every symbol include/pa.h declares.
EXPORTS = ["pa_prepare_metadata", "pa_slot_mapping", "pa_write_kv", "pa_attention_workspace_bytes",
           "pa_attention", "pa_write_kv_attention", "pa_write_kv_attention_noalloc",
           "pa_noalloc_scratch_bytes", "pa_kv_cache_bytes", "pa_kv_elem_offset",
           "pa_status_string",
           "pa_last_error", "pa_profile_enable", "pa_profile_read",
           "pa_kv_manager_create", "pa_kv_manager_destroy", "pa_kv_manager_num_free_blocks",
           "pa_kv_manager_get_computed_blocks", "pa_kv_manager_allocate_slots",
           "pa_kv_manager_cache_blocks", "pa_kv_manager_free", "pa_kv_manager_block_ids",
           "pa_kv_manager_ref_count", "pa_zero_blocks", "pa_placement_check"]


class PaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class PaKvPool(C.Structure):
    _fields_ = [("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("num_blocks", C.c_int32),
                ("block_size", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("kv_dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float)]


class PaBatch(C.Structure):
    _fields_ = [("num_seqs", C.c_int32), ("num_tokens", C.c_int32),
                ("query_start_loc", C.c_void_p), ("seq_lens", C.c_void_p),
                ("block_table", C.c_void_p), ("bt_stride", C.c_int32),
                ("query_start_loc_host", C.c_void_p), ("seq_lens_host", C.c_void_p),
                ("num_common_prefix_blocks", C.c_int32)]


class PaPlacement(C.Structure):
    _fields_ = [("compute_units", C.c_int32), ("xcds", C.c_int32), ("one_wave_alone", C.c_float),
                ("two_wave_paired", C.c_float), ("xcd_round_robin", C.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_pool_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    pool_p, batch_p = C.POINTER(PaKvPool), C.POINTER(PaBatch)
    sig = {
        "pa_prepare_metadata": (i32, [i32, P, P, P, P]),
        "pa_slot_mapping": (i32, [batch_p, i32, P, P]),
        "pa_write_kv": (i32, [pool_p, P, P, i32, P, i32, P]),
        "pa_attention_workspace_bytes": (C.c_size_t, [pool_p, batch_p, i32]),
        "pa_attention": (i32, [pool_p, batch_p, P, i32, i32, f32, i32, P, P, C.c_size_t, P]),
        "pa_write_kv_attention": (i32, [pool_p, batch_p, P, P, P, i32, i32, f32, i32, P, P, P,
                                        C.c_size_t, P]),
        "pa_write_kv_attention_noalloc": (i32, [pool_p, batch_p, P, P, P, i32, i32, f32, i32, P, P, P]),
        "pa_noalloc_scratch_bytes": (C.c_size_t, []),
        "pa_kv_cache_bytes": (C.c_size_t, [pool_p]),
        "pa_kv_elem_offset": (i64, [pool_p, i32, i64, i32, i32, i32]),
        "pa_status_string": (C.c_char_p, [i32]),
        "pa_last_error": (C.c_char_p, []),
        "pa_profile_enable": (i32, [i32]),
        "pa_profile_read": (i32, [C.c_char_p, C.POINTER(i32), C.POINTER(C.c_double)]),
        "pa_kv_manager_create": (i32, [i32, i32, C.POINTER(P)]),
        "pa_kv_manager_destroy": (None, [P]),
        "pa_kv_manager_num_free_blocks": (i32, [P]),
        "pa_kv_manager_get_computed_blocks": (i32, [P, P, i32, C.c_uint64, P, i32, C.POINTER(i32)]),
        "pa_kv_manager_allocate_slots": (i32, [P, i64, i32, P, i32, P, i32, C.POINTER(i32)]),
        "pa_kv_manager_cache_blocks": (i32, [P, i64, P, i32, C.c_uint64]),
        "pa_kv_manager_free": (i32, [P, i64]),
        "pa_kv_manager_block_ids": (i32, [P, i64, P, i32, C.POINTER(i32)]),
        "pa_kv_manager_ref_count": (i32, [P, i32, C.POINTER(i32)]),
        "pa_zero_blocks": (i32, [pool_p, P, i32, P]),
        "pa_placement_check": (i32, [C.POINTER(PaPlacement)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    return L


lib = _load()


def _check(st: int) -> None:
    if st != 0:
        raise PaError(st, lib.pa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def torch_dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


# ---------------------------------------------------------------- objects --

@dataclass
class KVPool:
    """A paged KV pool in device memory (layout: see include/pa.h)."""
    k_cache: torch.Tensor   # uint8 [pa_kv_cache_bytes]
    v_cache: torch.Tensor
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    k_scale: float = 1.0
    v_scale: float = 1.0

    @staticmethod
    def spec(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, k_scale=1.0, v_scale=1.0):
        return PaKvPool(None, None, num_blocks, block_size, num_kv_heads, head_dim, DTYPES[kv_dtype],
                        k_scale, v_scale)

    @classmethod
    def allocate(cls, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, k_scale=1.0,
                 v_scale=1.0, device="cuda", fill_byte: Optional[int] = None) -> "KVPool":
        nbytes = lib.pa_kv_cache_bytes(C.byref(cls.spec(num_blocks, block_size, num_kv_heads,
                                                         head_dim, kv_dtype, k_scale, v_scale)))
        if nbytes == 0:
            raise PaError(1, "invalid pool shape")
        k = torch.empty(nbytes, dtype=torch.uint8, device=device)
        v = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if fill_byte is not None:
            k.fill_(fill_byte)
            v.fill_(fill_byte)
        return cls(k, v, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, k_scale, v_scale)

    def struct(self) -> PaKvPool:
        return PaKvPool(self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.num_blocks,
                        self.block_size, self.num_kv_heads, self.head_dim, DTYPES[self.kv_dtype],
                        self.k_scale, self.v_scale)

    def elem_offset(self, which: int, block: int, offset: int, head: int, dim: int) -> int:
        return int(lib.pa_kv_elem_offset(C.byref(self.struct()), which, block, offset, head, dim))

    def logical(self, which: str, blocks: Optional[np.ndarray] = None) -> np.ndarray:
        """Copy of K or V in logical [num_blocks][block_size][num_kv_heads][head_dim]
        order, as raw element values (float32, uint16 bf16 bits, or uint8 codes).
        With `blocks`, only those blocks, in that order ([len(blocks)][...])."""
        dev = self.k_cache if which == "k" else self.v_cache
        nb = self.num_blocks
        if blocks is not None:
            idx = torch.as_tensor(np.asarray(blocks, dtype=np.int64), device=dev.device)
            dev = dev.view(nb, -1).index_select(0, idx)
            nb = int(idx.numel())
        raw = dev.cpu().numpy().reshape(-1)
        npd = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[self.kv_dtype]
        el = raw.view(npd)
        S, H, D = self.block_size, self.num_kv_heads, self.head_dim
        if which == "k":
            E = 16 // el.itemsize
            return el.reshape(nb, H, D // E, S, E).transpose(0, 3, 1, 2, 4).reshape(nb, S, H, D).copy()
        return el.reshape(nb, H, D, S).transpose(0, 3, 1, 2).copy()


@dataclass
class Batch:
    """One step's ragged batch: device arrays plus their host mirrors."""
    query_start_loc: torch.Tensor   # int32 device [N+1]
    seq_lens: torch.Tensor          # int32 device [N]
    block_table: torch.Tensor       # int32 device [N, W]
    qsl_host: np.ndarray            # int32 [N+1]
    seq_lens_host: np.ndarray       # int32 [N]
    num_common_prefix_blocks: int = 0   # shared-prefix hint (pa.h)

    @classmethod
    def from_host(cls, qsl: np.ndarray, seq_lens: np.ndarray, block_table: np.ndarray,
                  device="cuda", num_common_prefix_blocks: int = 0) -> "Batch":
        qsl = np.ascontiguousarray(qsl, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        return cls(torch.from_numpy(qsl).to(device), torch.from_numpy(sl).to(device),
                   torch.from_numpy(bt).to(device), qsl, sl, int(num_common_prefix_blocks))

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens_host.size)

    @property
    def num_tokens(self) -> int:
        return int(self.qsl_host[-1])

    def struct(self) -> PaBatch:
        bt = self.block_table
        return PaBatch(self.num_seqs, self.num_tokens, self.query_start_loc.data_ptr(),
                       self.seq_lens.data_ptr(), bt.data_ptr(), bt.stride(0) if bt.dim() == 2 else 0,
                       self.qsl_host.ctypes.data, self.seq_lens_host.ctypes.data,
                       self.num_common_prefix_blocks)


# ---------------------------------------------------------------- calls ----

def prepare_metadata(num_computed, num_scheduled):
    """a0 on the host: (query_start_loc [N+1], seq_lens [N]) as int32 numpy arrays."""
    nc = np.ascontiguousarray(num_computed, dtype=np.int32)
    ns = np.ascontiguousarray(num_scheduled, dtype=np.int32)
    qsl = np.empty(nc.size + 1, dtype=np.int32)
    sl = np.empty(nc.size, dtype=np.int32)
    _check(lib.pa_prepare_metadata(nc.size, _np_ptr(nc), _np_ptr(ns), _np_ptr(qsl), _np_ptr(sl)))
    return qsl, sl


def slot_mapping(batch: Batch, block_size: int, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(batch.num_tokens, dtype=torch.int64, device=batch.seq_lens.device)
    b = batch.struct()
    _check(lib.pa_slot_mapping(C.byref(b), block_size, _ptr(out), _stream(stream)))
    return out


def write_kv(pool: KVPool, key: torch.Tensor, value: torch.Tensor, slots: torch.Tensor,
             stream=None) -> None:
    assert key.is_contiguous() and value.is_contiguous() and slots.is_contiguous()
    assert slots.dtype == torch.int64
    p = pool.struct()
    _check(lib.pa_write_kv(C.byref(p), _ptr(key), _ptr(value), torch_dtype_code(key), _ptr(slots),
                           int(slots.numel()), _stream(stream)))


def attention_workspace_bytes(pool: KVPool, batch: Batch, num_q_heads: int) -> int:
    p, b = pool.struct(), batch.struct()
    n = int(lib.pa_attention_workspace_bytes(C.byref(p), C.byref(b), num_q_heads))
    if n == 0:
        raise PaError(1, lib.pa_last_error().decode())
    return n


def attention(pool: KVPool, batch: Batch, query: torch.Tensor, num_q_heads: int,
              softmax_scale: float, causal: bool = True, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    assert query.is_contiguous()
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:
        workspace = torch.empty(attention_workspace_bytes(pool, batch, num_q_heads),
                                dtype=torch.uint8, device=query.device)
    p, b = pool.struct(), batch.struct()
    _check(lib.pa_attention(C.byref(p), C.byref(b), _ptr(query), torch_dtype_code(query),
                            num_q_heads, softmax_scale, int(causal), _ptr(out), _ptr(workspace),
                            workspace.numel(), _stream(stream)))
    return out


def write_kv_attention(pool: KVPool, batch: Batch, query: torch.Tensor, key: torch.Tensor,
                       value: torch.Tensor, num_q_heads: int, softmax_scale: float,
                       causal: bool = True, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       slots: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_write_kv_attention: the KV update and the attention in one call."""
    assert query.is_contiguous() and key.is_contiguous() and value.is_contiguous()
    assert key.dtype == query.dtype and value.dtype == query.dtype
    assert slots is None or (slots.dtype == torch.int64 and slots.is_contiguous())
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:
        workspace = torch.empty(attention_workspace_bytes(pool, batch, num_q_heads),
                                dtype=torch.uint8, device=query.device)
    p, b = pool.struct(), batch.struct()
    _check(lib.pa_write_kv_attention(C.byref(p), C.byref(b), _ptr(query), _ptr(key), _ptr(value),
                                     torch_dtype_code(query), num_q_heads, softmax_scale,
                                     int(causal), _ptr(slots), _ptr(out), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))
    return out


def write_kv_attention_noalloc(pool: KVPool, batch: Batch, query: torch.Tensor, key: torch.Tensor,
                               value: torch.Tensor, num_q_heads: int, softmax_scale: float,
                               causal: bool = True, out: Optional[torch.Tensor] = None,
                               slots: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_write_kv_attention_noalloc: the one call with the KV update, its
    scratch in the library's static device array (no workspace)."""
    assert query.is_contiguous() and key.is_contiguous() and value.is_contiguous()
    assert key.dtype == query.dtype and value.dtype == query.dtype
    assert slots is None or (slots.dtype == torch.int64 and slots.is_contiguous())
    if out is None:
        out = torch.empty_like(query)
    p, b = pool.struct(), batch.struct()
    _check(lib.pa_write_kv_attention_noalloc(C.byref(p), C.byref(b), _ptr(query), _ptr(key),
                                             _ptr(value), torch_dtype_code(query), num_q_heads,
                                             softmax_scale, int(causal), _ptr(slots), _ptr(out),
                                             _stream(stream)))
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib.pa_noalloc_scratch_bytes())


class KVManager:
    """The library's host block pool (pa_kv_manager_*): allocate_slots, free,
    reference counts, the free queue and block-hash prefix hits."""

    def __init__(self, num_blocks: int, block_size: int):
        h = C.c_void_p()
        _check(lib.pa_kv_manager_create(num_blocks, block_size, C.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self) -> None:
        if self._h:
            lib.pa_kv_manager_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free_blocks(self) -> int:
        return int(lib.pa_kv_manager_num_free_blocks(self._h))

    def get_computed_blocks(self, token_ids, extra_key: int = 0) -> list:
        t = np.ascontiguousarray(token_ids, dtype=np.int32)
        out = np.empty(max(1, t.size // self.block_size + 1), dtype=np.int32)
        n = C.c_int32(0)
        _check(lib.pa_kv_manager_get_computed_blocks(self._h, _np_ptr(t), t.size, extra_key,
                                                     _np_ptr(out), out.size, C.byref(n)))
        return out[:n.value].tolist()

    def allocate_slots(self, request_id: int, num_tokens: int, computed_blocks=()) -> Optional[list]:
        """New block ids, or None when the pool has too few free blocks."""
        cb = np.ascontiguousarray(list(computed_blocks), dtype=np.int32)
        out = np.empty(max(1, -(-num_tokens // self.block_size)), dtype=np.int32)
        n = C.c_int32(0)
        st = lib.pa_kv_manager_allocate_slots(self._h, request_id, num_tokens,
                                              _np_ptr(cb) if cb.size else None, cb.size,
                                              _np_ptr(out), out.size, C.byref(n))
        if st == 6:
            return None
        _check(st)
        return out[:n.value].tolist()

    def cache_blocks(self, request_id: int, token_ids, num_tokens: int, extra_key: int = 0) -> None:
        t = np.ascontiguousarray(token_ids, dtype=np.int32)
        assert num_tokens <= t.size
        _check(lib.pa_kv_manager_cache_blocks(self._h, request_id, _np_ptr(t), num_tokens, extra_key))

    def free(self, request_id: int) -> None:
        _check(lib.pa_kv_manager_free(self._h, request_id))

    def block_ids(self, request_id: int) -> list:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = C.c_int32(0)
        _check(lib.pa_kv_manager_block_ids(self._h, request_id, _np_ptr(out), out.size, C.byref(n)))
        return out[:n.value].tolist()

    def ref_count(self, block: int) -> int:
        r = C.c_int32(0)
        _check(lib.pa_kv_manager_ref_count(self._h, block, C.byref(r)))
        return int(r.value)


def zero_blocks(pool: KVPool, block_ids: torch.Tensor, stream=None) -> None:
    assert block_ids.dtype == torch.int32 and block_ids.is_contiguous()
    p = pool.struct()
    _check(lib.pa_zero_blocks(C.byref(p), _ptr(block_ids), int(block_ids.numel()), _stream(stream)))


def profile_enable(on: bool) -> None:
    _check(lib.pa_profile_enable(1 if on else 0))


def profile_read(kernel: str):
    n = C.c_int32(0)
    ms = C.c_double(0)
    _check(lib.pa_profile_read(kernel.encode(), C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)


def placement_check() -> dict:
    """Dispatch placement on the current device (pa_placement_check): the
    fractions of probe workgroups placed as the planners assume."""
    r = PaPlacement()
    _check(lib.pa_placement_check(C.byref(r)))
    return {"compute_units": int(r.compute_units), "xcds": int(r.xcds),
            "one_wave_alone": round(float(r.one_wave_alone), 4),
            "two_wave_paired": round(float(r.two_wave_paired), 4),
            "xcd_round_robin": round(float(r.xcd_round_robin), 4)}


def status_string(code: int) -> str:
    return lib.pa_status_string(code).decode()

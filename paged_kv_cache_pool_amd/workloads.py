"""Seeded synthetic inputs for one paged-attention step.

This module only draws inputs: request lengths, the physical blocks each
request owns (the allocator's outcome), and the K/V/Q values.  It contains
none of the method's arithmetic -- no query_start_loc prefix sum, no slot
derivation, no KV write, no attention.  Both the HIP path and the CPU oracle
consume the same arrays from here and each derives everything else with its
own code.

Conventions
-----------
* ``num_computed[i]``: tokens of request ``i`` already in the KV pool before
  this step; ``num_scheduled[i]``: tokens computed in this step (``c_i``).
  The page "vLLM 推理流程分析" §5.1.2 defines the step's per-request length as
  computed + scheduled; that sum is left to the consumers.
* ``block_table[i, b]``: physical block holding logical block ``b`` of
  request ``i``; rows are padded with -1 beyond the blocks the request owns.
* ``history``: a list of "earlier steps" that populate the pool before the
  measured step.  Each entry gives, per request, how many tokens it writes
  (``count``) and how many the request holds after it (``total``), plus the
  rows it writes in request order.  Consumers apply it with their own slot
  derivation and KV write.
* Values: i.i.d. N(0, 1) drawn in float32 from numpy's PCG64, rounded to
  nearest-even into bfloat16 when the workload is bf16.  bf16 arrays are
  returned as ``uint16`` bit patterns; fp32 arrays as ``float32``.

Draw order for a seed: lengths, then the block permutation, both from
``default_rng(seed)``.  Value arrays come from independent child streams keyed
by (seed, role, ...) in chunks of 2**22 elements (see ``_normal``), so they
can be drawn in parallel and reproduced in any order.  fp8 scales are a fixed convention computed from the drawn rows
(amax / 448, float32).
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import List, Optional

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8"

FP8_E4M3_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class HistoryBatch:
    count: np.ndarray      # int32 [N]  tokens written by this earlier step
    total: np.ndarray      # int32 [N]  tokens the request holds after it
    key: np.ndarray        # [sum(count), Hkv, d]  (uint16 bf16 bits or float32)
    value: np.ndarray      # same shape/dtype as key
    requests: np.ndarray   # int32 [N]  which rows of block_table this batch uses


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str           # f32 | bf16 | fp8  (pool element type)
    io_dtype: str           # f32 | bf16       (q/k/v/output element type)
    num_computed: np.ndarray    # int32 [N]
    num_scheduled: np.ndarray   # int32 [N]
    block_table: np.ndarray     # int32 [N, W], -1 padded
    history: List[HistoryBatch]
    query: np.ndarray       # [T, Hq, d]
    key: np.ndarray         # [T, Hkv, d]
    value: np.ndarray       # [T, Hkv, d]
    k_scale: float = 1.0
    v_scale: float = 1.0
    shared_prefix_blocks: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.num_computed.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query.shape[0])

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))


_CHUNK = 1 << 22  # elements per independent child stream


def _normal(key, shape, io_dtype: str) -> np.ndarray:
    """N(0, 1) values of ``shape``; element chunk ``c`` comes from the PCG64 stream
    seeded by ``SeedSequence(key + [c])``, so the result does not depend on how
    many threads draw it."""
    total = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(total, dtype=np.uint16 if io_dtype == BF16 else np.float32)
    nchunks = -(-total // _CHUNK)

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(total, (c + 1) * _CHUNK)
        r = np.random.default_rng(np.random.SeedSequence(list(key) + [c]))
        x = r.standard_normal(size=hi - lo, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(x) if io_dtype == BF16 else x

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        workers = max(1, min(16, os.cpu_count() or 1, nchunks))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _as_f32(a: np.ndarray, io_dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if io_dtype == BF16 else a


def _blocks_needed(n_tokens: int, block_size: int) -> int:
    return -(-int(n_tokens) // block_size)


def build(name: str, seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
          block_size: int, num_blocks: int, kv_dtype: str, io_dtype: str,
          num_computed, num_scheduled, shared_prefix_tokens: int = 0,
          rng: Optional[np.random.Generator] = None) -> Workload:
    """Assemble a workload from per-request lengths (already drawn)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    nc = np.asarray(num_computed, dtype=np.int32)
    ns = np.asarray(num_scheduled, dtype=np.int32)
    n = nc.shape[0]
    totals = nc.astype(np.int64) + ns
    S = block_size
    sp_blocks = shared_prefix_tokens // S
    assert shared_prefix_tokens % S == 0
    need = [_blocks_needed(t, S) for t in totals]
    unique_need = sum(max(0, b - sp_blocks) for b in need) + sp_blocks
    assert unique_need <= num_blocks, (unique_need, num_blocks)
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = max(1, max(need) if need else 1)
    bt = np.full((n, width), -1, dtype=np.int32)
    cursor = sp_blocks
    for i in range(n):
        if sp_blocks:
            bt[i, :sp_blocks] = perm[:sp_blocks]
        own = need[i] - sp_blocks if sp_blocks else need[i]
        bt[i, sp_blocks:sp_blocks + own] = perm[cursor:cursor + own]
        cursor += own

    H, d = num_kv_heads, head_dim
    history: List[HistoryBatch] = []
    if sp_blocks:
        # The shared prefix is written once, through request 0's table.
        cnt = np.array([shared_prefix_tokens], dtype=np.int32)
        history.append(HistoryBatch(count=cnt, total=cnt.copy(),
                                    key=_normal([seed, 1, 0, 0], (shared_prefix_tokens, H, d), io_dtype),
                                    value=_normal([seed, 1, 0, 1], (shared_prefix_tokens, H, d), io_dtype),
                                    requests=np.array([0], dtype=np.int32)))
        own_cnt = (nc - shared_prefix_tokens).astype(np.int32)
        assert (own_cnt >= 0).all()
    else:
        own_cnt = nc.copy()
    if int(own_cnt.sum()) > 0:
        t = int(own_cnt.sum())
        history.append(HistoryBatch(count=own_cnt, total=nc.copy(),
                                    key=_normal([seed, 1, 1, 0], (t, H, d), io_dtype),
                                    value=_normal([seed, 1, 1, 1], (t, H, d), io_dtype),
                                    requests=np.arange(n, dtype=np.int32)))

    T = int(ns.sum())
    q = _normal([seed, 2, 0], (T, num_q_heads, d), io_dtype)
    k = _normal([seed, 2, 1], (T, H, d), io_dtype)
    v = _normal([seed, 2, 2], (T, H, d), io_dtype)

    k_scale = v_scale = 1.0
    if kv_dtype == FP8:
        ka = max([float(np.abs(_as_f32(h.key, io_dtype)).max()) for h in history] +
                 [float(np.abs(_as_f32(k, io_dtype)).max()) if T else 0.0])
        va = max([float(np.abs(_as_f32(h.value, io_dtype)).max()) for h in history] +
                 [float(np.abs(_as_f32(v, io_dtype)).max()) if T else 0.0])
        k_scale = float(np.float32(ka) / np.float32(FP8_E4M3_MAX))
        v_scale = float(np.float32(va) / np.float32(FP8_E4M3_MAX))

    return Workload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=H,
                    head_dim=d, block_size=S, num_blocks=num_blocks, kv_dtype=kv_dtype,
                    io_dtype=io_dtype, num_computed=nc, num_scheduled=ns, block_table=bt,
                    history=history, query=q, key=k, value=v, k_scale=k_scale,
                    v_scale=v_scale, shared_prefix_blocks=sp_blocks)


# --------------------------------------------------------------------------
# The five reference workloads.  Lengths follow the configuration text:
# "context len" is the request's length including this step's tokens.
# Requests are ordered decodes first, then prefill chunks.
# --------------------------------------------------------------------------

def tiny_f32(seed: int = 0) -> Workload:
    """4 requests, 4 q = 4 kv heads, d = 64, S = 16, 32-block pool, fp32.
    Context lengths {17, 33, 1, 64}: three decode tokens and one 8-token chunk."""
    rng = np.random.default_rng(seed)
    ctx = np.array([17, 33, 1, 64], dtype=np.int32)
    ns = np.array([1, 1, 1, 8], dtype=np.int32)
    return build("tiny_f32", seed, num_q_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
                 num_blocks=32, kv_dtype=F32, io_dtype=F32, num_computed=ctx - ns,
                 num_scheduled=ns, rng=rng)


def llama8b_decode(seed: int = 0, num_seqs: int = 64, lo: int = 512, hi: int = 4096,
                   num_blocks: int = 40000) -> Workload:
    """64 decode requests, 32 q / 8 kv heads, d = 128, S = 16, bf16, context U[512, 4096]."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    ns = np.ones(num_seqs, dtype=np.int32)
    return build("llama8b_decode", seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=16, num_blocks=num_blocks, kv_dtype=BF16, io_dtype=BF16,
                 num_computed=ctx - ns, num_scheduled=ns, rng=rng)


def mixed_step(seed: int = 0, num_decode: int = 48, lo: int = 256, hi: int = 8192,
               chunk_a: int = 512, chunk_b: int = 1488, chunk_b_cached: int = 1536,
               num_blocks: int = 40000) -> Workload:
    """Token budget 2048: 48 decodes (context U[256, 8192]) + a 512-token chunk with no
    history + a 1488-token chunk after 1536 cached tokens.  32 q / 8 kv, d = 128, bf16."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=num_decode).astype(np.int32)
    nc = np.concatenate([ctx - 1, [0, chunk_b_cached]]).astype(np.int32)
    ns = np.concatenate([np.ones(num_decode), [chunk_a, chunk_b]]).astype(np.int32)
    return build("mixed_step", seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=16, num_blocks=num_blocks, kv_dtype=BF16, io_dtype=BF16,
                 num_computed=nc, num_scheduled=ns, rng=rng)


def long_decode_70b(seed: int = 0, num_seqs: int = 8, lo: int = 32 * 1024, hi: int = 128 * 1024,
                    num_blocks: int = 81920) -> Workload:
    """8 decode requests, 64 q / 8 kv heads, d = 128, bf16, context U[32k, 128k] (k = 1024)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    ns = np.ones(num_seqs, dtype=np.int32)
    return build("long_decode_70b", seed, num_q_heads=64, num_kv_heads=8, head_dim=128,
                 block_size=16, num_blocks=num_blocks, kv_dtype=BF16, io_dtype=BF16,
                 num_computed=ctx - ns, num_scheduled=ns, rng=rng)


def prefix_fp8_decode(seed: int = 0, num_seqs: int = 128, prefix: int = 2048, lo: int = 64,
                      hi: int = 512, num_blocks: int = 40000) -> Workload:
    """128 decode requests sharing a 2048-token (128-block) prefix plus unique suffixes of
    U[64, 512] tokens; fp8 e4m3 pool with per-tensor fp32 scales; q/k/v/out bf16."""
    rng = np.random.default_rng(seed)
    suffix = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    ctx = prefix + suffix
    ns = np.ones(num_seqs, dtype=np.int32)
    return build("prefix_fp8_decode", seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=16, num_blocks=num_blocks, kv_dtype=FP8, io_dtype=BF16,
                 num_computed=ctx - ns, num_scheduled=ns, shared_prefix_tokens=prefix, rng=rng)


def spec_verify(seed: int = 0, num_seqs: int = 64, lo: int = 512, hi: int = 4096, c_lo: int = 2,
                c_hi: int = 8, num_blocks: int = 40000) -> Workload:
    """Speculative-decoding verify step on the Llama-3-8B decode layer: 64 requests, each
    with a chunk of U[2, 8] draft tokens after a history such that the context is
    U[512, 4096] tokens; 32 q / 8 kv heads, d = 128, bf16: the shape of a batch that
    checks draft tokens (each request has a few new rows over a long history)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    ns = rng.integers(c_lo, c_hi + 1, size=num_seqs).astype(np.int32)
    return build("spec_verify", seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=16, num_blocks=num_blocks, kv_dtype=BF16, io_dtype=BF16,
                 num_computed=ctx - ns, num_scheduled=ns, rng=rng)


def long_prefill(seed: int = 0, num_seqs: int = 2, chunk: int = 4096, cached: int = 2048,
                 num_blocks: int = 40000) -> Workload:
    """Chunked prefill of long prompts on the Llama-3-8B layer: 2 requests, each a
    4096-token chunk after 2048 cached tokens (causal over chunk + history); 32 q / 8 kv
    heads, d = 128, bf16.  A batch large enough to fill the chip with prefill tiles."""
    rng = np.random.default_rng(seed)
    nc = np.full(num_seqs, cached, dtype=np.int32)
    ns = np.full(num_seqs, chunk, dtype=np.int32)
    return build("long_prefill", seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=16, num_blocks=num_blocks, kv_dtype=BF16, io_dtype=BF16,
                 num_computed=nc, num_scheduled=ns, rng=rng)


CONFIGS = {
    1: tiny_f32,
    2: llama8b_decode,
    3: mixed_step,
    4: long_decode_70b,
    5: prefix_fp8_decode,
    6: spec_verify,
    7: long_prefill,
}


def make(config: int, seed: int = 0, **overrides) -> Workload:
    return CONFIGS[config](seed, **overrides)


def random_small(seed: int, *, max_seqs: int = 4, max_len: int = 64, block_size: int = 16,
                 num_q_heads: int = 4, num_kv_heads: int = 2, head_dim: int = 64,
                 kv_dtype: str = F32, io_dtype: str = F32, max_chunk: Optional[int] = None,
                 spare_blocks: int = 8) -> Workload:
    """Tiny randomized batch (for brute-force and edge-case checks)."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, max_seqs + 1))
    total = rng.integers(1, max_len + 1, size=n).astype(np.int32)
    cap = total if max_chunk is None else np.minimum(total, max_chunk)
    ns = np.array([int(rng.integers(1, c + 1)) for c in cap], dtype=np.int32)
    nc = total - ns
    need = sum(_blocks_needed(t, block_size) for t in total)
    return build(f"random_small_{seed}", seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, block_size=block_size, num_blocks=need + spare_blocks,
                 kv_dtype=kv_dtype, io_dtype=io_dtype, num_computed=nc, num_scheduled=ns, rng=rng)


def to_f32(a: np.ndarray, io_dtype: str) -> np.ndarray:
    """Values of an io array as float32 (bf16 bits widened exactly)."""
    return _as_f32(a, io_dtype)


def work_summary(w: Workload) -> dict:
    tot = (w.num_computed.astype(np.int64) + w.num_scheduled)
    return {
        "workload": w.name, "seed": w.seed, "num_seqs": w.num_seqs, "num_tokens": w.num_tokens,
        "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
        "block_size": w.block_size, "num_blocks": w.num_blocks, "kv_dtype": w.kv_dtype,
        "io_dtype": w.io_dtype, "context_total": int(tot.sum()),
        "context_min": int(tot.min()), "context_max": int(tot.max()),
    }


__all__ = ["Workload", "HistoryBatch", "build", "make", "CONFIGS", "random_small",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "to_f32", "work_summary",
           "F32", "BF16", "FP8", "FP8_E4M3_MAX"]


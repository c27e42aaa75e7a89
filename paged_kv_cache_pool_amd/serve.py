"""A continuous-batching loop around the attention step.

Each step follows the scheduler and model-runner passes of "vLLM 推理流程分析":
  * schedule (§4.2-4.3): running requests first, each with its next tokens
    (one for a decode, the rest of the prompt up to the token budget for a
    chunked prefill), through allocate_slots.  Then waiting requests, each
    looked up in the prefix cache (get_computed_blocks) and admitted while
    the token budget and the pool allow.  A request is admitted only when
    the free blocks cover its whole length (prompt and new tokens) on top of
    what the running requests may still take, so a running request's
    allocation never fails and no request is ever preempted (preemption is
    control plane, left out);
  * execute (§5.1.1-5.1.3, §6): the newly allocated blocks are zeroed, the
    batch metadata (query_start_loc, seq_lens, the block table) is built on
    the host and copied to the device, and the one-call step writes the new
    tokens' K/V and runs the attention;
  * commit (§7-8): every scheduled request's computed count advances, its
    full blocks enter the prefix cache, a request whose known tokens are all
    computed emits its next token, and a request with all its tokens is
    freed (§8.1).

Model stand-in: there are no weights, so a token's K/V (and its query) is a
deterministic function of the token ids up to it and the request's extra
key, drawn from a seeded normal generator; requests that share a prefix
therefore produce the same K/V for it, which is what makes a prefix-cache
hit valid.  The "sampled" next token is a deterministic function of the
same chain.  The host block pool is the library's pa_kv_manager.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding as B
from .workloads import BF16, f32_to_bf16_bits

_VOCAB = 32000


def _chain(prev: int, token: int, extra_key: int) -> int:
    # 64-bit mix of the previous chain value, the token and the extra key
    # (splitmix64 finaliser); the chain value keys the token's K/V rows
    x = (prev ^ ((token & 0xFFFFFFFF) * 0x9E3779B97F4A7C15) ^ (extra_key * 0xD1B54A32D192ED03)) & ((1 << 64) - 1)
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
    return x ^ (x >> 31)


@dataclasses.dataclass
class Request:
    req_id: int
    prompt: List[int]
    max_new_tokens: int
    extra_key: int = 0
    tokens: List[int] = dataclasses.field(default_factory=list)
    chain: List[int] = dataclasses.field(default_factory=list)   # chain value after each token
    num_computed: int = 0
    generated: int = 0
    status: str = "waiting"

    def __post_init__(self):
        if not self.tokens:
            self.tokens = list(self.prompt)
        if not self.chain:
            c = 0
            for t in self.tokens:
                c = _chain(c, t, self.extra_key)
                self.chain.append(c)


@dataclasses.dataclass
class StepPlan:
    """One step's batch, built on the host (the scheduler's output plus the
    metadata the model runner derives from it)."""
    req_ids: List[int]
    num_computed: np.ndarray      # per scheduled request, before the step
    num_scheduled: np.ndarray
    query_start_loc: np.ndarray
    seq_lens: np.ndarray
    block_table: np.ndarray       # [N][width], -1 past each request's blocks
    new_blocks: List[int]         # new_block_ids_to_zero
    prefix_hits: Dict[int, int]   # request -> hit blocks, for requests admitted this step
    query: np.ndarray             # [T][Hq][D] io dtype (bf16 bits or float32)
    key: np.ndarray               # [T][Hkv][D]
    value: np.ndarray

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])


class ServingLoop:
    def __init__(self, pool: B.KVPool, num_q_heads: int, io_dtype: str = BF16,
                 token_budget: int = 256, max_num_seqs: int = 64, enable_prefix_cache: bool = True,
                 device: str = "cuda"):
        self.pool, self.device = pool, device
        self.S = pool.block_size
        self.Hq, self.Hkv, self.D = num_q_heads, pool.num_kv_heads, pool.head_dim
        self.io_dtype = io_dtype
        self.scale = 1.0 / np.sqrt(self.D)
        self.budget, self.max_num_seqs = token_budget, max_num_seqs
        self.prefix_cache = enable_prefix_cache
        self.manager = B.KVManager(pool.num_blocks, pool.block_size)
        self.requests: Dict[int, Request] = {}
        self.waiting: List[int] = []
        self.running: List[int] = []
        self.finished: List[int] = []
        self.steps = 0
        self.admission_waits = 0      # steps whose admission stopped for want of blocks

    # ------------------------------------------------------------ requests --
    def add_request(self, req: Request) -> None:
        if self._total_blocks(req) > self.pool.num_blocks:
            raise ValueError(f"request {req.req_id} needs {self._total_blocks(req)} blocks, "
                             f"the pool has {self.pool.num_blocks}")
        self.requests[req.req_id] = req
        self.waiting.append(req.req_id)

    def done(self) -> bool:
        return not self.waiting and not self.running

    def _rows(self, req: Request, lo: int, hi: int):
        """Query, key and value rows of tokens lo .. hi-1 of the request."""
        n = hi - lo
        q = np.empty((n, self.Hq, self.D), np.float32)
        k = np.empty((n, self.Hkv, self.D), np.float32)
        v = np.empty((n, self.Hkv, self.D), np.float32)
        for i in range(n):
            g = np.random.default_rng(req.chain[lo + i])
            q[i] = g.standard_normal((self.Hq, self.D), dtype=np.float32)
            k[i] = g.standard_normal((self.Hkv, self.D), dtype=np.float32)
            v[i] = g.standard_normal((self.Hkv, self.D), dtype=np.float32)
        return q, k, v

    # ------------------------------------------------------------ schedule --
    def _total_blocks(self, req: Request) -> int:
        # blocks of the request's whole length (an upper bound: the last new
        # token is never computed)
        return -(-(len(req.prompt) + req.max_new_tokens) // self.S)

    def _outstanding(self) -> int:
        # blocks the running requests may still allocate
        return sum(max(0, self._total_blocks(self.requests[r]) - len(self.manager.block_ids(r)))
                   for r in self.running)

    def schedule(self) -> Optional[StepPlan]:
        budget = self.budget
        sched: List[int] = []
        nsched: Dict[int, int] = {}
        new_blocks: List[int] = []
        hits_of: Dict[int, int] = {}
        # running requests (decodes and unfinished chunked prefills)
        i = 0
        while i < len(self.running) and budget > 0:
            rid = self.running[i]
            req = self.requests[rid]
            n = min(len(req.tokens) - req.num_computed, budget)
            if n <= 0:
                i += 1
                continue
            new = self.manager.allocate_slots(rid, req.num_computed + n)
            if new is None:
                raise RuntimeError(f"request {rid}: no free block although its blocks were reserved")
            new_blocks += new
            sched.append(rid)
            nsched[rid] = n
            budget -= n
            i += 1
        # waiting requests, admitted while their whole length fits (hit
        # blocks counted as new: a hit on a free cached block takes it from
        # the free queue)
        while self.waiting and budget > 0 and len(self.running) < self.max_num_seqs:
            rid = self.waiting[0]
            req = self.requests[rid]
            if self._total_blocks(req) > self.manager.num_free_blocks() - self._outstanding():
                self.admission_waits += 1
                break
            hits = self.manager.get_computed_blocks(req.tokens, req.extra_key) if self.prefix_cache else []
            computed = len(hits) * self.S
            n = min(len(req.tokens) - computed, budget)
            new = self.manager.allocate_slots(rid, computed + n, hits)
            if new is None:
                raise RuntimeError(f"request {rid}: no free block although the admission check passed")
            self.waiting.pop(0)
            self.running.append(rid)
            req.status, req.num_computed = "running", computed
            hits_of[rid] = len(hits)
            new_blocks += new
            sched.append(rid)
            nsched[rid] = n
            budget -= n
        if not sched:
            return None
        return self._build(sched, nsched, new_blocks, hits_of)

    def _build(self, sched, nsched, new_blocks, hits_of) -> StepPlan:
        nc = np.array([self.requests[r].num_computed for r in sched], np.int32)
        ns = np.array([nsched[r] for r in sched], np.int32)
        qsl, sl = B.prepare_metadata(nc, ns)
        rows = [self.manager.block_ids(r) for r in sched]
        width = max(len(x) for x in rows)
        bt = np.full((len(sched), width), -1, np.int32)
        for i, x in enumerate(rows):
            bt[i, :len(x)] = x
        qs, ks, vs = [], [], []
        for r, c, n in zip(sched, nc, ns):
            q, k, v = self._rows(self.requests[r], int(c), int(c + n))
            qs.append(q), ks.append(k), vs.append(v)
        q, k, v = (np.concatenate(x) for x in (qs, ks, vs))
        if self.io_dtype == BF16:
            q, k, v = (f32_to_bf16_bits(x) for x in (q, k, v))
        return StepPlan(list(sched), nc, ns, qsl, sl, bt, list(new_blocks), dict(hits_of), q, k, v)

    # ------------------------------------------------------------- execute --
    def _dev(self, a: np.ndarray) -> torch.Tensor:
        if self.io_dtype == BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(self.device)

    def execute(self, plan: StepPlan, stream=None):
        """Zero the new blocks, then the step (one call with the KV update).
        Returns (output [T][Hq][D] tensor, slot_mapping tensor)."""
        if plan.new_blocks:
            ids = torch.tensor(plan.new_blocks, dtype=torch.int32, device=self.device)
            B.zero_blocks(self.pool, ids, stream=stream)
        batch = B.Batch.from_host(plan.query_start_loc, plan.seq_lens, plan.block_table, self.device)
        q, k, v = self._dev(plan.query), self._dev(plan.key), self._dev(plan.value)
        slots = torch.empty(plan.num_tokens, dtype=torch.int64, device=self.device)
        out = B.write_kv_attention(self.pool, batch, q, k, v, self.Hq, float(self.scale), causal=True,
                                   slots=slots, stream=stream)
        return out, slots

    # -------------------------------------------------------------- commit --
    def commit(self, plan: StepPlan) -> List[int]:
        """Advance the scheduled requests; returns the ids finished this step."""
        done = []
        for r, n in zip(plan.req_ids, plan.num_scheduled):
            req = self.requests[r]
            req.num_computed += int(n)
            if self.prefix_cache:
                self.manager.cache_blocks(r, req.tokens, req.num_computed, req.extra_key)
            if req.num_computed == len(req.tokens):
                tok = int(req.chain[-1] % _VOCAB)
                req.tokens.append(tok)
                req.chain.append(_chain(req.chain[-1], tok, req.extra_key))
                req.generated += 1
                if req.generated >= req.max_new_tokens:
                    req.status = "finished"
                    self.manager.free(r)
                    self.running.remove(r)
                    self.finished.append(r)
                    done.append(r)
        self.steps += 1
        return done

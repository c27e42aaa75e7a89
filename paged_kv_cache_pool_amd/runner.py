"""Run a synthetic workload's step on the GPU through libpa.so.

Device set-up for tests, the smoke check and the benchmark: allocate the
pool (every byte 0xFF, a NaN in each element type, so unwritten slots are
canaries), populate it with the workload's earlier steps using the library's
own metadata, slot derivation and KV write, and then run the step:
slot derivation -> KV write -> attention, all on one stream (or the one call
that does all three).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import BF16, Workload


def to_device(a: np.ndarray, io_dtype: str, device="cuda") -> torch.Tensor:
    if io_dtype == BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class GpuStep:
    def __init__(self, w: Workload, device: str = "cuda", canary: bool = True, causal: bool = True,
                 stream: Optional[torch.cuda.Stream] = None, shared_prefix: bool = True,
                 fused: bool = False):
        self.w, self.device, self.causal, self.fused = w, device, causal, fused
        self.stream = stream or torch.cuda.current_stream()
        self.pool = B.KVPool.allocate(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                      w.kv_dtype, w.k_scale, w.v_scale, device=device,
                                      fill_byte=0xFF if canary else 0)
        with torch.cuda.stream(self.stream):
            for h in w.history:
                qsl, sl = B.prepare_metadata(h.total - h.count, h.count)
                hb = B.Batch.from_host(qsl, sl, w.block_table[h.requests], device)
                slots = B.slot_mapping(hb, w.block_size, stream=self.stream)
                B.write_kv(self.pool, to_device(h.key, w.io_dtype, device),
                           to_device(h.value, w.io_dtype, device), slots, stream=self.stream)
            qsl, sl = B.prepare_metadata(w.num_computed, w.num_scheduled)
            # the workload's common prefix (blocks every request starts with) is
            # passed as the scheduler's shared-prefix hint unless disabled
            npref = w.shared_prefix_blocks if shared_prefix else 0
            self.batch = B.Batch.from_host(qsl, sl, w.block_table, device, num_common_prefix_blocks=npref)
            self.query = to_device(w.query, w.io_dtype, device)
            self.key = to_device(w.key, w.io_dtype, device)
            self.value = to_device(w.value, w.io_dtype, device)
            self.slots = torch.empty(w.num_tokens, dtype=torch.int64, device=device)
            self.out = torch.empty_like(self.query)
            self.ws_bytes = B.attention_workspace_bytes(self.pool, self.batch, w.num_q_heads)
            self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.stream.synchronize()

    def run(self) -> torch.Tensor:
        """One step: a1 slots, a2 KV write, a3-a7 attention (asynchronous); with
        `fused`, all of them in the one call that includes the KV update."""
        w = self.w
        if self.fused:
            B.write_kv_attention(self.pool, self.batch, self.query, self.key, self.value,
                                 w.num_q_heads, w.softmax_scale, causal=self.causal, out=self.out,
                                 workspace=self.workspace, slots=self.slots, stream=self.stream)
            return self.out
        B.slot_mapping(self.batch, w.block_size, out=self.slots, stream=self.stream)
        B.write_kv(self.pool, self.key, self.value, self.slots, stream=self.stream)
        B.attention(self.pool, self.batch, self.query, w.num_q_heads, w.softmax_scale,
                    causal=self.causal, out=self.out, workspace=self.workspace, stream=self.stream)
        return self.out

    def out_f64(self) -> np.ndarray:
        return self.out.float().cpu().numpy().astype(np.float64)

"""The entry point that allocates nothing, pa_write_kv_attention_noalloc,
through the C ABI, against the entry point with a workspace
(pa_write_kv_attention) on the same inputs.

Calls in a row on one device share the library's static scratch: the mixed
2048-token step (every kernel of the path: the scatter pass, the wide extend
launch, the split-K decode and the merge), the fp8 shared-prefix step (prefix
items and the prefix row lists in the split-K launch), then a smaller batch
(the source-map page's mixed batch).  Each call's slots, pool bytes and output
must equal the workspace entry point's exactly (same plan, same kernels), and
the output must match the oracle within the attention tolerance.  A batch
whose plan does not fit the static scratch is refused before any launch.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_pool_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-5, W.BF16: 2e-2, W.FP8: 2e-2}


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
    sys.stdout.flush()


def _used_blocks(w):
    return np.unique(w.block_table[w.block_table >= 0])


def _page_mixed():
    return W.build("page_mixed", 3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                   num_blocks=200, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[1024, 512, 600],
                   num_scheduled=[1, 256, 3])


def test_noalloc_matches_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import binding as B
    from paged_kv_cache_pool_amd import runner
    for w in (W.make(3), W.make(5), _page_mixed()):
        say("workload", w.name, "tokens", w.num_tokens)
        ref_step = runner.GpuStep(w, fused=True)       # pa_write_kv_attention, own workspace
        ref_step.run()
        step = runner.GpuStep(w, fused=True)           # same pool contents before the call
        step.out.fill_(float("nan"))
        step.slots.fill_(-7)
        B.write_kv_attention_noalloc(step.pool, step.batch, step.query, step.key, step.value,
                                     w.num_q_heads, w.softmax_scale, causal=True, out=step.out,
                                     slots=step.slots, stream=step.stream)
        torch.cuda.synchronize()
        assert torch.equal(step.slots, ref_step.slots)
        blocks = _used_blocks(w)
        for which in ("k", "v"):
            assert (step.pool.logical(which, blocks) == ref_step.pool.logical(which, blocks)).all(), which
        assert torch.equal(step.out.view(torch.uint8), ref_step.out.view(torch.uint8))
        ref = O.run_step(w).out
        err = float(np.abs(step.out_f64() - ref).max())
        say(w.name, "equal to the workspace entry point; max_abs_err vs oracle", err)
        assert err <= TOL[w.kv_dtype]
        del ref_step, step


def test_noalloc_refuses_a_batch_beyond_the_scratch(monkeypatch):
    """Four decode rows of 16k keys cut into 64-key partitions need 1024
    partial slots of 64 heads (about 34 MB, more than the 32 MiB scratch):
    refused with PA_ERR_WORKSPACE on the host, nothing launched, the pool
    untouched."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import binding as B
    from paged_kv_cache_pool_amd import runner
    w = W.build("noalloc_big", 1, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=4 * 16384 // 16 + 8, kv_dtype=W.BF16, io_dtype=W.BF16,
                num_computed=[16383] * 4, num_scheduled=[1] * 4)
    step = runner.GpuStep(w, fused=True)
    monkeypatch.setenv("PA_PARTITION_KEYS", "64")
    monkeypatch.setenv("PA_DECODE_PAIRS", "0")
    need = B.attention_workspace_bytes(step.pool, step.batch, w.num_q_heads)
    assert need > B.noalloc_scratch_bytes()
    before = step.pool.k_cache.clone()
    with pytest.raises(B.PaError) as e:
        B.write_kv_attention_noalloc(step.pool, step.batch, step.query, step.key, step.value,
                                     w.num_q_heads, w.softmax_scale, out=step.out, slots=step.slots,
                                     stream=step.stream)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.equal(step.pool.k_cache, before)

"""GPU parity at the workloads' full sizes, every row, both forms of the step.

For each seeded workload (the five reference configurations, the verify
batch and the long prefill; seeds 1-4 on configurations 1, 2, 3 and 5, seeds
1-2 on the long-context decode and the verify batch) the
HIP path runs once as three calls (pa_slot_mapping -> pa_write_kv ->
pa_attention) and once as the one call with the KV update
(pa_write_kv_attention), in the launch configuration bench.py times, and is
compared with the CPU oracle on the same inputs:

* slots: equal to the oracle's slot derivation;
* pool bytes: every block any request uses, plus 64 unused blocks that must
  still hold their canaries, byte for byte through logical (block, offset,
  head, dim) indexing (this covers the blocks that receive the new tokens);
* attention: every output row, max |O_gpu - O_oracle| <= 1e-5 (fp32 pool) or
  2e-2 (bf16 / fp8 pools).

The long prefill (8192 rows of 6144 keys) is compared in four row slices so
that each test stays short; its GPU output is computed once per form.
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
    print("[gpu-fullsize]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def R():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import runner
    return runner


# The oracle's step of the latest (config, seed), shared by the two forms
# (the cases below list both forms of a workload one after the other).
_ORACLE = {}


def _oracle_step(cfg, seed):
    key = (cfg, seed)
    if key not in _ORACLE:
        _ORACLE.clear()
        w = W.make(cfg, seed)
        _ORACLE[key] = (w, O.run_step(w))
    return _ORACLE[key]


def _compare_blocks(w, step, orc_pool):
    used = np.unique(w.block_table[w.block_table >= 0])
    rng = np.random.default_rng(w.seed + 17)
    unused = np.setdiff1d(np.arange(w.num_blocks), used)
    blocks = np.sort(np.concatenate([used, rng.choice(unused, size=min(64, unused.size), replace=False)])
                     if unused.size else used)
    for which in ("k", "v"):
        g = step.pool.logical(which, blocks)
        o = (orc_pool.k if which == "k" else orc_pool.v)[blocks]
        gv = g.view(np.uint32) if g.dtype == np.float32 else g
        ov = o.view(np.uint32) if o.dtype == np.float32 else o
        bad = np.argwhere(gv != ov)
        assert bad.size == 0, f"{which} pool differs at {bad[:5].tolist()} (of {len(bad)})"
    return len(used)


def _compare_rows(w, got, ref):
    assert got.shape == ref.shape
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    worst = np.unravel_index(err.argmax(), err.shape)
    say(w.name, "seed", w.seed, "rows", ref.shape[0], "max_abs_err", float(err.max()),
        "mean", float(err.mean()), "max|O|", float(np.abs(ref).max()), "at", worst)
    assert err.max() <= TOL[w.kv_dtype], (float(err.max()), worst)


CASES = [(c, 0, f) for c in (1, 2, 3, 4, 5, 6) for f in (False, True)] + \
        [(c, s, f) for c in (1, 2, 3, 5) for s in (1, 2, 3, 4) for f in (False, True)] + \
        [(c, s, f) for c in (4, 6) for s in (1, 2) for f in (False, True)]


@pytest.mark.parametrize("cfg,seed,fused", CASES,
                         ids=[f"cfg{c}-seed{s}-{'one_call' if f else 'three_calls'}" for c, s, f in CASES])
def test_full_step(R, cfg, seed, fused):
    say("config", cfg, "seed", seed, "one call" if fused else "three calls")
    w, ref = _oracle_step(cfg, seed)
    step = R.GpuStep(w, fused=fused)
    step.run()
    torch.cuda.synchronize()
    assert (step.slots.cpu().numpy() == ref.slots).all(), "slots differ from the oracle"
    n_used = _compare_blocks(w, step, ref.pool)
    say("pool bytes equal on", n_used, "used blocks")
    _compare_rows(w, step.out_f64(), ref.out)


# ------------------------------------------------------------ long prefill --

_LP = {}


def _long_prefill_gpu(R, fused):
    if fused not in _LP:
        w = W.make(7)
        step = R.GpuStep(w, fused=fused)
        step.run()
        torch.cuda.synchronize()
        qsl = O.query_start_loc(w.num_scheduled)
        sl = O.seq_lens(w.num_computed, w.num_scheduled)
        assert (step.slots.cpu().numpy() == O.slot_mapping(qsl, sl, w.block_table, w.block_size)).all()
        _LP[fused] = (w, step.out_f64())
        del step
        torch.cuda.empty_cache()
    return _LP[fused]


_LP_REF = {}


@pytest.mark.parametrize("part", range(4))
def test_long_prefill_rows(R, part):
    """Every row of the long prefill (two 4096-row chunks after 2048 cached
    tokens), a quarter per test, in both forms of the step."""
    say("long prefill rows, part", part)
    w_gpu, _ = _long_prefill_gpu(R, False)
    T = w_gpu.num_tokens
    rows = np.arange(part * T // 4, (part + 1) * T // 4, dtype=np.int32)
    if part not in _LP_REF:
        _LP_REF.clear()
        _LP_REF[part] = O.run_step(w_gpu, tokens=rows).out
    ref = _LP_REF[part]
    for fused in (False, True):
        w, got = _long_prefill_gpu(R, fused)
        _compare_rows(w, got[rows], ref)


def test_long_prefill_pool(R):
    """The long prefill's written pool blocks, byte for byte, in both forms."""
    say("long prefill pool")
    w = W.make(7)
    orc = O.build_pool(w)
    qsl = O.query_start_loc(w.num_scheduled)
    sl = O.seq_lens(w.num_computed, w.num_scheduled)
    O.write_kv(orc, w.key, w.value, w.io_dtype, O.slot_mapping(qsl, sl, w.block_table, w.block_size))
    for fused in (False, True):
        step = R.GpuStep(w, fused=fused)
        step.run()
        torch.cuda.synchronize()
        _compare_blocks(w, step, orc)
        del step
    _LP.clear()

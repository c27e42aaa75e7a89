"""GPU parity of the wide prefill kernel (256 columns per workgroup) and of its
key pieces, against the CPU oracle on the same seeded inputs.

Requests with more than 128 (token, head) columns go to the wide kernel; when
their items are long compared with the average load of a compute unit, their
key ranges are cut into pieces whose partial (m, l, o) the merge kernel
combines.  PA_WIDE_PIECES forces the number of pieces, so small batches cover
the piece path; PA_DISABLE_WIDE routes the same rows to the key-split kernel.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_pool_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[gpu-wide]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def R():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import runner
    return runner


def _chunk_batch(name, g, c, hist, kv, extra_decode=True):
    nq = [hist, 70] if extra_decode else [hist]
    ns = [c, 1] if extra_decode else [c]
    total = c + hist + 80
    return W.build(name, total, num_q_heads=2 * g, num_kv_heads=2, head_dim=128, block_size=16,
                   num_blocks=-(-total // 16) + 40, kv_dtype=kv, io_dtype=W.BF16,
                   num_computed=nq, num_scheduled=ns)


def _run(R, w, causal=True):
    step = R.GpuStep(w, causal=causal)
    step.run()
    torch.cuda.synchronize()
    return step


def _err(w, step, causal=True):
    ref = O.run_step(w, causal=causal).out
    got = step.out_f64()
    assert np.isfinite(got).all()
    return float(np.abs(got - ref).max())


# (g, c, hist): every case has more than 128 (token, head) columns, so it
# reaches the wide kernel (g = 1 takes longer chunks for that)
WIDE_CASES = [(g, c, h) for g in (1, 4, 8, 16)
              for c, h in ([(140, 0), (200, 37)] if g == 1 else [(40, 0), (100, 37)]) + [(257, 300), (600, 1000)]]


@pytest.mark.parametrize("pieces", ["1", "2", "3"])
@pytest.mark.parametrize("g,c,hist", WIDE_CASES)
def test_wide_chunks(R, monkeypatch, pieces, g, c, hist):
    """Causal chunks with history on the wide kernel, whole key range or cut
    into 2 / 3 pieces, with ragged column blocks (c * g not a multiple of
    256) and a decode row in the same batch."""
    assert c * g > 128
    monkeypatch.setenv("PA_WIDE_PIECES", pieces)
    say("wide g", g, "c", c, "hist", hist, "pieces", pieces)
    w = _chunk_batch(f"wide_{g}_{c}_{hist}", g, c, hist, W.BF16)
    err = _err(w, _run(R, w))
    say("  max_abs_err", err)
    assert err <= TOL


@pytest.mark.parametrize("pieces", ["1", "2"])
@pytest.mark.parametrize("g", [4, 8, 16])
@pytest.mark.parametrize("c,hist", [(100, 37), (600, 1000)])
def test_wide_chunks_fp8(R, monkeypatch, pieces, g, c, hist):
    """The same over an fp8 pool (k_scale folded into the scores, v_scale
    into the output and into the pieces' partials)."""
    monkeypatch.setenv("PA_WIDE_PIECES", pieces)
    say("wide fp8 g", g, "c", c, "hist", hist, "pieces", pieces)
    w = _chunk_batch(f"wide8_{g}_{c}_{hist}", g, c, hist, W.FP8)
    err = _err(w, _run(R, w))
    say("  max_abs_err", err)
    assert err <= TOL


@pytest.mark.parametrize("pieces", ["1", "2"])
def test_wide_noncausal(R, monkeypatch, pieces):
    monkeypatch.setenv("PA_WIDE_PIECES", pieces)
    say("wide non-causal, pieces", pieces)
    w = W.build("wide_nc", 4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=60, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[300, 0, 20],
                num_scheduled=[200, 90, 1])
    err = _err(w, _run(R, w, causal=False), causal=False)
    say("  max_abs_err", err)
    assert err <= TOL


def test_wide_matches_key_split_kernel(R, monkeypatch):
    """The wide kernel and the key-split kernel on the same rows: both within
    the tolerance of the oracle, and close to each other (they differ only in
    the order of fp32 additions and where P is rounded)."""
    w = _chunk_batch("wide_vs_split", 4, 333, 555, W.BF16)
    monkeypatch.setenv("PA_WIDE_PIECES", "2")
    a = _run(R, w).out_f64()
    monkeypatch.setenv("PA_DISABLE_WIDE", "1")
    b = _run(R, w).out_f64()
    ref = O.run_step(w).out
    say("wide", float(np.abs(a - ref).max()), "key-split", float(np.abs(b - ref).max()),
        "between", float(np.abs(a - b).max()))
    assert np.abs(a - ref).max() <= TOL and np.abs(b - ref).max() <= TOL
    assert np.abs(a - b).max() <= TOL


@pytest.mark.parametrize("pieces", ["1", "2", "3"])
def test_one_hot_probe_wide_bit_exact(R, monkeypatch, pieces):
    """One-hot probe through the wide kernel and the piece merge: 100 new rows
    x 4 heads (400 columns) all select one history position j*; every other
    weight underflows to exactly 0 in fp32, in its own piece as well as in
    the merge, so O = v[j*] exactly."""
    monkeypatch.setenv("PA_WIDE_PIECES", pieces)
    H, D, hist, c = 2, 128, 16 * 20 + 3, 100
    w = W.build("probe_wide", 1, num_q_heads=8, num_kv_heads=H, head_dim=D, block_size=16,
                num_blocks=40, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[hist],
                num_scheduled=[c])
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    vals = np.arange(hist)[:, None, None] * sign[None, None, :] * np.ones((1, H, 1))
    w.history[0].value[:] = W.f32_to_bf16_bits(vals.astype(np.float32))
    w.value[:] = W.f32_to_bf16_bits((200.0 * sign + np.zeros((c, H, D))).astype(np.float32))
    w.query[:] = W.f32_to_bf16_bits(np.ones((c, 8, D), np.float32))
    w.key[:] = 0
    for jstar in [0, 70, 200, hist - 1]:
        say("probe pieces", pieces, "j*", jstar)
        w.history[0].key[:] = 0
        w.history[0].key[jstar] = W.f32_to_bf16_bits(np.full((H, D), 16.0, np.float32))
        step = _run(R, w)
        got = step.out.float().cpu().numpy()
        assert (got == (jstar * sign)[None, None, :]).all(), (jstar, got[0, 0, :6])


def test_wide_default_large_prefill(R, monkeypatch):
    """Two 4096-token prefill chunks, each after 2048 cached tokens (8 kv
    heads, g = 4), and a decode row: large enough that the planner's own rule
    picks the wide kernel (its longest item, 96 tiles, is below half of a
    compute unit's average load).  Sampled rows (the first and last of each
    chunk among them) against the oracle, which computes them one by one."""
    monkeypatch.delenv("PA_WIDE_PIECES", raising=False)
    monkeypatch.delenv("PA_DISABLE_WIDE", raising=False)
    w = W.build("wide_large", 11, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=2 * (2048 + 4096) // 16 + 80, kv_dtype=W.BF16, io_dtype=W.BF16,
                num_computed=[2048, 2048, 70], num_scheduled=[4096, 4096, 1])
    step = _run(R, w)
    rng = np.random.default_rng(3)
    must = {0, 4095, 4096, 8191, 8192}
    tokens = np.array(sorted(must | set(rng.choice(8192, 30, replace=False).tolist())), np.int32)
    ref = O.run_step(w, tokens=tokens).out
    got = step.out_f64()[tokens]
    err = float(np.abs(got - ref).max())
    say("large prefill sampled max_abs_err", err)
    assert np.isfinite(got).all() and err <= TOL


@pytest.mark.parametrize("plan_copy", ["", "1"])
@pytest.mark.parametrize("fused", [True, False])
def test_wide_pieces_graph_capture(R, monkeypatch, fused, plan_copy):
    """A step with wide items cut into two key pieces (so the merge runs too),
    captured into a HIP graph: every replay equals the eager step bit for bit,
    with an eager step of another batch between replays, and matches the
    oracle; a replay reads new query contents and matches the oracle for
    them."""
    monkeypatch.setenv("PA_WIDE_PIECES", "2")
    monkeypatch.setenv("PA_GRAPH_PLAN_COPY", plan_copy)
    w = _chunk_batch("wide_graph", 4, 600, 1000, W.BF16)
    s = torch.cuda.Stream()
    step = R.GpuStep(w, stream=s, fused=fused)
    with torch.cuda.stream(s):
        step.run()
    s.synchronize()
    eager = step.out.clone()
    assert _err(w, step) <= TOL
    other = R.GpuStep(_chunk_batch("wide_graph_other", 8, 257, 300, W.BF16), fused=True)
    g = torch.cuda.CUDAGraph()
    step.out.zero_()
    with torch.cuda.graph(g, stream=s):
        step.run()
    torch.cuda.synchronize()
    for rep in range(3):
        say("wide graph replay", rep, "fused", fused)
        step.out.fill_(float("nan"))
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out.view(torch.uint8), eager.view(torch.uint8)), rep
    step.query.mul_(0.5)
    g.replay()
    torch.cuda.synchronize()
    replayed = step.out.clone()
    # halving is exact in bf16 for these values: the oracle gets the same query
    half = dataclasses.replace(w, query=W.f32_to_bf16_bits(W.to_f32(w.query, W.BF16) * np.float32(0.5)))
    err = _err(half, step)
    say("replay after the query change, max_abs_err", err)
    assert err <= TOL
    with torch.cuda.stream(s):
        step.run()
    s.synchronize()
    assert torch.equal(replayed.view(torch.uint8), step.out.view(torch.uint8))

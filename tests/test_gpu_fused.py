"""GPU parity of the attention call that includes the KV update
(pa_write_kv_attention), through the C ABI.

* slots and pool bytes: bit-exact against the oracle's slot derivation and
  scatter, and identical to what the separate calls (pa_slot_mapping,
  pa_write_kv) leave in the pool;
* attention: within the same tolerance as pa_attention against the oracle
  (the newest key of a decode row may be added in another order than in the
  separate path, so the two outputs agree to rounding, not bit for bit).
"""
import ctypes as C
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_pool_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-5, W.BF16: 2e-2, W.FP8: 2e-2}


def say(*a):
    print("[gpu-fused]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def R():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import runner
    return runner


def _pool_bits(pool, which):
    a = pool.logical(which)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _assert_same_pool(p1, p2):
    for which in ("k", "v"):
        a, b = _pool_bits(p1, which), _pool_bits(p2, which)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{which} pools differ at {bad[:5].tolist()} (of {len(bad)})"


def _assert_pool_is_oracle(w, pool):
    orc = O.build_pool(w)
    O.write_kv(orc, w.key, w.value, w.io_dtype, _want_slots(w))
    for which in ("k", "v"):
        o = orc.k if which == "k" else orc.v
        o = o.view(np.uint32) if o.dtype == np.float32 else o
        bad = np.argwhere(_pool_bits(pool, which) != o)
        assert bad.size == 0, f"{which} pool differs from the oracle at {bad[:5].tolist()} (of {len(bad)})"


def _want_slots(w):
    qsl = O.query_start_loc(w.num_scheduled)
    sl = O.seq_lens(w.num_computed, w.num_scheduled)
    return O.slot_mapping(qsl, sl, w.block_table, w.block_size)


def _check_out(w, step, tokens=None):
    ref = O.run_step(w, tokens=tokens).out
    got = step.out_f64()
    if tokens is not None:
        got = got[tokens]
    err = np.abs(got - ref)
    say(w.name, "max_abs_err", float(err.max()), "max|O|", float(np.abs(ref).max()))
    assert np.isfinite(got).all()
    assert err.max() <= TOL[w.kv_dtype], (float(err.max()), np.unravel_index(err.argmax(), err.shape))


def _sample(w, n, seed):
    rng = np.random.default_rng(seed)
    if w.num_tokens <= n:
        return np.arange(w.num_tokens, dtype=np.int32)
    qsl = O.query_start_loc(w.num_scheduled)
    must = {int(qsl[i]) for i in range(w.num_seqs) if w.num_scheduled[i] > 0}
    must |= {int(qsl[i + 1]) - 1 for i in range(w.num_seqs) if w.num_scheduled[i] > 0}
    must = set(sorted(must)[: n // 2])
    rest = rng.choice(w.num_tokens, size=max(0, n - len(must)), replace=False).tolist()
    return np.array(sorted(must | set(rest)), dtype=np.int32)


def _halved(w):
    """The workload's query rows times 0.5 (exact for normal values)."""
    q = W.to_f32(w.query, w.io_dtype) * np.float32(0.5)
    return W.f32_to_bf16_bits(q) if w.io_dtype == W.BF16 else q.astype(np.float32)


def _fused_and_separate(R, w, **kw):
    fused = R.GpuStep(w, fused=True, **kw)
    fused.run()
    sep = R.GpuStep(w, **kw)
    sep.run()
    torch.cuda.synchronize()
    return fused, sep


# routes of a short chunk (2 .. 32 / g rows): multi-row items of the split-K
# kernel (PA_MULTIROW), one split-K unit per row, or the MFMA extend kernel
# (the default)
ROUTES = {"multi": {"PA_MULTIROW": "1"}, "rows": {"PA_EXTEND_MIN_ROWS": "64"},
          "extend": {"PA_EXTEND_MIN_ROWS": "2"}}


def _route(monkeypatch, route):
    for k in ("PA_MULTIROW", "PA_EXTEND_MIN_ROWS"):
        monkeypatch.delenv(k, raising=False)
    for k, v in ROUTES[route].items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("seed", range(30))
def test_fused_equals_separate_random(R, seed):
    """Random ragged batches over every pool type, head size and GQA ratio:
    the one call leaves the same pool bytes and slots as the separate calls,
    and both outputs match the oracle."""
    kv = [W.F32, W.BF16, W.FP8][seed % 3]
    io = W.F32 if kv == W.F32 else W.BF16
    g = [1, 2, 4, 8, 16][(seed // 3) % 5]
    D = [64, 128][(seed // 15) % 2]
    say("fused random", seed, kv, "g", g, "D", D)
    w = W.random_small(seed + 100, max_seqs=6, max_len=300, num_q_heads=2 * g, num_kv_heads=2,
                       head_dim=D, kv_dtype=kv, io_dtype=io, spare_blocks=4)
    if kv == W.FP8:
        w = W.build(w.name, seed + 100, num_q_heads=2 * g, num_kv_heads=2, head_dim=D,
                    block_size=16, num_blocks=w.num_blocks, kv_dtype=W.FP8, io_dtype=W.BF16,
                    num_computed=w.num_computed, num_scheduled=w.num_scheduled)
    fused, sep = _fused_and_separate(R, w)
    assert (fused.slots.cpu().numpy() == sep.slots.cpu().numpy()).all()
    _assert_same_pool(fused.pool, sep.pool)
    _assert_pool_is_oracle(w, fused.pool)
    _check_out(w, fused)
    _check_out(w, sep)


@pytest.mark.parametrize("pairs", ["0", "1", "2"])
@pytest.mark.parametrize("route", ["multi", "rows", "extend"])
@pytest.mark.parametrize("kv", [W.BF16, W.FP8])
def test_fused_decode_partitions_and_verify_rows(R, monkeypatch, kv, route, pairs):
    """Decode rows split into 64-key partitions or into the paired layout's
    pieces, one wave per bin or per piece (the newest key is written by the
    row's last item, which may hold that key alone), next to
    speculative-verify-sized chunks of 2 to 8 rows and one prefill chunk.  The
    chunks' K/V are written by the scatter pass before the attention kernels
    read them; the verify chunks run as multi-row items of the split-K kernel,
    as one split-K unit per row, or on the MFMA extend kernel (the default)."""
    monkeypatch.setenv("PA_PARTITION_KEYS", "64")
    monkeypatch.setenv("PA_DECODE_PAIRS", pairs)
    _route(monkeypatch, route)
    say("fused partitions + verify rows", kv, "route", route, "pairs", pairs)
    nc = [64, 0, 127, 128, 300, 5, 64, 200, 40]
    ns = [1, 1, 1, 1, 1, 4, 8, 2, 24]
    w = W.build(f"fused_parts_{kv}", 7, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=140, kv_dtype=kv, io_dtype=W.BF16, num_computed=nc, num_scheduled=ns)
    fused, sep = _fused_and_separate(R, w)
    assert (fused.slots.cpu().numpy() == _want_slots(w)).all()
    _assert_same_pool(fused.pool, sep.pool)
    _assert_pool_is_oracle(w, fused.pool)
    _check_out(w, fused)


@pytest.mark.parametrize("prefix_pass", ["", "1"])
@pytest.mark.parametrize("pairs", ["0", "1", "2"])
@pytest.mark.parametrize("kv", [W.BF16, W.FP8])
def test_fused_cascade(R, monkeypatch, kv, pairs, prefix_pass):
    """The shared prefix with the KV update: the decode rows' own keys
    (written inside the split-K kernel) follow the prefix, whose attention
    comes from prefix items of the split-K kernel or from the MFMA prefix
    pass (PA_PREFIX_PASS=1); partition form or paired layout (one wave per
    bin or per piece)."""
    monkeypatch.setenv("PA_DECODE_PAIRS", pairs)
    monkeypatch.setenv("PA_PREFIX_PASS", prefix_pass)
    say("fused cascade", kv, "pairs", pairs, "prefix pass", prefix_pass)
    own = [0, 1, 17, 33, 60, 9, 5]
    w = W.build(f"fused_casc_{kv}", 11, num_q_heads=8, num_kv_heads=2, head_dim=128,
                block_size=16, num_blocks=80, kv_dtype=kv, io_dtype=W.BF16,
                num_computed=[48 + o for o in own], num_scheduled=[1, 1, 1, 1, 1, 3, 20],
                shared_prefix_tokens=48)
    fused, sep = _fused_and_separate(R, w)
    _assert_same_pool(fused.pool, sep.pool)
    _assert_pool_is_oracle(w, fused.pool)
    _check_out(w, fused)


@pytest.mark.parametrize("seed", range(24))
def test_multirow_chunks_random(R, monkeypatch, seed):
    """Random batches of short chunks (1 .. 32 / g rows over random histories)
    as multi-row items: g in {1, 2, 4, 8, 16} (so 16 or 32 MFMA columns),
    head dims 64 and 128, bf16 and fp8 pools, causal and not, in the paired
    layout (one wave per bin or per piece) and with forced 64-key partitions,
    so rows' causal limits fall inside, at the start of and after key pieces.
    Both step forms: pool bytes and slots exact, every row against the
    oracle."""
    rng = np.random.default_rng(seed + 500)
    monkeypatch.setenv("PA_MULTIROW", "1")
    kv = [W.BF16, W.FP8][seed % 2]
    g = [1, 2, 4, 8, 16][(seed // 2) % 5]
    D = [128, 64][(seed // 10) % 2]
    causal = seed % 7 != 3
    pairs, part = [("1", None), ("2", None), ("0", "64")][seed % 3]
    monkeypatch.setenv("PA_DECODE_PAIRS", pairs)
    if part:
        monkeypatch.setenv("PA_PARTITION_KEYS", part)
    n = int(rng.integers(1, 12))
    ns = rng.integers(1, max(1, 32 // g) + 1, n)
    nc = rng.integers(0, 400, n)
    say("multi-row random", seed, kv, "g", g, "D", D, "causal", causal, "pairs", pairs, "part", part,
        "rows", ns.tolist())
    w = W.build(f"multirow_{seed}", seed + 500, num_q_heads=2 * g, num_kv_heads=2, head_dim=D,
                block_size=16, num_blocks=int(sum(-(-(a + b) // 16) for a, b in zip(nc, ns))) + 6,
                kv_dtype=kv, io_dtype=W.BF16, num_computed=nc.astype(np.int32),
                num_scheduled=ns.astype(np.int32))
    fused = R.GpuStep(w, fused=True, causal=causal)
    fused.run()
    sep = R.GpuStep(w, causal=causal)
    sep.run()
    torch.cuda.synchronize()
    assert (fused.slots.cpu().numpy() == _want_slots(w)).all()
    _assert_same_pool(fused.pool, sep.pool)
    _assert_pool_is_oracle(w, fused.pool)
    for step in (fused, sep):
        ref = O.run_step(w, causal=causal).out
        err = np.abs(step.out_f64() - ref)
        assert np.isfinite(step.out_f64()).all()
        assert err.max() <= TOL[kv], (float(err.max()), np.unravel_index(err.argmax(), err.shape))


def test_fused_page_mixed_batch(R):
    """The source-map page's mixed batch (one decode row, a 256-token chunk, a
    3-token chunk) through the one call."""
    say("fused page mixed batch")
    w = W.build("page_mixed", 3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=200, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[1024, 512, 600],
                num_scheduled=[1, 256, 3])
    fused, sep = _fused_and_separate(R, w)
    _assert_same_pool(fused.pool, sep.pool)
    _check_out(w, fused)


def test_fused_block_id_outside_pool(R):
    """New tokens whose blocks lie outside the pool: as with the separate calls,
    their slots are reported but nothing is written, and those keys take no
    part in the attention.  Covers a decode row's own write and a 5-token
    chunk split over a valid and an invalid block (scatter pass)."""
    say("fused invalid block id")
    w = W.build("fused_bad_block", 4, num_q_heads=4, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=20, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[16, 40, 70, 30],
                num_scheduled=[1, 1, 1, 5])
    bt = w.block_table.copy()
    bt[0, 1] = -1                   # request 0's new token (position 16)
    bt[1, 2] = w.num_blocks + 3     # request 1's new token (position 40)
    bt[3, 2] = -1                   # request 3's tokens at positions 32..34
    w = dataclasses.replace(w, block_table=bt)
    fused, sep = _fused_and_separate(R, w)
    fs, ss = fused.slots.cpu().numpy(), sep.slots.cpu().numpy()
    assert (fs == ss).all() and fs[0] < 0 and fs[1] >= w.num_blocks * 16
    assert (fs[3:5] >= 0).all() and (fs[5:8] < 0).all()
    _assert_same_pool(fused.pool, sep.pool)
    a, b = fused.out_f64(), sep.out_f64()
    assert np.isfinite(a).all()
    assert np.abs(a - b).max() <= TOL[W.BF16]


def test_fused_rejects_null_rows(R):
    from paged_kv_cache_pool_amd import binding as B
    say("fused null key")
    w = W.make(1)
    step = R.GpuStep(w, fused=True)
    p, b = step.pool.struct(), step.batch.struct()
    st = B.lib.pa_write_kv_attention(C.byref(p), C.byref(b), B._ptr(step.query), None, None,
                                     B.torch_dtype_code(step.query), w.num_q_heads,
                                     w.softmax_scale, 1, None, B._ptr(step.out),
                                     B._ptr(step.workspace), step.workspace.numel(), None)
    assert st == 1


@pytest.mark.parametrize("route", ["multi", "rows", "extend"])
def test_spec_verify_workload(R, monkeypatch, route):
    """The speculative-verify workload (64 requests with 2..8 draft tokens after
    long histories) with the verify chunks as multi-row items of the split-K
    kernel, as one split-K unit per row, and on the MFMA extend kernel (the
    default), one call with the KV update: every row against the oracle,
    slots exact."""
    _route(monkeypatch, route)
    say("spec verify, route", route)
    w = W.make(6)
    step = R.GpuStep(w, fused=True)
    step.run()
    torch.cuda.synchronize()
    assert (step.slots.cpu().numpy() == _want_slots(w)).all()
    _check_out(w, step)


# ------------------------------------------------------------- HIP graphs --

@pytest.mark.parametrize("plan_copy", ["", "1"])
@pytest.mark.parametrize("cfg,fused", [(1, True), (1, False), (2, True), (5, True), (6, True)])
def test_graph_capture_replays(R, monkeypatch, cfg, fused, plan_copy):
    """A step captured into a HIP graph (torch's stream capture around the
    library's calls) replays the same batch: every replay equals the eager
    step bit for bit, with unrelated eager steps of another batch (other
    pool, own plans) run between the replays, and both match the oracle; new
    query contents written between replays are read by the next replay, whose
    output matches the oracle's for the new query.  The captured work lists
    live in the library's captured-plan arena, or (plan_copy) are copied
    into the workspace by kernels inside the graph."""
    monkeypatch.setenv("PA_GRAPH_PLAN_COPY", plan_copy)
    say("graph capture config", cfg, "fused", fused, "plan copy", plan_copy)
    w = W.make(cfg)
    s = torch.cuda.Stream()
    step = R.GpuStep(w, stream=s, fused=fused)
    with torch.cuda.stream(s):
        step.run()
    s.synchronize()
    eager = step.out.clone()
    eager_pool_k = step.pool.k_cache.clone()
    _check_out(w, step)
    other = R.GpuStep(W.make(1, seed=5), fused=True)
    g = torch.cuda.CUDAGraph()
    step.out.zero_()
    with torch.cuda.graph(g, stream=s):
        step.run()
    torch.cuda.synchronize()
    for rep in range(4):
        step.out.fill_(float("nan"))
        other.run()                      # eager calls between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out.view(torch.uint8), eager.view(torch.uint8)), rep
        assert torch.equal(step.pool.k_cache, eager_pool_k)
    # new query contents: the replay reads them (halving is exact in bf16 and
    # fp32 for these values, so the oracle gets the same query)
    step.query.mul_(0.5)
    g.replay()
    torch.cuda.synchronize()
    replayed = step.out.clone()
    half = dataclasses.replace(w, query=_halved(w))
    _check_out(half, step)
    with torch.cuda.stream(s):
        step.run()
    s.synchronize()
    assert torch.equal(replayed.view(torch.uint8), step.out.view(torch.uint8))
    assert not torch.equal(replayed.view(torch.uint8), eager.view(torch.uint8))


@pytest.mark.parametrize("kv", [W.BF16, W.FP8])
@pytest.mark.parametrize("launch", ["", "1"])
def test_scatter_and_merge_carried_by_other_launches(R, monkeypatch, kv, launch):
    """The one-call step of a mixed batch: the scatter of prefill-chunk rows
    is carried by workgroups appended to the split-K launch (the default when
    only extend items read the rows), and the merge of the split-K partials by
    workgroups appended to the extend launch; or each runs as a launch of its
    own (PA_SCATTER_LAUNCH=1, PA_MERGE_LAUNCH=1).  Decode rows (long enough to
    be cut into pieces), chunks whose rows the extend items write themselves,
    and wide chunks with history (ragged segments at both ends of a block).
    Pool bytes and slots equal the oracle's and the three-call form's,
    outputs match the oracle, and the launch profile shows which form ran."""
    from paged_kv_cache_pool_amd import binding as B
    monkeypatch.setenv("PA_SCATTER_LAUNCH", launch)
    monkeypatch.setenv("PA_MERGE_LAUNCH", launch)
    monkeypatch.setenv("PA_PARTITION_KEYS", "128")
    monkeypatch.setenv("PA_DECODE_PAIRS", "0")
    say("scatter and merge carried by other launches, kv", kv, "own launches", launch)
    w = W.build(f"carried_{kv}", 21, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                num_blocks=260, kv_dtype=kv, io_dtype=W.BF16,
                num_computed=[300, 0, 77, 1000, 45, 513, 64],
                num_scheduled=[1, 70, 1, 150, 9, 200, 1])
    B.profile_enable(True)
    fused = R.GpuStep(w, fused=True)
    fused.run()
    torch.cuda.synchronize()
    n_scatter, _ = B.profile_read("k_write_new")
    n_merge, _ = B.profile_read("k_merge")
    B.profile_enable(False)
    assert (n_scatter == 0) == (launch == ""), n_scatter
    assert (n_merge == 0) == (launch == ""), n_merge
    sep = R.GpuStep(w)
    sep.run()
    torch.cuda.synchronize()
    assert (fused.slots.cpu().numpy() == sep.slots.cpu().numpy()).all()
    _assert_same_pool(fused.pool, sep.pool)
    _assert_pool_is_oracle(w, fused.pool)
    _check_out(w, fused)
    _check_out(w, sep)


@pytest.mark.parametrize("seed", range(12))
def test_carried_work_random(R, seed):
    """Random mixed batches that take both carried paths by default: decode
    rows over long histories (cut into pieces, so rows are merged) and
    prefill chunks of more than 128 (row, head) columns per kv head with
    history (their rows scattered by the split-K launch), bf16 and fp8 pools,
    g in {1, 2, 4, 8, 16}.  One call against the three-call form (pool bytes
    and slots exact) and against the oracle (every row)."""
    rng = np.random.default_rng(seed + 900)
    kv = [W.BF16, W.FP8][seed % 2]
    g = [1, 2, 4, 8, 16][seed % 5]
    hkv = int(rng.choice([1, 2, 4]))
    n_dec = int(rng.integers(2, 9))
    n_ext = int(rng.integers(1, 4))
    lo_c = -(-129 // g)                          # more than 128 columns per kv head
    nc = [int(x) for x in rng.integers(200, 2500, n_dec)] + [int(x) for x in rng.integers(0, 700, n_ext)]
    ns = [1] * n_dec + [int(x) for x in rng.integers(lo_c, lo_c + 300, n_ext)]
    order = rng.permutation(len(nc))
    nc = [nc[k] for k in order]
    ns = [ns[k] for k in order]
    nb = sum(-(-(a + b) // 16) for a, b in zip(nc, ns)) + 16
    say("carried random", seed, kv, "g", g, "hkv", hkv, "computed", nc, "scheduled", ns)
    w = W.build(f"carried_rand_{seed}", seed + 900, num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=128,
                block_size=16, num_blocks=nb, kv_dtype=kv, io_dtype=W.BF16,
                num_computed=nc, num_scheduled=ns)
    fused, sep = _fused_and_separate(R, w)
    assert (fused.slots.cpu().numpy() == sep.slots.cpu().numpy()).all()
    _assert_same_pool(fused.pool, sep.pool)
    _assert_pool_is_oracle(w, fused.pool)
    _check_out(w, fused)
    _check_out(w, sep)


@pytest.mark.parametrize("plan_copy", ["", "1"])
def test_graph_of_several_layers(R, monkeypatch, plan_copy):
    """The attention layers of one model step captured into one HIP graph:
    four one-call steps, each on its own pool and inputs (a decode layer, a
    mixed batch with a prefill chunk, the verify shape, the fp8 shared-prefix
    shape, at reduced sizes), captured in turn on one stream.  Every replay
    gives each layer's eager output bit for bit, with eager calls of another
    batch between replays, and each matches the oracle; after new query
    contents in two of the layers, the next replay matches the oracle for
    them."""
    monkeypatch.setenv("PA_GRAPH_PLAN_COPY", plan_copy)
    ws = [W.llama8b_decode(seed=3, num_seqs=24, lo=100, hi=1200, num_blocks=2200),
          W.mixed_step(seed=4, num_decode=12, lo=64, hi=900, chunk_a=96, chunk_b=200,
                       chunk_b_cached=150, num_blocks=900),
          W.spec_verify(seed=5, num_seqs=10, lo=80, hi=700, num_blocks=600),
          W.prefix_fp8_decode(seed=6, num_seqs=20, prefix=256, lo=16, hi=120, num_blocks=400)]
    s = torch.cuda.Stream()
    layers = [R.GpuStep(w, stream=s, fused=True) for w in ws]
    eager = []
    for w, ly in zip(ws, layers):
        say("layer", w.name)
        with torch.cuda.stream(s):
            ly.run()
        s.synchronize()
        _check_out(w, ly)
        eager.append(ly.out.clone())
    other = R.GpuStep(W.make(1, seed=7), fused=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for ly in layers:
            ly.run()
    torch.cuda.synchronize()
    for rep in range(3):
        say("several-layer graph replay", rep, "plan copy", plan_copy)
        for ly in layers:
            ly.out.fill_(float("nan"))
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ly in enumerate(layers):
            assert torch.equal(ly.out.view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
    for k in (0, 2):
        layers[k].query.mul_(0.5)
    g.replay()
    torch.cuda.synchronize()
    for k, (w, ly) in enumerate(zip(ws, layers)):
        _check_out(dataclasses.replace(w, query=_halved(w)) if k in (0, 2) else w, ly)


def test_graph_capture_rejects_validation(R, monkeypatch):
    from paged_kv_cache_pool_amd import binding as B
    say("graph capture + PA_VALIDATE")
    w = W.make(1)
    s = torch.cuda.Stream()
    step = R.GpuStep(w, stream=s, fused=True)
    monkeypatch.setenv("PA_VALIDATE", "1")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(B.PaError) as e:
        with torch.cuda.graph(g, stream=s):
            step.run()
    assert e.value.status == 2
    torch.cuda.synchronize()


def test_staging_ring_across_streams(R):
    """The plan's staging buffers are reused after 16 calls: 48 calls that
    alternate between two streams (two batches, the decode layer and a mixed
    batch) and a third stream used once, with every call's output equal to
    the same batch's first output bit for bit.  A buffer is released by the
    next call on its own stream; the buffer of the stream used once is waited
    for by a device synchronisation."""
    say("staging ring across streams")
    wa = W.llama8b_decode(seed=2, num_seqs=40, lo=100, hi=1500, num_blocks=4200)
    wb = W.build("ring_b", 4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                 num_blocks=90, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[300, 40, 0, 77],
                 num_scheduled=[1, 1, 120, 9])
    sa, sb, sc = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    a = R.GpuStep(wa, stream=sa, fused=True)
    b = R.GpuStep(wb, stream=sb, fused=True)
    c = R.GpuStep(wb, stream=sc, fused=True)
    a.run()
    b.run()
    c.run()
    torch.cuda.synchronize()
    ref_a, ref_b = a.out.clone(), b.out.clone()
    assert torch.equal(c.out.view(torch.uint8), ref_b.view(torch.uint8))
    _check_out(wa, a)
    _check_out(wb, b)
    for k in range(48):
        (a if k % 2 == 0 else b).run()
        if k % 8 == 7:
            torch.cuda.synchronize()
            assert torch.equal(a.out.view(torch.uint8), ref_a.view(torch.uint8)), k
            assert torch.equal(b.out.view(torch.uint8), ref_b.view(torch.uint8)), k
    torch.cuda.synchronize()
    assert torch.equal(a.out.view(torch.uint8), ref_a.view(torch.uint8))
    assert torch.equal(b.out.view(torch.uint8), ref_b.view(torch.uint8))


@pytest.mark.parametrize("case", ["mixed", "prefix_pass"])
def test_later_work_lists_in_device_or_host_memory(R, monkeypatch, case):
    """The work lists of the launches after the split-K one (merge, extend and
    prefix-pass items) are copied into the workspace by copy workgroups of the
    split-K launch, and read there; with PA_LISTS_IN_HOST=1 they are read
    from the host staging buffer.  Both give the same output bits and pool
    bytes, and match the oracle: a mixed batch (split decode rows, prefill
    chunks, carried scatter and merge) and a shared-prefix batch through the
    MFMA prefix pass."""
    if case == "mixed":
        monkeypatch.setenv("PA_PARTITION_KEYS", "128")
        w = W.build("lists_mixed", 23, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                    num_blocks=260, kv_dtype=W.BF16, io_dtype=W.BF16,
                    num_computed=[300, 0, 77, 1000, 45, 513, 64],
                    num_scheduled=[1, 70, 1, 150, 9, 200, 1])
    else:
        monkeypatch.setenv("PA_PREFIX_PASS", "1")
        w = W.prefix_fp8_decode(seed=5, num_seqs=24, prefix=512, lo=16, hi=200, num_blocks=900)
    outs = []
    for in_host in ("", "1"):
        monkeypatch.setenv("PA_LISTS_IN_HOST", in_host)
        say("work lists", case, "in host memory" if in_host else "copied to the workspace")
        step = R.GpuStep(w, fused=True)
        step.run()
        torch.cuda.synchronize()
        _check_out(w, step)
        outs.append(step)
    a, b = outs
    assert torch.equal(a.out.view(torch.uint8), b.out.view(torch.uint8))
    assert (a.slots.cpu().numpy() == b.slots.cpu().numpy()).all()
    _assert_same_pool(a.pool, b.pool)

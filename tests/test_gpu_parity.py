"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

* slot derivation and the KV write: bit-exact (the pool is compared through
  logical (block, offset, head, dim) indexing; unwritten slots must still
  hold their canaries);
* attention: max |O_gpu - O_oracle| <= 1e-5 for the fp32 workload and
  <= 2e-2 for bf16 / fp8 pools (fp32 accumulation, bf16 output);
* the workloads at full size, every row and both forms of the step, are in
  test_gpu_fullsize.py; this file holds the small and edge cases.
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
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def R():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import runner
    return runner


def _tol(w):
    return TOL[w.kv_dtype]


def _oracle_pool(w):
    return O.build_pool(w)


def _compare_pool(w, gpu_pool, orc_pool, blocks=None):
    for which in ("k", "v"):
        g = gpu_pool.logical(which)
        o = orc_pool.k if which == "k" else orc_pool.v
        if blocks is not None:
            g, o = g[blocks], o[blocks]
        gv = g.view(np.uint32) if g.dtype == np.float32 else g
        ov = o.view(np.uint32) if o.dtype == np.float32 else o
        bad = np.argwhere(gv != ov)
        assert bad.size == 0, f"{which} pool differs at {bad[:5].tolist()} (of {len(bad)})"


def _sample_tokens(w, n, seed=0):
    rng = np.random.default_rng(seed)
    T = w.num_tokens
    if T <= n:
        return np.arange(T, dtype=np.int32)
    # always include the first and last rows of every request with > 1 row
    qsl = O.query_start_loc(w.num_scheduled)
    must = set()
    for i in range(w.num_seqs):
        if w.num_scheduled[i] > 1:
            must |= {int(qsl[i]), int(qsl[i + 1]) - 1}
    rest = rng.choice(T, size=max(0, n - len(must)), replace=False).tolist()
    return np.array(sorted(must | set(rest)), dtype=np.int32)


def _check_attention(w, step, tokens=None, tol=None):
    tol = _tol(w) if tol is None else tol
    ref = O.run_step(w, tokens=tokens).out
    got = step.out_f64()
    if tokens is not None:
        got = got[tokens]
    err = np.abs(got - ref)
    say(w.name, "max_abs_err", float(err.max()), "mean", float(err.mean()), "max|O|", float(np.abs(ref).max()))
    assert np.isfinite(got).all()
    assert err.max() <= tol, (float(err.max()), np.unravel_index(err.argmax(), err.shape))


# ------------------------------------------------------------ slots / write --

@pytest.mark.parametrize("seed", range(12))
def test_write_random_small_bit_exact(R, seed):
    kv = [W.F32, W.BF16, W.FP8][seed % 3]
    io = W.F32 if kv == W.F32 else W.BF16
    D = [64, 128][(seed // 3) % 2]
    say("write random", seed, kv, D)
    w = W.random_small(seed, max_seqs=5, max_len=150, num_q_heads=4, num_kv_heads=2, head_dim=D,
                       kv_dtype=kv, io_dtype=io, spare_blocks=5)
    if kv == W.FP8:
        w = W.build(w.name, seed, num_q_heads=4, num_kv_heads=2, head_dim=D, block_size=16,
                    num_blocks=w.num_blocks, kv_dtype=W.FP8, io_dtype=W.BF16,
                    num_computed=w.num_computed, num_scheduled=w.num_scheduled)
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    orc = O.run_step(w).pool
    _compare_pool(w, step.pool, orc)


def test_write_negative_and_out_of_range_slots_skipped(R):
    from paged_kv_cache_pool_amd import binding as B
    say("write negative slots")
    pool = B.KVPool.allocate(4, 16, 2, 64, "bf16", fill_byte=0xFF)
    key = torch.arange(5 * 2 * 64, dtype=torch.float32, device="cuda").reshape(5, 2, 64).bfloat16()
    val = -key
    slots = torch.tensor([3, -1, 63, 64, 1 << 40], dtype=torch.int64, device="cuda")
    B.write_kv(pool, key, val, slots)
    torch.cuda.synchronize()
    lk = pool.logical("k")
    kb = key.cpu().view(torch.int16).numpy().view(np.uint16)
    assert (lk[0, 3] == kb[0]).all() and (lk[3, 15] == kb[2]).all()
    mask = np.ones((4, 16), bool)
    mask[0, 3] = mask[3, 15] = False
    assert (lk[mask] == 0xFFFF).all()


def test_fp8_encode_every_bf16(R):
    """Every bf16 bit pattern through pa_write_kv into an fp8 pool (scale 1 and
    a non-power-of-two scale) gives the oracle's code."""
    from paged_kv_cache_pool_amd import binding as B
    for scale in (1.0, 0.0137):
        say("fp8 exhaustive scale", scale)
        bits = np.arange(1 << 16, dtype=np.uint16)
        T = (1 << 16) // 128
        key = torch.from_numpy(bits.view(np.int16).reshape(T, 1, 128)).cuda().view(torch.bfloat16)
        pool = B.KVPool.allocate(T // 16, 16, 1, 128, "fp8", scale, scale, fill_byte=0)
        slots = torch.arange(T, dtype=torch.int64, device="cuda")
        B.write_kv(pool, key, key, slots)
        torch.cuda.synchronize()
        got_k = pool.logical("k").reshape(-1)
        got_v = pool.logical("v").reshape(-1)
        x = (bits.astype(np.uint32) << 16).view(np.float32)
        y = (x / np.float32(scale)).astype(np.float32)
        want = O.e4m3_encode(y)
        assert (got_k == want).all(), np.argwhere(got_k != want)[:5]
        assert (got_v == want).all()


# ------------------------------------------------------------- attention --

def test_attention_tiny_f32_config(R):
    say("attention config 1")
    w = W.make(1)
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


@pytest.mark.parametrize("pairs", [None, "1"])
@pytest.mark.parametrize("seed", range(30))
def test_attention_random_small(R, monkeypatch, seed, pairs):
    """Random small batches over pool dtypes, GQA ratios and head dims, in
    the planner's own decode form and with the paired form forced (its
    matrix-core kernel for both head dims; fp32 pools keep their kernel)."""
    if pairs:
        monkeypatch.setenv("PA_DECODE_PAIRS", pairs)
    kv = [W.F32, W.BF16, W.FP8][seed % 3]
    io = W.F32 if kv == W.F32 else W.BF16
    g = [1, 2, 4, 8, 16][(seed // 3) % 5]
    D = [64, 128][(seed // 15) % 2]
    say("attention random", seed, kv, "g", g, "D", D, "pairs", pairs)
    w = W.random_small(seed, max_seqs=5, max_len=300, num_q_heads=2 * g, num_kv_heads=2,
                       head_dim=D, kv_dtype=kv, io_dtype=io, spare_blocks=4)
    if kv == W.FP8:
        w = W.build(w.name, seed, num_q_heads=2 * g, num_kv_heads=2, head_dim=D, block_size=16,
                    num_blocks=w.num_blocks, kv_dtype=W.FP8, io_dtype=W.BF16,
                    num_computed=w.num_computed, num_scheduled=w.num_scheduled)
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


@pytest.mark.parametrize("pairs", ["0", "1", "2"])
def test_attention_long_and_split(R, monkeypatch, pairs):
    """Several partials per row and long rows: forced 64-key partitions
    (pairs "0"), or the paired layout (one wave runs a bin's two pieces, "1";
    or each piece its own wave, "2"), whose bins (512 for 2 kv heads) cut
    these rows into pieces of a step or two."""
    monkeypatch.setenv("PA_PARTITION_KEYS", "64")
    monkeypatch.setenv("PA_DECODE_PAIRS", pairs)
    say("attention split, pairs", pairs)
    w = W.llama8b_decode(seed=3, num_seqs=6, lo=1, hi=700, num_blocks=400)
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


@pytest.mark.parametrize("charge", ["0", "2", "7"])
def test_paired_bins_second_piece_charge(R, monkeypatch, charge):
    """The paired layout with the second piece of a bin charged 0, 2 (the
    default) or 7 steps.  For this batch (40 rows of 512-6000 keys, bins of
    18 steps) a charge of 2 fits and two-piece bins carry fewer steps, and 7
    does not fit, so the plan falls back to no charge.  The attention matches
    the oracle on every row in the one-call form."""
    monkeypatch.setenv("PA_PAIR_PENALTY", charge)
    say("paired bins, second-piece charge", charge)
    w = W.llama8b_decode(seed=11, num_seqs=40, lo=512, hi=6000, num_blocks=16000)
    step = R.GpuStep(w, fused=True)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


@pytest.mark.parametrize("n,lo,hi", [(200, 512, 1500), (300, 16, 400)])
def test_attention_many_decode_rows(R, n, lo, hi):
    """Many decode rows on the Llama-3-8B layer shape: 200 rows of 512-1500
    keys fit the paired layout (128 bins of two pieces), 300 rows do not
    (more rows than two per bin) and take the partition form.  Sampled rows
    against the oracle."""
    say("attention", n, "decode rows")
    w = W.llama8b_decode(seed=5, num_seqs=n, lo=lo, hi=hi, num_blocks=n * (hi // 16 + 2) + 64)
    step = R.GpuStep(w, fused=True)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step, tokens=_sample_tokens(w, 40, seed=n))


def test_attention_zero_token_requests_and_noncausal(R):
    say("attention c=0 requests + non-causal")
    w = W.build("zeros", 5, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=60, kv_dtype=W.BF16, io_dtype=W.BF16,
                num_computed=[10, 100, 0, 37, 64], num_scheduled=[0, 1, 3, 0, 5])
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)
    step_nc = R.GpuStep(w, causal=False)
    step_nc.run()
    torch.cuda.synchronize()
    ref = O.run_step(w, causal=False).out
    assert np.abs(step_nc.out_f64() - ref).max() <= 2e-2


def test_one_hot_probe_bit_exact(R):
    """All keys zero except one aligned with q and large: every other weight
    underflows to 0 in fp32, so the output equals that key's value exactly.
    Values encode their position, so any block/offset mistake in the attention
    kernel shows as a wrong number."""
    say("one-hot probe")
    H, D = 2, 128
    L = 16 * 9 + 5
    w = W.build("probe", 0, num_q_heads=4, num_kv_heads=H, head_dim=D, block_size=16,
                num_blocks=40, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[L - 1],
                num_scheduled=[1])
    pos = np.arange(L - 1)
    # value of position j, dim e: +j for even e, -j for odd e (exact in bf16, j < 256)
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    vals = pos[:, None, None] * sign[None, None, :] * np.ones((1, H, 1))
    w.history[0].value[:] = W.f32_to_bf16_bits(vals.astype(np.float32))
    w.value[:] = W.f32_to_bf16_bits(((L - 1) * sign + np.zeros((1, H, D))).astype(np.float32))
    q = np.ones((1, 4, D), np.float32)
    w.query[:] = W.f32_to_bf16_bits(q)
    w.key[:] = 0
    for jstar in [0, 15, 16, 77, L - 2]:
        w.history[0].key[:] = 0
        w.history[0].key[jstar] = W.f32_to_bf16_bits(np.full((H, D), 16.0, np.float32))
        step = R.GpuStep(w)
        step.run()
        torch.cuda.synchronize()
        got = step.out.float().cpu().numpy()[0]
        want = jstar * sign
        assert (got == want[None, :]).all(), (jstar, got[0, :8], want[:8])


def test_nan_canaries_never_read(R):
    """Unwritten pool slots hold NaN and trailing block-table entries are -1:
    outputs stay finite (covers partially filled last blocks)."""
    say("nan canaries")
    w = W.build("canary", 9, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=80, kv_dtype=W.BF16, io_dtype=W.BF16,
                num_computed=[0, 16, 17, 30, 129], num_scheduled=[1, 1, 1, 2, 20])
    w.block_table = np.concatenate([w.block_table, np.full((w.num_seqs, 3), -1, np.int32)], axis=1)
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    assert np.isfinite(step.out_f64()).all()
    _check_attention(w, step)


def test_page_mixed_batch(R):
    """The mixed batch the source-map page walks through ("vLLM 源码完全拆解（十六）",
    fourth walk-through path): one decode row, a 256-token chunk and a 3-token
    chunk, with 1024, 512 and 600 tokens already computed, so seq_lens =
    [1025, 768, 603] and query_start_loc = [0, 1, 257, 260].  Every row of
    the three paths (decode, MFMA extend, short chunk through the split-K
    kernel) is compared with the oracle."""
    say("page mixed batch")
    w = W.build("page_mixed", 3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=200, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[1024, 512, 600],
                num_scheduled=[1, 256, 3])
    assert O.query_start_loc(w.num_scheduled).tolist() == [0, 1, 257, 260]
    assert O.seq_lens(w.num_computed, w.num_scheduled).tolist() == [1025, 768, 603]
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


# ------------------------------------------------------ shared prefix ------

def _cascade_workload(kv, g, seed=11):
    """Seven requests sharing a 3-block prefix: five decodes (own history 0 ..
    60 tokens), a 3-token chunk (split-K rows, also cascaded) and a 20-token
    chunk (MFMA prefill rows, not cascaded)."""
    own = [0, 1, 17, 33, 60, 9, 5]
    ns = [1, 1, 1, 1, 1, 3, 20]
    nc = [48 + o for o in own]
    return W.build(f"casc_{kv}_{g}", seed, num_q_heads=2 * g, num_kv_heads=2, head_dim=128,
                   block_size=16, num_blocks=80, kv_dtype=kv, io_dtype=W.BF16, num_computed=nc,
                   num_scheduled=ns, shared_prefix_tokens=48)


@pytest.mark.parametrize("prefix_pass", ["", "1"])
@pytest.mark.parametrize("kv", [W.BF16, W.FP8])
@pytest.mark.parametrize("g", [1, 4, 8, 16])
def test_cascade_shared_prefix(R, monkeypatch, kv, g, prefix_pass):
    """Cascade attention: the rows' attention over the shared prefix comes from
    prefix items of the split-K kernel (or, with PA_PREFIX_PASS=1, from the
    MFMA prefix pass) and is merged with their own keys; equal to the oracle
    (plain attention), with and without the hint."""
    monkeypatch.setenv("PA_PREFIX_PASS", prefix_pass)
    say("cascade", kv, "g", g, "prefix pass", prefix_pass)
    w = _cascade_workload(kv, g)
    assert w.shared_prefix_blocks == 3
    for hint in (True, False):
        step = R.GpuStep(w, shared_prefix=hint)
        step.run()
        torch.cuda.synchronize()
        _check_attention(w, step)


@pytest.mark.parametrize("case", range(8))
def test_cascade_many_rows(R, monkeypatch, case):
    """Many decode rows over one shared prefix (40 .. 300 rows, g 1 .. 16, so
    that the prefix rows' columns fall below and above the split-K kernel's
    limit for prefix items), bf16 and fp8, in the paired layout and with
    forced 64-key partitions (many prefix pieces per unit), causal: every row
    against the oracle."""
    rng = np.random.default_rng(900 + case)
    kv = [W.BF16, W.FP8][case % 2]
    g = [1, 4, 16, 8][(case // 2) % 4]
    rows = [300, 40, 60, 150][(case // 2) % 4]
    if case >= 6:
        monkeypatch.setenv("PA_DECODE_PAIRS", "0")
        monkeypatch.setenv("PA_PARTITION_KEYS", "64")
    own = rng.integers(0, 200, rows)
    P = 16 * int(rng.integers(4, 40))
    say("cascade many rows", case, kv, "g", g, "rows", rows, "prefix", P)
    w = W.build(f"casc_many_{case}", 900 + case, num_q_heads=2 * g, num_kv_heads=2, head_dim=128,
                block_size=16, num_blocks=int(sum(-(-(P + o + 1) // 16) for o in own)) + 8,
                kv_dtype=kv, io_dtype=W.BF16, num_computed=(P + own).astype(np.int32),
                num_scheduled=np.ones(rows, np.int32), shared_prefix_tokens=P)
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


def test_cascade_hint_ignored_when_not_history(R):
    """A hint that no request can honour (more prefix blocks than any request
    holds in its history) is ignored: the result is still the oracle's."""
    say("cascade hint ignored")
    from paged_kv_cache_pool_amd import binding as B
    w = _cascade_workload(W.BF16, 4)
    step = R.GpuStep(w)
    step.batch.num_common_prefix_blocks = 50
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)
    assert B.attention_workspace_bytes(step.pool, step.batch, w.num_q_heads) > 0


def test_cascade_wrong_hint_rejected_under_validation(R, monkeypatch):
    """With PA_VALIDATE the block tables are checked against the hint."""
    say("cascade wrong hint")
    from paged_kv_cache_pool_amd import binding as B
    w = W.build("casc_bad", 5, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=40, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[40, 50],
                num_scheduled=[1, 1])
    step = R.GpuStep(w)
    step.batch.num_common_prefix_blocks = 2      # the two requests' blocks differ
    monkeypatch.setenv("PA_VALIDATE", "1")
    with pytest.raises(B.PaError) as e:
        step.run()
    assert e.value.status == 4


# ------------------------------------------------------------ MFMA extend --

@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("c,hist", [(16, 0), (17, 5), (33, 64), (100, 37), (129, 300), (257, 16)])
def test_extend_chunks(R, g, c, hist):
    """Prefill chunks (c >= 16 rows go to the MFMA kernel) with ragged column
    tiles, history before the chunk and a decode row in the same batch."""
    say("extend g", g, "c", c, "hist", hist)
    w = W.build(f"ext_{g}_{c}_{hist}", c + hist, num_q_heads=2 * g, num_kv_heads=2, head_dim=128,
                block_size=16, num_blocks=-(-(c + hist) // 16) + 40, kv_dtype=W.BF16,
                io_dtype=W.BF16, num_computed=[hist, 70], num_scheduled=[c, 1])
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


@pytest.mark.parametrize("g", [1, 4, 8, 16])
@pytest.mark.parametrize("c,hist", [(16, 0), (100, 37), (129, 300), (257, 16)])
def test_extend_chunks_fp8(R, g, c, hist):
    """Prefill chunks over an fp8 pool (per-tensor scales) through the MFMA
    kernel: the codes are widened to bf16 exactly in LDS, scores take
    k_scale and the output v_scale."""
    say("extend fp8 g", g, "c", c, "hist", hist)
    w = W.build(f"ext8_{g}_{c}_{hist}", c + hist + 1, num_q_heads=2 * g, num_kv_heads=2, head_dim=128,
                block_size=16, num_blocks=-(-(c + hist) // 16) + 40, kv_dtype=W.FP8,
                io_dtype=W.BF16, num_computed=[hist, 70], num_scheduled=[c, 1])
    step = R.GpuStep(w)
    step.run()
    torch.cuda.synchronize()
    _check_attention(w, step)


def test_extend_noncausal(R):
    say("extend non-causal")
    w = W.build("ext_nc", 4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=30, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[50, 0],
                num_scheduled=[70, 40])
    step = R.GpuStep(w, causal=False)
    step.run()
    torch.cuda.synchronize()
    ref = O.run_step(w, causal=False).out
    err = np.abs(step.out_f64() - ref).max()
    say("extend non-causal err", err)
    assert err <= 2e-2


def test_one_hot_probe_extend_bit_exact(R):
    """The one-hot probe through the MFMA kernel: 40 new rows all select the
    same history position; P = 1 and 0 are exact in bf16, so O = v exactly."""
    say("one-hot probe (extend)")
    H, D, hist, c = 2, 128, 16 * 7 + 3, 40
    w = W.build("probe_ext", 1, num_q_heads=8, num_kv_heads=H, head_dim=D, block_size=16,
                num_blocks=30, kv_dtype=W.BF16, io_dtype=W.BF16, num_computed=[hist],
                num_scheduled=[c])
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    vals = np.arange(hist)[:, None, None] * sign[None, None, :] * np.ones((1, H, 1))
    w.history[0].value[:] = W.f32_to_bf16_bits(vals.astype(np.float32))
    w.value[:] = W.f32_to_bf16_bits((200.0 * sign + np.zeros((c, H, D))).astype(np.float32))
    w.query[:] = W.f32_to_bf16_bits(np.ones((c, 8, D), np.float32))
    w.key[:] = 0
    for jstar in [0, 31, 64, hist - 1]:
        w.history[0].key[:] = 0
        w.history[0].key[jstar] = W.f32_to_bf16_bits(np.full((H, D), 16.0, np.float32))
        step = R.GpuStep(w)
        step.run()
        torch.cuda.synchronize()
        got = step.out.float().cpu().numpy()
        assert (got == (jstar * sign)[None, None, :]).all(), (jstar, got[0, 0, :6])

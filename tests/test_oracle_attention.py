"""Pins for the oracle's attention (and, through it, its pool write).

Each check ties the oracle to something other than itself:
* brute force: a dense float64 numpy attention over the workload's raw rows
  rebuilt in logical order (no pool, no block table, explicit bottom-right
  causal mask) on many random tiny batches;
* a library special case: torch's scaled_dot_product_attention in float64
  for prefill chunks without history;
* closed forms: one visible key, all keys equal, q = 0, a one-hot probe;
* invariants the pages state or imply: block permutation does not change the
  result, probability rows sum to one, a decode step equals the last row of
  the matching prefill, chunked prefill equals one-shot prefill, GQA equals
  MHA with replicated K/V heads, and any partition of the keys merged with
  the rescaling rule gives the same result ("vLLM 源码完全拆解（十六）",
  third walk-through path: page and partition boundaries must not change the
  mathematical result).
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_pool_amd import workloads as W


def _rows(w, a):
    return W.to_f32(a, w.io_dtype).astype(np.float64)


def _kv_as_stored(w, x, which):
    """Row values as the pool holds them (fp8: quantised with torch's codec)."""
    x = W.to_f32(x, w.io_dtype)
    if w.kv_dtype != W.FP8:
        return x.astype(np.float64)
    s = np.float32(w.k_scale if which == "k" else w.v_scale)
    y = (x / s).astype(np.float32)
    code = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return code.to(torch.float32).numpy().astype(np.float64) * float(s)


def dense_reference(w, causal=True):
    """Dense fp64 attention per request from the raw rows in logical order."""
    n, H, d, Hq = w.num_seqs, w.num_kv_heads, w.head_dim, w.num_q_heads
    g = Hq // H
    L = (w.num_computed + w.num_scheduled).astype(int)
    Ks = [np.full((L[i], H, d), np.nan) for i in range(n)]
    Vs = [np.full((L[i], H, d), np.nan) for i in range(n)]
    for hb in w.history:
        k, v = _kv_as_stored(w, hb.key, "k"), _kv_as_stored(w, hb.value, "v")
        r = 0
        for j, req in enumerate(hb.requests):
            c, tot = int(hb.count[j]), int(hb.total[j])
            reqs = [req] if w.shared_prefix_blocks == 0 or len(hb.requests) > 1 else range(n)
            for rq in reqs:
                Ks[rq][tot - c:tot] = k[r:r + c]
                Vs[rq][tot - c:tot] = v[r:r + c]
            r += c
    kn, vn = _kv_as_stored(w, w.key, "k"), _kv_as_stored(w, w.value, "v")
    q = _rows(w, w.query)
    out = np.zeros((w.num_tokens, Hq, d))
    tok = 0
    for i in range(n):
        c = int(w.num_scheduled[i])
        Ks[i][L[i] - c:] = kn[tok:tok + c]
        Vs[i][L[i] - c:] = vn[tok:tok + c]
        for t in range(c):
            p = L[i] - c + t
            nv = p + 1 if causal else L[i]
            for h in range(Hq):
                kk, vv = Ks[i][:nv, h // g], Vs[i][:nv, h // g]
                s = (kk @ q[tok + t, h]) * np.float64(np.float32(w.softmax_scale))
                e = np.exp(s - s.max())
                out[tok + t, h] = (e[:, None] * vv).sum(0) / e.sum()
        tok += c
    return out


@pytest.mark.parametrize("seed", range(60))
def test_brute_force_random_small(orc, seed):
    S = [1, 4, 16][seed % 3]
    g = [1, 2, 4][(seed // 3) % 3]
    kv = [W.F32, W.BF16, W.FP8][(seed // 9) % 3]
    io = W.F32 if kv == W.F32 else W.BF16
    w = W.random_small(seed, max_seqs=4, max_len=64, block_size=S, num_q_heads=2 * g,
                       num_kv_heads=2, head_dim=16, kv_dtype=kv, io_dtype=io)
    if kv == W.FP8:
        w = W.build(w.name, seed, num_q_heads=2 * g, num_kv_heads=2, head_dim=16, block_size=S,
                    num_blocks=w.num_blocks, kv_dtype=W.FP8, io_dtype=W.BF16,
                    num_computed=w.num_computed, num_scheduled=w.num_scheduled)
    res = orc.run_step(w)
    ref = dense_reference(w)
    assert np.abs(res.out - ref).max() < 1e-12


def test_brute_force_noncausal(orc):
    w = W.random_small(11, max_seqs=3, max_len=40, block_size=4, head_dim=8)
    res = orc.run_step(w, causal=False)
    assert np.abs(res.out - dense_reference(w, causal=False)).max() < 1e-12


@pytest.mark.parametrize("cfg", [1])
def test_brute_force_tiny_config(orc, cfg):
    w = W.make(cfg)
    res = orc.run_step(w)
    assert np.abs(res.out - dense_reference(w)).max() < 1e-12


def _prefill_workload(seed, L, Hq=4, H=2, d=16, S=4, io=W.F32, kv=W.F32, chunks=None):
    """One request with a prompt of length L processed as one step (or the last of
    several chunks when `chunks` lists earlier chunk sizes)."""
    chunks = chunks or []
    done = sum(chunks)
    return W.build(f"prefill_{seed}", seed, num_q_heads=Hq, num_kv_heads=H, head_dim=d,
                   block_size=S, num_blocks=-(-L // S) + 3, kv_dtype=kv, io_dtype=io,
                   num_computed=[done], num_scheduled=[L - done])


def test_sdpa_no_history_prefill(orc):
    for seed, (L, Hq, H) in enumerate([(37, 4, 2), (64, 8, 8), (5, 4, 1)]):
        w = _prefill_workload(seed, L, Hq, H)
        res = orc.run_step(w)
        q = torch.from_numpy(_rows(w, w.query)).permute(1, 0, 2)          # [Hq, L, d]
        k = torch.from_numpy(_rows(w, w.key)).permute(1, 0, 2)
        v = torch.from_numpy(_rows(w, w.value)).permute(1, 0, 2)
        g = Hq // H
        k = k.repeat_interleave(g, 0)
        v = v.repeat_interleave(g, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, is_causal=True, scale=float(np.float32(w.softmax_scale)))
        assert np.abs(res.out - ref.permute(1, 0, 2).numpy()).max() < 1e-12


def test_single_visible_key_returns_its_value(orc):
    w = W.make(1)  # request 2 has context length 1
    res = orc.run_step(w)
    tok = int(res.qsl[2])
    v = w.value[tok]  # [H, d]
    assert (res.out[tok] == v.astype(np.float64)).all()


def test_equal_keys_and_zero_query_give_mean(orc):
    w = W.random_small(5, max_seqs=3, max_len=50, block_size=4, head_dim=8)
    # every key row identical -> uniform weights
    w.key[:] = 0.5
    for hb in w.history:
        hb.key[:] = 0.5
    res = orc.run_step(w)
    ref = dense_reference(w)
    assert np.abs(res.out - ref).max() < 1e-12
    # the mean of the visible values
    L = w.num_computed + w.num_scheduled
    vals = {}
    r = 0
    for hb in w.history:
        for j, req in enumerate(hb.requests):
            c, tot = int(hb.count[j]), int(hb.total[j])
            vals.setdefault(int(req), {}).update({tot - c + t: hb.value[r + t] for t in range(c)})
            r += c
    tok = 0
    for i in range(w.num_seqs):
        c = int(w.num_scheduled[i])
        for t in range(c):
            vals.setdefault(i, {})[L[i] - c + t] = w.value[tok + t]
        for t in range(c):
            p = L[i] - c + t
            m = np.mean([vals[i][j].astype(np.float64) for j in range(p + 1)], axis=0)
            g = w.num_q_heads // w.num_kv_heads
            for h in range(w.num_q_heads):
                assert np.abs(res.out[tok + t, h] - m[h // g]).max() < 1e-12
        tok += c
    # q = 0 gives the same means with arbitrary keys
    w2 = W.random_small(5, max_seqs=3, max_len=50, block_size=4, head_dim=8)
    w2.query[:] = 0
    res2 = orc.run_step(w2)
    assert np.abs(res2.out - res.out).max() < 1e-12


def test_one_hot_probe_selects_one_position(orc):
    """All keys zero except key j*, which is aligned with q and large: the
    softmax puts all weight on j*, so the output is v_{j*} (to double
    precision).  Values encode their own position, so a wrong block or offset
    lookup shows up as a wrong number."""
    S, H, d, L = 4, 1, 8, 23
    w = _prefill_workload(1, L, Hq=1, H=1, d=d, S=S, chunks=[15])
    for hb in w.history:
        hb.key[:] = 0
        pos = np.arange(15)
        hb.value[:] = (pos[:, None, None] * 1.0 + np.arange(d)[None, None, :] / 16.0).astype(np.float32)
    w.key[:] = 0
    w.value[:] = ((15 + np.arange(8))[:, None, None] + np.arange(d)[None, None, :] / 16.0).astype(np.float32)
    q = np.ones(d, np.float32)
    w.query[:] = q
    for jstar in [0, 3, 4, 9, 14]:
        for hb in w.history:
            hb.key[:] = 0
            hb.key[jstar, 0, :] = 200.0 * q / np.linalg.norm(q)
        res = orc.run_step(w)
        # every token of the chunk sees j* (positions 15..22 >= j*)
        want = jstar + np.arange(d) / 16.0
        assert np.abs(res.out[:, 0, :] - want).max() < 1e-30 + 1e-12 * np.abs(want).max()


def test_block_permutation_invariance(orc):
    base = W.random_small(9, max_seqs=4, max_len=90, block_size=4, head_dim=16)
    res_a = orc.run_step(base)
    rng = np.random.default_rng(123)
    perm = rng.permutation(base.num_blocks).astype(np.int32)
    bt2 = np.where(base.block_table >= 0, perm[np.maximum(base.block_table, 0)], -1).astype(np.int32)
    base.block_table = bt2
    res_b = orc.run_step(base)
    assert (res_a.out == res_b.out).all()
    assert (res_a.slots != res_b.slots).any()


@pytest.mark.parametrize("seed", range(4))
def test_probabilities_sum_to_one(orc, seed):
    w = W.random_small(seed, max_seqs=3, max_len=80, block_size=16, head_dim=16)
    res = orc.run_step(w)
    for tok in range(w.num_tokens):
        for h in range(w.num_q_heads):
            p = orc.attention_probs(res.pool, res.qsl, res.seq_lens, w.block_table, w.query,
                                    w.io_dtype, w.num_q_heads, w.softmax_scale, tok, h)
            assert abs(p.sum() - 1.0) < 1e-12 and (p >= 0).all()


def test_decode_equals_last_prefill_row(orc):
    L = 41
    one_shot = _prefill_workload(3, L, S=4)
    # same rows: positions 0..L-2 as history, the last as a decode step
    dec = _prefill_workload(3, L, S=4, chunks=[L - 1])
    dec.history[0].key[:] = one_shot.key[:L - 1]
    dec.history[0].value[:] = one_shot.value[:L - 1]
    dec.key[:] = one_shot.key[L - 1:]
    dec.value[:] = one_shot.value[L - 1:]
    dec.query[:] = one_shot.query[L - 1:]
    dec.block_table = one_shot.block_table.copy()
    a = orc.run_step(one_shot).out[L - 1]
    b = orc.run_step(dec).out[0]
    assert (a == b).all()


@pytest.mark.parametrize("split", [[8], [1, 20], [16, 16]])
def test_chunked_equals_one_shot(orc, split):
    L = 45
    one = _prefill_workload(4, L, S=4)
    ref = orc.run_step(one).out
    pool = orc.Pool(one.num_blocks, one.block_size, one.num_kv_heads, one.head_dim, "f32")
    done = 0
    outs = []
    for c in split + [L - sum(split)]:
        qsl = orc.query_start_loc([c])
        sl = orc.seq_lens([done], [c])
        slots = orc.slot_mapping(qsl, sl, one.block_table, one.block_size)
        orc.write_kv(pool, one.key[done:done + c], one.value[done:done + c], "f32", slots)
        outs.append(orc.attention(pool, qsl, sl, one.block_table, one.query[done:done + c], "f32",
                                  one.num_q_heads, one.softmax_scale))
        done += c
    assert (np.concatenate(outs) == ref).all()


def test_gqa_equals_replicated_mha(orc):
    g, H = 4, 2
    w = W.random_small(21, max_seqs=3, max_len=70, block_size=16, num_q_heads=g * H,
                       num_kv_heads=H, head_dim=16)
    out_gqa = orc.run_step(w).out
    rep = W.build("rep", 21, num_q_heads=g * H, num_kv_heads=g * H, head_dim=16, block_size=16,
                  num_blocks=w.num_blocks, kv_dtype=W.F32, io_dtype=W.F32,
                  num_computed=w.num_computed, num_scheduled=w.num_scheduled)
    rep.block_table = w.block_table
    rep.query = w.query
    rep.key = np.repeat(w.key, g, axis=1)
    rep.value = np.repeat(w.value, g, axis=1)
    for a, b in zip(rep.history, w.history):
        a.key = np.repeat(b.key, g, axis=1)
        a.value = np.repeat(b.value, g, axis=1)
    out_mha = orc.run_step(rep).out
    assert (out_gqa == out_mha).all()


@pytest.mark.parametrize("part", [1, 2, 7, 16, 64, 100000])
def test_partition_merge_invariance(orc, part):
    w = W.random_small(31, max_seqs=4, max_len=200, block_size=16, head_dim=16)
    res = orc.run_step(w)
    merged = orc.attention_partitioned(res.pool, res.qsl, res.seq_lens, w.block_table, w.query,
                                       w.io_dtype, w.num_q_heads, w.softmax_scale, part)
    assert np.abs(merged - res.out).max() < 1e-12


def test_unwritten_slots_are_never_read(orc):
    """Pool slots beyond every request's length hold NaN canaries and block-table
    entries past the last needed block are -1: the output stays finite."""
    w = W.random_small(2, max_seqs=4, max_len=61, block_size=16, head_dim=16, spare_blocks=6)
    res = orc.run_step(w)
    assert np.isfinite(res.out).all()
    assert np.isnan(res.pool.k).any()

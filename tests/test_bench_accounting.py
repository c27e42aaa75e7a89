"""The byte and flop counts bench.py divides by kernel time (CPU only).

Each count is checked against a closed form of the workload's shape, or
against another count that must agree with it, not against a retyped copy
of the same formula.
"""
import importlib.util
import os

import numpy as np
import pytest

from paged_kv_cache_pool_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _meta(w):
    qsl = np.concatenate([[0], np.cumsum(w.num_scheduled)]).astype(np.int64)
    return w.num_computed + w.num_scheduled, qsl


def test_decode_layer_counts_agree(bench):
    """No block is shared: the per-row table walk and the distinct slots read are
    the same bytes, sum(L) keys of K and V per kv head."""
    w = W.make(2)
    sl, qsl = _meta(w)
    expect = int(sl.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    assert bench.table_walk_kv_bytes(w, sl, qsl) == expect
    assert bench.unique_kv_bytes(w, sl, qsl) == expect
    dec = bench.algorithmic_work(w, sl, qsl)[0]
    # plus q rows and block ids only
    ids = sum(-(-int(L) // 16) for L in sl) * 4
    assert dec == expect + w.num_tokens * w.num_q_heads * w.head_dim * 2 + ids


def test_shared_prefix_counts(bench):
    """fp8 shared prefix: the table walk counts the 2048-key prefix once per row,
    the distinct slots once in all (prefix blocks are shared, suffix blocks are
    each request's own), and the cascade's algorithmic bytes once per kv head."""
    w = W.make(5)
    sl, qsl = _meta(w)
    row = w.num_kv_heads * w.head_dim * 2 * 1
    P = w.shared_prefix_blocks * w.block_size
    assert P == 2048
    assert bench.table_walk_kv_bytes(w, sl, qsl) == int(sl.sum()) * row
    P_used, in_decode = bench.cascade_prefix(w, sl, qsl)
    assert P_used == P
    assert bench.unique_kv_bytes(w, sl, qsl, 0 if in_decode else P) == (P + int((sl - P).sum())) * row


def test_long_prefill_flops_closed_form(bench):
    """Two 4096-token chunks after 2048 cached tokens: row t sees 2048 + t + 1 keys."""
    w = W.make(7)
    sl, qsl = _meta(w)
    c, h = 4096, 2048
    pairs = c * h + c * (c + 1) // 2
    assert bench.algorithmic_work(w, sl, qsl)[1] == 2 * 4 * w.num_q_heads * w.head_dim * pairs


def test_multirow_items_read_kv_once(bench, monkeypatch):
    """Verify chunks as multi-row split-K items read each request's K/V once, as
    the extend kernel does: the two algorithmic byte counts differ only by the
    block ids and the new rows' write."""
    w = W.make(6)
    sl, qsl = _meta(w)
    ext_bytes = bench.algorithmic_work(w, sl, qsl, fused=True)[2]
    monkeypatch.setenv("PA_MULTIROW", "1")
    dec_bytes = bench.algorithmic_work(w, sl, qsl, extend_on=False, fused=True)[0]
    assert abs(dec_bytes - ext_bytes) / ext_bytes < 0.01
    monkeypatch.delenv("PA_MULTIROW")
    per_row = bench.algorithmic_work(w, sl, qsl, extend_on=False, fused=True)[0]
    assert per_row > 3 * dec_bytes      # one walk per row instead

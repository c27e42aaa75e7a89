"""The continuous-batching loop's host side (scheduling, the block pool,
metadata), dry-run on the CPU: every step's batch passes the oracle's
metadata checks, new tokens go to distinct slots in their own request's
blocks, the token budget and the running-request cap hold, prefix hits
happen, admission waits for blocks (the pool cannot hold every request at
once) without any running request running out, and every request finishes
with all blocks returned."""
import numpy as np
import pytest

import oracle as O
from paged_kv_cache_pool_amd import binding as B
from paged_kv_cache_pool_amd import serve

import serving_scenario as SC


def test_dry_run_scenario():
    pool = B.KVPool.allocate(SC.POOL["num_blocks"], SC.POOL["block_size"],
                             SC.POOL["num_kv_heads"], SC.POOL["head_dim"], "bf16", device="cpu")
    loop = serve.ServingLoop(pool, device="cpu", **SC.LOOP)
    for r in SC.requests():
        loop.add_request(r)
    hits = steps = 0
    while not loop.done():
        plan = loop.schedule()
        assert plan is not None, "nothing schedulable while requests remain"
        steps += 1
        assert steps < 1000
        T = plan.num_tokens
        assert 0 < T <= SC.LOOP["token_budget"]
        assert len(loop.running) <= SC.LOOP["max_num_seqs"]
        assert O.validate(plan.query_start_loc, plan.seq_lens, plan.block_table, 16,
                          SC.POOL["num_blocks"], T) == 0
        slots = O.slot_mapping(plan.query_start_loc, plan.seq_lens, plan.block_table, 16)
        assert len(set(slots.tolist())) == T
        for i, r in enumerate(plan.req_ids):
            own = set(loop.manager.block_ids(r))
            for s in slots[plan.query_start_loc[i]:plan.query_start_loc[i + 1]]:
                assert int(s) // 16 in own
        assert plan.query.shape == (T, SC.LOOP["num_q_heads"], 128)
        hits += sum(plan.prefix_hits.values())
        loop.commit(plan)
    assert sorted(loop.finished) == list(range(12))
    assert loop.manager.num_free_blocks() == SC.POOL["num_blocks"]
    assert hits > 0 and loop.admission_waits > 0, (hits, loop.admission_waits)
    for r in loop.requests.values():
        assert r.generated == r.max_new_tokens
        assert len(r.tokens) == len(r.prompt) + r.max_new_tokens


def test_request_longer_than_pool_refused():
    pool = B.KVPool.allocate(4, 16, 2, 64, "bf16", device="cpu")
    loop = serve.ServingLoop(pool, num_q_heads=4, device="cpu")
    with pytest.raises(ValueError):
        loop.add_request(serve.Request(0, list(range(60)), 5))
    loop.add_request(serve.Request(1, list(range(59)), 5))


def test_same_prefix_same_rows():
    """Requests that share a prefix (and extra key) get the same K/V rows for
    it, so a prefix-cache hit reuses valid contents; another key differs."""
    pool = B.KVPool.allocate(8, 16, 2, 64, "bf16", device="cpu")
    loop = serve.ServingLoop(pool, num_q_heads=4, device="cpu")
    a = serve.Request(0, [5, 6, 7, 8, 9], 1)
    b = serve.Request(1, [5, 6, 7, 1], 1)
    c = serve.Request(2, [5, 6, 7, 8, 9], 1, extra_key=1)
    ra, rb, rc = (loop._rows(x, 0, 3) for x in (a, b, c))
    for i in (1, 2):
        assert np.array_equal(ra[i], rb[i])
        assert not np.array_equal(ra[i], rc[i])

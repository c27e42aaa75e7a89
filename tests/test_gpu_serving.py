"""GPU parity of the continuous-batching loop: every step's one-call
attention (with the KV update and the zeroing of new blocks) against the
oracle run on the same batch metadata, and the pool after the whole run
against the oracle's pool, bit for bit.  Also the zeroing kernel itself."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_pool_amd import workloads as W

import serving_scenario as SC

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-serving]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_pool_amd import binding
    return binding


def test_zero_blocks(B):
    say("zero blocks")
    for kv, D in (("bf16", 128), ("fp8", 64), ("f32", 64)):
        pool = B.KVPool.allocate(12, 16, 3, D, kv, fill_byte=0xAB)
        ids = torch.tensor([3, 7, -1, 12, 0], dtype=torch.int32, device="cuda")
        B.zero_blocks(pool, ids)
        torch.cuda.synchronize()
        for which in ("k", "v"):
            a = pool.logical(which).view(np.uint8).reshape(12, -1)
            for b in range(12):
                want = 0 if b in (0, 3, 7) else 0xAB
                assert (a[b] == want).all(), (kv, which, b)


def test_serving_loop_against_oracle(B):
    from paged_kv_cache_pool_amd import serve
    say("serving loop scenario")
    pool = B.KVPool.allocate(SC.POOL["num_blocks"], SC.POOL["block_size"], SC.POOL["num_kv_heads"],
                             SC.POOL["head_dim"], "bf16", fill_byte=0xFF)
    loop = serve.ServingLoop(pool, **SC.LOOP)
    for r in SC.requests():
        loop.add_request(r)
    orc = O.Pool(SC.POOL["num_blocks"], 16, SC.POOL["num_kv_heads"], SC.POOL["head_dim"], "bf16")
    steps = worst = 0
    while not loop.done():
        plan = loop.schedule()
        assert plan is not None
        out, slots = loop.execute(plan)
        torch.cuda.synchronize()
        # the oracle: zero the same blocks, write with its own slots, attend
        if plan.new_blocks:
            orc.k[plan.new_blocks] = 0
            orc.v[plan.new_blocks] = 0
        want_slots = O.slot_mapping(plan.query_start_loc, plan.seq_lens, plan.block_table, 16)
        assert (slots.cpu().numpy() == want_slots).all(), steps
        O.write_kv(orc, plan.key, plan.value, "bf16", want_slots)
        ref = O.attention(orc, plan.query_start_loc, plan.seq_lens, plan.block_table, plan.query,
                          "bf16", SC.LOOP["num_q_heads"], loop.scale)
        got = out.float().cpu().numpy().astype(np.float64)
        err = float(np.abs(got - ref).max())
        worst = max(worst, err)
        assert np.isfinite(got).all() and err <= 2e-2, (steps, err)
        loop.commit(plan)
        steps += 1
        assert steps < 1000
    say("steps", steps, "max_abs_err", worst)
    assert sorted(loop.finished) == list(range(12))
    for which in ("k", "v"):
        g = pool.logical(which)
        o = orc.k if which == "k" else orc.v
        assert (g == o).all(), which

"""The host block pool: the library's pa_kv_manager against the pages' worked
examples and against the plain reference model oracle/kv_manager.py (written
from the pages; no shared code), plus invariants.  CPU only.

Pins of the model itself: the pages' lifecycle examples (§10.1-10.3 of
"vLLM 推理流程分析", tests/golden/page_examples.txt), the published FNV-1a 64
test vectors for the block hash, and invariants any block pool keeps
(every block is either in the free queue or referenced; reference counts
equal the number of requests holding a block; a hit returns blocks whose
cached tokens are the lookup's own)."""
import os

import numpy as np
import pytest

from oracle import kv_manager as OM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.txt")


@pytest.fixture(scope="module")
def B():
    from paged_kv_cache_pool_amd import binding
    return binding


def _pool_examples():
    out = []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, fields, cite = [x.strip() for x in line.split("|", 2)]
        if k != "pool":
            continue
        d = {"cite": cite}
        for f in fields.split():
            key, val = f.split("=", 1)
            d[key] = val if key == "name" else [int(x) for x in val.split(",")]
        out.append(d)
    return out


def test_fnv1a64_published_vectors():
    # test vectors of the FNV reference (Fowler, Noll, Vo): 64-bit FNV-1a
    assert OM.fnv1a64(b"") == 0xCBF29CE484222325
    assert OM.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert OM.fnv1a64(b"foobar") == 0x85944171F73967E8


def _managers(B, nb, S):
    return [OM.KVManagerModel(nb, S), B.KVManager(nb, S)]


@pytest.mark.parametrize("ex", _pool_examples(), ids=lambda e: e["name"])
def test_page_lifecycle_examples(B, ex):
    S = ex["S"][0]
    a = ex["a"]
    for m in _managers(B, 16, S):
        assert m.allocate_slots(1, len(a)) == list(range(-(-len(a) // S)))
        blocks = m.block_ids(1)
        if "blocks_a" in ex:
            assert blocks == ex["blocks_a"], ex["cite"]
            slots = [blocks[p // S] * S + p % S for p in range(len(a))]
            assert slots == ex["slots_a"], ex["cite"]
        if "decode" in ex:
            grew = []
            for step in range(1, ex["decode"][0] + 1):
                new = m.allocate_slots(1, len(a) + step)
                if new:
                    grew.append(step)
            assert grew == ex["grow_at"], ex["cite"]
        if "b" in ex:
            m.cache_blocks(1, a, len(a))
            hit = m.get_computed_blocks(ex["b"])
            assert hit == ex["hit"], ex["cite"]
            assert m.ref_count(hit[0]) == 1
            new = m.allocate_slots(2, len(ex["b"]), hit)
            assert m.ref_count(hit[0]) == ex["ref_after"][0], ex["cite"]
            assert len(hit) * S == ex["computed"][0], ex["cite"]
            assert m.block_ids(2)[0] == hit[0] and new and new[0] not in m.block_ids(1)


def _check_invariants(models, live):
    ref, lib = models
    nb = ref.num_blocks
    held = np.zeros(nb, dtype=int)
    for r in live:
        for b in ref.block_ids(r):
            held[b] += 1
    for b in range(nb):
        assert ref.ref_count(b) == held[b] == lib.ref_count(b)
    assert ref.num_free_blocks() == lib.num_free_blocks() == int((held == 0).sum())
    assert sorted(ref.free_queue) == [b for b in range(nb) if held[b] == 0]


@pytest.mark.parametrize("seed", range(12))
def test_library_matches_model_random_ops(B, seed):
    """Random lives of requests that share prefixes (a few system prompts,
    two extra keys), under capacity pressure: every call gives the same
    answer in the library and in the model, and the invariants hold."""
    rng = np.random.default_rng(seed)
    S = [4, 16, 1, 8][seed % 4]
    nb = int(rng.integers(12, 60))
    models = _managers(B, nb, S)
    prompts = [rng.integers(0, 50, size=int(rng.integers(1, 6 * S))).tolist() for _ in range(4)]
    live, toks, keys = {}, {}, {}
    next_id = 0
    for op in range(300):
        kind = rng.integers(0, 4)
        if kind == 0 or not live:              # a new request: prefix hit + prompt
            base = prompts[int(rng.integers(0, len(prompts)))]
            t = base + rng.integers(0, 50, size=int(rng.integers(0, 2 * S))).tolist()
            if not t:
                t = [1]
            key = int(rng.integers(0, 2))
            hits = [m.get_computed_blocks(t, key) for m in models]
            assert hits[0] == hits[1]
            for i, b in enumerate(hits[0]):    # a hit holds exactly these tokens
                assert models[0].block_key[b][1][1:] == (key, tuple(t[i * S:(i + 1) * S]))
            res = [m.allocate_slots(next_id, len(t), hits[0]) for m in models]
            assert res[0] == res[1]
            if res[0] is not None:
                live[next_id], toks[next_id], keys[next_id] = len(t), t, key
                for m in models:
                    m.cache_blocks(next_id, t, len(t), key)
            next_id += 1
        elif kind == 1:                        # grow a running request (decode / chunk)
            r = list(live)[int(rng.integers(0, len(live)))]
            n = live[r] + int(rng.integers(1, 3 * S))
            res = [m.allocate_slots(r, n) for m in models]
            assert res[0] == res[1]
            if res[0] is not None:
                toks[r] = toks[r] + rng.integers(0, 50, size=n - live[r]).tolist()
                live[r] = n
                for m in models:
                    m.cache_blocks(r, toks[r], n, keys[r])
        else:                                  # finish (free) a request
            r = list(live)[int(rng.integers(0, len(live)))]
            for m in models:
                m.free(r)
            del live[r]
        for r in live:
            assert models[0].block_ids(r) == models[1].block_ids(r)
        _check_invariants(models, live)


def test_hit_needs_same_extra_key_and_survives_free_until_reuse(B):
    for m in _managers(B, 6, 4):
        t = list(range(100, 113))
        m.allocate_slots(1, len(t))
        m.cache_blocks(1, t, len(t), 7)
        assert m.get_computed_blocks(t, 7) == [0, 1, 2]
        assert m.get_computed_blocks(t, 8) == []                 # other identity
        assert m.get_computed_blocks(t[:12], 7) == [0, 1]        # last token's block never hits
        m.free(1)                                                # ref 0, still cached
        assert m.num_free_blocks() == 6
        assert m.get_computed_blocks(t, 7) == [0, 1, 2]
        # queue order after the free: 4, 5 (never used), then 3, 2, 1, 0
        assert m.allocate_slots(2, 4 * 3) == [4, 5, 3]
        assert m.get_computed_blocks(t, 7) == [0, 1, 2]          # block 3 was not cached
        assert m.allocate_slots(3, 4) == [2]                     # block 2 is reused ...
        assert m.get_computed_blocks(t, 7) == [0, 1]             # ... and no longer a hit


def test_capacity_failure_changes_nothing(B):
    for m in _managers(B, 4, 4):
        assert m.allocate_slots(1, 12) == [0, 1, 2]
        before = (m.num_free_blocks(), [m.ref_count(b) for b in range(4)])
        assert m.allocate_slots(2, 8) is None
        assert (m.num_free_blocks(), [m.ref_count(b) for b in range(4)]) == before
        assert m.allocate_slots(2, 4) == [3]


def test_library_argument_errors(B):
    m = B.KVManager(4, 4)
    with pytest.raises(B.PaError):
        m.free(99)
    with pytest.raises(B.PaError):
        m.block_ids(99)
    m.allocate_slots(1, 4)
    with pytest.raises(B.PaError):
        m.allocate_slots(1, 8, [0])      # computed blocks for a request that has blocks
    with pytest.raises(B.PaError):
        m.allocate_slots(2, 8, [3])      # block 3 holds no cached content

"""A shared continuous-batching scenario for the serving-loop tests: twelve
requests built on three system prompts (so later requests hit the prefix
cache), two extra keys, prompts of 18..130 tokens, 2..10 new tokens each,
a 30-block pool of 16-token blocks (too small to admit every request at
once, so admission waits for blocks), a
128-token budget and at most 8 running requests."""
import numpy as np

from paged_kv_cache_pool_amd import serve


def requests(seed=0, n=12):
    rng = np.random.default_rng(seed)
    systems = [rng.integers(0, 32000, size=int(L)).tolist() for L in (40, 64, 17)]
    out = []
    for i in range(n):
        sp = systems[i % 3]
        tail = rng.integers(0, 32000, size=int(rng.integers(1, 66))).tolist()
        out.append(serve.Request(req_id=i, prompt=sp + tail, max_new_tokens=int(rng.integers(2, 11)),
                                 extra_key=int(i % 4 == 3)))
    return out


POOL = dict(num_blocks=30, block_size=16, num_kv_heads=2, head_dim=128)
LOOP = dict(num_q_heads=8, token_budget=128, max_num_seqs=8)

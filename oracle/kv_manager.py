"""Reference model of the host block pool -- TEST INFRASTRUCTURE ONLY.

Plain Python, written from the pages, with no code shared with the library's
pa_kv_manager (only tests/ import it):

* "vLLM 推理流程分析" §4.2-4.3: allocate_slots gives a request physical blocks
  for its new tokens, after taking the blocks a prefix-cache hit found
  (get_computed_blocks: hash each full block of the prompt, look the hash up
  in the block-hash map, return the hit blocks);
* §8.1: free decrements the reference count of every block of the request,
  and a block whose count reaches zero goes back to the free queue;
* §10.1-10.3: a prompt's blocks are allocated as it grows; a decode step
  needs a new block only when the last one is full; a second request with
  the same prefix hits the first request's block and raises its reference
  count from 1 to 2;
* "vLLM 源码完全拆解（十六）", second walk-through path: a block with
  reference count zero keeps its contents for hits until it is reused; the
  cache key covers the parent prefix and extra identity besides the block's
  tokens.

Where the pages leave the policy open the model takes the plainest reading,
the same the library documents: the free queue starts in ascending block
order and hands blocks out from its front; a freed request returns its
blocks last block first; a block handed out again is no longer a hit; the
block holding a prompt's last token is never a hit (one token is always
computed).  The block hash is FNV-1a 64 (Fowler-Noll-Vo, offset basis
0xcbf29ce484222325, prime 0x100000001b3) over the little-endian bytes of the
parent hash (0 first), the extra key and the block's token ids as int32; a
hit also requires the stored key to be equal.

The free queue is a plain list (O(n) removals): fine for test sizes.
"""
from __future__ import annotations

import struct
from typing import Dict, List, Optional, Sequence, Tuple

_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = _FNV_OFFSET) -> int:
    for byte in data:
        h ^= byte
        h = (h * _FNV_PRIME) & _MASK
    return h


def block_hash(parent: int, extra_key: int, tokens: Sequence[int]) -> int:
    data = struct.pack("<QQ", parent & _MASK, extra_key & _MASK)
    data += struct.pack("<%di" % len(tokens), *tokens)
    return fnv1a64(data)


class KVManagerModel:
    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.free_queue: List[int] = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.block_key: Dict[int, Tuple[int, Tuple[int, int, Tuple[int, ...]]]] = {}
        self.hash_to_block: Dict[int, int] = {}
        self.req_blocks: Dict[int, List[int]] = {}

    def num_free_blocks(self) -> int:
        return len(self.free_queue)

    def get_computed_blocks(self, token_ids: Sequence[int], extra_key: int = 0) -> List[int]:
        S = self.block_size
        usable = max(0, len(token_ids) - 1) // S        # blocks before the last token's block
        hits, parent = [], 0
        for i in range(usable):
            toks = tuple(int(t) for t in token_ids[i * S:(i + 1) * S])
            h = block_hash(parent, extra_key, toks)
            b = self.hash_to_block.get(h)
            if b is None or self.block_key[b][1] != (parent, extra_key, toks):
                break
            hits.append(b)
            parent = h
        return hits

    def allocate_slots(self, req: int, num_tokens: int, computed: Sequence[int] = ()) -> Optional[List[int]]:
        have = self.req_blocks.get(req, [])
        if have and computed:
            raise ValueError("computed blocks only for a request without blocks")
        need = -(-num_tokens // self.block_size)
        fresh = need - len(have) - len(computed)
        in_queue = sum(1 for b in computed if b in self.free_queue)
        if fresh > 0 and fresh > len(self.free_queue) - in_queue:
            return None
        blocks = self.req_blocks.setdefault(req, [])
        for b in computed:                                  # touch
            if b in self.free_queue:
                self.free_queue.remove(b)
            self.ref[b] += 1
            blocks.append(b)
        new = []
        for _ in range(max(0, fresh)):
            b = self.free_queue.pop(0)
            if b in self.block_key:                         # reused: no longer a hit
                h, _key = self.block_key.pop(b)
                if self.hash_to_block.get(h) == b:
                    del self.hash_to_block[h]
            self.ref[b] = 1
            blocks.append(b)
            new.append(b)
        return new

    def cache_blocks(self, req: int, token_ids: Sequence[int], num_tokens: int, extra_key: int = 0) -> None:
        S = self.block_size
        blocks = self.req_blocks[req]
        parent = 0
        for i in range(min(num_tokens // S, len(blocks))):
            toks = tuple(int(t) for t in token_ids[i * S:(i + 1) * S])
            h = block_hash(parent, extra_key, toks)
            b = blocks[i]
            if b not in self.block_key and h not in self.hash_to_block:
                self.block_key[b] = (h, (parent, extra_key, toks))
                self.hash_to_block[h] = b
            parent = h

    def free(self, req: int) -> None:
        for b in reversed(self.req_blocks.pop(req)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free_queue.append(b)

    def block_ids(self, req: int) -> List[int]:
        return list(self.req_blocks[req])

    def ref_count(self, block: int) -> int:
        return self.ref[block]

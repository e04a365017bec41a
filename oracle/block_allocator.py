"""Plain model of the host-side block allocator of a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It follows the
behaviour the pages describe, step by step, with plain Python containers:

* faulkner, "Prefix Caching 与 Copy-on-Write": a full block is identified by
  a chained hash H_k = Hash(H_{k-1}, tokens of block k) with H_{-1} = 0; a
  block whose reference count drops to zero is not wiped but parked in an
  LRU pool of evictable blocks, indexed by its hash; a new prompt matches
  its leading full blocks against that index (H_0, H_1, ... in order), and
  a hit only increments the block's reference count; copy-on-write splits a
  partly filled tail block shared by several sequences (ref_count > 1) when
  one of them appends: a fresh block gets the existing slots plus the new
  token, and the old block's count drops by one.
* faulkner, "块分配器与 Prefix Caching 参考实现": the hash is BLAKE2b with an
  8-byte digest over the parent hash (8 bytes, little-endian) followed by
  each token id (4 bytes, little-endian); blocks are taken from the least
  recently used end of the evictable pool (all blocks, in id order, at the
  start), losing any hash they had; running out of blocks raises
  ``MemoryError``; prefix matching stops at the first full block that
  misses (or at the partial last block), and later full blocks of the
  prompt are registered under their hashes; freeing a sequence decrements
  each of its blocks and parks the ones that reach zero at the most
  recently used end; appending a token to a full tail block takes a new
  block.  Where a hash was registered again on a fresh block (after the
  first block of that chain was evicted), taking the older block removes
  the index entry only if it still names that block.  The listing raises
  partway through a prompt; here an allocation
  that cannot be met changes nothing (the blocks a failed prompt would have
  taken would otherwise stay owned by no sequence), the plainest reading
  that keeps the reference counts exact.
* qwbw section 4.3: sequences sharing a prompt prefix point their block
  tables at the same physical blocks (copy-on-write), and preempted
  sequences' blocks can be swapped out to host memory and back.
"""

from __future__ import annotations

import hashlib
from collections import OrderedDict

import numpy as np


def block_hash(parent: int, tokens) -> int:
    """Chained hash of one full block: BLAKE2b-64 over the parent hash and
    the block's token ids (faulkner, allocator reference implementation)."""
    h = hashlib.blake2b(digest_size=8)
    h.update(int(parent).to_bytes(8, "little", signed=False))
    for t in tokens:
        h.update(int(t).to_bytes(4, "little", signed=False))
    return int.from_bytes(h.digest(), "little", signed=False)


class BlockAllocator:
    """Reference counts, chained-hash prefix reuse, LRU eviction and
    copy-on-write over ``num_blocks`` physical blocks of ``block_size``
    slots.  ``order`` is the initial evictable order (default: block ids in
    increasing order)."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.hash: list[int | None] = [None] * num_blocks
        self.tokens: list[list[int]] = [[] for _ in range(num_blocks)]
        ids = range(num_blocks) if order is None else [int(i) for i in order]
        if sorted(ids) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        self.evictable: OrderedDict[int, None] = OrderedDict((i, None) for i in ids)
        self.by_hash: dict[int, int] = {}

    # -- one fresh block from the LRU end of the evictable pool
    def _take(self) -> int:
        if not self.evictable:
            raise MemoryError("out of KV cache blocks")
        blk, _ = self.evictable.popitem(last=False)
        if self.hash[blk] is not None:
            # the index entry goes only if it still names this block: after an
            # eviction a later prompt can register the same hash on a fresh
            # block, and that entry must stay
            if self.by_hash.get(self.hash[blk]) == blk:
                del self.by_hash[self.hash[blk]]
            self.hash[blk] = None
        self.tokens[blk] = []
        self.ref[blk] = 1
        return blk

    def allocate_prompt(self, token_ids) -> tuple[list[int], int]:
        """Block table of a new prompt and how many of its tokens were found
        cached."""
        bs = self.block_size
        # all or nothing: count the leading hits (and those parked in the
        # evictable pool, which leave it), then the fresh blocks still needed
        hits, parked, parent = 0, set(), 0
        for start in range(0, len(token_ids), bs):
            chunk = [int(t) for t in token_ids[start:start + bs]]
            if len(chunk) < bs:
                break
            parent = block_hash(parent, chunk)
            hit = self.by_hash.get(parent)
            if hit is None:
                break
            hits += 1
            if self.ref[hit] == 0:
                parked.add(hit)
        need = -(-len(token_ids) // bs) - hits
        if need > len(self.evictable) - len(parked):
            raise MemoryError("out of KV cache blocks")
        table: list[int] = []
        cached = 0
        parent = 0
        matching = True
        for start in range(0, len(token_ids), bs):
            chunk = [int(t) for t in token_ids[start:start + bs]]
            full = len(chunk) == bs
            if matching and full:
                h = block_hash(parent, chunk)
                hit = self.by_hash.get(h)
                if hit is not None:
                    if self.ref[hit] == 0:
                        del self.evictable[hit]
                    self.ref[hit] += 1
                    table.append(hit)
                    cached += bs
                    parent = h
                    continue
            matching = False
            blk = self._take()
            self.tokens[blk] = list(chunk)
            if full:
                h = block_hash(parent, chunk)
                self.hash[blk] = h
                self.by_hash[h] = blk
                parent = h
            table.append(blk)
        return table, cached

    def append_token(self, table: list[int], token: int):
        """Append one decoded token to a sequence (its table is updated in
        place).  Returns ``(src, dst)`` when copy-on-write moved the tail
        block (the device copies block src's rows to dst), else ``None``."""
        last = table[-1]
        if len(self.tokens[last]) == self.block_size:
            blk = self._take()
            self.tokens[blk] = [int(token)]
            table.append(blk)
            return None
        if self.ref[last] > 1:
            blk = self._take()
            self.ref[last] -= 1
            self.tokens[blk] = list(self.tokens[last]) + [int(token)]
            table[-1] = blk
            return (last, blk)
        self.tokens[last].append(int(token))
        return None

    def fork(self, table: list[int]) -> list[int]:
        """A second sequence sharing all of ``table``'s blocks (parallel
        sampling / beam search share the prompt and its tail block: qwbw
        section 4.3)."""
        for blk in table:
            self.ref[blk] += 1
        return list(table)

    def free_sequence(self, table) -> None:
        for blk in table:
            self.ref[blk] -= 1
            if self.ref[blk] < 0:
                raise ValueError("block freed more often than taken")
            if self.ref[blk] == 0:
                self.evictable[blk] = None

    def num_free(self) -> int:
        return len(self.evictable)


def copy_blocks(pool: np.ndarray, pairs) -> np.ndarray:
    """Copy every slot of block ``src`` onto block ``dst`` for each pair
    (the device side of copy-on-write), bit for bit, in the order given."""
    out = np.array(pool, copy=True)
    for src, dst in pairs:
        out[int(dst)] = out[int(src)]
    return out


def swap_out(pool: np.ndarray, blocks) -> np.ndarray:
    """Rows of the listed blocks, in order, as a host array ``[n, ...]``
    (qwbw section 4.3 and faulkner's preemption section: a preempted
    sequence's blocks move to host memory)."""
    return np.stack([np.array(pool[int(b)], copy=True) for b in blocks]) if len(blocks) else \
        np.zeros((0,) + pool.shape[1:], dtype=pool.dtype)


def swap_in(pool: np.ndarray, host: np.ndarray, blocks) -> np.ndarray:
    """The inverse move: host row i goes back into block ``blocks[i]``."""
    out = np.array(pool, copy=True)
    for i, b in enumerate(blocks):
        out[int(b)] = host[i]
    return out

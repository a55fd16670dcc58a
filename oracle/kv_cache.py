"""Paged KV cache append and block allocator -- TEST INFRASTRUCTURE ONLY.

Oracle for the KV-append step of the paged path.  Only ``tests/`` and the
CPU-baseline leg of ``bench.py`` may use it; the product library never does.
Plain Python and numpy; the arithmetic is byte copies and integer index math.

What it follows:

* The block allocator of "Flash Attention and Paged Attention", section 3
  (the PagedKVCache class): the pool has ``num_blocks`` physical blocks, a
  free list of their ids, ``allocate`` takes ceil(num_tokens / block_size)
  ids off the END of the free list (one pop per block) and fails with a
  RuntimeError when too few are free, ``release`` puts ids back on the end.
* The growth rule of the same section: a request that grows only gets new
  physical blocks and new page-table entries; its existing blocks stay put.
* The decode step of "Sequence length doubles, inference time quadruples"
  (prefill and decode stages): every new token's K and V are appended to the
  cache after the tokens already there.
* The address of token t of a request ("Chunked attention ... 70x slower",
  section 2.1): logical block t // block_size, physical block from the
  request's page table, slot t % block_size; the pool is
  [num_blocks, 2, H, block_size, d] with K at index 0 and V at index 1.

A batch append is all-or-nothing and allocates in request order: request
0's new blocks first, each taken with one pop, then request 1's, ... -- the
same ids, in the same table slots, as calling ``allocate`` once per request
in order.  Before anything changes the whole batch is checked: a request
whose table would need more than ``max_blocks`` entries fails with status
TABLE_FULL, otherwise a batch needing more blocks than are free fails with
status EXHAUSTED.
"""
from __future__ import annotations

import numpy as np

OK, EXHAUSTED, TABLE_FULL = 0, 1, 2


class CacheFull(RuntimeError):
    """Raised when an append cannot be done; ``status`` says why."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks holding num_tokens tokens: ceil(num_tokens / block_size)."""
    return -(-int(num_tokens) // int(block_size))


class BlockAllocator:
    """The pages' free-list allocator over physical block ids."""

    def __init__(self, num_blocks: int, block_size: int, free=None):
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad allocator geometry")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free = list(range(num_blocks)) if free is None else [int(b) for b in free]

    def allocate_blocks(self, count: int) -> list:
        if count > len(self.free):
            raise CacheFull(EXHAUSTED, "KV cache exhausted: need %d blocks, %d free" % (count, len(self.free)))
        return [self.free.pop() for _ in range(count)]

    def allocate(self, num_tokens: int) -> list:
        return self.allocate_blocks(blocks_for(num_tokens, self.block_size))

    def release(self, blocks) -> None:
        self.free.extend(int(b) for b in blocks)


def append(pool: np.ndarray, block_table: np.ndarray, ctx_lens, new_lens, k_new: np.ndarray, v_new: np.ndarray,
           alloc: BlockAllocator):
    """Append new_lens[r] tokens to every request r of a batch.

    pool        : [num_blocks, 2, H, block_size, d], modified in place
    block_table : int32 [num_seqs, max_blocks], modified in place; entries
                  [0, ceil(ctx / bs)) are the request's blocks on entry
    ctx_lens    : tokens already cached per request
    new_lens    : tokens to append per request (>= 0)
    k_new, v_new: packed [sum(new_lens), H, d]; request r's rows start at
                  sum_{s<r} new_lens[s]
    alloc       : the free list (modified)
    Returns the new context lengths ctx + new.  Raises CacheFull (nothing
    modified) when the batch does not fit.
    """
    bs = alloc.block_size
    ctx = [int(c) for c in ctx_lens]
    new = [int(n) for n in new_lens]
    num_seqs, max_blocks = block_table.shape
    have = [blocks_for(c, bs) for c in ctx]
    want = [blocks_for(c + n, bs) for c, n in zip(ctx, new)]
    for r in range(num_seqs):
        if want[r] > max_blocks:
            raise CacheFull(TABLE_FULL, "request %d needs %d table entries, the table has %d"
                            % (r, want[r], max_blocks))
    total = sum(w - h for w, h in zip(want, have))
    if total > len(alloc.free):
        raise CacheFull(EXHAUSTED, "KV cache exhausted: need %d blocks, %d free" % (total, len(alloc.free)))
    for r in range(num_seqs):
        block_table[r, have[r]:want[r]] = alloc.allocate_blocks(want[r] - have[r])
    row = 0
    for r in range(num_seqs):
        for i in range(new[r]):
            t = ctx[r] + i
            pb = int(block_table[r, t // bs])
            pool[pb, 0, :, t % bs, :] = k_new[row + i]
            pool[pb, 1, :, t % bs, :] = v_new[row + i]
        row += new[r]
    return [c + n for c, n in zip(ctx, new)]

"""Pins of the KV-append oracle (oracle/kv_cache.py) against what the pages fix.

* The allocator of "Flash Attention and Paged Attention", section 3: ceil
  division of tokens into blocks, ids taken one pop at a time off the end of
  the free list, release appending to it, RuntimeError when too few are free.
  The expected ids below are worked out by hand from that description.
* Appending K/V ("Sequence length doubles ...", decode stage) must leave
  every request's logical sequence -- read back token by token through its
  page table with the address of "Chunked attention ... 70x slower", section
  2.1 -- equal to its old tokens followed by the new ones, and must leave
  every other slot of the pool untouched.  The read-back below is written
  here, independently of the oracle's write path.
"""
import numpy as np
import pytest

from oracle import kv_cache as kc


def test_allocator_worked_example():
    a = kc.BlockAllocator(10, 16)
    assert kc.blocks_for(33, 16) == 3 and kc.blocks_for(32, 16) == 2 and kc.blocks_for(0, 16) == 0
    assert a.allocate(33) == [9, 8, 7]          # three pops off the end
    assert a.allocate(16) == [6]
    assert a.allocate(0) == []
    a.release([8, 9])
    assert a.free == [0, 1, 2, 3, 4, 5, 8, 9]
    assert a.allocate(1) == [9]                  # last released, first reused
    with pytest.raises(RuntimeError):
        a.allocate(16 * 8)                       # 8 blocks wanted, 7 free
    assert a.free == [0, 1, 2, 3, 4, 5, 8]       # a failed allocate takes nothing


def logical_view(pool, table, ctx_lens, bs):
    """Per-token read-back: token t of request r sits in block table[r, t//bs], slot t%bs."""
    out = []
    for r, c in enumerate(ctx_lens):
        k = np.stack([pool[table[r, t // bs], 0, :, t % bs, :] for t in range(c)]) if c else None
        v = np.stack([pool[table[r, t // bs], 1, :, t % bs, :] for t in range(c)]) if c else None
        out.append((k, v))
    return out


def make_state(rng, num_blocks, bs, H, d, ctx_lens, max_blocks):
    pool = rng.standard_normal((num_blocks, 2, H, bs, d)).astype(np.float32)
    alloc = kc.BlockAllocator(num_blocks, bs, free=rng.permutation(num_blocks).tolist())
    table = np.full((len(ctx_lens), max_blocks), -1, dtype=np.int32)
    for r, c in enumerate(ctx_lens):
        blocks = alloc.allocate(c)
        table[r, :len(blocks)] = blocks
    return pool, table, alloc


@pytest.mark.parametrize("seed", range(6))
def test_append_extends_every_logical_sequence(seed):
    rng = np.random.default_rng(seed)
    bs, H, d = [16, 32][seed % 2], 2, 8
    ctx = [0, 1, bs - 1, bs, bs + 5, 3 * bs, 7][: 3 + seed % 5]
    new = [int(x) for x in rng.integers(0, 2 * bs + 3, len(ctx))]
    new[0] = 0 if seed % 3 == 0 else new[0]
    max_blocks = max(kc.blocks_for(c + n, bs) for c, n in zip(ctx, new)) + 1
    pool, table, alloc = make_state(rng, 64, bs, H, d, ctx, max_blocks)
    before = logical_view(pool, table, ctx, bs)
    pool0, table0 = pool.copy(), table.copy()
    k_new = rng.standard_normal((sum(new), H, d)).astype(np.float32)
    v_new = rng.standard_normal((sum(new), H, d)).astype(np.float32)
    free0 = list(alloc.free)
    ctx1 = kc.append(pool, table, ctx, new, k_new, v_new, alloc)
    assert ctx1 == [c + n for c, n in zip(ctx, new)]
    after = logical_view(pool, table, ctx1, bs)
    row = 0
    for r in range(len(ctx)):
        kb, vb = before[r]
        ka, va = after[r]
        if ctx[r]:
            assert np.array_equal(ka[:ctx[r]], kb) and np.array_equal(va[:ctx[r]], vb)
        if new[r]:
            assert np.array_equal(ka[ctx[r]:], k_new[row:row + new[r]])
            assert np.array_equal(va[ctx[r]:], v_new[row:row + new[r]])
        row += new[r]
        # existing table entries keep their blocks
        h = kc.blocks_for(ctx[r], bs)
        assert np.array_equal(table[r, :h], table0[r, :h])
    # blocks taken = exactly the ones missing from the free list, off its end
    taken = len(free0) - len(alloc.free)
    assert alloc.free == free0[:len(free0) - taken]
    # every slot not holding a new token is untouched
    written = np.zeros(pool.shape[:1] + pool.shape[3:4], dtype=bool)
    for r in range(len(ctx)):
        for t in range(ctx[r], ctx1[r]):
            written[table[r, t // bs], t % bs] = True
    for b in range(pool.shape[0]):
        for s in range(bs):
            if not written[b, s]:
                assert np.array_equal(pool[b, :, :, s, :], pool0[b, :, :, s, :])


def test_batch_allocation_equals_per_request_allocation():
    """Batched append takes the same ids, in the same table slots, as one
    allocate() per request in request order (the reading the GPU path uses)."""
    rng = np.random.default_rng(11)
    bs, H, d = 16, 1, 4
    ctx = [5, 0, 16, 40]
    new = [30, 17, 1, 0]
    pool, table, alloc = make_state(rng, 40, bs, H, d, ctx, 8)
    ref_alloc = kc.BlockAllocator(40, bs, free=list(alloc.free))
    ref_table = table.copy()
    for r in range(len(ctx)):
        h, w = kc.blocks_for(ctx[r], bs), kc.blocks_for(ctx[r] + new[r], bs)
        ref_table[r, h:w] = ref_alloc.allocate_blocks(w - h)
    kc.append(pool, table, ctx, new, np.zeros((sum(new), H, d), np.float32), np.zeros((sum(new), H, d), np.float32),
              alloc)
    assert np.array_equal(table, ref_table) and alloc.free == ref_alloc.free


@pytest.mark.parametrize("case", ["exhausted", "table_full"])
def test_failed_append_changes_nothing(case):
    rng = np.random.default_rng(5)
    bs, H, d = 16, 2, 4
    ctx = [3, 20]
    pool, table, alloc = make_state(rng, 6, bs, H, d, ctx, 3)
    new = [40, 20] if case == "exhausted" else [10, 40]    # 3 blocks wanted, 2 free / 4 table entries needed
    if case == "exhausted":
        alloc.free = alloc.free[:2]
    pool0, table0, free0 = pool.copy(), table.copy(), list(alloc.free)
    with pytest.raises(RuntimeError) as ei:
        kc.append(pool, table, ctx, new, np.ones((sum(new), H, d), np.float32), np.ones((sum(new), H, d), np.float32),
                  alloc)
    assert ei.value.status == (kc.EXHAUSTED if case == "exhausted" else kc.TABLE_FULL)
    assert np.array_equal(pool, pool0) and np.array_equal(table, table0) and alloc.free == free0


def test_partial_block_filled_before_a_new_one():
    """A request ending mid-block first fills that block's free slots."""
    rng = np.random.default_rng(2)
    bs, H, d = 16, 1, 2
    pool, table, alloc = make_state(rng, 8, bs, H, d, [10], 4)
    first = int(table[0, 0])
    nfree = len(alloc.free)
    k_new = np.arange(8 * H * d, dtype=np.float32).reshape(8, H, d)
    kc.append(pool, table, [10], [6], k_new[:6], k_new[:6], alloc)
    assert len(alloc.free) == nfree                    # 10 + 6 = 16 still one block
    assert np.array_equal(pool[first, 0, :, 10:16, :].transpose(1, 0, 2), k_new[:6])
    kc.append(pool, table, [16], [2], k_new[6:], k_new[6:], alloc)
    assert len(alloc.free) == nfree - 1                # token 16 opens block 1
    assert np.array_equal(pool[int(table[0, 1]), 0, :, 0:2, :].transpose(1, 0, 2), k_new[6:])

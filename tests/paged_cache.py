"""Host-side block allocator used by the tests to build block tables.

It mirrors the allocator semantics of the ipipp.com page, section 3
(PagedKVCache): a free list of physical block ids, ``allocate(num_tokens)``
hands out ceil(num_tokens / block_size) blocks taken from the end of the free
list, ``release`` returns blocks to it, and running out raises RuntimeError.
The physical pool itself lives in device memory and is created by the tests;
this class only manages ids.  It is test scaffolding, not part of the product.
"""


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad allocator geometry")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks))

    def blocks_needed(self, num_tokens: int) -> int:
        return -(-num_tokens // self.block_size)

    def allocate(self, num_tokens: int) -> list:
        need = self.blocks_needed(num_tokens)
        if need > len(self.free):
            raise RuntimeError("KV cache exhausted: need %d blocks, %d free" % (need, len(self.free)))
        return [self.free.pop() for _ in range(need)]

    def release(self, blocks) -> None:
        self.free.extend(blocks)

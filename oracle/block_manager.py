"""Plain reference model of the paged KV block manager (host side).

TEST INFRASTRUCTURE ONLY: imported by tests/ and the smoke check, never by
the product path.

Sources (the pages this follows):
  [B1] "PagedAttention and vLLM Architecture: Virtual Memory for LLM Serving",
       section 1: physical memory is a fixed pool of blocks set up at start,
       each holding the K and V of B tokens; a block table kept by the serving
       engine maps each request's logical block b to a physical block.
  [B2] same page, "Why Internal Fragmentation is Bounded": a request gets a
       new block only when a token overflows its current last block, so only
       the last block of a sequence is partly empty (at most B - 1 idle slots).
  [B3] same page, section 3, "Copy-on-Write (CoW) for Parallel Sampling &
       Beam Search": the N streams forked from one prompt share its physical
       blocks, each with reference count N.  When a stream must write into a
       block whose count is above 1, the engine takes a fresh block from the
       free pool, copies the block's tokens into it, lowers the old block's
       count by one and points the stream's table at the copy; later writes
       of that stream go to its private block.
  [A3] "PagedAttention Paper Breakdown: Virtual Memory Allocation for LLM KV
       Cache Serving", section 3, "Dynamic Copy-on-Write (CoW) Parallel
       Sampling": the copy is made only for the writing stream; the shared
       prompt blocks stay untouched for the others.

Readings where the pages are silent (each one is listed in the design notes):
  * the free pool hands out the lowest-numbered free block first (any order
    is correct; this one makes the result unique, so two implementations can
    be compared exactly);
  * a fork makes one child that shares every block of its parent (forking a
    prompt three times gives the four streams of [B3], count 4);
  * a write lands in an existing block only when the sequence's length is
    not a multiple of B; a length that is a multiple of B opens a fresh block
    ([B2]), so a full shared block is never copied;
  * the copy of [B3] copies the whole block (all B token rows of K and V);
  * freeing a sequence lowers the count of each of its blocks; a block whose
    count reaches 0 returns to the free pool;
  * sequence ids are handed out 0, 1, 2, ... and never reused;
  * an operation that would need more free blocks than the pool holds, or a
    table longer than max_blocks, fails and changes nothing;
  * swapping ("PagedAttention Paper Breakdown", Engineering Limitations:
    under memory pressure blocks move between CPU and GPU over PCIe): a
    swap-out saves every block of the sequence to host memory and drops the
    sequence's hold on them (blocks no one else holds return to the pool); a
    swap-in gives the sequence fresh private blocks, lowest first, into
    which the saved contents return.  A swapped sequence cannot append,
    fork or be swapped out again until it is swapped in.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class RefBlockManager:
    """[B1]-[B3] written out with plain Python containers."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks: int):
        assert num_blocks > 0 and block_size > 0 and max_blocks > 0
        self.num_blocks = num_blocks
        self.B = block_size
        self.max_blocks = max_blocks
        self.ref = [0] * num_blocks        # [B3] reference count per physical block
        self.tables = {}                   # [B1] seq id -> list of physical block ids
        self.lens = {}                     # seq id -> tokens held
        self.swapped = {}                  # seq id -> tokens held while on the host
        self.next_id = 0

    # -- the free pool ([B1]); reading: lowest-numbered free block first
    def free_blocks(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def _take_block(self) -> int:
        for b in range(self.num_blocks):
            if self.ref[b] == 0:
                self.ref[b] = 1
                return b
        raise OutOfBlocks()

    # -- sequences
    def add_sequence(self) -> int:
        s = self.next_id
        self.next_id += 1
        self.tables[s] = []
        self.lens[s] = 0
        return s

    def fork(self, parent: int) -> int:
        """[B3]: the child shares every block of the parent."""
        child = self.add_sequence()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def free(self, s: int) -> None:
        if s in self.swapped:                # a swapped sequence holds no blocks
            del self.swapped[s]
            return
        for b in self.tables.pop(s):
            self.ref[b] -= 1
        del self.lens[s]

    def _needs(self, s: int, n: int):
        """Fresh blocks and copies an append of n tokens to s needs."""
        L = self.lens[s]
        B = self.B
        cow = 1 if (n > 0 and L % B != 0 and self.ref[self.tables[s][-1]] > 1) else 0
        held = len(self.tables[s])
        new = max(0, -(-(L + n) // B) - held)
        return new, cow

    def append(self, s: int, n: int):
        """Reserve the slots of n new tokens of sequence s at positions
        L .. L+n-1.  Returns (slots, copies): copies are (src, dst) block
        pairs whose contents must be copied before the tokens are written."""
        new, cow = self._needs(s, n)
        if new + cow > self.free_blocks():
            raise OutOfBlocks()
        if -(-(self.lens[s] + n) // self.B) > self.max_blocks:
            raise OutOfBlocks()
        table = self.tables[s]
        copies = []
        if cow:
            # [B3]: the write would land in a shared block -> private copy
            old = table[-1]
            fresh = self._take_block()
            copies.append((old, fresh))
            self.ref[old] -= 1
            table[-1] = fresh
        slots = []
        for _ in range(n):
            p = self.lens[s]
            if p % self.B == 0:
                table.append(self._take_block())   # [B2]: overflow opens a block
            slots.append(table[p // self.B] * self.B + p % self.B)
            self.lens[s] = p + 1
        return slots, copies

    # -- swapping
    def swap_out(self, s: int):
        """Blocks to save (in table order); the sequence leaves the device."""
        blocks = self.tables.pop(s)
        for b in blocks:
            self.ref[b] -= 1
        self.swapped[s] = self.lens.pop(s)
        return blocks

    def swap_in(self, s: int):
        """Fresh blocks (in table order) that receive the saved contents."""
        L = self.swapped[s]
        need = -(-L // self.B)
        if need > self.free_blocks():
            raise OutOfBlocks()
        del self.swapped[s]
        self.tables[s] = [self._take_block() for _ in range(need)]
        self.lens[s] = L
        return list(self.tables[s])

    # -- views
    def table(self, s: int):
        return list(self.tables[s])

    def length(self, s: int) -> int:
        return self.lens[s]

    def live(self):
        return sorted(self.tables)


def copy_blocks(pool, pairs):
    """Apply (src, dst) whole-block copies to a pool shaped [num_blocks, ...],
    in order, and return the new pool (the input is left untouched)."""
    out = pool.copy()
    for src, dst in pairs:
        out[dst] = out[src]
    return out

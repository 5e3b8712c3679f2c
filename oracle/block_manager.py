"""CPU oracle: the block allocator above the paged cache (free list, block
tables, reference counts, copy-on-write) and the block copy it asks the GPU
for.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the library's allocator or kernels.

From the pages:

* Blocks are allocated on demand: a sequence takes a new block only when its
  last one is full (position % block_size == 0), so it wastes at most
  block_size - 1 slots, all in its last block; a finished sequence returns
  its blocks to the free list at once (KV-cache post, "PagedAttention: the KV
  cache in blocks"; serving lesson, "PagedAttention (Kwon et al., 2023)":
  waste bound).

* Free-list order, from the brunomaga post's ``PagedKVCache``: the free list
  starts as 0 .. num_blocks-1, allocation takes the *last* entry, and freeing
  a sequence appends its table's blocks in table order.  Running out of free
  blocks is an error the scheduler must handle (preemption).

* Sharing and copy-on-write (serving lesson, "Sharing (section 4.4)"; KV-cache
  post, "Sharing"; brunomaga post): a physical block may sit in several
  block tables; a reference count says how many.  A forked sequence (another
  sample of the same prompt) maps its blocks to the parent's and each count
  goes up by one.  Before a sequence writes into a block whose count is above
  1, it takes a private copy: a new block receives the old one's contents
  (that copy is the only device work), the old block's count drops by 1, and
  the sequence's table points at the copy.  The last sharer finds a count of 1
  and writes in place.  Only a partly filled last block can be written, so an
  append copies at most one block.

* The serving lesson's exercise 3 fixes the numbers: three samples of a
  100-token prompt in 16-token blocks take 21 blocks unshared and 7 shared
  (count 3); when each sample writes its first new token, the first two copy
  the last block (its count drops to 2, then 1) and the third writes in
  place: 9 blocks.

An append that needs more blocks than are free changes nothing and raises.
"""

from __future__ import annotations

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks))           # allocation pops the last entry
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}

    # -- sequences ------------------------------------------------------------------
    def add(self, seq: int):
        if seq in self.tables:
            raise KeyError(seq)
        self.tables[seq] = []
        self.lengths[seq] = 0

    def fork(self, parent: int, child: int):
        """child shares every block of parent (parallel samples of one prompt)."""
        if child in self.tables or parent not in self.tables:
            raise KeyError((parent, child))
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int):
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lengths[seq]

    def _blocks_needed(self, seq: int, n: int) -> int:
        table, length, bs = self.tables[seq], self.lengths[seq], self.block_size
        new = -(-(length + n) // bs) - len(table)
        cow = 1 if n > 0 and length % bs != 0 and self.ref[table[length // bs]] > 1 else 0
        return max(new, 0) + cow

    def append_slots(self, seq: int, n: int) -> list[tuple[int, int]]:
        """Make room for n new tokens of seq (positions length .. length+n-1).
        Returns the (source, destination) block copies copy-on-write needs."""
        if self._blocks_needed(seq, n) > len(self.free):
            raise OutOfBlocks("out of KV cache blocks: the scheduler must preempt a sequence")
        table, bs = self.tables[seq], self.block_size
        copies = []
        for pos in range(self.lengths[seq], self.lengths[seq] + n):
            lb = pos // bs
            if lb == len(table):                      # the last block is full: a new one
                b = self.free.pop()
                self.ref[b] = 1
                table.append(b)
            elif self.ref[table[lb]] > 1:             # shared: copy before writing
                old = table[lb]
                b = self.free.pop()
                self.ref[b] = 1
                self.ref[old] -= 1
                table[lb] = b
                copies.append((old, b))
        self.lengths[seq] += n
        return copies

    # -- views ------------------------------------------------------------------------
    def used_blocks(self) -> int:
        return self.num_blocks - len(self.free)

    def block_tables(self, seqs, max_blocks: int):
        """int32 [len(seqs), max_blocks] tables (-1 padded) and int32 lengths."""
        out = np.full((len(seqs), max_blocks), -1, np.int32)
        lens = np.zeros(len(seqs), np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            out[i, :len(t)] = t
            lens[i] = self.lengths[s]
        return out, lens


def copy_blocks(pools, pairs):
    """Apply copy-on-write copies: for each (src, dst), every pool's block dst
    becomes a copy of block src (all KV heads and slots; for an e4m3 cache
    the per-(block, head) scales are pools too).  Returns new arrays."""
    out = [np.array(p, copy=True) for p in pools]
    for src, dst in pairs:
        for o, p in zip(out, pools):
            o[dst] = p[src]
    return out

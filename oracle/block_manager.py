"""Block manager of a paged KV cache: on-demand allocation, freeing, sharing
by reference counts and copy-on-write at divergence; plus the block copy the
copy-on-write step asks for.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

What the pages fix:

* The cache is a pool of fixed-size physical blocks (16 or 32 tokens) and each
  sequence's table maps its logical positions to blocks; blocks are taken only
  as tokens are generated, so only a sequence's last block can have unused
  slots (How vLLM gets real throughput on H100s, "PagedAttention borrows from
  operating systems"; vLLM architecture, memory and benchmarks deep dive,
  "PagedAttention: a 1960s idea for modern GPUs").
* A request that needs space takes any free block from the pool, and a
  finished request's blocks go back to the pool at once, ready for the next
  request (Dissecting vLLM, "PagedAttention: Virtual Memory for KV Cache";
  How vLLM gets real throughput on H100s, "Continuous batching removes
  straggler bubbles").
* Rollouts or samples of one prompt point their tables at the prompt's
  physical blocks; a block is duplicated only when a sequence that shares it
  diverges, i.e. writes into it (copy-on-write, the same three sections).

Readings where the pages are silent:

* The free pool is a stack: the most recently freed block is reused first;
  initially block 0 is taken first, then 1, 2, ...
* ``free`` releases a sequence's blocks from its last logical block to its
  first; each block whose count drops to zero goes onto the stack.
* ``fork`` gives the child the parent's table and length; every block's
  count grows by one.
* ``append`` of k tokens to a sequence of n tokens: a position p with
  p % bs == 0 takes a new block; if n % bs != 0 and the last block is shared
  (count > 1), that block is first copied to a new block (copy-on-write,
  whole-block copy) and the sequence's table entry moved to the copy. The
  call either succeeds whole or changes nothing: it fails when the pool
  lacks the blocks it needs or the table would exceed its capacity.
"""

import numpy as np

OK = "ok"
OUT_OF_BLOCKS = "out_of_blocks"
STATE = "state"
SHAPE = "shape"


class BlockManagerRef:
    def __init__(self, num_blocks, block_size, max_blocks_per_seq):
        if num_blocks <= 0 or block_size <= 0 or max_blocks_per_seq <= 0:
            raise ValueError("sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.capacity = max_blocks_per_seq
        self.free_stack = list(range(num_blocks - 1, -1, -1))   # pop() -> 0, 1, 2, ...
        self.refcount = [0] * num_blocks
        self.tables = {}    # seq -> list of physical blocks
        self.lengths = {}   # seq -> tokens
        self.copies = []    # pending (src, dst) block copies

    # -- queries ----------------------------------------------------------------
    def num_free(self):
        return len(self.free_stack)

    def length(self, seq):
        return self.lengths.get(seq, -1)

    def table(self, seq):
        return list(self.tables[seq])

    def blocks_needed(self, seq, k):
        """Blocks an append of k tokens would take from the pool."""
        n = self.lengths[seq]
        bs = self.block_size
        new = sum(1 for p in range(n, n + k) if p % bs == 0)
        cow = 1 if (k > 0 and n % bs != 0 and self.refcount[self.tables[seq][-1]] > 1) else 0
        return new + cow

    def take_copies(self):
        out, self.copies = self.copies, []
        return out

    # -- operations -------------------------------------------------------------
    def add(self, seq):
        if seq in self.tables:
            return STATE
        self.tables[seq] = []
        self.lengths[seq] = 0
        return OK

    def fork(self, parent, child):
        if parent not in self.tables or child in self.tables:
            return STATE
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            self.refcount[blk] += 1
        return OK

    def _take(self):
        blk = self.free_stack.pop()
        self.refcount[blk] = 1
        return blk

    def append(self, seq, k):
        """Reserve k new positions; returns (status, slots)."""
        if seq not in self.tables:
            return STATE, []
        if k < 0:
            return SHAPE, []
        n = self.lengths[seq]
        bs = self.block_size
        if -(-(n + k) // bs) > self.capacity:
            return SHAPE, []
        if self.blocks_needed(seq, k) > self.num_free():
            return OUT_OF_BLOCKS, []
        table = self.tables[seq]
        if k > 0 and n % bs != 0 and self.refcount[table[-1]] > 1:
            src = table[-1]
            dst = self._take()
            self.refcount[src] -= 1
            table[-1] = dst
            self.copies.append((src, dst))
        slots = []
        for p in range(n, n + k):
            if p % bs == 0:
                table.append(self._take())
            slots.append(table[p // bs] * bs + p % bs)
        self.lengths[seq] = n + k
        return OK, slots

    def free(self, seq):
        if seq not in self.tables:
            return STATE
        for blk in reversed(self.tables[seq]):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free_stack.append(blk)
        del self.tables[seq]
        del self.lengths[seq]
        return OK


def copy_blocks_ref(key_cache, value_cache, pairs):
    """Copies of the caches with block ``dst`` set to block ``src`` for every
    pair, in order (all heads, all rows; a bit copy)."""
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for src, dst in pairs:
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc


def move_blocks_ref(src_key, src_value, dst_key, dst_value, pairs):
    """Copies of the destination pools with block ``dst`` set to source block
    ``src`` for every pair (swapping between the device cache and a host pool:
    Dissecting vLLM, "Continuous Batching: Breaking the Sequence Barrier")."""
    dk = np.array(dst_key, copy=True)
    dv = np.array(dst_value, copy=True)
    for src, dst in pairs:
        dk[dst] = src_key[src]
        dv[dst] = src_value[src]
    return dk, dv

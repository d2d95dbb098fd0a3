"""Pins of the block-manager oracle: the pages' Figure 1/2 allocation, closed
forms for prompt sharing, pool invariants, all-or-nothing failure, and a
brute-force content simulation in which every sequence must read back its
own token history through its table after any mix of add / fork / append /
free (the property copy-on-write exists for)."""

import json
import os

import numpy as np
import pytest

from oracle import accounting
from oracle.block_manager import (OK, OUT_OF_BLOCKS, SHAPE, STATE, BlockManagerRef,
                                  copy_blocks_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _invariants(bm):
    held = {}
    for seq, table in bm.tables.items():
        assert len(table) == -(-bm.lengths[seq] // bm.block_size)   # only the last block partial
        for blk in table:
            held[blk] = held.get(blk, 0) + 1
    for blk in range(bm.num_blocks):
        assert bm.refcount[blk] == held.get(blk, 0)
    assert len(set(bm.free_stack)) == len(bm.free_stack)
    assert set(bm.free_stack).isdisjoint(held)
    assert len(bm.free_stack) + len(held) == bm.num_blocks


def test_figures_1_2_paged_allocation():
    g = json.load(open(os.path.join(GOLDEN, "figs_1_2_allocation.json")))
    bm = BlockManagerRef(num_blocks=9, block_size=g["block_size"], max_blocks_per_seq=3)
    for seq, n in enumerate(g["request_lengths"]):
        assert bm.add(seq) == OK
        status, slots = bm.append(seq, n)
        assert status == OK and len(slots) == n
    per = [len(bm.table(s)) for s in range(len(g["request_lengths"]))]
    assert per == g["paged"]["blocks_per_request"]
    reserved = (bm.num_blocks - bm.num_free()) * bm.block_size
    assert reserved == g["paged"]["reserved"]
    assert reserved - sum(g["request_lengths"]) == g["paged"]["unused"]
    assert g["contiguous"]["reserved"] - reserved == g["paged"]["freed_vs_contiguous"]
    _invariants(bm)


def test_stack_order_and_immediate_reuse():
    bm = BlockManagerRef(8, 4, 8)
    bm.add("a")
    assert bm.append("a", 9)[1] == [0, 1, 2, 3, 4, 5, 6, 7, 8]   # blocks 0, 1, 2
    bm.add("b")
    assert bm.append("b", 1)[1] == [12]                          # block 3
    bm.free("a")                   # blocks go back last-to-first: 2, 1, 0 -> 0 on top
    bm.add("c")
    assert bm.append("c", 5)[1] == [0, 1, 2, 3, 4]               # blocks 0, 1
    _invariants(bm)


@pytest.mark.parametrize("prompt,rollouts,bs", [(4096, 16, 16), (4100, 8, 16), (45, 5, 32),
                                               (3, 4, 4)])
def test_prompt_sharing_closed_form(prompt, rollouts, bs):
    rng = np.random.default_rng(prompt + rollouts)
    tails = [int(x) for x in rng.integers(1, 300, size=rollouts)]
    bm = BlockManagerRef(10_000, bs, 1024)
    bm.add(0)
    bm.append(0, prompt)
    for r in range(1, rollouts + 1):
        assert bm.fork(0, r) == OK
    bm.free(0)
    for r in range(1, rollouts + 1):
        assert bm.append(r, tails[r - 1])[0] == OK
    full, partial = divmod(prompt, bs)
    copies = bm.take_copies()
    if partial == 0:
        expected = full + sum(-(-t // bs) for t in tails)
        assert copies == []
    else:
        # every rollout but the last one to write copies the shared partial block
        expected = full + 1 + (rollouts - 1) + sum(
            -(-(prompt + t) // bs) - (full + 1) for t in tails)
        assert len(copies) == rollouts - 1
        src = {s for s, _ in copies}
        assert len(src) == 1
    assert bm.num_blocks - bm.num_free() == expected
    _invariants(bm)


def test_internal_fragmentation_bound():
    # waste is the last block's slack: < 4 % once n > 24 (bs - 1)
    for bs in (16, 32):
        bm = BlockManagerRef(100_000, bs, 100_000)
        lens = [24 * (bs - 1) + 1 + k for k in range(0, 3000, 7)]
        for i, n in enumerate(lens):
            bm.add(i)
            bm.append(i, n)
        reserved = (bm.num_blocks - bm.num_free()) * bs
        assert reserved == accounting.paged_slots(lens, bs)
        for n in lens:
            assert accounting.internal_fragmentation([n], bs) < 0.04


def test_failure_changes_nothing():
    bm = BlockManagerRef(3, 4, 3)
    bm.add(0)
    bm.append(0, 6)
    bm.fork(0, 1)
    before = (list(bm.free_stack), list(bm.refcount), {k: list(v) for k, v in bm.tables.items()},
              dict(bm.lengths))
    # seq 1 writing at position 6 needs a copy of the shared block plus, for
    # 3 tokens, one more block: 2 > 1 free
    assert bm.blocks_needed(1, 3) == 2
    assert bm.append(1, 3) == (OUT_OF_BLOCKS, [])
    assert bm.append(0, 7)[0] == SHAPE          # 13 tokens need 4 blocks > capacity 3
    assert bm.append(7, 1)[0] == STATE
    assert bm.fork(0, 1) == STATE and bm.fork(9, 10) == STATE and bm.add(0) == STATE
    after = (list(bm.free_stack), list(bm.refcount), {k: list(v) for k, v in bm.tables.items()},
             dict(bm.lengths))
    assert before == after
    assert bm.take_copies() == []


def _simulate(bm_factory, seed, steps=400):
    """Random add / fork / append / free; a content array stands in for the
    cache, copies are applied before the appended tokens are written, and
    every live sequence must read back its own history."""
    rng = np.random.default_rng(seed)
    bm = bm_factory()
    content = np.full(bm.num_blocks * bm.block_size, -1, dtype=np.int64)
    history = {}
    next_id, next_tok = 0, 0
    for _ in range(steps):
        op = rng.choice(["add", "fork", "append", "append", "append", "free"])
        live = list(history)
        if op == "add" or not live:
            assert bm.add(next_id) == OK
            history[next_id] = []
            next_id += 1
        elif op == "fork":
            parent = live[rng.integers(len(live))]
            assert bm.fork(parent, next_id) == OK
            history[next_id] = list(history[parent])
            next_id += 1
        elif op == "append":
            seq = live[rng.integers(len(live))]
            k = int(rng.integers(1, 3 * bm.block_size))
            status, slots = bm.append(seq, k)
            if status != OK:
                continue
            for src, dst in bm.take_copies():
                bs = bm.block_size
                content[dst * bs:(dst + 1) * bs] = content[src * bs:(src + 1) * bs]
            toks = list(range(next_tok, next_tok + k))
            next_tok += k
            content[slots] = toks
            history[seq].extend(toks)
        else:
            seq = live[rng.integers(len(live))]
            assert bm.free(seq) == OK
            del history[seq]
        for seq, hist in history.items():
            table = bm.table(seq)
            bs = bm.block_size
            got = [int(content[table[p // bs] * bs + p % bs]) for p in range(len(hist))]
            assert got == hist, f"sequence {seq} reads back the wrong tokens"
    return bm


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_keep_every_history(seed):
    bm = _simulate(lambda: BlockManagerRef(64, 4, 64), seed)
    _invariants(bm)


def test_copy_blocks_ref():
    rng = np.random.default_rng(0)
    kc = rng.integers(0, 1 << 16, size=(6, 2, 4, 8), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(6, 2, 4, 8), dtype=np.uint16)
    nk, nv = copy_blocks_ref(kc, vc, [(1, 4), (4, 5)])
    assert np.array_equal(nk[4], kc[1]) and np.array_equal(nk[5], kc[1])   # in order
    assert np.array_equal(nv[4], vc[1]) and np.array_equal(nv[5], vc[1])
    for b in (0, 1, 2, 3):
        assert np.array_equal(nk[b], kc[b]) and np.array_equal(nv[b], vc[b])


# ---- sensitivity: planted mistakes must fail a pin --------------------------------------

class _NoCow(BlockManagerRef):
    """Writes into a shared block in place (no copy-on-write)."""

    def blocks_needed(self, seq, k):
        n = self.lengths[seq]
        return sum(1 for p in range(n, n + k) if p % self.block_size == 0)

    def append(self, seq, k):
        if seq not in self.tables:
            return STATE, []
        n, bs = self.lengths[seq], self.block_size
        if self.blocks_needed(seq, k) > self.num_free():
            return OUT_OF_BLOCKS, []
        table, slots = self.tables[seq], []
        for p in range(n, n + k):
            if p % bs == 0:
                table.append(self._take())
            slots.append(table[p // bs] * bs + p % bs)
        self.lengths[seq] = n + k
        return OK, slots


class _CopyAlways(BlockManagerRef):
    def blocks_needed(self, seq, k):
        n = self.lengths[seq]
        extra = 1 if (k > 0 and n % self.block_size) else 0
        return sum(1 for p in range(n, n + k) if p % self.block_size == 0) + extra

    def append(self, seq, k):
        if seq in self.tables and k > 0 and self.lengths[seq] % self.block_size:
            t = self.tables[seq]
            self.refcount[t[-1]] += 1     # pretend shared: always copy
            status, slots = super().append(seq, k)
            if status != OK:
                self.refcount[t[-1]] -= 1
            return status, slots
        return super().append(seq, k)


class _LeakOnFree(BlockManagerRef):
    def free(self, seq):
        if seq in self.tables:
            for blk in self.tables[seq]:
                self.refcount[blk] -= 1
            del self.tables[seq]
            del self.lengths[seq]
            return OK
        return STATE


class _ForkNoRef(BlockManagerRef):
    def fork(self, parent, child):
        if parent not in self.tables or child in self.tables:
            return STATE
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        return OK


@pytest.mark.parametrize("cls", [_NoCow, _CopyAlways, _LeakOnFree, _ForkNoRef])
def test_planted_block_manager_mistake_fails_a_pin(cls):
    def fails(fn):
        try:
            fn()
        except (AssertionError, IndexError, KeyError):
            return True
        return False

    def sharing():
        bm = cls(10_000, 16, 1024)
        bm.add(0)
        bm.append(0, 4100)
        for r in range(1, 9):
            bm.fork(0, r)
        bm.free(0)
        for r in range(1, 9):
            assert bm.append(r, 20)[0] == OK
        assert len(bm.take_copies()) == 7
        # 256 full prompt blocks, the partial one, 7 copies, one new block each
        assert bm.num_blocks - bm.num_free() == 256 + 1 + 7 + 8
        _invariants(bm)

    def simulation():
        for seed in range(3):
            bm = _simulate(lambda: cls(64, 4, 64), seed)
            _invariants(bm)

    assert fails(sharing) or fails(simulation)


def test_move_blocks_ref_round_trip():
    from oracle.block_manager import move_blocks_ref
    rng = np.random.default_rng(2)
    dk = rng.integers(0, 1 << 16, size=(8, 2, 4, 8), dtype=np.uint16)
    dv = rng.integers(0, 1 << 16, size=(8, 2, 4, 8), dtype=np.uint16)
    hk = np.zeros((5, 2, 4, 8), np.uint16)
    hv = np.zeros((5, 2, 4, 8), np.uint16)
    hk2, hv2 = move_blocks_ref(dk, dv, hk, hv, [(6, 0), (1, 4)])
    assert np.array_equal(hk2[0], dk[6]) and np.array_equal(hv2[4], dv[1])
    assert not hk2[1:4].any() and not hv2[1:4].any()
    back_k, back_v = move_blocks_ref(hk2, hv2, np.zeros_like(dk), np.zeros_like(dv), [(0, 2), (4, 7)])
    assert np.array_equal(back_k[2], dk[6]) and np.array_equal(back_v[7], dv[1])

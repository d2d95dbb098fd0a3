"""Pins of the continuous-batching scheduler oracle: the pages' straggler
example (static batching's idle slots, the closed-form admission and finish
iterations of iteration-level batching), a content simulation through
preemption (swap out, swap in) in which every sequence must read back its own
history, and liveness / batch-size invariants."""

import numpy as np
import pytest

from oracle.scheduler import (FINISHED, PREFILLING, RUNNING, SchedulerRef,
                              static_batching_idle_slots)

STRAGGLERS = [50, 120, 240, 1024]   # the pages' four requests' output lengths


def _run(sched, limit=100_000):
    plans = []
    while not sched.done():
        plans.append(sched.step())
        assert len(plans) < limit, "scheduler made no progress"
    return plans


def test_static_batching_bubble():
    # one static batch of the four requests: three slots idle while the 1024-token one runs
    assert static_batching_idle_slots(STRAGGLERS) == 974 + 904 + 784


def test_iteration_level_admission_closed_form():
    # 4 slots, 16 requests (the four output lengths cycling), prompts of 16
    # tokens prefilled in one iteration: a request admitted at iteration a
    # prefills at a, decodes at a+1 .. a+o and leaves at a+o+1, where the next
    # waiting request is admitted in the same iteration
    outs = STRAGGLERS * 4
    sched = SchedulerRef([(16, o) for o in outs], num_blocks=10_000, num_host_blocks=16,
                         block_size=16, max_blocks_per_seq=128, max_batch=4, chunk_tokens=64)
    plans = _run(sched)
    admitted = {s: p["iteration"] for p in plans for s in p["admitted"]}
    finished = {s: p["iteration"] for p in plans for s in p["finished"]}
    for s, o in enumerate(outs):
        assert finished[s] == admitted[s] + o + 1
    # the slot a request frees is refilled in the same iteration (FCFS order)
    slot_free_at = sorted(finished.values())
    later = [admitted[s] for s in range(4, len(outs))]
    assert later == slot_free_at[: len(later)]
    # no slot ever idles while requests wait: every iteration before the
    # queue drains decodes max_batch - (prefilling this iteration) sequences
    last_admit = max(admitted.values())
    for p in plans[1:last_admit + 1]:
        assert len(p["decode"]) + sum(1 for _ in p["admitted"]) == 4
    # fewer iterations than static batches of 4 would take
    static = sum(max(outs[i:i + 4]) + 2 for i in range(0, len(outs), 4))
    assert len(plans) < static


def _simulate(seed, num_blocks, max_batch, chunk, host_blocks=512, bs=4):
    """Content simulation: device and host pools hold token ids; each plan is
    applied (swap in, swap out, then the iteration's writes) and every live
    sequence must read back its prompt and generated tokens."""
    rng = np.random.default_rng(seed)
    reqs = [(int(rng.integers(1, 40)), int(rng.integers(1, 60))) for _ in range(30)]
    sched = SchedulerRef(reqs, num_blocks=num_blocks, num_host_blocks=host_blocks, block_size=bs,
                         max_blocks_per_seq=64, max_batch=max_batch, chunk_tokens=chunk)
    dev = np.full(num_blocks * bs, -1, dtype=np.int64)
    host = np.full(host_blocks * bs, -1, dtype=np.int64)

    def tok(seq, pos):
        return seq * 100_000 + pos

    plans = []
    preemptions = 0
    while not sched.done():
        plan = sched.step()
        plans.append(plan)
        assert len(plans) < 20_000
        for hb, db in plan["swap_in"]:
            dev[db * bs:(db + 1) * bs] = host[hb * bs:(hb + 1) * bs]
        for db, hb in plan["swap_out"]:
            host[hb * bs:(hb + 1) * bs] = dev[db * bs:(db + 1) * bs]
        preemptions += len(plan["preempted"])
        for ch in plan["prefill"]:
            for i, slot in enumerate(ch["slots"]):
                dev[slot] = tok(ch["seq"], ch["start"] + i)
        for d in plan["decode"]:
            dev[d["slot"]] = tok(d["seq"], d["context"] - 1)
        live = [s for s in sched.admit_order]
        assert len(live) <= max_batch
        for s in live:
            table = sched.bm.table(s)
            n = sched.prefilled[s] + sched.generated[s] if sched.state[s] == RUNNING \
                else sched.prefilled[s]
            got = [int(dev[table[p // bs] * bs + p % bs]) for p in range(n)]
            assert got == [tok(s, p) for p in range(n)], f"seq {s} lost its cache"
    for s, (p, o) in enumerate(reqs):
        assert sched.state[s] == FINISHED and sched.generated[s] == o
    return plans, preemptions


@pytest.mark.parametrize("seed", range(5))
def test_preemption_keeps_every_cache(seed):
    plans, preemptions = _simulate(seed, num_blocks=40, max_batch=8, chunk=24)
    assert preemptions > 0            # the small pool forces swapping


@pytest.mark.parametrize("seed", range(3))
def test_ample_pool_never_preempts(seed):
    plans, preemptions = _simulate(seed, num_blocks=2000, max_batch=6, chunk=17)
    assert preemptions == 0


def test_chunk_budget_and_order():
    reqs = [(100, 3), (10, 3), (37, 2)]
    sched = SchedulerRef(reqs, num_blocks=1000, num_host_blocks=4, block_size=16,
                         max_blocks_per_seq=64, max_batch=4, chunk_tokens=32)
    p0 = sched.step()
    assert [(c["seq"], c["start"], c["rows"]) for c in p0["prefill"]] == [(0, 0, 32)]
    p1 = sched.step()
    assert [(c["seq"], c["start"], c["rows"]) for c in p1["prefill"]] == [(0, 32, 32)]
    sched.step()
    p3 = sched.step()   # seq 0's last 4 rows, then seq 1's 10, then 18 of seq 2
    assert [(c["seq"], c["start"], c["rows"]) for c in p3["prefill"]] == \
        [(0, 96, 4), (1, 0, 10), (2, 0, 18)]
    assert p3["decode"] == []             # nobody has finished prefilling before this one
    p4 = sched.step()
    assert [d["seq"] for d in p4["decode"]] == [0, 1]
    assert sched.state[2] == RUNNING and sched.prefilled[2] == 37
    assert all(sched.state[s] != PREFILLING for s in range(3))


# ---- sensitivity: planted mistakes must fail a pin ---------------------------------------

class _NoSwapCopy(SchedulerRef):
    def step(self):
        plan = super().step()
        plan["swap_out"] = []           # frees blocks without saving them
        return plan


class _LateAdmit(SchedulerRef):
    """Admits only on even iterations (a freed slot can stay empty)."""

    def step(self):
        if self.iteration % 2 == 0:
            return super().step()
        saved = self.next_waiting
        self.next_waiting = len(self.requests)
        try:
            return super().step()
        finally:
            self.next_waiting = saved


@pytest.mark.parametrize("cls", [_NoSwapCopy, _LateAdmit])
def test_planted_scheduler_mistake_fails_a_pin(cls, monkeypatch):
    import oracle.scheduler as m
    monkeypatch.setattr(m, "SchedulerRef", cls)
    monkeypatch.setitem(globals(), "SchedulerRef", cls)
    failed = False
    for fn in (test_iteration_level_admission_closed_form,
               lambda: test_preemption_keeps_every_cache(0)):
        try:
            fn()
        except AssertionError:
            failed = True
    assert failed

"""Iteration-level (continuous) batching scheduler over a paged KV cache, and
the host swap space it preempts into.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

What the pages fix:

* The scheduler decides at the boundary of every forward pass (one token per
  running sequence), not at request boundaries. A sequence that emits its
  end-of-sequence token gives its blocks back to the pool at once and a
  waiting request takes the freed slot on the next iteration (How vLLM gets
  real throughput on H100s, "Continuous batching removes straggler bubbles";
  vLLM architecture, memory and benchmarks deep dive, "Continuous batching and
  the straggler problem").
* After each iteration it can eject finished sequences, admit waiting
  requests and preempt running sequences when memory runs short; a preempted
  sequence's blocks are swapped to host memory, its GPU blocks freed, and it
  resumes later without losing its context (Dissecting vLLM, "Continuous
  Batching: Breaking the Sequence Barrier").
* Long prompts are cut into chunks interleaved with decode tokens (vLLM
  architecture... deep dive, "Hardware-level optimizations").

Readings where the pages are silent:

* Requests are served first come, first served; every request is present from
  iteration 0 (an offline batch); a request is (prompt_len, output_len) and
  is finished once it has generated output_len tokens (its "end of sequence").
* The batch holds at most max_batch sequences (prefilling or running).
* Iteration t, in order:
  1. eject: running sequences with generated == output_len are freed;
  2. resume: while swapped sequences wait (oldest preemption first), the batch
     has room and the pool has length + 1 blocks' worth (blocks for its
     length plus one), the sequence gets fresh blocks for its whole length
     and its host blocks are copied back and released;
  3. admit: only when no sequence is swapped out; while requests wait and the
     batch has room and the pool has the blocks of prompt_len + 1 tokens, the
     next request is admitted and its whole prompt's blocks reserved;
  4. prefill: up to chunk_tokens prompt rows in total, taken from the
     prefilling sequences in admission order, each a chunk of consecutive
     rows; a sequence whose prompt is complete starts decoding on the next
     iteration;
  5. decode: every running sequence appends one token; while the pool cannot
     hold them all, the running sequence admitted last is preempted (its
     blocks swapped to host blocks, then freed). The appended tokens are the
     iteration's decode batch, in admission order.
* Host swap space is a pool of host blocks of the same size with the same
  stack policy as the device pool; a preemption takes one host block per
  device block, in the order of the sequence's table.
"""

from .block_manager import BlockManagerRef

WAITING, PREFILLING, RUNNING, SWAPPED, FINISHED = "waiting", "prefilling", "running", "swapped", \
    "finished"


class SchedulerRef:
    def __init__(self, requests, *, num_blocks, num_host_blocks, block_size, max_blocks_per_seq,
                 max_batch, chunk_tokens):
        self.requests = [(int(p), int(o)) for p, o in requests]
        self.bm = BlockManagerRef(num_blocks, block_size, max_blocks_per_seq)
        self.host_free = list(range(num_host_blocks - 1, -1, -1))
        self.block_size = block_size
        self.max_batch = max_batch
        self.chunk_tokens = chunk_tokens
        self.state = [WAITING] * len(self.requests)
        self.prefilled = [0] * len(self.requests)
        self.generated = [0] * len(self.requests)
        self.admit_order = []          # batch members, admission order
        self.swapped = []              # preempted, oldest first
        self.host_blocks = {}          # seq -> host blocks holding its cache
        self.next_waiting = 0
        self.iteration = 0

    def _need(self, tokens):
        return -(-tokens // self.block_size)

    def done(self):
        return all(s == FINISHED for s in self.state)

    def step(self):
        """One iteration's plan (a dict of host lists)."""
        bm = self.bm
        plan = {"iteration": self.iteration, "finished": [], "swap_out": [], "swap_in": [],
                "admitted": [], "prefill": [], "decode": [], "preempted": [], "resumed": []}
        # 1. eject
        for seq in list(self.admit_order):
            p, o = self.requests[seq]
            if self.state[seq] == RUNNING and self.generated[seq] == o:
                bm.free(seq)
                self.state[seq] = FINISHED
                self.admit_order.remove(seq)
                plan["finished"].append(seq)
        # 2. resume swapped sequences
        while self.swapped and len(self.admit_order) < self.max_batch:
            seq = self.swapped[0]
            length = self.requests[seq][0] + self.generated[seq]
            if bm.num_free() < self._need(length) + 1:
                break
            self.swapped.pop(0)
            bm.add(seq)
            status, _ = bm.append(seq, length)
            assert status == "ok"
            table = bm.table(seq)
            hosts = self.host_blocks.pop(seq)
            plan["swap_in"].extend(zip(hosts, table))
            for hb in reversed(hosts):
                self.host_free.append(hb)
            self.state[seq] = RUNNING
            self.admit_order.append(seq)
            plan["resumed"].append(seq)
        # 3. admit
        while (not self.swapped and self.next_waiting < len(self.requests)
               and len(self.admit_order) < self.max_batch):
            seq = self.next_waiting
            prompt = self.requests[seq][0]
            if bm.num_free() < self._need(prompt + 1):
                break
            bm.add(seq)
            status, slots = bm.append(seq, prompt)
            assert status == "ok"
            self.state[seq] = PREFILLING
            self.admit_order.append(seq)
            self.next_waiting += 1
            plan["admitted"].append(seq)
        # 4. prefill chunks
        budget = self.chunk_tokens
        became_running = []
        for seq in self.admit_order:
            if budget == 0:
                break
            if self.state[seq] != PREFILLING:
                continue
            prompt = self.requests[seq][0]
            take = min(budget, prompt - self.prefilled[seq])
            start = self.prefilled[seq]
            table = bm.table(seq)
            bs = self.block_size
            slots = [table[p // bs] * bs + p % bs for p in range(start, start + take)]
            plan["prefill"].append({"seq": seq, "start": start, "rows": take, "slots": slots})
            self.prefilled[seq] += take
            budget -= take
            if self.prefilled[seq] == prompt:
                became_running.append(seq)
        # 5. decode (sequences that finished their prompt this iteration wait)
        runners = [s for s in self.admit_order if self.state[s] == RUNNING]
        while runners and sum(bm.blocks_needed(s, 1) for s in runners) > bm.num_free():
            victim = runners.pop()      # admitted last
            table = bm.table(victim)
            if len(self.host_free) < len(table):
                raise RuntimeError("host swap space exhausted")
            hosts = [self.host_free.pop() for _ in table]
            plan["swap_out"].extend(zip(table, hosts))
            self.host_blocks[victim] = hosts
            bm.free(victim)
            self.state[victim] = SWAPPED
            self.admit_order.remove(victim)
            self.swapped.append(victim)
            plan["preempted"].append(victim)
        for seq in runners:
            status, slots = bm.append(seq, 1)
            assert status == "ok"
            self.generated[seq] += 1
            plan["decode"].append({"seq": seq, "slot": int(slots[0]),
                                   "context": self.requests[seq][0] + self.generated[seq]})
        for seq in became_running:
            self.state[seq] = RUNNING
        self.iteration += 1
        return plan


def static_batching_idle_slots(output_lens):
    """Idle slot-iterations of one static batch: every slot waits for the
    longest request (the pages' bubble)."""
    longest = max(output_lens)
    return sum(longest - n for n in output_lens)

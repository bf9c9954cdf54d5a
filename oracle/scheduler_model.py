"""Oracle model of the continuous-batching loop over a serving trace (test
infrastructure).

What the pages fix:

* Iteration-level scheduling: every step first removes the requests that have
  finished and gives their pages back, then admits waiting requests while free
  pages remain, then runs one forward step for every running request and
  appends each one's new token (hihuo.com "vLLM 原理：PagedAttention 和
  Continuous Batching", vLLM 的调度 > 调度流程; ksqn.cn "大模型推理性能优化：
  PagedAttention与Continuous Batching原理与实践", section 2.3).
* When memory runs short a low-priority request is suspended, its pages are
  released for the others, and it resumes later by recomputing its cache
  (hihuo.com page, Preemption（抢占）, recompute mode).

Readings where the pages are silent (the library's scheduler takes the same):

* Arrivals join the tail of the waiting queue; admission is first come, first
  served, and stops at the first request whose prompt does not fit in the free
  blocks (head-of-line blocking).  The pseudo-code pops from a Python list; it
  is read as FCFS because the allocation sample on the same pages is FIFO.
* Admission allocates blocks for the whole prompt at once; the prompt is then
  written in chunks of at most `chunk` tokens, one chunk per request per step,
  in admission order.  Chunks are planned after the step's decode appends, so a
  request preempted by an append has no chunk in that step (its blocks may
  already hold another request's token).  Prefill attention itself is not
  modelled.
* A request decodes from the step after its prompt is fully written; each
  decode step appends one token (its slot reserved by the allocator, with a
  new block when the token crosses a block boundary) and attends over every
  cached token, the new one included.  It finishes when it has produced its
  output length, and is released at the start of the next step.
* Decode appends run in admission order.  When an append finds no free block,
  the running request admitted last (the lowest first-come priority, possibly
  the requester itself) is preempted: its blocks are released, and it goes back
  to the head of the waiting queue with its prompt extended by the tokens it
  has generated so far (recompute).  The append is then retried.

* With prefix caching on, an arrival carries its prompt's token IDs and
  admission goes through ``add_prefix``: the cached opening is not prefilled
  (prefill starts after it), and the first request that does not fit blocks the
  queue as before.  Each prompt chunk's full blocks are registered when the
  chunk is planned (its K/V are written in that step, before any later step can
  reuse them); after that, every decoding request's newly full blocks are
  registered, in admission order.  Generated tokens have IDs
  given by the workload; a preempted request is admitted again with its prompt
  plus the tokens it generated, so its own cached blocks can serve the
  recompute.

* With a host pool (swap preemption, hihuo.com page, Preemption（抢占）: Swap),
  the preempted request is swapped out instead of released when the host pool
  can hold it (else it is recomputed as above); it keeps its progress.  Swapped
  requests come back first, in swap-out order, each step before any admission;
  while one of them does not fit, no new request is admitted.  A request swapped
  back in rejoins the running list at its end.  The step's device work runs in
  the order: swap-in copies, prompt writes and prefill, swap-out copies, decode
  writes and decode; a request swapped out in a step has no chunk in it.

Pins: a hand-worked trace on a four-block pool (tests/test_scheduler.py) that
exercises admission, chunking, release, head-of-line blocking, and preemption
of another request and of the requester itself; conservation of blocks after
every step; the library scheduler equals this model step by step.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

from .allocator_model import AllocatorModel, OutOfBlocks


@dataclass
class Request:
    rid: int
    prompt: int
    out_len: int
    generated: int = 0
    prompt_eff: int = 0      # tokens to prefill at the latest admission
    prefilled: int = 0       # of prompt_eff written so far
    ready: bool = False      # prompt fully written in an earlier step
    tokens: list = field(default_factory=list)  # prompt + generated token IDs (prefix caching)

    def finished(self) -> bool:
        return self.generated >= self.out_len


@dataclass
class StepRecord:
    step: int
    finished: list = field(default_factory=list)
    arrived: list = field(default_factory=list)
    admitted: list = field(default_factory=list)
    prefill: list = field(default_factory=list)      # (rid, start, count, slots)
    preempted: list = field(default_factory=list)
    decode: list = field(default_factory=list)       # (rid, position, slot, cow)
    cached: list = field(default_factory=list)       # (rid, cached prompt tokens) per admission
    swapped_in: list = field(default_factory=list)   # (rid, [(host, device) block pairs])
    swapped_out: list = field(default_factory=list)  # (rid, [(device, host) block pairs])


class SchedulerModel:
    def __init__(self, num_blocks: int, block_size: int, chunk: int, initial_free_order=None,
                 gen_token=None, num_host_blocks: int = 0):
        """gen_token(rid, position) -> token ID turns prefix caching on; arrivals
        then carry (prompt token IDs, out_len).  num_host_blocks > 0 turns swap
        preemption on."""
        self.alloc = AllocatorModel(num_blocks, block_size, initial_free_order,
                                    num_host_blocks=num_host_blocks)
        self.swap = num_host_blocks > 0
        self.swapped_q: deque[Request] = deque()
        self.gen_token = gen_token
        self.B = block_size
        self.chunk = chunk
        self.waiting: deque[Request] = deque()
        self.running: list[Request] = []
        self.next_rid = 0

    def step(self, n: int, arrivals) -> StepRecord:
        """One iteration; `arrivals` is a list of (prompt, out_len)."""
        rec = StepRecord(n)
        # 1. finished requests give their pages back
        for r in list(self.running):
            if r.finished():
                self.alloc.release(r.rid)
                self.running.remove(r)
                rec.finished.append(r.rid)
        # 2a. new requests queue up behind the waiting ones
        prefix = self.gen_token is not None
        for prompt, out_len in arrivals:
            if prefix:
                r = Request(self.next_rid, len(prompt), int(out_len), tokens=[int(t) for t in prompt])
            else:
                r = Request(self.next_rid, int(prompt), int(out_len))
            r.prompt_eff = r.prompt
            self.next_rid += 1
            self.waiting.append(r)
            rec.arrived.append(r.rid)
        # 2b. swapped requests come back first, in swap-out order
        while self.swapped_q:
            r = self.swapped_q[0]
            try:
                pairs = self.alloc.swap_in(r.rid)
            except OutOfBlocks:
                break
            self.swapped_q.popleft()
            self.running.append(r)
            rec.swapped_in.append((r.rid, pairs))
        # 2c. admit first come, first served while the whole prompt fits
        while self.waiting and not self.swapped_q:
            r = self.waiting[0]
            if prefix:
                try:
                    cached = self.alloc.add_prefix(r.rid, r.tokens[:r.prompt_eff])
                except OutOfBlocks:
                    break
                rec.cached.append((r.rid, cached))
            else:
                if -(-r.prompt_eff // self.B) > self.alloc.num_free():
                    break
                self.alloc.add(r.rid, r.prompt_eff)
                cached = 0
            r.prefilled = cached
            r.ready = False
            self.running.append(r)
            self.waiting.popleft()
            rec.admitted.append(r.rid)
        # 3a. every decoding request appends one token (preempting when out of blocks)
        decoders = [r for r in self.running if r.ready]
        for r in decoders:
            while r in self.running:
                try:
                    slot, cow = self.alloc.append(r.rid)
                except OutOfBlocks:
                    victim = self.running[-1]
                    if self.swap and len(self.alloc.block_table(victim.rid)) <= len(self.alloc.host_free):
                        rec.swapped_out.append((victim.rid, self.alloc.swap_out(victim.rid)))
                        self.running.remove(victim)
                        self.swapped_q.append(victim)
                        continue
                    self.alloc.release(victim.rid)
                    self.running.remove(victim)
                    victim.prompt_eff = victim.prompt + victim.generated
                    victim.prefilled = 0
                    victim.ready = False
                    self.waiting.appendleft(victim)
                    rec.preempted.append(victim.rid)
                    continue
                pos = self.alloc.length(r.rid) - 1
                rec.decode.append((r.rid, pos, slot, cow))
                r.generated += 1
                if prefix:
                    r.tokens.append(self.gen_token(r.rid, pos))
                break
        # 3b. prompts still running are written one chunk per request per step; a
        # request preempted by an append above has no chunk here
        for r in self.running:
            if r.prefilled < r.prompt_eff:
                c = min(self.chunk, r.prompt_eff - r.prefilled)
                rec.prefill.append((r.rid, r.prefilled, c,
                                    self.alloc.slots(r.rid, r.prefilled, c)))
                r.prefilled += c
                if prefix:
                    self.alloc.register(r.rid, r.tokens[:r.prefilled])
        if prefix:
            running = {r.rid: r for r in self.running}
            for rid, *_ in rec.decode:
                if rid in running:
                    self.alloc.register(rid, running[rid].tokens)
        # a prompt written this step decodes from the next one
        for r in self.running:
            if not r.ready and r.prefilled == r.prompt_eff:
                r.ready = True
        return rec

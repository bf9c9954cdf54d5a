"""Continuous batching over the library's block allocator: the host side of a
serving loop that feeds the paged cache.

Each step (hihuo.com "vLLM 原理：PagedAttention 和 Continuous Batching",
vLLM 的调度 > 调度流程; ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
Batching原理与实践", section 2.3):

1. requests that have produced their whole output release their blocks;
2. arrivals queue up behind the waiting requests, which are admitted first come,
   first served while the whole prompt fits in the free blocks (the first one
   that does not fit blocks the queue);
3. a request whose prompt was complete before this step appends one decode
   token, in admission order; when no block is free for an append, the running
   request admitted last is preempted: its blocks are released and it rejoins
   the head of the queue to recompute its prompt plus the tokens it has
   generated (hihuo.com page, Preemption（抢占）);
4. every request still running whose prompt is not yet written gets its next
   chunk of at most `chunk` prompt tokens, in admission order (after the
   appends, so that no preempted request keeps a chunk of this step).

With prefix caching (``gen_token`` given), arrivals carry their prompts' token
IDs; admission reuses the cached opening of each prompt through the allocator's
``add_prefix`` (hihuo.com page, 优势 > 3. 支持共享), prefill starts after it, each
planned chunk's full blocks are registered, and then every decoding request's
newly full blocks are registered, in admission order.

With a host pool (``num_host_blocks`` > 0) a preempted request is swapped out
when the pool can hold it (hihuo.com page, Preemption（抢占）: Swap), else
recomputed; swapped requests come back first, in swap-out order, before any new
admission.  A request swapped out in a step has no chunk planned in it.  The
caller runs a step's device work in the order: swap-in copies, prompt writes
and prefill, swap-out copies, decode writes and decode.

The plan a step returns says which slots to write and which sequences to decode;
the caller performs the device work (cache writes, then attention).
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

from . import _native as N
from .allocator import BlockAllocator


@dataclass
class _Req:
    rid: int
    prompt: int
    out_len: int
    generated: int = 0
    prompt_eff: int = 0
    prefilled: int = 0
    ready: bool = False
    length: int = 0   # tokens held in the cache
    tokens: np.ndarray = None  # prompt + generated token IDs (prefix caching), int32, with room
    ntok: int = 0

    def push(self, t: int):
        if self.ntok == len(self.tokens):
            self.tokens = np.concatenate([self.tokens, np.empty_like(self.tokens)])
        self.tokens[self.ntok] = t
        self.ntok += 1


@dataclass
class StepPlan:
    step: int
    finished: list = field(default_factory=list)
    arrived: list = field(default_factory=list)
    admitted: list = field(default_factory=list)
    preempted: list = field(default_factory=list)
    prefill: list = field(default_factory=list)   # (rid, start, count, slots int64[count])
    decode_rids: np.ndarray = None                # int64[n], admission order
    decode_pos: np.ndarray = None                 # int64[n]: position of the new token
    decode_slots: np.ndarray = None               # int64[n]
    decode_cows: np.ndarray = None                # int32[n, 2], -1 = no copy
    cached: list = field(default_factory=list)    # (rid, cached prompt tokens) per admission
    swapped_in: list = field(default_factory=list)   # (rid, int32[n, 2] (host, device) pairs)
    swapped_out: list = field(default_factory=list)  # (rid, int32[n, 2] (device, host) pairs)

    def prefill_tokens(self) -> int:
        return sum(c for _, _, c, _ in self.prefill)


class TraceScheduler:
    def __init__(self, num_blocks: int, block_size: int, chunk: int, initial_free_order=None,
                 gen_token=None, num_host_blocks: int = 0):
        """gen_token(rid, position) -> token ID turns prefix caching on; arrivals
        then carry (prompt token IDs, out_len).  num_host_blocks > 0 turns swap
        preemption on."""
        self.alloc = BlockAllocator(num_blocks, block_size, initial_free_order)
        self.swap = num_host_blocks > 0
        if self.swap:
            self.alloc.set_host_pool(num_host_blocks)
        self.swapped_q: deque[_Req] = deque()
        self.gen_token = gen_token
        self.B = block_size
        self.chunk = chunk
        self.waiting: deque[_Req] = deque()
        self.running: list[_Req] = []
        self.next_rid = 0

    def step(self, n: int, arrivals) -> StepPlan:
        """One iteration; `arrivals` is an iterable of (prompt, out_len)."""
        plan = StepPlan(n)
        alloc = self.alloc
        keep = []
        for r in self.running:
            if r.generated >= r.out_len:
                alloc.free(r.rid)
                plan.finished.append(r.rid)
            else:
                keep.append(r)
        self.running = keep
        prefix = self.gen_token is not None
        for prompt, out_len in arrivals:
            if prefix:
                p = np.asarray(prompt, dtype=np.int32)
                r = _Req(self.next_rid, len(p), int(out_len))
                r.tokens = np.empty(len(p) + int(out_len) + 1, dtype=np.int32)
                r.tokens[:len(p)] = p
                r.ntok = len(p)
            else:
                r = _Req(self.next_rid, int(prompt), int(out_len))
            r.prompt_eff = r.prompt
            self.next_rid += 1
            self.waiting.append(r)
            plan.arrived.append(r.rid)
        while self.swapped_q:
            r = self.swapped_q[0]
            try:
                pairs = alloc.swap_in(r.rid)
            except N.PagedKVError as e:
                if e.status != N.PA_ERR_OOM:
                    raise
                break
            self.swapped_q.popleft()
            self.running.append(r)
            plan.swapped_in.append((r.rid, pairs))
        while self.waiting and not self.swapped_q:
            r = self.waiting[0]
            if prefix:
                try:
                    cached = alloc.add_prefix(r.rid, r.tokens[:r.prompt_eff])
                except N.PagedKVError as e:
                    if e.status != N.PA_ERR_OOM:
                        raise
                    break
                plan.cached.append((r.rid, cached))
            else:
                if -(-r.prompt_eff // self.B) > alloc.num_free():
                    break
                alloc.add(r.rid, r.prompt_eff)
                cached = 0
            r.length = r.prompt_eff
            r.prefilled = cached
            r.ready = False
            self.running.append(r)
            self.waiting.popleft()
            plan.admitted.append(r.rid)
        decoders = [r for r in self.running if r.ready]
        rids, slots, cows, pos = [], [], [], []
        pending = decoders
        while pending:
            ids = np.fromiter((r.rid for r in pending), dtype=np.int64, count=len(pending))
            st, done, sl, cw, _, _ = alloc.append_batch(ids)
            for k in range(done):
                rids.append(pending[k].rid)
                slots.append(sl[k])
                cows.append(cw[k])
                pos.append(pending[k].length)
                if prefix:
                    pending[k].push(self.gen_token(pending[k].rid, pending[k].length))
                pending[k].length += 1
                pending[k].generated += 1
            if st == N.PA_OK:
                break
            if st != N.PA_ERR_OOM:
                N.check(st, "seq_append_batch")
            # out of blocks at pending[done]: preempt the youngest running request
            victim = self.running.pop()
            if self.swap and alloc.info(victim.rid)[1] <= alloc.num_free_host():
                plan.swapped_out.append((victim.rid, alloc.swap_out(victim.rid)))
                self.swapped_q.append(victim)
                pending = [r for r in pending[done:] if r is not victim]
                continue
            alloc.free(victim.rid)
            victim.prompt_eff = victim.prompt + victim.generated
            victim.prefilled = 0
            victim.ready = False
            self.waiting.appendleft(victim)
            plan.preempted.append(victim.rid)
            pending = [r for r in pending[done:] if r is not victim]
        # Prompt chunks are planned after the decode appends, so that a request
        # preempted by an append never holds a planned chunk: its blocks may
        # already serve the request that needed one.
        for r in self.running:
            if r.prefilled < r.prompt_eff:
                c = min(self.chunk, r.prompt_eff - r.prefilled)
                plan.prefill.append((r.rid, r.prefilled, c, alloc.slots(r.rid, r.prefilled, c)))
                r.prefilled += c
                if prefix:
                    alloc.register(r.rid, r.tokens[:r.prefilled])
        if prefix:
            # only a token that completes a block can add one to the cache; the
            # other calls would change nothing
            running = {r.rid: r for r in self.running}
            for rid, p in zip(rids, pos):
                if (p + 1) % self.B == 0 and rid in running:
                    rr = running[rid]
                    alloc.register(rid, rr.tokens[:rr.ntok])
        for r in self.running:
            if not r.ready and r.prefilled == r.prompt_eff:
                r.ready = True
        plan.decode_rids = np.asarray(rids, dtype=np.int64)
        plan.decode_slots = np.asarray(slots, dtype=np.int64)
        plan.decode_cows = (np.asarray(cows, dtype=np.int32).reshape(-1, 2) if cows
                            else np.zeros((0, 2), dtype=np.int32))
        plan.decode_pos = np.asarray(pos, dtype=np.int64)
        return plan

    def running_ids(self) -> list[int]:
        return [r.rid for r in self.running]

    def waiting_ids(self) -> list[int]:
        return [r.rid for r in self.waiting]

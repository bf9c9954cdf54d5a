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

Every step runs in the library's C++ scheduler (pa_sched_*); this module only
marshals arrivals in and the plan out.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass, field

import numpy as np

from . import _native as N
from .allocator import BlockAllocator


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _arr(p, n: int, dtype) -> np.ndarray:
    """A copy of n elements at a plan pointer."""
    out = np.empty(max(int(n), 0), dtype=dtype)
    if n > 0:
        ctypes.memmove(out.ctypes.data, ctypes.cast(p, ctypes.c_void_p).value, out.nbytes)
    return out


@dataclass
class Arrivals:
    """A step's arrivals packed for pa_sched_add_requests: prompt lengths, output
    lengths, and with prefix caching the prompts' token IDs and the tokens each
    request generates, concatenated."""
    prompt_lens: np.ndarray
    out_lens: np.ndarray
    prompt_tokens: np.ndarray = None
    out_tokens: np.ndarray = None

    def __len__(self):
        return int(self.prompt_lens.shape[0])


@dataclass
class StepPlan:
    step: int
    finished: list = field(default_factory=list)
    arrived: list = field(default_factory=list)
    admitted: list = field(default_factory=list)
    preempted: list = field(default_factory=list)
    prefill: list = field(default_factory=list)   # (rid, start, count, slots int64[count])
    decode_rids: np.ndarray = None                # int64[n], running order
    decode_pos: np.ndarray = None                 # int64[n]: position of the new token
    decode_slots: np.ndarray = None               # int64[n]
    decode_cows: np.ndarray = None                # int32[n, 2], -1 = no copy
    num_decode_cows: int = 0                      # rows of decode_cows with a copy
    cached: list = field(default_factory=list)    # (rid, cached prompt tokens) per admission
    swapped_in: list = field(default_factory=list)   # (rid, int32[n, 2] (host, device) pairs)
    swapped_out: list = field(default_factory=list)  # (rid, int32[n, 2] (device, host) pairs)
    prefill_rids: np.ndarray = None               # int64[chunks]
    prefill_start: np.ndarray = None              # int32[chunks]
    prefill_count: np.ndarray = None              # int32[chunks]
    prefill_slots: np.ndarray = None              # int64[tokens], chunk after chunk

    def prefill_tokens(self) -> int:
        return int(self.prefill_slots.shape[0]) if self.prefill_slots is not None else 0


class _Handle:
    """Owns one pa_scheduler."""

    def __init__(self, lib, h):
        self._lib, self.h = lib, h

    def __del__(self):
        try:
            if self.h:
                self._lib.pa_sched_destroy(self.h)
                self.h = None
        except Exception:
            pass


class TraceScheduler:
    def __init__(self, num_blocks: int, block_size: int, chunk: int, initial_free_order=None,
                 gen_token=None, num_host_blocks: int = 0, gen_tokens=None):
        """Prefix caching is on when gen_token(rid, position) -> token ID or
        gen_tokens(rid, first_position, count) -> int32 token IDs is given; arrivals
        then carry (prompt token IDs, out_len) and the tokens each request will
        generate are taken from it at arrival (a replayed trace knows them).
        num_host_blocks > 0 turns swap preemption on."""
        self._lib = N.lib()
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("initial_free_order must have num_blocks entries")
        h = ctypes.c_void_p()
        self.gen_token = gen_token
        self.gen_tokens = gen_tokens
        self.prefix = gen_token is not None or gen_tokens is not None
        N.check(self._lib.pa_sched_create(num_blocks, block_size,
                                          None if order is None else _ptr(order), chunk,
                                          int(self.prefix), num_host_blocks, ctypes.byref(h)),
                "pa_sched_create")
        self._handle = _Handle(self._lib, h)
        self._h = h
        self.alloc = BlockAllocator.borrowed(self._lib.pa_sched_allocator(h), num_blocks,
                                             block_size, self._handle)
        self.B = block_size
        self.chunk = chunk
        self.swap = num_host_blocks > 0
        self.next_rid = 0
        self._plan = N.SchedPlan()

    def _outputs(self, rid: int, start: int, count: int) -> np.ndarray:
        if self.gen_tokens is not None:
            return np.asarray(self.gen_tokens(rid, start, count), dtype=np.int32)
        return np.fromiter((self.gen_token(rid, start + g) for g in range(count)), dtype=np.int32,
                           count=count)

    def pack(self, arrivals, first_rid: int | None = None) -> Arrivals:
        """Pack (prompt, out_len) pairs (prefix caching: (prompt token IDs, out_len))
        whose requests will get IDs first_rid, first_rid + 1, ... (default: the next
        IDs this scheduler hands out)."""
        if isinstance(arrivals, Arrivals):
            return arrivals
        arrivals = list(arrivals)
        n = len(arrivals)
        rid0 = self.next_rid if first_rid is None else first_rid
        outs = np.fromiter((int(o) for _, o in arrivals), dtype=np.int32, count=n)
        if not self.prefix:
            plens = np.fromiter((int(p) for p, _ in arrivals), dtype=np.int32, count=n)
            return Arrivals(plens, outs)
        prompts = [np.asarray(p, dtype=np.int32) for p, _ in arrivals]
        plens = np.fromiter((len(p) for p in prompts), dtype=np.int32, count=n)
        ptoks = np.concatenate(prompts) if n else np.zeros(0, dtype=np.int32)
        outs_tok = [self._outputs(rid0 + k, int(plens[k]), int(outs[k])) for k in range(n)]
        if all(o.size == 0 for o in outs_tok):
            otoks = None  # a live loop: token IDs come later, through push_tokens
        elif all(o.size == int(outs[k]) for k, o in enumerate(outs_tok)):
            otoks = np.concatenate(outs_tok)
        else:
            raise ValueError("the token source must give each request all of its outputs, or none")
        return Arrivals(plens, outs, ptoks, otoks)

    def push_tokens(self, rids, tokens) -> None:
        """Pass sampled token IDs (one per named request, in order) to the scheduler."""
        r = np.ascontiguousarray(rids, dtype=np.int64)
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if r.shape != t.shape:
            raise ValueError("one token per request")
        N.check(self._lib.pa_sched_push_tokens(self._h, _ptr(r), _ptr(t), int(r.shape[0])),
                "pa_sched_push_tokens")

    def add_requests(self, arrivals) -> list[int]:
        """Queue arrivals (pairs or packed) for the next step; returns their IDs."""
        a = self.pack(arrivals)
        n = len(a)
        if n == 0:
            return []
        rids = np.empty(n, dtype=np.int64)
        ot = a.out_tokens
        N.check(self._lib.pa_sched_add_requests(
            self._h, n, _ptr(a.prompt_lens), _ptr(a.out_lens),
            None if a.prompt_tokens is None or a.prompt_tokens.size == 0 else _ptr(a.prompt_tokens),
            None if ot is None or ot.size == 0 else _ptr(ot), _ptr(rids)), "pa_sched_add_requests")
        self.next_rid += n
        return rids.tolist()

    def step(self, n: int, arrivals) -> StepPlan:
        """One iteration; `arrivals` is an iterable of (prompt, out_len), or packed."""
        self.add_requests(arrivals)
        p = self._plan
        N.check(self._lib.pa_sched_step(self._h, ctypes.byref(p)), "pa_sched_step")
        plan = StepPlan(n)
        plan.finished = _arr(p.finished, p.num_finished, np.int64).tolist()
        plan.arrived = _arr(p.arrived, p.num_arrived, np.int64).tolist()
        plan.admitted = _arr(p.admitted, p.num_admitted, np.int64).tolist()
        plan.preempted = _arr(p.preempted, p.num_preempted, np.int64).tolist()
        if self.prefix:
            cached = _arr(p.admitted_cached, p.num_admitted, np.int32).tolist()
            plan.cached = list(zip(plan.admitted, cached))
        plan.prefill_rids = _arr(p.prefill_rid, p.num_prefill, np.int64)
        plan.prefill_start = _arr(p.prefill_start, p.num_prefill, np.int32)
        plan.prefill_count = _arr(p.prefill_count, p.num_prefill, np.int32)
        plan.prefill_slots = _arr(p.prefill_slots, p.num_prefill_tokens, np.int64)
        off = np.concatenate([[0], np.cumsum(plan.prefill_count, dtype=np.int64)])
        plan.prefill = [(int(plan.prefill_rids[k]), int(plan.prefill_start[k]),
                         int(plan.prefill_count[k]), plan.prefill_slots[off[k]:off[k + 1]])
                        for k in range(p.num_prefill)]
        plan.decode_rids = _arr(p.decode_rid, p.num_decode, np.int64)
        plan.decode_pos = _arr(p.decode_pos, p.num_decode, np.int64)
        plan.decode_slots = _arr(p.decode_slot, p.num_decode, np.int64)
        plan.decode_cows = _arr(p.decode_cow, 2 * p.num_decode, np.int32).reshape(-1, 2)
        plan.num_decode_cows = int(p.num_decode_cows)
        for which in ("in", "out"):
            m = getattr(p, f"num_swapped_{which}")
            if m == 0:
                continue
            rids = _arr(getattr(p, f"swapped_{which}"), m, np.int64)
            cnt = _arr(getattr(p, f"swapped_{which}_pairs"), m, np.int32)
            pairs = _arr(getattr(p, f"swap_{which}"), 2 * int(cnt.sum()), np.int32).reshape(-1, 2)
            o = np.concatenate([[0], np.cumsum(cnt, dtype=np.int64)])
            setattr(plan, f"swapped_{which}",
                    [(int(rids[k]), pairs[o[k]:o[k + 1]]) for k in range(m)])
        return plan

    def running_info(self):
        """(rids int64, prompt lengths int32, tokens held int32) of the running
        requests, in running order."""
        n = self._lib.pa_sched_running(self._h, None, None, None, 0)
        rids = np.empty(max(n, 1), dtype=np.int64)
        prompts = np.empty(max(n, 1), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        self._lib.pa_sched_running(self._h, _ptr(rids), _ptr(prompts), _ptr(lens), n)
        return rids[:n], prompts[:n], lens[:n]

    def running_ids(self) -> list[int]:
        return self.running_info()[0].tolist()

    def waiting_ids(self) -> list[int]:
        n = self._lib.pa_sched_waiting(self._h, None, 0)
        out = np.empty(max(n, 1), dtype=np.int64)
        self._lib.pa_sched_waiting(self._h, _ptr(out), n)
        return out[:n].tolist()

"""The C++ scheduler's entry points from the host: argument checks, the prefix
mode's need for decode token IDs (PA_ERR_STATE with nothing changed when one is
missing), and a live loop that passes each sampled token with
pa_sched_push_tokens planning exactly what the replayed trace plans."""

import ctypes

import numpy as np
import pytest

from paged_kv_cache_397_amd import _native as N
from paged_kv_cache_397_amd.scheduler import TraceScheduler
from workloads import CONFIGS, gen


def _events(plan):
    return (plan.finished, plan.admitted, plan.preempted, plan.cached,
            [(r, s, c, list(map(int, sl))) for r, s, c, sl in plan.prefill],
            plan.decode_rids.tolist(), plan.decode_pos.tolist(), plan.decode_slots.tolist(),
            plan.decode_cows.tolist(),
            [(r, p.tolist()) for r, p in plan.swapped_in], [(r, p.tolist()) for r, p in plan.swapped_out])


def test_argument_checks():
    lib = N.lib()
    h = ctypes.c_void_p()
    assert lib.pa_sched_create(16, 16, None, 0, 0, 0, ctypes.byref(h)) == N.PA_ERR_INVALID_ARG
    assert lib.pa_sched_create(16, 16, None, 8, 0, -1, ctypes.byref(h)) == N.PA_ERR_INVALID_ARG
    assert lib.pa_sched_create(0, 16, None, 8, 0, 0, ctypes.byref(h)) == N.PA_ERR_INVALID_ARG
    assert lib.pa_sched_create(16, 16, None, 8, 1, 0, ctypes.byref(h)) == N.PA_OK
    try:
        one = np.ones(1, dtype=np.int32)
        p = one.ctypes.data_as(ctypes.c_void_p)
        # prefix caching needs the prompt's token IDs
        assert lib.pa_sched_add_requests(h, 1, p, p, None, None, None) == N.PA_ERR_INVALID_ARG
        neg = np.array([-1], dtype=np.int32)
        assert lib.pa_sched_add_requests(h, 1, neg.ctypes.data_as(ctypes.c_void_p), p, p, None,
                                         None) == N.PA_ERR_INVALID_ARG
        rid = np.array([5], dtype=np.int64)
        assert lib.pa_sched_push_tokens(h, rid.ctypes.data_as(ctypes.c_void_p), p, 1) == N.PA_ERR_STATE
        assert lib.pa_sched_step(h, None) == N.PA_ERR_INVALID_ARG
    finally:
        lib.pa_sched_destroy(h)


def test_partial_token_source_is_refused():
    """A token source that gives some requests fewer outputs than they generate would
    leave the scheduler reading past the tokens given: the binding refuses it."""
    s = TraceScheduler(8, 4, 4, gen_tokens=lambda rid, first, count: np.zeros(min(count, 1), dtype=np.int32))
    with pytest.raises(ValueError):
        s.add_requests([(np.arange(6, dtype=np.int32), 2)])


def test_missing_decode_token_changes_nothing():
    """A request whose next token ID was never given: the step fails before any
    change, and runs as planned once the token is pushed."""
    s = TraceScheduler(8, 4, 4, gen_tokens=lambda rid, first, count: np.zeros(0, dtype=np.int32))
    ref = TraceScheduler(8, 4, 4, gen_token=lambda rid, p: 7)
    for t in (s, ref):
        t.step(0, [(np.arange(6, dtype=np.int32), 2)])   # admitted, two chunks
        t.step(1, [])
    free_before = s.alloc.free_list()
    with pytest.raises(N.PagedKVError) as e:
        s.step(2, [])                                     # decodes position 6: no ID
    assert e.value.status == N.PA_ERR_STATE
    assert s.alloc.free_list() == free_before and s.alloc.length(0) == 6
    s.push_tokens([0], [7])
    assert _events(s.step(2, [])) == _events(ref.step(2, []))


@pytest.mark.parametrize("num_blocks,host", [(None, 0), (120, 0), (120, 40)])
def test_live_token_push_equals_replay(num_blocks, host):
    """Prefix caching with the token IDs passed one by one as a live loop samples
    them (the token a request appends at position p, pushed before the step that
    appends it) plans the same steps as the replay that knows them at arrival."""
    cfg = CONFIGS["trace_prefix_small"]
    N_ = num_blocks or cfg.num_blocks
    order = gen.pool_permutation(cfg.seed, N_)
    replay = TraceScheduler(N_, cfg.block_size, cfg.chunk, order, gen_tokens=cfg.gen_tokens,
                            num_host_blocks=host)
    live = TraceScheduler(N_, cfg.block_size, cfg.chunk, order,
                          gen_tokens=lambda rid, first, count: np.zeros(0, dtype=np.int32),
                          num_host_blocks=host)
    prompt, known, gen_count = {}, {}, {}
    preempted = 0
    for n in range(cfg.steps):
        arr = cfg.arrivals(n)
        for k, (p, _) in enumerate(arr):
            rid = live.next_rid + k
            prompt[rid], known[rid], gen_count[rid] = len(p), 0, 0
        # the live loop: every live request that may append this step knows the ID
        # of the token it appends next (position prompt + generated)
        if n > 0:
            need = [r for r in prompt if r < live.next_rid and known[r] <= gen_count[r]]
            if need:
                ids = np.array(need, dtype=np.int64)
                toks = np.array([cfg.gen_token(r, prompt[r] + gen_count[r]) for r in need], dtype=np.int32)
                live.push_tokens(ids, toks)
                for r in need:
                    known[r] += 1
        a = live.step(n, arr)
        b = replay.step(n, arr)
        assert _events(a) == _events(b), n
        for r in a.decode_rids.tolist():
            gen_count[r] += 1
        for r in a.finished:
            del prompt[r], known[r], gen_count[r]
        preempted += len(a.preempted) + len(a.swapped_out)
    assert live.alloc.prefix_stats() == replay.alloc.prefix_stats()
    if num_blocks is not None:
        assert preempted > 0

#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

One step is one pass of the whole decode hot path over the batch:
  host bookkeeping (library allocator: reserve every sequence's next slot,
  copy-on-write pairs, changed table entries) -> one host-to-device copy of
  that metadata -> block copies and table updates -> cache write of the new
  tokens' K/V -> decode attention (one kernel: gather + attention, with the
  merge of split sequences folded in).
All inputs (cache contents, per-step q / k / v) are resident in HBM before the
timed region.  The host part of step n+1 overlaps the device part of step n.

Prints one JSON line (the benchmark contract) with the whole-step effective
KV bandwidth as `value`, the pass-1 roofline (HIP events on the launch stream)
and the CPU oracle timed on a sample of the same batch.
"""

from __future__ import annotations

import argparse
import collections
import gc
import json
import math
import os
import platform
import sys
import time

import numpy as np

# Kernel arguments in device memory instead of host memory (a documented HIP runtime
# option, read when the runtime starts): the dispatch of each launch then does not
# fetch its arguments over the host link.  Measured on the batch-256 GQA step:
# 226.6-227.0 against 230.9-231.2 us/step.  Set before anything starts HIP; a value
# in the environment wins.
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

METRIC = "paged decode attention: effective KV GB/s (% HBM peak) + µs/step, batch 256"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gqa_b256",
                    choices=["gqa_b256", "llama2_7b_b64", "tiny_f32", "shared_prefix_b16", "shared_prefix_b32",
                             "trace_13b", "trace_prefix", "prefill_13b", "prefill_gqa", "swap_13b", "blocksize_sweep",
                             "hbm_ceiling"])
    ap.add_argument("--units", type=int, default=0, help="decode work units (0 = library default)")
    ap.add_argument("--step-launch", choices=["one", "two"], default="two",
                    help="a decode step as one launch (pa_decode_step: cache writes folded into "
                         "the decode kernel) or as two (pa_append_tokens, then pa_paged_attn_decode)")
    ap.add_argument("--metadata", choices=["pinned", "upload"], default="pinned",
                    help="the write kernel reads a step's metadata from its pinned ring slot in "
                         "place, or from a device copy uploaded ahead on a copy stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, copy a MIB-MiB device buffer 5 times (a plain "
                         "copy of known size, used to scale hardware byte counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int):
    """Device-to-device copies of a known size: the reference for FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    t = min(times)
    print(json.dumps({"copy_calibration_bytes": n, "reads_bytes": n, "writes_bytes": n,
                      "best_us": round(t * 1e6, 2),
                      "read_plus_write_gbps": round(2 * n / t / 1e9, 1)}), flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_397_amd", "csrc", f)
                  for f in ("decode_kernels.h", "decode_variant.hip", "kernels_decode.hip",
                            "kernels_common.h", "pagedkv_internal.h")]


PREFILL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_397_amd", "csrc", f)
                   for f in ("kernels_prefill.hip", "kernels_common.h", "pagedkv_internal.h")]


def measured_traffic(config_name: str, kind: str = "decode", sources=None):
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or
    None when there is none for this workload or the kernel source has changed since."""
    import hashlib
    sources = DECODE_SOURCES if sources is None else sources
    stem = config_name if config_name.startswith(kind) else f"{kind}_{config_name}"
    path = os.path.join(ROOT, "profiles", f"{stem}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            fields[k.strip()] = v.strip()
    digest = hashlib.sha256(b"".join(open(f, "rb").read() for f in sources)).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(cfg, ctx, q_host, seconds):
    """Time the fp64 oracle (as it stands) on every 4th sequence of step 0's batch."""
    from oracle.attention import paged_decode
    from oracle.cache import reshape_and_cache
    from oracle.layout import CacheLayout
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    sample = list(range(0, len(ctx), 4))
    B = cfg.block_size
    nblk = [-(-int(ctx[i]) // B) for i in sample]
    lay = CacheLayout(sum(nblk), cfg.num_kv_heads, B, cfg.head_dim, cfg.dtype)
    kc, vc = lay.empty_cache(), lay.empty_cache()
    tables = np.full((len(sample), max(nblk)), -1, dtype=np.int64)
    pos = 0
    for r, i in enumerate(sample):
        tables[r, :nblk[r]] = np.arange(pos, pos + nblk[r])
        pos += nblk[r]
        K, V = gen.seq_kv(cfg.seed, i, int(ctx[i]), cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
        slots = tables[r, np.arange(int(ctx[i])) // B] * B + np.arange(int(ctx[i])) % B
        reshape_and_cache(lay, K, V, slots, kc, vc)
    sctx = ctx[sample]
    q = q_host[sample]
    times = []
    t_end = time.perf_counter() + seconds
    while not times or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        paged_decode(lay, q, kc, vc, tables, sctx, cfg.scale)
        times.append(time.perf_counter() - t0)
    kv_bytes = int(sctx.sum()) * cfg.kv_bytes_per_token()
    t = float(np.median(times))
    # the same sample on one thread (BLAS limited to one), a shorter budget
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1s = []
            t_end = time.perf_counter() + seconds / 2
            while not t1s or time.perf_counter() < t_end:
                t0 = time.perf_counter()
                paged_decode(lay, q, kc, vc, tables, sctx, cfg.scale)
                t1s.append(time.perf_counter() - t0)
        single = {"value": kv_bytes / float(np.median(t1s)) / 1e9, "unit": "GB/s", "cores": 1,
                  "runs": len(t1s), "seconds_per_run": float(np.median(t1s))}
    except Exception as exc:  # pragma: no cover
        single = {"error": repr(exc)}
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": kv_bytes / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle (gather + textbook softmax) on every 4th sequence of "
                       f"the batch ({len(sample)} seqs, {int(sctx.sum())} tokens, "
                       f"{kv_bytes / 1e9:.3f} GB of KV), median of {len(times)} runs"),
            "seconds_per_run": t, "cpu_model": cpu, "affinity_cpus": len(os.sched_getaffinity(0)),
            "single_thread": single}


def _trace_end_to_end(cfg, spec, kc, vc, packed, max_blocks, pmax, smax, cmax, units, ws, order,
                      gtok, overlap=False):
    """The trace as a serving loop: each step the host plans it with a fresh library
    scheduler, writes its metadata into a pinned ring slot, uploads the slot with
    one copy and launches the step's kernels; the device runs behind the host, so
    the host's planning of step n + 1 overlaps the device's step n.  Returns the
    device timeline per step (events at step `lo` and after the last step: host
    bubbles included) and the host's own time per step.  overlap: a step's prompt
    phase (chunk writes and prefill attention) runs on a second stream beside its
    decode phase (token writes and decode attention) - they touch disjoint blocks
    and sequences - and the two join before the next step, whose work may depend on
    either (a finished request's blocks reused, a completed prompt decoding)."""
    import torch
    from paged_kv_cache_397_amd import ops
    from paged_kv_cache_397_amd.scheduler import TraceScheduler

    B, D, Hq, Hkv = spec.block_size, spec.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    sched = TraceScheduler(cfg.num_blocks, B, cfg.chunk, order, gen_tokens=gtok)
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 1)
    dt = spec.torch_dtype
    pool = {"pk": (pmax, Hkv), "pv": (pmax, Hkv), "pq": (pmax, Hq), "k": (smax, Hkv),
            "v": (smax, Hkv), "q": (smax, Hq)}
    pool = {k: torch.randn(n, h, D, generator=g, device="cuda", dtype=dt) for k, (n, h) in pool.items()}
    pout = torch.empty(pmax, Hq, D, device="cuda", dtype=dt)
    dout = torch.empty(smax, Hq, D, device="cuda", dtype=dt)
    # one slot's layout: (name, dtype, count), each field 256-byte aligned
    fields = [("pslots", np.int64, pmax), ("pqs", np.int32, cmax + 1), ("pctx", np.int32, cmax),
              ("ptables", np.int32, cmax * max_blocks), ("dslots", np.int64, smax),
              ("cows", np.int32, 2 * smax), ("tables", np.int32, smax * max_blocks),
              ("ctx", np.int32, smax)]
    offs, o = {}, 0
    for name, dtp, cnt in fields:
        offs[name] = (o, dtp, cnt)
        o += -(-cnt * np.dtype(dtp).itemsize // 256) * 256
    slot_bytes = o
    ring = 4
    pinned = [torch.empty(slot_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(ring)]
    host_views = [{n: p.numpy()[a:a + c * np.dtype(t).itemsize].view(t) for n, (a, t, c) in offs.items()}
                  for p in pinned]
    # two device staging buffers: step n + 1's upload (on a copy stream) overlaps step
    # n's kernels, and waits only for step n - 1's, the last user of its buffer
    devs = [torch.empty(slot_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    tdt = {np.int64: torch.int64, np.int32: torch.int32}
    dev_viewss = [{n: d[a:a + c * np.dtype(t).itemsize].view(tdt[t]) for n, (a, t, c) in offs.items()}
                  for d in devs]
    copy_stream = torch.cuda.Stream()  # default priority
    done_ev = [None, None]
    ring_ev = [None] * ring
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream() if overlap else stream  # default priority
    lo = min(50, cfg.steps - 1)
    ev_lo, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host_s, wait_s = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in range(cfg.steps):
        h0 = time.perf_counter()
        if n == lo:
            ev_lo.record(stream)
        plan = sched.step(n, packed[n])
        k = n % ring
        w0 = time.perf_counter()
        if ring_ev[k] is not None:
            ring_ev[k].synchronize()  # the slot's previous upload has been read
        wait_s.append(time.perf_counter() - w0)
        hv = host_views[k]
        P, C, S = plan.prefill_tokens(), len(plan.prefill_rids), len(plan.decode_rids)
        if P:
            hv["pslots"][:P] = plan.prefill_slots
            hv["pqs"][0] = 0
            np.cumsum(plan.prefill_count, out=hv["pqs"][1:C + 1])
            hv["pctx"][:C] = plan.prefill_start + plan.prefill_count
            sched.alloc.batch_metadata(plan.prefill_rids, max_blocks,
                                       tables=hv["ptables"][:C * max_blocks].reshape(C, max_blocks),
                                       ctx=np.empty(C, dtype=np.int32))
        if S:
            hv["dslots"][:S] = plan.decode_slots
            hv["cows"][:2 * S] = plan.decode_cows.reshape(-1)
            sched.alloc.batch_metadata(plan.decode_rids, max_blocks,
                                       tables=hv["tables"][:S * max_blocks].reshape(S, max_blocks),
                                       ctx=hv["ctx"][:S])
        bsel = n & 1
        dev_views = dev_viewss[bsel]
        if done_ev[bsel] is not None:
            copy_stream.wait_event(done_ev[bsel])
        with torch.cuda.stream(copy_stream):
            devs[bsel].copy_(pinned[k], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(copy_stream)
        ring_ev[k] = ev
        stream.wait_event(ev)
        if P:
            if overlap:
                side.wait_stream(stream)  # the upload, and every earlier step
            with torch.cuda.stream(side):
                ops.reshape_and_cache(spec, pool["pk"][:P], pool["pv"][:P], dev_views["pslots"][:P],
                                      kc, vc)
                ops.paged_attn_prefill(spec, pout[:P], pool["pq"][:P], kc, vc,
                                       dev_views["ptables"][:C * max_blocks].view(C, max_blocks),
                                       dev_views["pqs"][:C + 1], dev_views["pctx"][:C], cfg.scale,
                                       max_query_len=int(plan.prefill_count.max()))
        if S:
            ops.append_tokens(spec, pool["k"][:S], pool["v"][:S], dev_views["dslots"][:S], kc, vc,
                              cow_pairs=(dev_views["cows"][:2 * S].view(S, 2)
                                         if plan.num_decode_cows else None))
            ops.paged_attn_decode(spec, dout[:S], pool["q"][:S], kc, vc,
                                  dev_views["tables"][:S * max_blocks].view(S, max_blocks),
                                  dev_views["ctx"][:S], cfg.scale, units, ws,
                                  keep_cached=bool(cfg.prefix))
        if overlap and P:
            stream.wait_stream(side)  # join before the next step
        dv = torch.cuda.Event()
        dv.record(stream)
        done_ev[bsel] = dv
        host_s.append(time.perf_counter() - h0)
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = ev_lo.elapsed_time(ev_end) * 1e3 / (cfg.steps - lo)
    ws_ = np.array(wait_s[lo:]) * 1e6
    hs = np.array(host_s[lo:]) * 1e6 - ws_
    return {"note": "a fresh scheduler plans each step while the device runs the previous ones; "
                    "one pinned-to-device copy of the step's metadata per step, on a copy stream "
                    "ahead of the kernels (two device staging buffers); device timeline "
                    "from step %d to the end over the steps, host bubbles included" % lo
                    + ("; prompt and decode phases of a step on two streams, joined per step"
                       if overlap else ""),
            "us_per_step": round(float(per), 2),
            "host_us_per_step": {"mean": round(float(hs.mean()), 2),
                                 "p99": round(float(np.percentile(hs, 99)), 2),
                                 "note": "planning, metadata and launches; the wait for a free "
                                         "ring slot (the host is ahead of the device) excluded"},
            "ring_wait_us_per_step_mean": round(float(ws_.mean()), 2),
            "wall_ms_all_steps": round(wall * 1e3, 2),
            "metadata_bytes_per_upload": int(slot_bytes)}


def run_trace(args):
    """The continuous-batching trace: the library scheduler plans every step on the
    host (timed separately), then each step's device work runs on inputs already in
    HBM - the prompt chunks' cache writes, chunked-prefill attention over them, the
    decode tokens' writes, and decode attention over every decoding sequence - timed
    with events around each step.  With shared prompt openings (prefix caching) the
    cached part of a prompt is neither written nor attended again."""
    import torch
    from paged_kv_cache_397_amd import ops, _native
    from paged_kv_cache_397_amd.scheduler import TraceScheduler
    from workloads import CONFIGS, gen

    _native.lib()
    cfg = CONFIGS[args.config]
    B, D, Hq, Hkv = cfg.block_size, cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    spec = ops.CacheSpec(cfg.num_blocks, B, Hkv, D, cfg.dtype)
    max_blocks = -(-(cfg.prompt_hi + cfg.out_hi) // B)
    if cfg.prefix:
        max_blocks = -(-(cfg.open_hi + cfg.suffix_hi + cfg.out_hi) // B)
    order = gen.pool_permutation(cfg.seed, cfg.num_blocks)
    gtok = cfg.gen_tokens if cfg.prefix else None
    sched = TraceScheduler(cfg.num_blocks, B, cfg.chunk, order, gen_tokens=gtok)
    arrivals = [cfg.arrivals(n) for n in range(cfg.steps)]
    # The arrivals packed as the scheduler takes them (prompts' and replayed outputs'
    # token IDs included), outside every timed region: they are the trace's input.
    packed, rid = [], 0
    for a in arrivals:
        packed.append(sched.pack(a, rid))
        rid += len(packed[-1])
    plans, host_s = [], []
    for n in range(cfg.steps):
        t0 = time.perf_counter()
        plan = sched.step(n, packed[n])
        tables, ctx = sched.alloc.batch_metadata(plan.decode_rids, max_blocks)
        ptables, _ = sched.alloc.batch_metadata(plan.prefill_rids, max_blocks)
        host_s.append(time.perf_counter() - t0)
        plans.append((plan, tables, ctx, ptables))
    log(f"scheduled {cfg.steps} steps on the host")
    # the oracle scheduling model over the same trace, timed the same way (host side)
    from oracle.scheduler_model import SchedulerModel
    model = SchedulerModel(cfg.num_blocks, B, cfg.chunk, order,
                           gen_token=cfg.gen_token if cfg.prefix else None)
    model_s = []
    model_steps = min(cfg.steps, 40)  # a bounded sample: the model is plain Python
    for n in range(model_steps):
        t0 = time.perf_counter()
        model.step(n, arrivals[n])
        model_s.append(time.perf_counter() - t0)
    # Inputs resident in HBM: per-step metadata, and seeded synthetic K/V/q drawn on
    # the device (values do not affect timing; the parity of this loop is a test).
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    kc, vc = ops.empty_cache(spec)
    kc.zero_()
    vc.zero_()
    steps_dev = []
    for plan, tables, ctx, ptables in plans:
        P = plan.prefill_tokens()
        S = len(plan.decode_rids)
        d = {"P": P, "S": S, "ctx_sum": int(ctx.sum()),
             "cached": int(sum(c for _, c in plan.cached))}
        if P:
            d["pslots"] = torch.from_numpy(np.concatenate([sl for _, _, _, sl in plan.prefill])).cuda()
            d["pk"] = torch.randn(P, Hkv, D, generator=g, device="cuda", dtype=spec.torch_dtype)
            d["pv"] = torch.randn(P, Hkv, D, generator=g, device="cuda", dtype=spec.torch_dtype)
            cl = np.array([c for _, _, c, _ in plan.prefill], dtype=np.int64)
            st = np.array([s0 for _, s0, _, _ in plan.prefill], dtype=np.int64)
            d["pq"] = torch.randn(P, Hq, D, generator=g, device="cuda", dtype=spec.torch_dtype)
            d["pout"] = torch.empty(P, Hq, D, device="cuda", dtype=spec.torch_dtype)
            d["pqs"] = torch.from_numpy(np.concatenate([[0], np.cumsum(cl)]).astype(np.int32)).cuda()
            d["pctx"] = torch.from_numpy((st + cl).astype(np.int32)).cuda()
            d["ptables"] = torch.from_numpy(ptables).cuda()
            d["pmax"] = int(cl.max())
            d["pflops"] = float(sum(4.0 * D * Hq * (c * s0 + c * (c + 1) // 2)
                                    for s0, c in zip(st.tolist(), cl.tolist())))
        if S:
            d["dslots"] = torch.from_numpy(plan.decode_slots).cuda()
            # a step whose appends copy no block passes no pairs (one write launch)
            d["cows"] = (torch.from_numpy(np.ascontiguousarray(plan.decode_cows)).cuda()
                         if (plan.decode_cows[:, 0] >= 0).any() else None)
            d["tables"] = torch.from_numpy(tables).cuda()
            d["ctx"] = torch.from_numpy(ctx).cuda()
            d["k"] = torch.randn(S, Hkv, D, generator=g, device="cuda", dtype=spec.torch_dtype)
            d["v"] = torch.randn(S, Hkv, D, generator=g, device="cuda", dtype=spec.torch_dtype)
            d["q"] = torch.randn(S, Hq, D, generator=g, device="cuda", dtype=spec.torch_dtype)
            d["out"] = torch.empty(S, Hq, D, device="cuda", dtype=spec.torch_dtype)
        steps_dev.append(d)
    units = args.units if args.units > 0 else ops.default_units()
    ws = ops.decode_workspace(spec, Hq, units)
    torch.cuda.synchronize()
    log("trace inputs resident in HBM")
    stream = torch.cuda.current_stream()
    evs = []
    t0 = time.perf_counter()
    evp = []
    for d in steps_dev:
        e0, e1, e2, ep0, ep1 = (torch.cuda.Event(enable_timing=True) for _ in range(5))
        e0.record(stream)
        ep0.record(stream)
        if d["P"]:
            ops.reshape_and_cache(spec, d["pk"], d["pv"], d["pslots"], kc, vc)
            ops.paged_attn_prefill(spec, d["pout"], d["pq"], kc, vc, d["ptables"], d["pqs"],
                                   d["pctx"], cfg.scale, max_query_len=d["pmax"])
        ep1.record(stream)
        evp.append((ep0, ep1))
        if d["S"]:
            ops.append_tokens(spec, d["k"], d["v"], d["dslots"], kc, vc, cow_pairs=d["cows"])
            e1.record(stream)
            # prefix-cached prompts share blocks between sequences: keep them cached
            ops.paged_attn_decode(spec, d["out"], d["q"], kc, vc, d["tables"], d["ctx"], cfg.scale,
                                  units, ws, keep_cached=bool(cfg.prefix))
        else:
            e1.record(stream)
        e2.record(stream)
        evs.append((e0, e1, e2))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = np.array([a.elapsed_time(c) for a, _, c in evs]) * 1e-3
    t_attn = np.array([b.elapsed_time(c) for _, b, c in evs]) * 1e-3
    t_pre = np.array([a.elapsed_time(b) for a, b in evp]) * 1e-3
    pmax_all = max([d["P"] for d in steps_dev] + [1])
    smax_all = max([d["S"] for d in steps_dev] + [1])
    cmax_all = max([len(pl.prefill) for pl, _, _, _ in plans] + [1])
    for d in steps_dev:  # the per-step inputs; the end-to-end loop below draws from pools
        for k in [k for k, v in d.items() if isinstance(v, torch.Tensor)]:
            del d[k]
    torch.cuda.empty_cache()
    e2e = _trace_end_to_end(cfg, spec, kc, vc, packed, max_blocks, pmax_all, smax_all, cmax_all,
                            units, ws, order, gtok)
    e2e_ov = _trace_end_to_end(cfg, spec, kc, vc, packed, max_blocks, pmax_all, smax_all,
                               cmax_all, units, ws, order, gtok, overlap=True)
    pflops = np.array([d.get("pflops", 0.0) for d in steps_dev])
    kv_tok = 2 * Hkv * D * spec_elem_bytes(cfg.dtype)
    kv_bytes = np.array([d["ctx_sum"] for d in steps_dev], dtype=np.float64) * kv_tok
    lo = min(50, cfg.steps - 1)
    sel = slice(lo, cfg.steps)
    attn_gbps = float(kv_bytes[sel].sum() / t_attn[sel].sum() / 1e9)
    result = {
        "metric": "continuous-batching trace: device µs/step and effective decode KV GB/s",
        "value": round(attn_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": cfg.steps,
        "warmup": 0,
        "ms_per_step": round(float(t_step[sel].mean()) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.title}", "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "block_size": B, "pool_blocks": cfg.num_blocks, "seed": cfg.seed,
                   "units": units},
        "steps_measured": f"{lo}..{cfg.steps - 1}",
        "us_per_step": {"mean": round(float(t_step[sel].mean()) * 1e6, 2),
                        "median": round(float(np.median(t_step[sel])) * 1e6, 2),
                        "p99": round(float(np.percentile(t_step[sel], 99)) * 1e6, 2)},
        "attn_us_per_step_mean": round(float(t_attn[sel].mean()) * 1e6, 2),
        "pct_hbm_peak_attn": round(100 * attn_gbps / HBM_PEAK_GBPS, 2),
        "decode_seqs_last_step": steps_dev[-1]["S"],
        "decode_kv_gb_last_step": round(float(kv_bytes[-1]) / 1e9, 3),
        "prefill_tokens_per_step_mean": round(float(np.mean([d["P"] for d in steps_dev[lo:]])), 1),
        "prefill_us_per_step_mean": round(float(t_pre[sel].mean()) * 1e6, 2),
        "prefill_attn_tflops": round(float(pflops[sel].sum() / max(t_pre[sel].sum(), 1e-12) / 1e12), 2),
        "prefix_cache": ({"cached_prompt_tokens_per_step_mean":
                          round(float(np.mean([d["cached"] for d in steps_dev[lo:]])), 1),
                          "blocks_looked_up_reused_cached_now": list(sched.alloc.prefix_stats())}
                         if cfg.prefix else None),
        "host_scheduler_us_per_step": {"mean": round(float(np.mean(host_s[lo:])) * 1e6, 2),
                                       "p99": round(float(np.percentile(host_s[lo:], 99)) * 1e6, 2)},
        "oracle_scheduler": {"kind": "oracle", "steps": f"0..{model_steps - 1}",
                             "us_per_step_mean": round(float(np.mean(model_s)) * 1e6, 2),
                             "library_us_per_step_mean_same_steps":
                                 round(float(np.mean(host_s[:model_steps])) * 1e6, 2)},
        "wall_ms_all_steps": round(wall * 1e3, 2),
        "end_to_end": e2e,
        "end_to_end_phases_overlapped": e2e_ov,
    }
    print(json.dumps(result), flush=True)


def spec_elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def prefill_flops(offsets, chunk, num_q_heads, head_dim):
    """Algorithmic flops of causal chunk attention: a token at position p attends to
    p + 1 keys, 2 D flops each for QK^T and for PV, per query head."""
    keys = sum(int(o) * chunk + chunk * (chunk + 1) // 2 for o in offsets)
    return 4.0 * head_dim * num_q_heads * keys


def cpu_baseline_prefill(cfg, offsets, seconds):
    """Time the fp64 oracle (as it stands) on the first 32 rows of each of the first
    two chunks, with seeded data of the same shapes."""
    from oracle.attention import prefill_attention
    from oracle.layout import to_float64
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    rows = 32
    work = []
    for s in range(2):
        L = int(offsets[s]) + cfg.chunk
        K, V = gen.seq_kv(cfg.seed, s, L, cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
        q = gen.q_values(cfg.seed, 1 + s, rows, cfg.num_q_heads, cfg.head_dim, cfg.dtype)
        work.append((to_float64(q, cfg.dtype), to_float64(K, cfg.dtype), to_float64(V, cfg.dtype),
                     int(offsets[s])))
    flops = sum(4.0 * cfg.head_dim * cfg.num_q_heads * (rows * o + rows * (rows + 1) // 2)
                for _, _, _, o in work)
    times = []
    t_end = time.perf_counter() + seconds
    while not times or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        for q, K, V, o in work:
            prefill_attention(q, K[:o + rows], V[:o + rows], cfg.scale, o)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle on the first {rows} rows of chunks 0 and 1 "
                       f"(offsets {int(offsets[0])}, {int(offsets[1])}), median of {len(times)} runs"),
            "seconds_per_run": t}


def run_prefill(args):
    """Chunked-prefill attention: every sequence's cache holds its offset plus its
    chunk (written beforehand); one call attends every chunk token causally.  A step
    is one call over the whole batch of chunks, inputs resident in HBM."""
    import torch
    from paged_kv_cache_397_amd import ops, _native
    from paged_kv_cache_397_amd.batch import PagedKVCache
    from workloads import CONFIGS

    _native.lib()
    cfg = CONFIGS[args.config]
    S, Hq, Hkv, D, B, c = (cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                           cfg.block_size, cfg.chunk)
    spec = ops.CacheSpec(cfg.num_blocks, B, Hkv, D, cfg.dtype)
    offsets = cfg.offsets()
    L = (offsets + c).astype(np.int32)
    cache = PagedKVCache(spec, cfg.pool_order(), fill=0.0)
    for i in range(S):
        cache.alloc.add(i, int(L[i]))
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    # values do not change the timing; parity of this kernel is a test
    cache.k.copy_(torch.randn(cache.k.shape, generator=g, device="cuda", dtype=torch.float32))
    cache.v.copy_(torch.randn(cache.v.shape, generator=g, device="cuda", dtype=torch.float32))
    tables, ctx, _, _ = cache.metadata(range(S))
    T = S * c
    q = torch.randn(T, Hq, D, generator=g, device="cuda", dtype=torch.float32).to(spec.torch_dtype)
    out = torch.empty_like(q)
    qs = torch.arange(0, T + 1, c, dtype=torch.int32, device="cuda")
    ctx_dev = torch.from_numpy(L).cuda()
    stream = torch.cuda.current_stream()
    call = lambda: ops.paged_attn_prefill(spec, out, q, cache.k, cache.v, tables, qs, ctx_dev,
                                          cfg.scale, max_query_len=c, stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    per = []
    for _ in range(10):  # per-launch durations, untimed
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) * 1e-3)
    flops = prefill_flops(offsets, c, Hq, D)
    kv_bytes = float(L.sum()) * 2 * Hkv * D * spec_elem_bytes(cfg.dtype)
    tflops = flops / dev_s / 1e12
    result = {
        "metric": "chunked-prefill attention TFLOP/s (causal, paged K/V)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dev_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.title}", "seqs": S, "chunk": c,
                   "offsets": offsets.tolist(), "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block_size": B, "seed": cfg.seed},
        "wall_ms_timed": round(wall * 1e3, 3),
        "launch_us": {"median": round(float(np.median(per)) * 1e6, 2),
                      "min": round(float(np.min(per)) * 1e6, 2)},
        "flops_per_step": flops,
        "unique_kv_bytes_per_step": kv_bytes,
        "roofline": {"kernel": "prefill_kernel", "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name, "prefill", PREFILL_SOURCES),
                     "unique_kv_gbps": round(kv_bytes / dev_s / 1e9, 1)},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on the host)")
        result["cpu_baseline"] = cpu_baseline_prefill(cfg, offsets, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def run_tiny(args):
    """The tiny fp32 workload (4 sequences, ctx {1, 15, 16, 33}, 2 heads, D 64, a
    16-block pool): the sequences are admitted, then every sequence's next token is
    placed by the allocator (the third one takes a new block).  A step is that
    write of 4 tokens (reshape_and_cache) plus decode over the lengths after it.
    The same step is repeated (it rewrites the same slots with the same values), so
    the pool never runs out; at 70 KB of K/V the step is bound by launch latency,
    and its microseconds are the figure."""
    import torch
    from paged_kv_cache_397_amd import ops, _native
    from paged_kv_cache_397_amd.batch import PagedKVCache, to_device
    from workloads import CONFIGS, gen

    _native.lib()
    cfg = CONFIGS["tiny_f32"]
    S, Hq, Hkv, D, B = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    spec = ops.CacheSpec(cfg.num_blocks, B, Hkv, D, cfg.dtype)
    cache = PagedKVCache(spec, cfg.pool_order(), fill=0.0)
    ctx0 = cfg.context_lens()
    for i in range(S):
        K, V = gen.seq_kv(cfg.seed, i, int(ctx0[i]), Hkv, D, cfg.dtype)
        cache.add_sequence(i, K, V)
    st, done, slots, cows, _, _ = cache.alloc.append_batch(np.arange(S, dtype=np.int64))
    if st != 0 or done != S:
        raise RuntimeError(f"append_batch failed: status {st}")
    kn, vn = gen.new_tokens(cfg.seed, 1, S, Hkv, D, cfg.dtype)
    k_new, v_new = to_device(kn, spec), to_device(vn, spec)
    slots_dev = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
    tables, ctx_dev, _, ctx_h = cache.metadata(range(S))
    q = to_device(gen.q_values(cfg.seed, 1, S, Hq, D, cfg.dtype), spec)
    out = torch.empty(S, Hq, D, dtype=spec.torch_dtype, device="cuda")
    units = args.units if args.units > 0 else 0
    ws = ops.decode_workspace(spec, Hq, units)
    stream = torch.cuda.current_stream()
    write = ops.bind_reshape_and_cache(spec, k_new, v_new, slots_dev, cache.k, cache.v, stream)
    decode = ops.bind_decode(spec, out, q, cache.k, cache.v, tables, ctx_dev, cfg.scale, units, ws)
    for _ in range(args.warmup):
        write()
        decode()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        write()
        decode()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_w, t_d = [], []
    for _ in range(100):  # per-launch durations, untimed
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        write()
        b.record(stream)
        decode()
        c.record(stream)
        torch.cuda.synchronize()
        t_w.append(a.elapsed_time(b) * 1e-3)
        t_d.append(b.elapsed_time(c) * 1e-3)
    kv_bytes = float(ctx_h.sum()) * cfg.kv_bytes_per_token()
    us = wall / args.steps * 1e6
    result = {
        "metric": "paged decode step latency (µs/step: cache write of the step's tokens + decode)",
        "value": round(us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.title}", "seqs": S, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "block_size": B, "pool_blocks": cfg.num_blocks,
                   "context_lens": [int(x) for x in ctx_h], "seed": cfg.seed,
                   "units": units or "library default"},
        "write_us": {"median": round(float(np.median(t_w)) * 1e6, 2), "min": round(float(np.min(t_w)) * 1e6, 2)},
        "decode_us": {"median": round(float(np.median(t_d)) * 1e6, 2), "min": round(float(np.min(t_d)) * 1e6, 2)},
        "kv_bytes_per_step": kv_bytes,
        "decode_kv_gbps_median": round(kv_bytes / float(np.median(t_d)) / 1e9, 3),
        "roofline": None,
        "note": "launch-latency bound: 70 KB of K/V is far below any bandwidth or compute limit",
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on the host)")
        from oracle.attention import paged_decode
        from oracle.cache import reshape_and_cache
        from oracle.layout import CacheLayout
        lay = CacheLayout(cfg.num_blocks, Hkv, B, D, cfg.dtype)
        kc, vc = lay.empty_cache(), lay.empty_cache()
        t_host = tables.cpu().numpy().astype(np.int64)
        for i in range(S):
            L = int(ctx0[i])
            K, V = gen.seq_kv(cfg.seed, i, L, Hkv, D, cfg.dtype)
            reshape_and_cache(lay, K, V, t_host[i, np.arange(L) // B] * B + np.arange(L) % B, kc, vc)
        q_h = gen.q_values(cfg.seed, 1, S, Hq, D, cfg.dtype)
        times = []
        for _ in range(1000):
            h0 = time.perf_counter()
            reshape_and_cache(lay, kn, vn, np.asarray(slots, dtype=np.int64), kc, vc)
            paged_decode(lay, q_h, kc, vc, t_host, ctx_h.astype(np.int64), cfg.scale)
            times.append(time.perf_counter() - h0)
        result["cpu_baseline"] = {"value": round(float(np.median(times)) * 1e6, 2), "unit": "us/step",
                                  "cores": 1, "kind": "oracle",
                                  "sample": "the whole step (cache write of 4 tokens + fp64 decode of the 4 "
                                            "sequences), median of 1000 runs"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def run_blocksize(args):
    """Block-size sweep.  Host: KV utilisation (tokens held / slots reserved) of the
    serving trace's running requests with on-demand paging at B = 8, 16, 32, 64,
    against contiguous reservation of prompt + the largest allowed output, read from
    the library allocator (equal pool tokens for every B).  GPU: decode attention
    over a Llama-2-7B-shaped batch at B = 8, 16, 32, 64 (equal pool tokens; at B = 8
    each 16-token tile is read from two blocks, so twice the table entries)."""
    import torch
    from paged_kv_cache_397_amd import ops, _native
    from paged_kv_cache_397_amd.allocator import BlockAllocator
    from paged_kv_cache_397_amd.scheduler import TraceScheduler
    from workloads import CONFIGS, gen

    _native.lib()
    tr = CONFIGS["trace_13b"]
    pool_tokens = tr.num_blocks * tr.block_size
    arrivals = [tr.arrivals(n) for n in range(tr.steps)]
    util = {}
    for B in (8, 16, 32, 64):
        N = pool_tokens // B
        sch = TraceScheduler(N, B, tr.chunk, gen.pool_permutation(tr.seed, N))
        pg, ct, fx = [], [], []
        for n in range(tr.steps):
            sch.step(n, arrivals[n])
            if n < 50:
                continue
            rids, prompts, lens = sch.running_info()
            if not len(rids):
                continue
            # tokens held over slots reserved: the allocator's own block count (paged),
            # prompt + the largest allowed output, and a fixed 4096 per request
            held = int(lens.sum())
            pg.append(held / ((N - sch.alloc.num_free()) * B))
            ct.append(held / int((prompts.astype(np.int64) + tr.out_hi).sum()))
            fx.append(held / (4096 * len(rids)))
        util[B] = {"paged_mean": round(float(np.mean(pg)), 4), "paged_min": round(float(np.min(pg)), 4),
                   "contiguous_mean": round(float(np.mean(ct)), 4),
                   "fixed_4096_mean": round(float(np.mean(fx)), 4)}
    log("utilisation simulated")

    dc = CONFIGS["llama2_7b_b64"]
    S, Hq, Hkv, D = dc.num_seqs, dc.num_q_heads, dc.num_kv_heads, dc.head_dim
    ctx = dc.context_lens()
    kv_bytes = float(ctx.sum()) * dc.kv_bytes_per_token()
    dec = {}
    stream = torch.cuda.current_stream()
    for B in (8, 16, 32, 64):
        N = dc.num_blocks * 16 // B
        spec = ops.CacheSpec(N, B, Hkv, D, "bf16")
        kc, vc = ops.empty_cache(spec)
        kc.normal_()
        vc.normal_()
        alloc = BlockAllocator(N, B, gen.pool_permutation(dc.seed, N))
        for i in range(S):
            alloc.add(i, int(ctx[i]))
        tables, lens = alloc.batch_metadata(np.arange(S), -(-int(ctx.max()) // B))
        t_dev, c_dev = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
        q = torch.randn(S, Hq, D, device="cuda").to(torch.bfloat16)
        out = torch.empty_like(q)
        ws = ops.decode_workspace(spec, Hq, 0)
        call = ops.bind_decode(spec, out, q, kc, vc, t_dev, c_dev, dc.scale, 0, ws)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps, 10)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3 / reps
        dec[B] = {"decode_us": round(t * 1e6, 2), "kv_gbps": round(kv_bytes / t / 1e9, 1),
                  "table_entries": int(S * tables.shape[1])}
        del kc, vc
        torch.cuda.empty_cache()
    # chunked prefill at each block size: the prefill_13b batch (8 chunks of 512 tokens
    # after U[0, 3584] cached tokens), the same pool tokens at every B
    pc = CONFIGS["prefill_13b"]
    offsets = pc.offsets()
    Lp = (offsets + pc.chunk).astype(np.int32)
    flops = prefill_flops(offsets, pc.chunk, pc.num_q_heads, pc.head_dim)
    pre = {}
    for B in (8, 16, 32, 64):
        N = pc.num_blocks * 16 // B
        spec = ops.CacheSpec(N, B, pc.num_kv_heads, pc.head_dim, "bf16")
        kc, vc = ops.empty_cache(spec)
        kc.normal_()
        vc.normal_()
        alloc = BlockAllocator(N, B, gen.pool_permutation(pc.seed, N))
        for i in range(pc.num_seqs):
            alloc.add(i, int(Lp[i]))
        tables, _ = alloc.batch_metadata(np.arange(pc.num_seqs), -(-int(Lp.max()) // B))
        t_dev = torch.from_numpy(tables).cuda()
        T = pc.num_seqs * pc.chunk
        q = torch.randn(T, pc.num_q_heads, pc.head_dim, device="cuda").to(torch.bfloat16)
        out = torch.empty_like(q)
        qs = torch.arange(0, T + 1, pc.chunk, dtype=torch.int32, device="cuda")
        c_dev = torch.from_numpy(Lp).cuda()
        call = lambda: ops.paged_attn_prefill(spec, out, q, kc, vc, t_dev, qs, c_dev, pc.scale,
                                              max_query_len=pc.chunk, stream=stream)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps, 10)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3 / reps
        pre[B] = {"prefill_us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1)}
        del kc, vc
        torch.cuda.empty_cache()
    result = {
        "metric": "KV utilisation by block size (paged vs contiguous max-length reservation) "
                  "and decode attention us by block size",
        "value": util[16]["paged_mean"],
        "unit": "fraction of reserved KV slots holding tokens (B = 16)",
        "n_gpus": 1, "steps": tr.steps, "warmup": 50, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"blocksize_sweep: {tr.name} ({tr.title}) steps 50..{tr.steps - 1}, "
                               f"pool {pool_tokens} tokens; decode on {dc.name}",
                   "contiguous_max_new": tr.out_hi, "prefill_batch": pc.name},
        "utilisation": {str(k): v for k, v in util.items()},
        "decode": {str(k): v for k, v in dec.items()},
        "prefill": {str(k): v for k, v in pre.items()},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction, raw


def run_swap(args):
    """Swap preemption's data path: blocks of a 13B-shaped layer (40 KV heads x 16
    tokens x 128 dims, bf16: 160 KiB of K plus 160 KiB of V per block) copied from
    HBM to pinned host memory and back with pa_swap_blocks, scattered block IDs on
    both sides.  A plain contiguous copy of the same bytes (DMA engine) is timed
    beside it as the link's achievable rate."""
    import torch
    from paged_kv_cache_397_amd import ops, _native
    from paged_kv_cache_397_amd.allocator import BlockAllocator
    from workloads import gen

    _native.lib()
    nblk, nswap = 4096, 1024
    spec = ops.CacheSpec(nblk, 16, 40, 128, "bf16")
    kc, vc = ops.empty_cache(spec)
    kc.normal_()
    vc.normal_()
    hk, hv = ops.host_pool(spec, nswap)
    alloc = BlockAllocator(nblk, 16, gen.pool_permutation(12, nblk))
    alloc.set_host_pool(nswap)
    alloc.add(0, nswap * 16)
    out_pairs = torch.from_numpy(alloc.swap_out(0)).cuda()
    in_pairs = torch.from_numpy(alloc.swap_in(0)).cuda()
    nbytes = nswap * 2 * spec.num_kv_heads * spec.block_size * spec.head_dim * 2
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    reps = max(args.steps // 10, 3)
    t_out = timed(lambda: ops.swap_blocks(spec, kc, vc, hk, hv, out_pairs), reps)
    t_in = timed(lambda: ops.swap_blocks(spec, hk, hv, kc, vc, in_pairs), reps)
    dma_host = torch.empty(nbytes // 2, dtype=torch.bfloat16, pin_memory=True)
    dma_dev = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    t_dma_out = timed(lambda: dma_host.copy_(dma_dev, non_blocking=True), reps)
    t_dma_in = timed(lambda: dma_dev.copy_(dma_host, non_blocking=True), reps)
    gbps_out, gbps_in = nbytes / t_out / 1e9, nbytes / t_in / 1e9
    result = {
        "metric": "swap preemption: HBM <-> pinned host block copy GB/s",
        "value": round(min(gbps_out, gbps_in), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": 1,
        "ms_per_step": round((t_out + t_in) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swap_13b: 1024 scattered blocks (40x16x128 bf16, K+V 320 KiB each) "
                               "out to pinned host memory and back", "bytes_per_direction": nbytes},
        "swap_out_gbps": round(gbps_out, 2),
        "swap_in_gbps": round(gbps_in, 2),
        "dma_contiguous_gbps": {"device_to_host": round(nbytes / t_dma_out / 1e9, 2),
                                "host_to_device": round(nbytes / t_dma_in / 1e9, 2)},
        "roofline": {"kernel": "swap_blocks_kernel", "bound": "pcie", "achieved": round(min(gbps_out, gbps_in), 2),
                     "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(min(gbps_out, gbps_in) / PCIE_PEAK_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        from oracle.cache import swap_blocks as oracle_swap
        from oracle.layout import CacheLayout
        lay = CacheLayout(64, 40, 16, 128, "bf16")
        src = np.zeros(lay.cache_elems, dtype=np.uint16)
        dst = np.zeros_like(src)
        pairs = np.stack([np.arange(64), np.arange(64)[::-1]], axis=1)
        times = []
        t_end = time.perf_counter() + min(args.cpu_seconds, 5.0)
        while not times or time.perf_counter() < t_end:
            t0 = time.perf_counter()
            oracle_swap(lay, src, src, lay, dst, dst, pairs)
            times.append(time.perf_counter() - t0)
        b = 64 * 2 * lay.block_elems() * 2
        result["cpu_baseline"] = {"value": round(b / float(np.median(times)) / 1e9, 2), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": "oracle whole-block copy of 64 blocks between two host pools"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def run_ceiling(args):
    """What the part delivers for the decode kernel's read pattern, without any
    attention work: the probe library's eight-wave workgroups read, per step, one
    32 KiB chunk of a K buffer and one of a V buffer (each wave its 4 KiB slice,
    one 16-byte load per lane per KiB), over 1.27 GB (the batch-256 GQA step's
    K/V).  Streaming = each workgroup walks its own contiguous run of chunks;
    gather = chunks in a seeded random order.  Non-temporal or ordinary loads, one
    tile in flight per wave (as decode) or two."""
    import ctypes

    import torch

    from paged_kv_cache_397_amd import build as B

    if not os.path.exists(B.PROBE_LIB):
        raise ImportError(f"{B.PROBE_LIB} is missing: build the package first")
    lib = ctypes.CDLL(B.PROBE_LIB)
    fn = lib.pa_probe_gather_read
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_void_p]
    chunk = 32 * 1024
    results = []
    stream = torch.cuda.current_stream()
    for groups, per in ((256, 76), (512, 38), (128, 152)):
        n = groups * per
        k = torch.empty(n * chunk // 4, dtype=torch.int32, device="cuda")
        v = torch.empty_like(k)
        k.fill_(1)
        v.fill_(2)
        sink = torch.empty(groups * 8, dtype=torch.int32, device="cuda")
        rng = np.random.default_rng(12345)
        orders = {"stream": np.arange(n, dtype=np.int32),
                  "gather": rng.permutation(n).astype(np.int32)}
        nbytes = 2.0 * n * chunk
        for mode, order in orders.items():
            od = torch.from_numpy(order).cuda()
            for nt in (1, 0):
                for inflight in (1, 2):
                    call = lambda: fn(k.data_ptr(), v.data_ptr(), n, od.data_ptr(), groups, per,
                                      sink.data_ptr(), nt, inflight, stream.cuda_stream)
                    times = []
                    for rep in range(13):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        rc = call()
                        e1.record(stream)
                        if rc != 0:
                            raise RuntimeError(f"probe launch failed ({rc})")
                        torch.cuda.synchronize()
                        if rep >= 3:
                            times.append(e0.elapsed_time(e1) * 1e-3)
                    t = float(np.median(times))
                    results.append({"waves": groups * 8, "mode": mode,
                                    "loads": "non-temporal" if nt else "ordinary",
                                    "tiles_in_flight": inflight, "us": round(t * 1e6, 2),
                                    "gbps": round(nbytes / t / 1e9, 1),
                                    "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4)})
                    log(f"{results[-1]}")
            # the gather through buffer loads with each cache-policy setting
            if mode == "gather":
                pol = lib.pa_probe_gather_read_policy
                pol.restype = ctypes.c_int32
                pol.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                ctypes.c_void_p]
                for cp, name in ((0, "default"), (1, "sc0"), (2, "nt"), (3, "sc0 nt"), (16, "sc1"),
                                 (17, "sc0 sc1"), (18, "sc1 nt"), (19, "sc0 sc1 nt")):
                    times = []
                    for rep in range(13):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        rc = pol(k.data_ptr(), v.data_ptr(), n, od.data_ptr(), groups, per,
                                 sink.data_ptr(), cp, stream.cuda_stream)
                        e1.record(stream)
                        if rc != 0:
                            raise RuntimeError(f"probe launch failed ({rc})")
                        torch.cuda.synchronize()
                        if rep >= 3:
                            times.append(e0.elapsed_time(e1) * 1e-3)
                    t = float(np.median(times))
                    results.append({"waves": groups * 8, "mode": mode,
                                    "loads": f"buffer, policy {name}", "tiles_in_flight": 1,
                                    "us": round(t * 1e6, 2), "gbps": round(nbytes / t / 1e9, 1),
                                    "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4)})
                    log(f"{results[-1]}")
        del k, v
        torch.cuda.empty_cache()
    best = max(r["gbps"] for r in results if r["mode"] == "gather")
    print(json.dumps({"metric": "read ceiling for the decode access pattern (probe, no attention)",
                      "value": best, "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                      "config": {"workload": "hbm_ceiling: 2 x 32 KiB chunks per workgroup step, "
                                             "1.27 GB per pass"},
                      "bytes_per_pass": int(2 * 256 * 76 * chunk), "runs": results}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode path "
              f"shards by sequence or KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.config.startswith("trace"):
        run_trace(args)
        return
    if args.config.startswith("prefill"):
        run_prefill(args)
        return
    if args.config == "swap_13b":
        run_swap(args)
        return
    if args.config == "blocksize_sweep":
        run_blocksize(args)
        return
    if args.config == "hbm_ceiling":
        run_ceiling(args)
        return
    if args.config == "tiny_f32":
        run_tiny(args)
        return
    import torch
    from paged_kv_cache_397_amd import ops, _native
    from paged_kv_cache_397_amd.batch import PagedKVCache, to_device
    from workloads import CONFIGS, gen

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    _native.lib()  # fail loudly if the HIP library is not built
    cfg = CONFIGS[args.config]
    spec = ops.CacheSpec(cfg.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
    S, Hq, Hkv, D, B = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    steps, warm = args.steps, args.warmup
    prof_steps = 10  # untimed steps for the per-launch breakdown, after the timed region
    total_steps = steps + warm + prof_steps

    # ---------------------------------------------------------------- resident inputs
    t0 = time.time()
    cache = PagedKVCache(spec, cfg.pool_order(), fill=0.0)
    ctx0 = cfg.context_lens()
    seq_ids = np.arange(S, dtype=np.int64)
    if cfg.ctx_kind == "shared_prefix":
        # one parent holds the shared prefix (ending in a partial block); the other
        # sequences fork it, then every sequence appends its private suffix token by
        # token, round robin, so each first append meets the shared partial block.
        prefix = cfg.shared_prefix + B // 2
        Kp, Vp = gen.seq_kv(cfg.seed, 0, prefix, Hkv, D, cfg.dtype)
        cache.add_sequence(0, Kp, Vp)
        for c in range(1, S):
            cache.alloc.fork(0, c)
        extra = ctx0.astype(np.int64) - prefix
        suffix = [gen.seq_kv(cfg.seed, 1000 + i, int(extra[i]), Hkv, D, cfg.dtype) for i in range(S)]
        written = np.zeros(S, dtype=np.int64)
        while (written < extra).any():
            active = np.nonzero(written < extra)[0]
            st, done, slots, cows, _, _ = cache.alloc.append_batch(active)
            assert st == 0 and done == len(active)
            pairs = cows[cows[:, 0] >= 0]
            if len(pairs):
                ops.copy_blocks(spec, cache.k, cache.v,
                                torch.from_numpy(np.ascontiguousarray(pairs)).cuda())
            kk = np.stack([suffix[i][0][written[i]] for i in active])
            vv = np.stack([suffix[i][1][written[i]] for i in active])
            cache.write_tokens(kk, vv, slots)
            written[active] += 1
    else:
        for i in range(S):
            K, V = gen.seq_kv(cfg.seed, i, int(ctx0[i]), Hkv, D, cfg.dtype)
            cache.add_sequence(i, K, V)
            if i % 32 == 31:
                log(f"cache fill: {i + 1}/{S} sequences")
    max_blocks = -(-(int(ctx0.max()) + total_steps + 1) // B)
    tables_h, ctx_h = cache.alloc.batch_metadata(seq_ids, max_blocks)
    assert np.array_equal(ctx_h, ctx0)
    tables = torch.from_numpy(tables_h).cuda()
    q_host0 = gen.q_values(cfg.seed, 0, S, Hq, D, cfg.dtype)
    qs, ks, vs = [], [], []
    for n in range(total_steps):
        qs.append(to_device(gen.q_values(cfg.seed, n + 1, S, Hq, D, cfg.dtype), spec))
        kn, vn = gen.new_tokens(cfg.seed, n + 1, S, Hkv, D, cfg.dtype)
        ks.append(to_device(kn, spec))
        vs.append(to_device(vn, spec))
    out = torch.empty(S, Hq, D, dtype=spec.torch_dtype, device="cuda")
    units = args.units if args.units > 0 else ops.default_units()
    one_launch = args.step_launch == "one"
    ws = (ops.decode_step_workspace(spec, Hq, S, units) if one_launch
          else ops.decode_workspace(spec, Hq, units))
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.time() - t0:.1f} s): {S} seqs, sum ctx {int(ctx0.sum())}, "
        f"{units} units, step as {'one launch' if one_launch else 'two launches'}")

    # ---------------------------------------------------------------- per-step staging
    # A ring of pinned host buffers holds each step's metadata; the cache-write
    # kernel reads it in place (no separate host-to-device copy) and forwards the
    # context lengths to the device array the decode kernels read.
    # Slot n % R is reused by step n + R, once step n's launches are done.  An event
    # recorded on the stream is a marker packet that holds the next launch back by
    # ~6 us, so one is recorded only every EV_EVERY steps (and on the sampled timed
    # steps); a later step's event also covers the earlier steps.
    R, EV_EVERY = 8, 4
    words = S * 2 + S + 3 * S + 2 * S  # int32 words: slots (int64), ctx, updates, cow pairs
    pin = [torch.empty(words, dtype=torch.int32, pin_memory=True) for _ in range(R)]
    upload = args.metadata == "upload"
    # upload: each slot also has a device copy, filled on a copy stream as soon as the
    # host has staged it (the host runs steps ahead, so the copy is done before the
    # device reaches the step); the write kernel then reads device memory.  Device
    # slot n % R is free again once the ring event covering step n - R has completed,
    # which the host checks before staging; the compute stream waits for each copy.
    dmeta = [torch.empty(words, dtype=torch.int32, device="cuda") for _ in range(R)] if upload else pin
    copy_stream = torch.cuda.Stream() if upload else None  # default priority
    ring_ev = collections.deque()  # (step, event), oldest first
    ctx_dev = torch.from_numpy(ctx0.astype(np.int32)).cuda()

    def views(buf):
        return (buf[:2 * S].view(torch.int64), buf[2 * S:3 * S], buf[3 * S:6 * S].view(S, 3),
                buf[6 * S:8 * S].view(S, 2))

    # numpy views of every pinned slot, and the allocator's append bound to each slot:
    # slots and copy-on-write pairs land in the slot, new table entries in two arrays
    pin_np = [tuple(x.numpy() for x in views(buf)) for buf in pin]
    new_blocks = np.empty(S, dtype=np.int32)
    new_cols = np.empty(S, dtype=np.int32)
    binds = [cache.alloc.bind_append_batch(seq_ids, ps, pp, new_blocks, new_cols)
             for ps, _, _, pp in pin_np]

    ctx_now = ctx0.astype(np.int64).copy()
    stream = torch.cuda.current_stream()
    kv_per_tok = cfg.kv_bytes_per_token()
    ev = []
    host = []  # per timed step: (allocator, ring-slot wait, staging, whole host side) seconds

    # Every launch of every step is bound once (arguments converted up front); the
    # per-step metadata has a fixed shape (a copy-on-write row and a table-update row
    # per sequence, -1 when there is none).  A step whose appends copy no block
    # passes no copy-on-write pairs, so its writes are one launch; a step with
    # copies runs them as a launch of their own first.
    # Sequences forked from one parent share its blocks: those are read with ordinary
    # loads so that the shared prefix stays cached; private contexts are streamed.
    # With one launch per step (pa_decode_step) the decode kernel itself writes each
    # sequence's new token (and a copy-on-write copy) from the pinned metadata, sets
    # the table entries and lengths, and attends.
    shared = cfg.ctx_kind == "shared_prefix"
    calls = []
    for n in range(total_steps):
        hs, hc, hu, hp = views(dmeta[n % R])
        if one_launch:
            step_args = (spec, out, qs[n], ks[n], vs[n], hs, hc, cache.k, cache.v, tables, ctx_dev)
            calls.append((
                ops.bind_decode_step(*step_args, scale=cfg.scale, num_units=units, workspace=ws,
                                     keep_cached=shared),
                ops.bind_decode_step(*step_args, cow_pairs=hp, scale=cfg.scale, num_units=units,
                                     workspace=ws, keep_cached=shared),
                None))
            continue
        write_args = dict(block_tables=tables, table_updates=hu, lens_in=hc, lens_out=ctx_dev)
        calls.append((
            ops.bind_append_tokens(spec, ks[n], vs[n], hs, cache.k, cache.v, **write_args),
            ops.bind_append_tokens(spec, ks[n], vs[n], hs, cache.k, cache.v, cow_pairs=hp,
                                   **write_args),
            ops.bind_decode(spec, out, qs[n], cache.k, cache.v, tables, ctx_dev, cfg.scale, units,
                            ws, keep_cached=shared)))

    def step(n, mode):
        """mode "warm": no timing events; "timed": events around the decode kernel
        (the kernel the roofline is taken on) on every 5th step; "profile": events
        around every launch.  A marker between the write and the decode launch delays
        the decode (measured: 2.3 us per step), so the other steps record at most the
        ring-slot event, after the decode."""
        h0 = time.perf_counter()
        # The step's metadata goes into pinned ring slot n % R, which the write kernel
        # reads in place; first wait until the launches of step n - R, its last user,
        # are done.
        r = n % R
        if n >= R:
            while ring_ev[0][0] < n - R:
                ring_ev.popleft()  # older than the slot's last user: covers nothing needed
            # the first event at or after step n - R (one is recorded at least every
            # EV_EVERY <= R steps); poll rather than block: a blocking wait may sleep
            # the thread, and a late wake-up leaves the GPU without work
            while not ring_ev[0][1].query():
                pass
        hw = time.perf_counter()
        # a1: host bookkeeping in the library allocator, which writes every sequence's
        # slot and copy-on-write pair straight into the ring slot
        st, done = binds[r]()
        if st != 0 or done != S:
            raise RuntimeError(f"append_batch failed at step {n}: status {st}")
        ctx_now[:] += 1
        ha = time.perf_counter()
        # a2: the rest of the step's metadata (lengths, table updates) into the slot
        ps, pc, pu, pp = pin_np[r]
        pc[:] = ctx_now
        pu[:, 0] = np.where(new_blocks >= 0, seq_ids, -1)  # (row, column, block); row -1 = no update
        pu[:, 1] = new_cols
        pu[:, 2] = new_blocks
        if upload:
            with torch.cuda.stream(copy_stream):
                dmeta[r].copy_(pin[r], non_blocking=True)
            ecp = torch.cuda.Event()
            ecp.record(copy_stream)
            stream.wait_event(ecp)
        h1 = time.perf_counter()
        plain, with_cow, decode = calls[n]
        append = with_cow if (pp[:, 0] >= 0).any() else plain  # (-1, -1) = no copy
        if decode is None:  # one launch: the step call does the writes and the decode
            append, decode = (lambda: None), append
        timing = mode == "profile" or (mode == "timed" and (n - warm) % 5 == 0)
        if timing:
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        if mode == "profile":
            e0.record(stream)
        # a3 + a4: copy-on-write block copies, the changed table entries, the cache
        # write of the step's new tokens and the context lengths (a launch of their
        # own with two launches per step)
        append()
        if timing:
            e1.record(stream)
        # a5-a11: decode attention, one kernel (gather + attention, split sequences
        # merged by the last of their pieces to finish)
        decode()
        if timing:
            e2.record(stream)
            ev[mode].append((e0, e1, e2, int(ctx_now.sum())))
        elif n % EV_EVERY == EV_EVERY - 1:
            e2 = torch.cuda.Event()
            e2.record(stream)
        else:
            e2 = None
        if e2 is not None:
            ring_ev.append((n, e2))  # slots of steps <= n are free once e2 has completed
        if mode == "timed":
            step_tok.append(int(ctx_now.sum()))
            # (allocator, waiting for the ring slot, staging the metadata, whole host side)
            host.append((ha - hw, hw - h0, h1 - ha, time.perf_counter() - h0))

    ev = {"timed": [], "profile": []}
    step_tok = []  # sum of context lengths of every timed step
    # A full collection of the interpreter's heap (hundreds of thousands of objects
    # once torch is imported) stalls the host for tens of milliseconds and leaves the
    # GPU without work; settle the heap now and keep the collector off while stepping.
    gc.collect()
    gc.freeze()
    gc.disable()
    for n in range(warm):
        step(n, "warm")
    torch.cuda.synchronize()
    log(f"warmup done ({warm} steps)")
    t0 = time.perf_counter()
    for n in range(warm, warm + steps):
        step(n, "timed")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {steps} steps in {wall * 1e3:.2f} ms")
    # untimed per-launch breakdown: events around every launch perturb the stream,
    # so they stay out of the timed region
    for n in range(warm + steps, total_steps):
        step(n, "profile")
    torch.cuda.synchronize()
    gc.enable()
    # Cold decode: the last step's decode run again (it reads the cache and writes
    # only its outputs, so nothing changes) after a 1 GiB pass, more than the 256 MB
    # MALL and every XCD's L2, so that its K/V come from HBM.  Two ways: right after
    # writing the buffer (the MALL then holds dirty lines that the decode's reads
    # evict and write back) and right after reading it (clean lines only).
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    flush.fill_(1.0)
    if one_launch:
        # the cold runs repeat the last step's attention with the plain decode call
        # (same kernel without the writes): the step itself would append again
        ws_cold = ops.decode_workspace(spec, Hq, units)
        last_decode = ops.bind_decode(spec, out, qs[total_steps - 1], cache.k, cache.v, tables,
                                      ctx_dev, cfg.scale, units, ws_cold, keep_cached=shared)
    else:
        last_decode = calls[total_steps - 1][2]
    cold = {"write": [], "read": []}
    for kind in ("write", "read"):
        for _ in range(5):
            if kind == "write":
                flush.fill_(1.0)
            else:
                flush.amax()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            last_decode()
            c1.record(stream)
            torch.cuda.synchronize()
            cold[kind].append(c0.elapsed_time(c1) * 1e-3)
    del flush
    cold_bytes = float(ctx_now.sum()) * kv_per_tok

    tok = np.array(step_tok, dtype=np.float64)  # every timed step
    kv_bytes = tok * kv_per_tok
    s_tok = np.array([e[3] for e in ev["timed"]], dtype=np.float64)  # the sampled steps
    s_bytes = s_tok * kv_per_tok
    t_dec = np.array([e[1].elapsed_time(e[2]) for e in ev["timed"]]) * 1e-3
    pe = ev["profile"]
    pbytes = np.array([e[3] for e in pe], dtype=np.float64) * kv_per_tok
    t_write = np.array([e[0].elapsed_time(e[1]) for e in pe]) * 1e-3
    t_attn = np.array([e[1].elapsed_time(e[2]) for e in pe]) * 1e-3
    value = float(kv_bytes.sum() / wall / 1e9)
    dec_gbps = float(np.median(s_bytes / t_dec) / 1e9)
    unique = None
    if cfg.ctx_kind == "shared_prefix":
        # Shared blocks are read by many sequences in one pass; count each physical
        # block once with the tokens it holds (the tables before the first step), plus
        # one private token per sequence for every step since (warm-up included).
        held = {}
        for i in range(S):
            L = int(ctx0[i])
            for kk in range(-(-L // B)):
                blk = int(tables_h[i, kk])
                held[blk] = max(held.get(blk, 0), min(B, L - kk * B))
        first = float(sum(held.values()))
        u_tok = first + S * (warm + 1 + np.arange(steps, dtype=np.float64))
        unique = {"note": "each physical block counted once, private appends added per step",
                  "unique_kv_bytes_first_timed_step": int(u_tok[0] * kv_per_tok),
                  "unique_gbps": round(float((u_tok * kv_per_tok).sum() / wall / 1e9), 2)}
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.title}", "seqs": S, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "block_size": B, "pool_blocks": cfg.num_blocks,
                   "sum_ctx_first_step": int(tok[0]), "units": units, "seed": cfg.seed,
                   "kv_loads": "cached (shared blocks)" if shared else "streamed (non-temporal)",
                   "step_launches": 1 if one_launch else 2,
                   "hip_force_dev_kernarg": os.environ.get("HIP_FORCE_DEV_KERNARG"),
                   "step_metadata": args.metadata},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "shared_prefix_unique": unique,
        "us_per_step": round(wall / steps * 1e6, 2),
        "breakdown": {
            "note": f"{len(pe)} untimed steps after the timed region, events around every launch",
            "device_us_per_step_median": round(float(np.median(t_write + t_attn)) * 1e6, 2),
            "write_us_median": round(float(np.median(t_write)) * 1e6, 2),
            "attn_us_median": round(float(np.median(t_attn)) * 1e6, 2),
            "attn_gbps_median": round(float(np.median(pbytes / t_attn) / 1e9), 2),
        },
        "cold_decode": {
            "note": "the last step's decode after a 1 GiB pass (MALL and L2 flushed), 5 runs each: "
                    "after writing the buffer (dirty lines written back during the decode) and "
                    "after reading it",
            "after_write_us_median": round(float(np.median(cold["write"])) * 1e6, 2),
            "after_write_gbps_median": round(cold_bytes / float(np.median(cold["write"])) / 1e9, 2),
            "after_read_us_median": round(float(np.median(cold["read"])) * 1e6, 2),
            "after_read_gbps_median": round(cold_bytes / float(np.median(cold["read"])) / 1e9, 2),
        },
        # useful matrix-core work of the grouped-query product (G > 1 runs on MFMA):
        # 4 Hq D flops per cached token, over the decode kernel's median time
        "mfma": ({"useful_tflops": round(4.0 * Hq * D * float(np.median(s_tok)) / float(np.median(t_dec)) / 1e12, 2),
                  "frac_of_bf16_peak": round(4.0 * Hq * D * float(np.median(s_tok)) / float(np.median(t_dec))
                                             / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
                 if Hq > Hkv and cfg.dtype == "bf16" else None),
        "host_bookkeeping_us_median": round(float(np.median([h[0] for h in host])) * 1e6, 2),
        "host_staging_us_median": round(float(np.median([h[2] for h in host])) * 1e6, 2),
        "host_ring_wait_us_median": round(float(np.median([h[1] for h in host])) * 1e6, 2),
        "host_step_us_median": round(float(np.median([h[3] for h in host])) * 1e6, 2),
        "host_step_us_max": round(float(np.max([h[3] for h in host])) * 1e6, 2),
        "host_note": "ring wait = waiting for the GPU to free the step's pinned ring slot (the "
                     "host runs ahead of the GPU); bookkeeping = the library allocator reserving "
                     "every sequence's next slot, its slots and copy-on-write pairs written "
                     "straight into the ring slot; staging = the rest of the step's metadata "
                     "(lengths, table updates) into the slot",
        "roofline": {
            "kernel": ("decode_pass1, decode-step form (the step's cache writes, gather + attention, "
                       "merge of split sequences, one cooperative launch)" if one_launch else
                       "decode_pass1 (gather + attention, merge of split sequences folded in)"),
            "bound": "hbm",
            "achieved": round(dec_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(cfg.name),
            "decode_us_mean": round(float(t_dec.mean()) * 1e6, 2),
            "decode_us_median": round(float(np.median(t_dec)) * 1e6, 2),
            "decode_us_max": round(float(np.max(t_dec)) * 1e6, 2),
            "timed_steps_sampled": len(t_dec),
            "note": "HIP events on the launch stream around the decode launch of every 5th timed "
                    "step; the interval starts at a marker after the write kernel, so it also holds "
                    "the dispatch gap before the decode (rocprofv3 kernel durations are in profiles/)",
            "algorithmic_bytes_per_launch": int(np.median(s_bytes)),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the batch")
        result["cpu_baseline"] = cpu_baseline(cfg, ctx0, q_host0, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    result["host"] = {"python": platform.python_version(), "torch": torch.__version__,
                      "device": torch.cuda.get_device_name(0)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

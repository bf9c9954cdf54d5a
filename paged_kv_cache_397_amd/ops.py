"""Device ops: thin wrappers that pass torch tensors' device pointers and the
current HIP stream to libpagedkv.  Every computation runs in the library's HIP
kernels; these functions only check shapes/dtypes and marshal arguments.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _native as N

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_PA_DTYPE = {"f32": 0, "bf16": 1}


@dataclass(frozen=True)
class CacheSpec:
    """Shape of one paged KV cache (see the layout contract in include/pagedkv.h)."""
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" | "f32"

    def desc(self) -> N.CacheDesc:
        return N.CacheDesc(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim,
                           _PA_DTYPE[self.dtype])

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    @property
    def elems(self) -> int:
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _acc(t: torch.Tensor, name: str, dtype=None):
    """Device pointer of a tensor the GPU may read: a GPU tensor or pinned host memory."""
    if t.is_cuda:
        return _dev(t, name, dtype)
    if not t.is_pinned():
        raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def cache_bytes(spec: CacheSpec) -> int:
    return int(N.lib().pa_cache_bytes(ctypes.byref(spec.desc())))


def empty_cache(spec: CacheSpec, device="cuda"):
    """Uninitialised K and V cache arrays (flat, spec.elems elements each)."""
    k = torch.empty(spec.elems, dtype=spec.torch_dtype, device=device)
    v = torch.empty(spec.elems, dtype=spec.torch_dtype, device=device)
    return k, v


def reshape_and_cache(spec: CacheSpec, k, v, slot_mapping, k_cache, v_cache, stream=None):
    """Write k[t], v[t] ([T, Hkv, D]) into slot slot_mapping[t] (int64, -1 = skip)."""
    T = slot_mapping.numel()
    if tuple(k.shape) != (T, spec.num_kv_heads, spec.head_dim) or k.shape != v.shape:
        raise ValueError("k and v must be [T, Hkv, D]")
    st = N.lib().pa_reshape_and_cache(
        ctypes.byref(spec.desc()), _dev(k, "k", spec.torch_dtype), _dev(v, "v", spec.torch_dtype),
        _dev(slot_mapping, "slot_mapping", torch.int64), T,
        _dev(k_cache, "k_cache", spec.torch_dtype), _dev(v_cache, "v_cache", spec.torch_dtype),
        _stream(stream))
    N.check(st, "pa_reshape_and_cache")


def copy_blocks(spec: CacheSpec, k_cache, v_cache, pairs, stream=None):
    """Copy block src onto dst for each row (src, dst) of pairs ([n, 2] int32)."""
    n = pairs.shape[0] if pairs.dim() == 2 else pairs.numel() // 2
    st = N.lib().pa_copy_blocks(
        ctypes.byref(spec.desc()), _dev(k_cache, "k_cache", spec.torch_dtype),
        _dev(v_cache, "v_cache", spec.torch_dtype), _dev(pairs, "pairs", torch.int32), n,
        _stream(stream))
    N.check(st, "pa_copy_blocks")


def host_pool(spec: CacheSpec, num_blocks: int):
    """Pinned host K and V arrays for a swap pool of num_blocks blocks of spec's geometry."""
    n = num_blocks * spec.num_kv_heads * spec.block_size * spec.head_dim
    return (torch.empty(n, dtype=spec.torch_dtype, pin_memory=True),
            torch.empty(n, dtype=spec.torch_dtype, pin_memory=True))


def swap_blocks(spec: CacheSpec, src_k, src_v, dst_k, dst_v, pairs, stream=None):
    """Copy block pairs[i, 0] of (src_k, src_v) onto block pairs[i, 1] of (dst_k, dst_v);
    either pool may be a GPU tensor or pinned host memory, as may pairs ([n, 2] int32)."""
    n = pairs.shape[0] if pairs.dim() == 2 else pairs.numel() // 2
    per = spec.num_kv_heads * spec.block_size * spec.head_dim
    st = N.lib().pa_swap_blocks(
        ctypes.byref(spec.desc()), _acc(src_k, "src_k", spec.torch_dtype),
        _acc(src_v, "src_v", spec.torch_dtype), src_k.numel() // per,
        _acc(dst_k, "dst_k", spec.torch_dtype), _acc(dst_v, "dst_v", spec.torch_dtype),
        dst_k.numel() // per, _acc(pairs, "pairs", torch.int32), n, _stream(stream))
    N.check(st, "pa_swap_blocks")


def _append_args(spec, k, v, slot_mapping, k_cache, v_cache, cow_pairs, block_tables,
                 table_updates, lens_in, lens_out, stream):
    T = slot_mapping.numel()
    if tuple(k.shape) != (T, spec.num_kv_heads, spec.head_dim) or k.shape != v.shape:
        raise ValueError("k and v must be [T, Hkv, D]")
    if cow_pairs is not None and cow_pairs.numel() != 2 * T:
        raise ValueError("cow_pairs must be [T, 2]")
    n_upd = 0 if table_updates is None else table_updates.numel() // 3
    rows, cols = (0, 0) if block_tables is None else tuple(block_tables.shape)
    n_lens = 0 if lens_in is None else lens_in.numel()
    if n_lens and (lens_out is None or lens_out.numel() < n_lens):
        raise ValueError("lens_out must hold lens_in")
    return (ctypes.byref(spec.desc()), _dev(k, "k", spec.torch_dtype),
            _dev(v, "v", spec.torch_dtype), _acc(slot_mapping, "slot_mapping", torch.int64),
            None if cow_pairs is None else _acc(cow_pairs, "cow_pairs", torch.int32), T,
            _dev(k_cache, "k_cache", spec.torch_dtype), _dev(v_cache, "v_cache", spec.torch_dtype),
            None if block_tables is None else _dev(block_tables, "block_tables", torch.int32),
            rows, cols,
            None if n_upd == 0 else _acc(table_updates, "table_updates", torch.int32), n_upd,
            None if n_lens == 0 else _acc(lens_in, "lens_in", torch.int32),
            None if n_lens == 0 else _dev(lens_out, "lens_out", torch.int32), n_lens,
            _stream(stream))


def append_tokens(spec: CacheSpec, k, v, slot_mapping, k_cache, v_cache, cow_pairs=None,
                  block_tables=None, table_updates=None, lens_in=None, lens_out=None,
                  stream=None):
    """A decode step's writes: copy-on-write copies (cow_pairs [T, 2], row t for
    token t, -1 = none; they run as a launch of their own first, so pass None when
    the step copies nothing), table updates ([n, 3] rows (row, column, block)), the
    scatter of k[t], v[t] ([T, Hkv, D]) into slot_mapping[t], and lens_out[:] =
    lens_in.  slot_mapping, cow_pairs, table_updates and lens_in may be pinned host
    tensors."""
    args = _append_args(spec, k, v, slot_mapping, k_cache, v_cache, cow_pairs, block_tables,
                        table_updates, lens_in, lens_out, stream)
    N.check(N.lib().pa_append_tokens(*args), "pa_append_tokens")


def update_block_tables(block_tables, updates, stream=None):
    """Apply (row, column, block) rows of updates ([n, 3] int32) to block_tables."""
    rows, cols = block_tables.shape
    n = updates.shape[0] if updates.dim() == 2 else updates.numel() // 3
    st = N.lib().pa_update_block_tables(
        _dev(block_tables, "block_tables", torch.int32), rows, cols,
        _dev(updates, "updates", torch.int32), n, _stream(stream))
    N.check(st, "pa_update_block_tables")


def default_units() -> int:
    return int(N.lib().pa_decode_default_units())


def decode_workspace_bytes(spec: CacheSpec, num_q_heads: int, num_units: int = 0) -> int:
    n = int(N.lib().pa_decode_workspace_bytes(ctypes.byref(spec.desc()), num_q_heads, num_units))
    if n == 0:
        raise N.PagedKVError(N.PA_ERR_INVALID_ARG, "pa_decode_workspace_bytes")
    return n


def decode_workspace(spec: CacheSpec, num_q_heads: int, num_units: int = 0, device="cuda"):
    """Zero-filled once: the single-call decode needs its split counts at zero before
    its first use (every completed call leaves them zero again)."""
    return torch.zeros(decode_workspace_bytes(spec, num_q_heads, num_units), dtype=torch.uint8,
                       device=device)


DECODE_KEEP_CACHED = 1  # PA_DECODE_KEEP_CACHED


def _decode(fn: str, spec: CacheSpec, out, q, k_cache, v_cache, block_tables, context_lens,
            scale, num_units, workspace, stream, keep_cached=False):
    S, Hq, D = q.shape
    if D != spec.head_dim or tuple(out.shape) != (S, Hq, D):
        raise ValueError("q and out must be [S, Hq, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, maxB] and context_lens [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = decode_workspace(spec, Hq, num_units, q.device)
    st = getattr(N.lib(), fn)(
        ctypes.byref(spec.desc()), _dev(out, "out", spec.torch_dtype),
        _dev(q, "q", spec.torch_dtype), _dev(k_cache, "k_cache", spec.torch_dtype),
        _dev(v_cache, "v_cache", spec.torch_dtype),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, block_tables.shape[1],
        float(scale), int(num_units), _dev(workspace, "workspace"), workspace.numel(),
        DECODE_KEEP_CACHED if keep_cached else 0, _stream(stream))
    N.check(st, fn)
    return out


def paged_attn_decode(spec: CacheSpec, out, q, k_cache, v_cache, block_tables, context_lens,
                      scale: float | None = None, num_units: int = 0, workspace=None,
                      stream=None, keep_cached: bool = False):
    """out[i, j] = softmax attention of q[i, j] over sequence i's cached tokens."""
    return _decode("pa_paged_attn_decode", spec, out, q, k_cache, v_cache, block_tables,
                   context_lens, scale, num_units, workspace, stream, keep_cached)


def paged_attn_decode_partial(spec: CacheSpec, out, q, k_cache, v_cache, block_tables,
                              context_lens, scale: float | None = None, num_units: int = 0,
                              workspace=None, stream=None, keep_cached: bool = False):
    """First kernel of paged_attn_decode (needs the same workspace in the merge)."""
    if workspace is None:
        raise ValueError("the partial/merge split needs an explicit shared workspace")
    return _decode("pa_paged_attn_decode_partial", spec, out, q, k_cache, v_cache, block_tables,
                   context_lens, scale, num_units, workspace, stream, keep_cached)


def paged_attn_decode_merge(spec: CacheSpec, out, q, k_cache, v_cache, block_tables,
                            context_lens, scale: float | None = None, num_units: int = 0,
                            workspace=None, stream=None, keep_cached: bool = False):
    """Second kernel of paged_attn_decode: merges the partial records of split sequences."""
    if workspace is None:
        raise ValueError("the partial/merge split needs an explicit shared workspace")
    return _decode("pa_paged_attn_decode_merge", spec, out, q, k_cache, v_cache, block_tables,
                   context_lens, scale, num_units, workspace, stream, keep_cached)


def decode_step_workspace(spec: CacheSpec, num_q_heads: int, num_seqs: int, num_units: int = 0,
                          device="cuda"):
    """Zero-filled workspace of a decode step (it also serves paged_attn_decode)."""
    n = int(N.lib().pa_decode_step_workspace_bytes(ctypes.byref(spec.desc()), num_q_heads,
                                                   num_units, num_seqs))
    if n == 0:
        raise N.PagedKVError(N.PA_ERR_INVALID_ARG, "pa_decode_step_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _step_args(spec, out, q, k_new, v_new, slot_mapping, cow_pairs, lens_in, k_cache, v_cache,
               block_tables, context_lens, scale, num_units, workspace, stream, keep_cached):
    S, Hq, D = q.shape
    if D != spec.head_dim or tuple(out.shape) != (S, Hq, D):
        raise ValueError("q and out must be [S, Hq, D]")
    if tuple(k_new.shape) != (S, spec.num_kv_heads, D) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [S, Hkv, D]")
    if slot_mapping.numel() != S or lens_in.numel() != S or context_lens.numel() != S:
        raise ValueError("slot_mapping, lens_in and context_lens must hold one entry per sequence")
    if cow_pairs is not None and cow_pairs.numel() != 2 * S:
        raise ValueError("cow_pairs must be [S, 2]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, maxB]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    desc = spec.desc()
    return desc, (
        ctypes.byref(desc), _dev(out, "out", spec.torch_dtype), _dev(q, "q", spec.torch_dtype),
        _dev(k_new, "k_new", spec.torch_dtype), _dev(v_new, "v_new", spec.torch_dtype),
        _acc(slot_mapping, "slot_mapping", torch.int64),
        None if cow_pairs is None else _acc(cow_pairs, "cow_pairs", torch.int32),
        _acc(lens_in, "lens_in", torch.int32), _dev(k_cache, "k_cache", spec.torch_dtype),
        _dev(v_cache, "v_cache", spec.torch_dtype),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, block_tables.shape[1],
        ctypes.c_float(scale), int(num_units), _dev(workspace, "workspace"), workspace.numel(),
        DECODE_KEEP_CACHED if keep_cached else 0, _stream(stream))


def decode_step(spec: CacheSpec, out, q, k_new, v_new, slot_mapping, lens_in, k_cache, v_cache,
                block_tables, context_lens, cow_pairs=None, scale: float | None = None,
                num_units: int = 0, workspace=None, stream=None, keep_cached: bool = False):
    """One decode step in one launch: sequence i's new token (k_new[i], v_new[i]) is
    written at slot_mapping[i] (after the copy cow_pairs[i], if any), block_tables and
    context_lens are updated for it (context_lens = lens_in), and out is decode
    attention over every cached token, the new ones included.  slot_mapping,
    cow_pairs and lens_in may be pinned host tensors."""
    if workspace is None:
        workspace = decode_step_workspace(spec, q.shape[1], q.shape[0], num_units, q.device)
    _, args = _step_args(spec, out, q, k_new, v_new, slot_mapping, cow_pairs, lens_in, k_cache,
                         v_cache, block_tables, context_lens, scale, num_units, workspace, stream,
                         keep_cached)
    N.check(N.lib().pa_decode_step(*args), "pa_decode_step")
    return out


def bind_decode_step(spec: CacheSpec, out, q, k_new, v_new, slot_mapping, lens_in, k_cache,
                     v_cache, block_tables, context_lens, cow_pairs=None,
                     scale: float | None = None, num_units: int = 0, workspace=None, stream=None,
                     keep_cached: bool = False) -> "BoundCall":
    """decode_step with its arguments fixed (same meaning as decode_step)."""
    if workspace is None:
        raise ValueError("a bound decode step needs an explicit workspace")
    desc, args = _step_args(spec, out, q, k_new, v_new, slot_mapping, cow_pairs, lens_in, k_cache,
                            v_cache, block_tables, context_lens, scale, num_units, workspace,
                            stream, keep_cached)
    return BoundCall("pa_decode_step", args, keep=desc)


def paged_attn_decode_noalloc(spec: CacheSpec, out, q, k_cache, v_cache, block_tables,
                              context_lens, scale: float | None = None, num_units: int = 0,
                              stream=None, keep_cached: bool = False):
    """paged_attn_decode without a workspace: the library's static per-GPU scratch
    buffer serves instead (PA_ERR_TOO_LARGE when the request needs more than it
    holds).  Calls that overlap in time on one GPU race."""
    S, Hq, D = q.shape
    if D != spec.head_dim or tuple(out.shape) != (S, Hq, D):
        raise ValueError("q and out must be [S, Hq, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, maxB] and context_lens [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = N.lib().pa_paged_attn_decode_noalloc(
        ctypes.byref(spec.desc()), _dev(out, "out", spec.torch_dtype),
        _dev(q, "q", spec.torch_dtype), _dev(k_cache, "k_cache", spec.torch_dtype),
        _dev(v_cache, "v_cache", spec.torch_dtype),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, block_tables.shape[1],
        float(scale), int(num_units), DECODE_KEEP_CACHED if keep_cached else 0, _stream(stream))
    N.check(st, "pa_paged_attn_decode_noalloc")
    return out


def paged_attn_prefill(spec: CacheSpec, out, q, k_cache, v_cache, block_tables, query_start,
                       context_lens, scale: float | None = None, max_query_len: int | None = None,
                       stream=None):
    """Chunked-prefill attention: rows query_start[s] .. query_start[s+1]-1 of q are the
    last tokens of sequence s's cache (context_lens[s] tokens, the chunk included), and
    each attends causally to its own position and every earlier one.

    query_start and context_lens are int32 GPU tensors.  max_query_len bounds every
    chunk length; when it is None it is read from query_start (a device-to-host copy,
    which synchronises: pass it in a serving loop)."""
    T, Hq, D = q.shape
    if D != spec.head_dim or tuple(out.shape) != (T, Hq, D):
        raise ValueError("q and out must be [T, Hq, D]")
    S = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise ValueError("block_tables must be [S, maxB], query_start [S + 1], context_lens [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if S else 0
    st = N.lib().pa_paged_attn_prefill(
        ctypes.byref(spec.desc()), _dev(out, "out", spec.torch_dtype),
        _dev(q, "q", spec.torch_dtype), _dev(k_cache, "k_cache", spec.torch_dtype),
        _dev(v_cache, "v_cache", spec.torch_dtype),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(query_start, "query_start", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, T, Hq, block_tables.shape[1],
        int(max_query_len), float(scale), _stream(stream))
    N.check(st, "pa_paged_attn_prefill")
    return out


class BoundCall:
    """A library call with every argument converted once, for tight serving loops:
    calling it costs one foreign-function call and a status check.  The buffers it
    names must outlive it; the stream is captured at bind time."""

    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, name: str, args, keep=None):
        self._name = name
        self._fn = getattr(N.lib(), name)
        self._args = tuple(args)
        self._keep = keep  # objects the converted arguments point into (the descriptor)

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            N.check(st, self._name)


def bind_reshape_and_cache(spec: CacheSpec, k, v, slot_mapping, k_cache, v_cache,
                           stream=None) -> BoundCall:
    """reshape_and_cache with its arguments fixed (same meaning as reshape_and_cache)."""
    T = slot_mapping.numel()
    if tuple(k.shape) != (T, spec.num_kv_heads, spec.head_dim) or k.shape != v.shape:
        raise ValueError("k and v must be [T, Hkv, D]")
    desc = spec.desc()
    return BoundCall("pa_reshape_and_cache", (
        ctypes.byref(desc), _dev(k, "k", spec.torch_dtype), _dev(v, "v", spec.torch_dtype),
        _dev(slot_mapping, "slot_mapping", torch.int64), T,
        _dev(k_cache, "k_cache", spec.torch_dtype), _dev(v_cache, "v_cache", spec.torch_dtype),
        _stream(stream)), keep=desc)


def bind_append_tokens(spec: CacheSpec, k, v, slot_mapping, k_cache, v_cache, cow_pairs=None,
                       block_tables=None, table_updates=None, lens_in=None, lens_out=None,
                       stream=None) -> BoundCall:
    """append_tokens with its arguments fixed (same meaning as append_tokens)."""
    args = _append_args(spec, k, v, slot_mapping, k_cache, v_cache, cow_pairs, block_tables,
                        table_updates, lens_in, lens_out, stream)
    return BoundCall("pa_append_tokens", args, keep=args[0])


def bind_decode(spec: CacheSpec, out, q, k_cache, v_cache, block_tables, context_lens,
                scale: float | None, num_units: int, workspace, stage: str = "both",
                stream=None, keep_cached: bool = False) -> BoundCall:
    """paged_attn_decode (stage "both"), or its first ("partial") or second ("merge")
    kernel, with its arguments fixed."""
    fn = {"both": "pa_paged_attn_decode", "partial": "pa_paged_attn_decode_partial",
          "merge": "pa_paged_attn_decode_merge"}[stage]
    S, Hq, D = q.shape
    if D != spec.head_dim or tuple(out.shape) != (S, Hq, D):
        raise ValueError("q and out must be [S, Hq, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S, maxB] and context_lens [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    desc = spec.desc()
    return BoundCall(fn, (
        ctypes.byref(desc), _dev(out, "out", spec.torch_dtype), _dev(q, "q", spec.torch_dtype),
        _dev(k_cache, "k_cache", spec.torch_dtype), _dev(v_cache, "v_cache", spec.torch_dtype),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, block_tables.shape[1],
        ctypes.c_float(scale), int(num_units), _dev(workspace, "workspace"), workspace.numel(),
        DECODE_KEEP_CACHED if keep_cached else 0, _stream(stream)), keep=desc)

"""Seeded random draws for the paged-decode workloads.

Every array comes from ``numpy.random.default_rng([seed, tag, ...])`` so that a
piece of data (one sequence's keys and values, one step's queries) can be
regenerated on its own, in any order, and always gives the same bits.  Values
are standard normal; bf16 data is the float32 draw rounded to nearest-even and
returned as raw ``uint16`` bit patterns, float32 data is returned as float32.
"""

from __future__ import annotations

import functools

import numpy as np

# Sub-stream tags: the second word of every seed sequence.
TAG_CTX = 1      # context lengths
TAG_PERM = 2     # permutation of the physical block pool (free-list order)
TAG_Q = 3        # queries, per decode step
TAG_KV = 4       # per-sequence key/value history, per token position
TAG_NEW = 5      # keys/values of the tokens written by a decode step
TAG_TRACE = 6    # arrivals / prompt lengths / output lengths of a serving trace

DTYPES = ("f32", "bf16")


def stream(seed: int, *tags: int) -> np.random.Generator:
    """Independent generator for (seed, tags...)."""
    return np.random.default_rng([int(seed), *[int(t) for t in tags]])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16, nearest-even; return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs stay below 0xFF800000, so the sum cannot wrap in 32 bits
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Standard-normal draw in the storage format of ``dtype``."""
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else bf16_bits_from_f32(x)


def seq_kv(seed: int, seq: int, ctx: int, num_kv_heads: int, head_dim: int,
           dtype: str):
    """Keys and values of tokens 0..ctx-1 of sequence ``seq``: two [ctx, Hkv, D].

    The draw is prefix-stable: token p has the same value whatever ``ctx`` is,
    so a sequence that grows (or is recomputed after preemption) rewrites the
    same bits at the same positions.
    """
    rng = stream(seed, TAG_KV, seq)
    kv = draw_values(rng, (ctx, 2, num_kv_heads, head_dim), dtype)
    return np.ascontiguousarray(kv[:, 0]), np.ascontiguousarray(kv[:, 1])


def new_tokens(seed: int, step: int, num_tokens: int, num_kv_heads: int,
               head_dim: int, dtype: str):
    """Keys and values of the tokens a decode step writes: two [T, Hkv, D]."""
    rng = stream(seed, TAG_NEW, step)
    kv = draw_values(rng, (num_tokens, 2, num_kv_heads, head_dim), dtype)
    return np.ascontiguousarray(kv[:, 0]), np.ascontiguousarray(kv[:, 1])


def q_values(seed: int, step: int, num_seqs: int, num_q_heads: int,
             head_dim: int, dtype: str) -> np.ndarray:
    """Queries of one decode step: [S, Hq, D]."""
    return draw_values(stream(seed, TAG_Q, step), (num_seqs, num_q_heads, head_dim), dtype)


def context_lens_uniform(seed: int, num_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths uniform on the integers [lo, hi] (int32)."""
    return stream(seed, TAG_CTX).integers(lo, hi + 1, num_seqs).astype(np.int32)


def context_lens_loguniform(seed: int, num_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths log-uniform on [lo, hi], rounded to integers (int32)."""
    u = stream(seed, TAG_CTX).uniform(np.log(lo), np.log(hi), num_seqs)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


def pool_permutation(seed: int, num_blocks: int) -> np.ndarray:
    """A seeded permutation of the physical block IDs 0..N-1 (int32)."""
    return stream(seed, TAG_PERM).permutation(num_blocks).astype(np.int32)


# ----------------------------------------------------------------------------- serving trace

TAG_TRACE_KV = 7   # keys/values of one token of one request of a serving trace
TAG_TRACE_Q = 8    # query of one decode step of one request of a serving trace


def trace_arrivals(seed: int, step: int, mean: float, prompt_lo: int, prompt_hi: int,
                   out_p: float, out_lo: int, out_hi: int):
    """Requests arriving at one step of a serving trace: Poisson(mean) of them, each
    with a prompt length uniform on [prompt_lo, prompt_hi] and an output length
    geometric(out_p) clipped to [out_lo, out_hi].  Returns (prompts, outputs)."""
    rng = stream(seed, TAG_TRACE, step)
    count = int(rng.poisson(mean))
    prompts = rng.integers(prompt_lo, prompt_hi + 1, count)
    outs = np.clip(rng.geometric(out_p, count), out_lo, out_hi)
    return prompts.astype(np.int64), outs.astype(np.int64)


def trace_token_kv(seed: int, req: int, positions, num_kv_heads: int, head_dim: int,
                   dtype: str):
    """Keys and values of tokens `positions` of request `req`: two [len, Hkv, D].

    Each token's values depend only on (seed, req, position), so a request that is
    preempted and prefilled again rewrites exactly the same bits."""
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    k = np.empty((len(positions), num_kv_heads, head_dim), dtype=np.float32 if dtype == "f32" else np.uint16)
    v = np.empty_like(k)
    for i, p in enumerate(positions.tolist()):
        kv = draw_values(stream(seed, TAG_TRACE_KV, req, p), (2, num_kv_heads, head_dim), dtype)
        k[i], v[i] = kv[0], kv[1]
    return k, v


def trace_query(seed: int, req: int, position: int, num_q_heads: int, head_dim: int,
                dtype: str) -> np.ndarray:
    """Query [Hq, D] of request `req` at the decode step that writes `position`."""
    return draw_values(stream(seed, TAG_TRACE_Q, req, position), (num_q_heads, head_dim), dtype)


# ----------------------------------------------------------------------------- shared prompt openings

TAG_TOKEN_KV = 9    # per-token and per-position tables of content-addressed keys/values
TAG_PROMPTS = 10    # token IDs of the prompts of a serving trace with shared openings
TAG_GEN_TOKEN = 11  # token IDs a request generates


@functools.lru_cache(maxsize=4)
def _token_kv_tables(seed: int, num_kv_heads: int, head_dim: int, vocab: int, max_pos: int):
    shape = (2, num_kv_heads, head_dim)
    tok_t = stream(seed, TAG_TOKEN_KV, 0).standard_normal((vocab, *shape), dtype=np.float32)
    pos_t = stream(seed, TAG_TOKEN_KV, 1).standard_normal((max_pos, *shape), dtype=np.float32)
    return tok_t, pos_t


def token_kv(seed: int, tokens, start: int, num_kv_heads: int, head_dim: int, dtype: str,
             vocab: int = 64, max_pos: int = 8192):
    """Keys and values of `tokens` at positions start, start+1, ...: two [n, Hkv, D].

    A token's values depend only on (seed, token ID, position) - a per-token draw
    plus a per-position draw, summed in float32 and rounded once - so prompts that
    share an opening hold identical bits there, as a model's cache would."""
    tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
    pos = start + np.arange(len(tokens))
    if len(tokens) and (tokens.min() < 0 or tokens.max() >= vocab or pos[-1] >= max_pos):
        raise ValueError("token or position outside the tables")
    tok_t, pos_t = _token_kv_tables(seed, num_kv_heads, head_dim, vocab, max_pos)
    x = (tok_t[tokens] + pos_t[pos]) * np.float32(0.7071067811865476)
    x = x if dtype == "f32" else bf16_bits_from_f32(x)
    return x[:, 0], x[:, 1]


def shared_opening_prompts(seed: int, step: int, count: int, openings: int, open_lo: int,
                           open_hi: int, suffix_lo: int, suffix_hi: int, vocab: int):
    """Token IDs of `count` prompts arriving at one step: each is one of `openings`
    fixed openings (a system prompt, its length uniform on [open_lo, open_hi] and
    drawn once per trace) followed by a private suffix of uniform length."""
    lens = stream(seed, TAG_PROMPTS, 0).integers(open_lo, open_hi + 1, openings)
    heads = [stream(seed, TAG_PROMPTS, 1, k).integers(0, vocab, int(lens[k])) for k in range(openings)]
    rng = stream(seed, TAG_PROMPTS, 2, step)
    out = []
    for _ in range(count):
        k = int(rng.integers(0, openings))
        tail = rng.integers(0, vocab, int(rng.integers(suffix_lo, suffix_hi + 1)))
        out.append(np.concatenate([heads[k], tail]).astype(np.int32))
    return out


_M64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    """One output of the SplitMix64 generator (Steele, Lea and Flood) for state x."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def generated_token(seed: int, req: int, position: int, vocab: int) -> int:
    """Token ID request `req` produces at `position` (a counter-based draw: cheap
    enough to call once per generated token)."""
    x = _splitmix64((int(seed) << 48) ^ (TAG_GEN_TOKEN << 40) ^ (int(req) << 20) ^ int(position))
    return int(x % vocab)


def generated_tokens(seed: int, req: int, first: int, count: int, vocab: int) -> np.ndarray:
    """generated_token for positions first .. first + count - 1, as int32 (the same
    SplitMix64 output, computed on uint64 arrays)."""
    with np.errstate(over="ignore"):
        pos = np.arange(first, first + count, dtype=np.uint64)
        z = (np.uint64((int(seed) << 48) ^ (TAG_GEN_TOKEN << 40) ^ (int(req) << 20)) ^ pos)
        z = z + np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return (z % np.uint64(vocab)).astype(np.int32)


# ----------------------------------------------------------------------------- full-size serving-trace values

TAG_TRACE_TABLE = 12   # value tables of the full-size trace parity runs
_TABLE_ROWS = 4093     # a prime: a request's positions 0 .. 4092 land on distinct rows


@functools.lru_cache(maxsize=2)
def _trace_value_table(seed: int, which: int, width: int, dtype: str) -> np.ndarray:
    return draw_values(stream(seed, TAG_TRACE_TABLE, which, width), (_TABLE_ROWS, width), dtype)


def trace_table_rows(req: int, positions) -> np.ndarray:
    """Table rows of tokens `positions` of request `req`: (7919 req + 104729 p) mod 4093.
    Distinct positions of one request (fewer than 4093 apart) get distinct rows."""
    p = np.asarray(positions, dtype=np.int64).reshape(-1)
    return (7919 * int(req) + 104729 * p) % _TABLE_ROWS


def trace_table_kv(seed: int, req: int, positions, num_kv_heads: int, head_dim: int,
                   dtype: str):
    """Keys and values of tokens `positions` of request `req`, two [len, Hkv, D], read
    from one seeded table of 4093 standard-normal rows (a row holds a token's K and
    V).  A cheap stand-in for per-token draws at the full trace sizes: a token's
    values depend only on (seed, req, position), so a recomputed prompt rewrites
    the same bits; tokens of different requests may share a row."""
    t = _trace_value_table(seed, 0, 2 * num_kv_heads * head_dim, dtype)
    x = t[trace_table_rows(req, positions)].reshape(-1, 2, num_kv_heads, head_dim)
    return np.ascontiguousarray(x[:, 0]), np.ascontiguousarray(x[:, 1])


def trace_table_query(seed: int, reqs, positions, num_q_heads: int, head_dim: int,
                      dtype: str) -> np.ndarray:
    """Queries [n, Hq, D] of requests `reqs` at the decode steps that write
    `positions`, from a second seeded table of the same kind."""
    t = _trace_value_table(seed, 1, num_q_heads * head_dim, dtype)
    rows = np.array([trace_table_rows(r, [p])[0] for r, p in zip(reqs, positions)], dtype=np.int64)
    return t[rows].reshape(-1, num_q_heads, head_dim)

"""Oracle decode attention: gather, then textbook softmax attention in float64.

Test infrastructure only.  What it follows:

* Decode runs one forward step per new token, and each step's attention looks
  back at the keys and values of every earlier token of the sequence, which is
  why they are cached (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
  Batching原理与实践", section 2 and 2.1).
* With paging, the kernel collects a sequence's scattered physical blocks into
  one temporary logical view before computing attention (same page, 2.2).  The
  oracle does exactly that: it materialises the view with its own layout reader
  (``oracle.layout``) and then computes plain softmax attention over it.
* Batches are ragged: every sequence has its own length (same page, 2.3, item 3);
  only the first ``context_lens[i]`` tokens of sequence i take part.

Readings where the pages are silent (listed with the others in the design notes):
query head j reads KV head j // G with G = Hq / Hkv; the score is
``scale * <q, k>``; no causal / sliding / ALiBi mask (one query attends to all
cached tokens); a sequence with no cached tokens gets an all-zero output.

Pins: torch's CPU float64 ``scaled_dot_product_attention`` on the same gathered
inputs; closed forms (one token returns its value row; constant values return
that constant; a zero query averages the values; two tokens give the logistic
weighting); invariance under permuting physical block IDs, identity vs scattered
tables, and shared vs private prefix blocks.

Prefill (chunked).  The prompt is processed before decoding starts, all of its
tokens in one pass (ksqn.cn page, section 2); a long prompt is written in chunks
(the scheduling readings in ``oracle.scheduler_model``).  Generation is
autoregressive: a token's attention looks at itself and the tokens before it,
never after it (same page, 2.1).  Reading where the pages are silent: a chunk of
c query tokens belongs to a sequence whose cache already holds L tokens with the
chunk's own keys and values among them (written before the attention call), so
chunk token i sits at position L - c + i and attends to cache positions
0 .. L - c + i.  Pins: torch's float64 SDPA with an explicit causal mask offset by
the chunk start; a position-0 token returns its value row; a zero query gives
the running mean of the values; any cut of a prompt into chunks gives the same
rows; a chunk's last row equals decode attention over the whole cache.
"""

from __future__ import annotations

import numpy as np

from .layout import CacheLayout, to_float64


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query token over L cached tokens, float64.

    q: [Hq, D]; K, V: [L, Hkv, D] (any real dtype, promoted to float64).
    Returns [Hq, D] float64.  L == 0 gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    G = Hq // Hkv
    for j in range(Hq):
        h = j // G
        s = scale * (K[:, h, :] @ q[j])       # one score per cached token
        p = np.exp(s - s.max())               # softmax numerator (max-shifted)
        out[j] = (p @ V[:, h, :]) / p.sum()   # weighted sum of the value rows
    return out


def paged_decode(layout: CacheLayout, q, k_cache, v_cache, block_tables, context_lens,
                 scale: float) -> np.ndarray:
    """Decode attention for a ragged batch stored in a paged cache.

    q: [S, Hq, D] in storage format; caches: flat arrays in storage format;
    block_tables: [S, maxB] int; context_lens: [S] int.
    Only table columns < ceil(L / B) are read.  Returns [S, Hq, D] float64.
    """
    q = np.asarray(q)
    S, Hq, D = q.shape
    B = layout.block_size
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for i in range(S):
        L = int(context_lens[i])
        if L == 0:
            continue
        nb = -(-L // B)
        K, V = layout.gather(k_cache, v_cache, np.asarray(block_tables[i][:nb]), L)
        out[i] = decode_attention(to_float64(q[i], layout.dtype),
                                  to_float64(K, layout.dtype),
                                  to_float64(V, layout.dtype), scale)
    return out


def contiguous_decode(q, K, V, scale: float, dtype: str) -> np.ndarray:
    """Decode attention of one sequence from its logical (unpaged) K/V.

    q: [Hq, D]; K, V: [L, Hkv, D], all in storage format.  Paging only changes
    where the bytes live, so this is the expected output for a sequence whose
    tokens were written into any set of blocks.
    """
    return decode_attention(to_float64(q, dtype), to_float64(K, dtype),
                            to_float64(V, dtype), scale)


def prefill_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                      start: int) -> np.ndarray:
    """Causal attention of a chunk of c query tokens at positions start .. start+c-1.

    q: [c, Hq, D]; K, V: [L, Hkv, D] with L >= start + c (the chunk's own keys and
    values included).  Row i attends to keys 0 .. start + i.  Returns [c, Hq, D]
    float64.
    """
    q = np.asarray(q, dtype=np.float64)
    c = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(c):
        n = start + i + 1          # keys visible to row i: itself and everything before
        out[i] = decode_attention(q[i], K[:n], V[:n], scale)
    return out


def paged_prefill(layout: CacheLayout, q, k_cache, v_cache, block_tables, query_start,
                  context_lens, scale: float) -> np.ndarray:
    """Chunked-prefill attention for a ragged batch stored in a paged cache.

    q: [T, Hq, D] in storage format, the chunks of all sequences one after another;
    sequence s owns rows query_start[s] .. query_start[s+1]-1 (c_s rows) and holds
    context_lens[s] >= c_s tokens in the cache, its chunk last.  Returns [T, Hq, D]
    float64.
    """
    q = np.asarray(q)
    T = q.shape[0]
    B = layout.block_size
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(len(context_lens)):
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        c, L = r1 - r0, int(context_lens[s])
        if c == 0:
            continue
        assert 0 < c <= L and r1 <= T
        nb = -(-L // B)
        K, V = layout.gather(k_cache, v_cache, np.asarray(block_tables[s][:nb]), L)
        out[r0:r1] = prefill_attention(to_float64(q[r0:r1], layout.dtype),
                                       to_float64(K, layout.dtype),
                                       to_float64(V, layout.dtype), scale, L - c)
    return out

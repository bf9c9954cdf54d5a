"""KV-cache memory utilisation: paged on-demand blocks against contiguous
max-length reservation (test infrastructure).

What the pages fix:

* Contiguous allocation has to reserve for the longest possible generation, so
  most of it is wasted when generations are short (internal fragmentation), and
  free memory splits into holes (external fragmentation) (ksqn.cn "大模型推理性能
  优化：PagedAttention与Continuous Batching原理与实践", 2.1 items 1 and 2;
  blog.gitcode.com "如何通过PagedAttention实现LLM高性能推理：实战指南", section 1:
  more than half of the space wasted).
* Paging reserves whole blocks on demand, so only a request's last block is
  partly empty; smaller blocks waste less but need more table lookups (ksqn.cn
  page, 3.4 on --block-size); the pages report utilisation rising from about 50%
  to about 95% (hihuo.com "vLLM 原理：PagedAttention 和 Continuous Batching", 优势 >
  1. 显存利用率高) and ask for more than 80% (blog.gitcode.com page, section 4).

Definitions (readings): utilisation = tokens held / token slots reserved, over the
requests admitted at a step.  Paged reservation of a request holding L tokens is
ceil(L / B) * B slots.  Contiguous reservation is the request's prompt plus the
largest output length the server allows (a request cannot know its own), i.e.
prompt + max_new, reserved at admission; the hihuo.com page's own example instead
reserves a fixed 4096 tokens for every request (优势 > 1), which fixed_reserved
gives.  External fragmentation is not modelled.

Pins: closed forms (lengths that are multiples of B give 1; one token per request
gives 1/B; a request that uses its whole allowance gives 1 contiguously) and the
library allocator's own block count over a serving trace.
"""

from __future__ import annotations


def paged_reserved(lengths, block_size: int) -> int:
    """Token slots reserved by on-demand paging for requests of these lengths."""
    B = int(block_size)
    return sum(-(-int(L) // B) * B for L in lengths)


def contiguous_reserved(prompts, max_new: int) -> int:
    """Token slots reserved at admission for prompt + the largest allowed output."""
    return sum(int(p) + int(max_new) for p in prompts)


def fixed_reserved(num_requests: int, max_len: int) -> int:
    """Token slots reserved when every request gets the same max_len slots."""
    return int(num_requests) * int(max_len)


def utilisation(used: int, reserved: int) -> float:
    return 1.0 if reserved == 0 else used / reserved

"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package draws random numbers and nothing else: it holds no step of the
paged-attention method (no cache layout, no allocation policy, no attention
arithmetic).  Both the HIP path and the CPU oracle take their inputs from here,
so that a comparison between the two always runs on identical bits.
"""

from .gen import (  # noqa: F401
    TAG_CTX, TAG_PERM, TAG_Q, TAG_KV, TAG_NEW, TAG_TRACE,
    stream, bf16_bits_from_f32, draw_values, seq_kv, new_tokens, q_values,
    context_lens_uniform, context_lens_loguniform, pool_permutation,
)
from .configs import CONFIGS, DecodeConfig, TraceConfig, get_config  # noqa: F401

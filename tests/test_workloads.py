"""The seeded generators: bf16 rounding, prefix stability, config shapes (CPU only)."""

import numpy as np
import torch

from workloads import CONFIGS, gen


def test_bf16_rounding_matches_torch_nearest_even():
    rng = gen.stream(1, 1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-40], np.float32)])
    ours = gen.bf16_bits_from_f32(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_seq_kv_is_prefix_stable():
    K1, V1 = gen.seq_kv(9, 3, 17, 2, 64, "bf16")
    K2, V2 = gen.seq_kv(9, 3, 50, 2, 64, "bf16")
    assert np.array_equal(K1, K2[:17]) and np.array_equal(V1, V2[:17])
    assert not np.array_equal(K2[0], V2[0])


def test_config_context_lengths():
    c = CONFIGS["gqa_b256"].context_lens()
    assert c.shape == (256,) and c.min() >= 16 and c.max() <= 8192
    c = CONFIGS["llama2_7b_b64"].context_lens()
    assert c.shape == (64,) and c.min() >= 128 and c.max() <= 4096
    c = CONFIGS["shared_prefix_b16"].context_lens()
    assert c.min() >= 1024 + 16 and c.max() <= 1024 + 512
    assert list(CONFIGS["tiny_f32"].context_lens()) == [1, 15, 16, 33]
    p = CONFIGS["tiny_f32"].pool_order()
    assert sorted(p) == list(range(16))


def test_generated_tokens_vectorised_equals_scalar():
    """The array form of the counter-based token draw gives the scalar form's IDs,
    including past 2^32 in the hashed state (large request IDs and positions)."""
    from workloads import gen
    for seed, req, first in ((9, 0, 0), (9, 123, 1000), (17, 70000, 1 << 19)):
        got = gen.generated_tokens(seed, req, first, 64, 64)
        assert got.tolist() == [gen.generated_token(seed, req, first + k, 64) for k in range(64)]

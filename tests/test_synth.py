"""The seeded workload generators: determinism and the length recipes."""
import numpy as np

from synth import CONFIGS, gen, get_config


def test_deterministic():
    for cfg in CONFIGS:
        assert np.array_equal(gen.context_lengths(cfg), gen.context_lengths(cfg))
        assert np.array_equal(gen.free_order(cfg), gen.free_order(cfg))


def test_free_order_is_permutation():
    for cfg in CONFIGS:
        fo = gen.free_order(cfg)
        assert np.array_equal(np.sort(fo), np.arange(cfg.num_blocks))


def test_length_recipes():
    c1 = get_config("gpt2_fp32")
    l1 = gen.context_lengths(c1)
    assert l1.min() >= 1 and l1.max() <= 1024 and len(l1) == 8
    c2 = get_config("chat_ragged")
    l2 = gen.context_lengths(c2)
    assert len(l2) == 256 and l2.min() >= 1 and l2.max() <= 1024
    assert 250 <= np.median(l2) <= 350
    c3 = get_config("gqa70b_32k")
    assert (gen.context_lengths(c3) == 32768).all()
    c4 = get_config("fork_cow")
    suf = gen.suffix_lengths(c4)
    assert suf.min() >= 256 and suf.max() <= 2048
    assert np.array_equal(gen.context_lengths(c4), 16392 + suf)
    c5 = get_config("offload")
    ch = gen.offload_choice(c5, 8192)
    assert ch.shape == (4, 4096)
    for row in ch:
        assert len(set(row.tolist())) == 4096 and row.max() < 8192


def test_lognormal_sigma_matches_chat_mean():
    # sigma chosen so that the uncapped mean exp(mu + sigma^2/2) is 371 at median 300
    c2 = get_config("chat_ragged")
    assert abs(300 * np.exp(c2.length_sigma ** 2 / 2) - 371) < 0.1


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, np.inf], np.float32)
    bits = gen.f32_to_bf16_bits(x).tolist()
    assert bits == [0x3F80, 0x3F82, 0x8000, 0x7F80]


def test_prefill_recipe():
    c = get_config("prefill_chunks")
    h = gen.prefill_histories(c)
    assert h.tolist() == [0, 512, 1024, 1536] * 4
    assert np.array_equal(gen.context_lengths(c), h + 512)
    assert (gen.context_lengths(c) <= c.length_max).all()
    assert c.seed == 8306

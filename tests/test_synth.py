"""The seeded input generator: storage rounding, determinism, order statistics."""
import numpy as np
import torch

from learned_kv_cache_amd import synth


def test_round_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 7
    ties = np.array([1.00390625, 1.01171875, -1.00390625, 2.0 ** -130, 0.0, -0.0], np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ref.view(np.uint32), synth.round_bf16(x).view(np.uint32))
    assert np.array_equal(synth.bf16_bits(ref), torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_draw_is_deterministic_and_decode_rows_match():
    a, b = synth.draw(synth.TINY), synth.draw(synth.TINY)
    for name in ("h", "q", "k", "v"):
        assert np.array_equal(a.tensor(name, 0), b.tensor(name, 0))
        assert np.array_equal(a.tensor(name, 0)[64:], a.decode_rows(name, 0))
    c = synth.draw(synth.TINY, run_id=1)
    assert not np.array_equal(a.tensor("k", 0), c.tensor("k", 0))


def test_offset_for_fraction_gives_exact_counts():
    u = np.random.default_rng(3).standard_normal(10001)
    for p in (0.0, 0.3, 0.85, 0.92, 1.0):
        o = synth.offset_for_fraction(u, p)
        assert int(np.sum(u - o > 0)) == int(round(p * u.size))


def test_ragged_contexts_are_log_uniform():
    d = synth.draw(synth.QWEN8B_FP8_SERVING)
    assert d.ctx.min() >= 1024 and d.ctx.max() <= 16384 and len(d.ctx) == 64
    assert d.T(0) == d.ctx[0] + 256

"""The seeded input generator: determinism, per-sequence streams, bf16 rounding
and the vectorised path hash."""
import numpy as np
import struct

from tree_draft_build_amd import workload as wl


def test_bf16_round_to_nearest_even():
    # exact bf16 values survive, halfway cases round to even, the rest to nearest
    vals = np.array([1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 3.0e38], np.float32)
    bits = wl.f32_to_bf16_bits(vals)
    back = wl.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == -2.5
    assert back[2] == 1.0                     # tie -> even mantissa
    assert back[3] == 1.0 + 4 * 2 ** -8       # tie -> even (upwards)
    assert back[4] == 1.0                     # below half ulp
    for v, b in zip(vals, bits):              # matches struct-level truncation check
        u = struct.unpack("<I", struct.pack("<f", v))[0]
        assert abs(int(b) - (u >> 16)) <= 1


def test_generation_is_deterministic_and_per_sequence():
    cfg = wl.CONFIGS["batched"]
    a = wl.make_logits(cfg, [3])
    b = wl.make_logits(cfg, [0, 3])
    np.testing.assert_array_equal(a[0], b[1])
    c = wl.make_attn_inputs(cfg.replace(batch=4), [2])
    d = wl.make_attn_inputs(cfg.replace(batch=4))
    off = d["ctx_offsets"]
    np.testing.assert_array_equal(c["k_ctx"], d["k_ctx"][off[2]:off[3]])
    np.testing.assert_array_equal(c["q"][0], d["q"][2])


def test_context_laws():
    lens = wl.ctx_lengths(wl.CONFIGS["batched"])
    assert lens.min() >= 512 and lens.max() <= 4096 and len(lens) == 16
    lens = wl.ctx_lengths(wl.CONFIGS["long"])
    assert lens.min() >= 1 and lens.max() <= 32768 and len(lens) == 64
    assert 4000 < np.median(lens) < 16000
    assert np.all(wl.ctx_lengths(wl.CONFIGS["qwen3_8b"]) == 4096)


def test_spike_law():
    cfg = wl.CONFIGS["qwen3_8b"]
    x = wl.logits_for_seq(cfg, 0)
    assert x.shape == (16, 151936)
    assert abs(float(np.median(x))) < 0.05 and 1.9 < float(np.std(x)) < 2.1


def test_path_uniforms_vectorised_matches_scalar():
    seeds = np.array([0, 1, 99, 2 ** 63 + 5], np.uint64)
    for path in [(), (5,), (151935, 7, 7)]:
        v = wl.path_uniforms(seeds, 3, path)
        s = [wl.path_uniform(int(x), 3, path) for x in seeds]
        np.testing.assert_array_equal(v, s)
        assert np.all((v >= 0) & (v < 1))

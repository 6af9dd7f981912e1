"""Seeded input generator: determinism, distributions and bf16 rounding."""
import numpy as np

from synth import CONFIGS, bf16_bits_from_f32, generate, zipf_router_bias


def test_same_seed_same_bits():
    cfg = CONFIGS["tiny_fp32"]
    a, b = generate(cfg), generate(cfg)
    for key in ("x", "w_gate", "w1", "w3", "w2"):
        assert a[key].tobytes() == b[key].tobytes()
    c = generate(cfg, seed=1)
    assert a["x"].tobytes() != c["x"].tobytes()


def test_streams_are_independent_per_tensor_and_layer():
    cfg = CONFIGS["tiny_fp32"]
    a = generate(cfg, layer=0)
    b = generate(cfg, layer=1)
    assert a["w1"].tobytes() != b["w1"].tobytes()
    assert a["w1"].tobytes() != a["w3"].tobytes()


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5, 3.0e38, 1e-40], np.float32)
    bits = bf16_bits_from_f32(f)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80          # tie -> even (down)
    assert bits[2] == 0x3F82          # tie -> even (up)
    assert bits[3] == 0x3F81          # above the tie -> up
    assert bits[4] == 0xC020
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back[:5] - f[:5]) <= np.abs(f[:5]) * 2 ** -8)


def test_distributions_match_recipe():
    cfg = CONFIGS["tiny_fp32"].with_(T=4096)
    g = generate(cfg)
    assert abs(g["x"].std() - 1.0) < 0.02
    assert abs(g["w_gate"].std() - 0.02) < 0.002
    assert abs(g["w1"].std() - 128 ** -0.5) < 0.002
    assert abs(g["w2"].std() - 256 ** -0.5) < 0.002
    dec = CONFIGS["mixtral_decode_t16"].with_(d=256, d_ff=256)
    x = generate(dec, tensors=("x",))["x"]
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(np.sqrt((xf ** 2).mean(axis=1)), 1.0, rtol=1e-2)


def test_zipf_bias():
    b = zipf_router_bias(8)
    p = np.exp(b.astype(np.float64))
    np.testing.assert_allclose(p.sum(), 1.0, rtol=1e-6)
    np.testing.assert_allclose(p[0], 0.4286, atol=1e-4)
    assert np.all(np.diff(b) < 0)

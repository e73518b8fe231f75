"""Seeded synthetic inputs: shapes, determinism, statistics, bf16 rounding."""
import numpy as np

import datagen


def test_bf16_round_to_nearest_even():
    f = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0xC0000000], dtype=np.uint32).view(np.float32)
    b = datagen.f32_to_bf16_bits(f)
    # 1 + 2^-8 is a tie between 1.0 (even) and 1 + 2^-7: goes to 1.0;
    # 1 + 3*2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even): goes up;
    # one bit above the first tie rounds up.
    assert list(b[:5]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000]
    assert np.array_equal(datagen.bf16_bits_to_f32(b[:5]), np.array([1.0, 1.0, 1.015625, 1.0078125, -2.0], np.float32))


def test_tiny_layer_recipe():
    lay = datagen.make_layer("tiny")
    assert lay["W"].shape == (64, 128) and lay["W"].dtype == np.float32
    assert lay["X"].shape == (128, 512) and lay["X"].dtype == np.float32
    std = lay["X"].std(axis=1)
    assert 12 < std[5] < 30 and 12 < std[77] < 30
    others = np.delete(std, [5, 77])
    assert 0.8 < others.min() and others.max() < 1.25
    assert 0.015 < lay["W"].std() < 0.025
    again = datagen.make_layer("tiny")
    assert np.array_equal(lay["W"], again["W"]) and np.array_equal(lay["X"], again["X"])
    other = datagen.make_layer("tiny", seed=1)
    assert not np.array_equal(lay["W"], other["W"])


def test_scaled_recipes_statistics():
    for name, mult in (("q_proj_7b", 15.0), ("down_proj_7b", 30.0), ("o_proj_70b", 20.0)):
        r = datagen.recipe(name, d_out=32, d_in=1024, n_tok=2048)
        X = datagen.make_activations(r, 0, threads=4)
        assert X.dtype == np.uint16 and X.shape == (1024, 2048)
        xf = datagen.bf16_bits_to_f32(X)
        k = int(round(r["outliers"][1] * 1024))
        med = np.median(np.abs(xf), axis=1)
        top = np.sort(med)[-k:]
        assert top.min() > 0.3 * mult * np.median(med)
        # threads do not change the bytes
        assert np.array_equal(X, datagen.make_activations(r, 0, threads=1))


def test_lognormal_channel_scales():
    r = datagen.recipe("up_proj_70b", d_out=16, d_in=512, n_tok=1024)
    X = datagen.bf16_bits_to_f32(datagen.make_activations(r, 0))
    logstd = np.log(X.std(axis=1))
    assert abs(logstd.mean()) < 0.2 and 0.8 < logstd.std() < 1.2

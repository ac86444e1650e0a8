"""The seeded synthetic generator: determinism and the stated distributions."""
import numpy as np

from weight_only_bit_moe_amd.inputs import (CONFIGS, LayerSpec, bf16_bits_to_f32, f32_to_bf16_bits,
                                            make_layer)


def small(**kw):
    base = dict(name="s", T=64, H=256, I=128, E=16, topk=4, bits13=2, group13=128, bits2=4,
                group2=64)
    base.update(kw)
    return LayerSpec(**base)


def test_same_seed_same_bytes():
    a, b = make_layer(small(), 3), make_layer(small(), 3)
    for f in ("x", "topk_ids", "topk_w", "w13", "s13", "w2", "s2"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_layer(small(), 4)
    assert not np.array_equal(a.w13, c.w13)


def test_bf16_rounding_nearest_even():
    v = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.5, 3e38], np.float32)
    r = bf16_bits_to_f32(f32_to_bf16_bits(v))
    assert list(r[:5]) == [1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -2.5]
    assert np.isfinite(r[5])


def test_shapes_and_ranges():
    L = make_layer(small(scale_lo=0.01, scale_hi=0.05), 1)
    assert L.w13.shape == (16, 256, 256 * 2 // 32) and L.w2.shape == (16, 256, 128 * 4 // 32)
    assert L.s13.shape == (16, 256, 2) and L.s2.shape == (16, 256, 2)
    assert L.s13.dtype == np.float16 and L.s13.min() >= np.float16(0.01) and L.s13.max() <= np.float16(0.05)
    assert np.allclose(L.topk_w.sum(1), 1.0, atol=1e-6)
    for t in range(64):
        assert len(set(L.topk_ids[t])) == 4          # distinct per token
    # every 2-bit field of the words is uniform over its 4 values
    fields = (L.w13[..., None] >> (np.arange(16, dtype=np.uint32) * 2)) & 3
    counts = np.bincount(fields.reshape(-1), minlength=4) / fields.size
    assert np.allclose(counts, 0.25, atol=0.01)


def test_zipf_routing_is_skewed_and_loguniform_scales():
    L = make_layer(small(T=2048, E=64, topk=6, routing="zipf", scale_dist="loguniform",
                         scale_lo=1e-3, scale_hi=5e-2), 2)
    counts = np.bincount(L.topk_ids.reshape(-1), minlength=64)
    assert counts.max() > 1000 and counts.min() < 100
    ls = np.log(L.s2.astype(np.float64))
    assert ls.min() >= np.log(1e-3) - 1e-3 and ls.max() <= np.log(5e-2) + 1e-3


def test_outlier_channels():
    L = make_layer(small(outlier_frac=0.05, x_sigma=2.0), 6)
    xf = bf16_bits_to_f32(L.x)
    assert len(L.outlier_channels) == round(0.05 * 256)
    big = np.abs(xf[:, L.outlier_channels]).mean()
    rest = np.abs(np.delete(xf, L.outlier_channels, axis=1)).mean()
    assert 7 < big / rest < 13


def test_named_configs_shapes():
    assert CONFIGS[2].T == 4 and CONFIGS[2].bits13 == 2 and CONFIGS[5].group2 == 64
    assert CONFIGS[4].clamp == 7.0 and CONFIGS[5].x_sigma == 2.0


def test_dense_weights_and_importance_recipe():
    from weight_only_bit_moe_amd.inputs import make_dense_weights, make_importance
    w = make_dense_weights(64, 1024, 5)
    assert w.dtype == np.uint16 and w.shape == (64, 1024)
    assert np.array_equal(w, make_dense_weights(64, 1024, 5))
    f = bf16_bits_to_f32(w).astype(np.float64)
    # t4 * 0.02: variance df/(df-2) * 0.02^2 = 8e-4; heavy tails (kurtosis > normal's 3)
    assert abs(f.var() / 8e-4 - 1) < 0.15
    assert ((f - f.mean()) ** 4).mean() / f.var() ** 2 > 4.0
    imp = make_importance(4096, 7)
    assert imp.dtype == np.float32 and imp.shape == (4096,) and np.all(imp > 0)
    assert np.sum(imp > 30) >= 30            # about 1% outlier channels at 100x
    assert np.array_equal(imp, make_importance(4096, 7))

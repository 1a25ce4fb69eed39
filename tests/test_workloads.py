"""The seeded input generators: bf16 rounding, determinism, layout."""
import numpy as np

from learned_token_pruning_amd import workloads as W


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is exactly halfway between two bf16 values: ties go to the even mantissa (1.0)
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 0.0, -0.0, np.inf, -np.inf], np.float32)
    back = W.bf16_bits_to_f32(W.f32_to_bf16_bits(vals))
    np.testing.assert_array_equal(back, np.array([1.0, 1.0, 1 + 4 * 2 ** -8, -2.5, 0.0, -0.0, np.inf, -np.inf],
                                                 np.float32))
    assert np.signbit(back[5])
    assert np.isnan(W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    err = np.abs(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)) - x) / np.abs(x)
    assert err.max() <= 2 ** -8  # unit roundoff of an 8-bit significand


def test_workload_1_is_deterministic_and_shaped():
    a, b = W.workload(1), W.workload(1)
    assert a.x.shape == (512, 256) and a.w1.shape == (64, 256)
    assert a.q.shape == (512, 4, 64) and a.k.shape == (512, 2, 64)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.q, b.q)
    assert a.segments.doc_end == [448] and a.segments.seg_start == [0, 512]
    assert a.needle_rows.size == 8 and np.all(a.needle_rows < 448)
    norms = np.linalg.norm(W.bf16_bits_to_f32(a.x), axis=1)
    assert norms[a.needle_rows].min() > 2.5 * np.median(norms)


def test_mixture_scores_shape():
    seg = W.single_segment(32704, 64, 2048)
    s = W.mixture_scores(3, seg, k_marks=(1024, 2048, 4096, 8192))
    doc = s[:32704]
    frac_hot = np.mean(doc > 2.5)
    assert 0.03 < frac_hot < 0.07
    assert np.unique(doc).size < doc.size * 0.995
    assert np.any((doc == 0) & np.signbit(doc)) and np.any((doc == 0) & ~np.signbit(doc))

"""Seeded input generators: shapes, determinism and the recipe's properties."""
import numpy as np
import pytest

from scale_deformable_attention_amd import workloads as wl


def test_pyramid_shapes_follow_strides():
    # ceil(800/s), ceil(1333/s) and ceil(1080/s), ceil(1920/s) for strides 8..64
    for (h, w), s in zip(wl.PYRAMID_800x1333, (8, 16, 32, 64)):
        assert (h, w) == (-(-800 // s), -(-1333 // s))
    for (h, w), s in zip(wl.PYRAMID_1920x1080, (8, 16, 32, 64)):
        assert (h, w) == (-(-1080 // s), -(-1920 // s))
    assert wl.WORKLOADS["encoder"].Nv == 22223
    assert wl.WORKLOADS["hires_bf16"].Nv == 43110
    assert list(wl.WORKLOADS["encoder"].level_start_index()) == [0, 16700, 20900, 21950]


def test_points_per_workload():
    assert wl.WORKLOADS["tiny"].points == 128
    assert wl.WORKLOADS["encoder"].points == 5_689_088
    assert wl.WORKLOADS["decoder"].points == 307_200
    assert wl.WORKLOADS["hires_bf16"].points == 22_072_320
    assert wl.WORKLOADS["encoder_train"].points == 11_378_176


def test_generation_is_deterministic_and_shaped():
    w = wl.WORKLOADS["tiny"]
    a, b = wl.generate(w), wl.generate(w)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["value"].shape == (1, 80, 2, 8) and a["value"].dtype == np.float32
    assert a["sampling_locations"].shape == (1, 16, 2, 2, 2, 2)
    assert a["attention_weights"].shape == (1, 16, 2, 2, 2)
    assert a["grad_output"].shape == (1, 16, 16)
    np.testing.assert_allclose(a["attention_weights"].reshape(1, 16, 2, 4).sum(-1), 1.0, rtol=1e-6)


def test_grid_reference_points_are_pixel_centres():
    w = wl.WORKLOADS["encoder"].scaled(B=1, M=1, K=1, sigma_px=0.0,
                                       shapes=((3, 5), (2, 2)))
    x = wl.generate(w)
    loc = x["sampling_locations"][0, :, 0, 0, 0]          # level-0 sample of each query
    assert loc.shape == (19, 2)
    np.testing.assert_allclose(loc[:15, 0], np.tile((np.arange(5) + 0.5) / 5, 3), rtol=1e-7)
    np.testing.assert_allclose(loc[:15, 1], np.repeat((np.arange(3) + 0.5) / 3, 5), rtol=1e-7)
    np.testing.assert_allclose(loc[15:, 0], np.tile((np.arange(2) + 0.5) / 2, 2), rtol=1e-7)


def test_batch_slice_is_a_subsample():
    w = wl.WORKLOADS["tiny"].scaled(B=3)
    full, part = wl.generate(w), wl.generate(w, batch_slice=slice(1, 2))
    assert np.array_equal(full["value"][1:2], part["value"])
    assert np.array_equal(full["sampling_locations"][1:2], part["sampling_locations"])


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, np.inf], np.float32)
    bits = wl.bf16_round(x)
    back = wl.bf16_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    assert back[1] == np.float32(1.0)
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert back[2] == np.float32(1.0 + 2 ** -6)
    assert back[3] == np.float32(-2.5) and np.isinf(back[5])
    assert np.isnan(wl.bf16_to_f32(wl.bf16_round(np.array([np.nan], np.float32))))[0]


@pytest.mark.parametrize("name", ["tiny", "decoder"])
def test_offsets_spread_matches_sigma(name):
    w = wl.WORKLOADS[name]
    x = wl.generate(w)
    ref = x["reference_points"]
    for l, (h, wd) in enumerate(w.shapes):
        d = (x["sampling_locations"][:, :, :, l].astype(np.float64)
             - ref[None, :, None, None, :]) * np.array([wd, h])
        tol = 4.0 / np.sqrt(d.size)          # a few standard errors of the estimate
        assert abs(d.mean()) < tol * w.sigma_px
        assert abs(d.std() / w.sigma_px - 1.0) < tol

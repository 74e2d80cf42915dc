"""The seeded input generators: determinism and the workload recipes (CPU only)."""

import numpy as np

import synth


def test_streams_are_deterministic_and_distinct():
    a = synth.gaussian_bf16(42, synth.TAG_DATA, (64, 128))
    b = synth.gaussian_bf16(42, synth.TAG_DATA, (64, 128))
    c = synth.gaussian_bf16(43, synth.TAG_DATA, (64, 128))
    assert a.dtype == np.uint16 and a.shape == (64, 128)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert not np.array_equal(a, synth.gaussian_bf16(42, synth.TAG_QUERY, (64, 128)))


def test_configs_name_seeds_not_matrices():
    """D and G are rebuilt from seeds by each side; a config carries only the seeds."""
    c = synth.config2(rows=16, cols=128)
    assert c["sign_seed"] == synth.BASE_SEED and c["proj_seed"] == synth.BASE_SEED
    assert "signs" not in c and "G" not in c


def test_bf16_cast_is_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0 - 2 ** -7 - 2 ** -20], dtype=np.float32)
    back = synth.bf16_to_f32(synth.bf16_from_f32(x))
    assert back[0] == 1.0 and back[1] == 1.0 + 2 ** -6 and back[2] == -2.0 - 2 ** -6


def test_config1_recipe():
    c = synth.config1()
    assert c["x"].shape == (256, 512) and c["x"].dtype == np.float32
    assert abs(np.std(c["x"]) - 0.02) < 0.001


def test_config2_recipe_small():
    x, pos = synth.weight_with_outlier_entries(0, 256, 512)
    assert len(pos) == int(0.001 * 256 * 512) and len(np.unique(pos)) == len(pos)
    v = np.abs(synth.bf16_to_f32(x).reshape(-1))
    assert np.median(v[pos]) > 5 * np.median(v)


def test_config3_layout():
    lay = synth.config3_layout()
    assert len(lay) == 224
    total = sum(r * c for _, _, _, r, c in lay)
    assert total == 6_979_321_856
    assert lay[4][2] == "gate" and lay[7][1] == 1


def test_config4_recipe_small():
    c = synth.config4(tokens=64)
    assert c["keys"].shape == (4, 8, 64, 128) and c["q"].shape == (4, 32, 128)
    k = synth.bf16_to_f32(c["keys"])
    for h in range(8):
        ch = c["outlier_channels"][h]
        assert np.mean(np.abs(k[:, h][..., ch])) > 10 * np.mean(np.abs(k[:, h]))

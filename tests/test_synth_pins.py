"""Pins of the seeded synthetic workloads (CPU only).

Voxel counts N follow from the generator recipe alone; the pair counts P
(rulebook entries >= 0, centre tap included) come from the oracle's rulebook.
Config 3b is a dense 128^3 box, where P = (3*128 - 2)^3 is a closed form.
"""
import numpy as np
import pytest

import synth
from oracle import submconv_ref as ref

EXPECTED = {
    # key: (N, per-item N, P)
    "1": (450, [450], 4_650),
    "2a": (22_406, [22_406], 403_774),
    "3a": (135_826, [135_826], 2_833_778),
    "3b": (2_097_152, [2_097_152], 55_742_968),
    "4": (1_664_012, [611_631, 536_367, 280_434, 235_580], 30_027_876),
    "5": (2_550_313, [1_274_422, 1_275_891], 17_117_513),
}


@pytest.mark.parametrize("key", ["1", "2a", "3a"])
def test_small_config_counts(key):
    c = synth.coords_for(key)
    n, per_item, p = EXPECTED[key]
    assert c.dtype == np.int32 and c.shape == (n, 4)
    assert [int((c[:, 0] == m).sum()) for m in range(len(per_item))] == per_item
    assert int((ref.rulebook_sorted(c) >= 0).sum()) == p


@pytest.mark.slow
@pytest.mark.parametrize("key", ["3b", "4", "5"])
def test_large_config_counts(key):
    c = synth.coords_for(key)
    n, per_item, p = EXPECTED[key]
    assert c.shape == (n, 4)
    assert [int((c[:, 0] == m).sum()) for m in range(len(per_item))] == per_item
    assert int((ref.rulebook_sorted(c) >= 0).sum()) == p


def test_dense_rulebook_agrees_with_dict_rulebook_on_small_configs():
    for key in ("1", "2a"):
        c = synth.coords_for(key)
        assert np.array_equal(ref.rulebook(c), ref.rulebook_sorted(c))


def test_values_are_rounded_and_seeded():
    f = synth.feats_for(3, 0, 10, 128, "bf16")
    g = synth.feats_for(3, 0, 10, 128, "bf16")
    assert f.dtype.is_floating_point and str(f.dtype) == "torch.bfloat16"
    assert (f == g).all()
    w = synth.weight_for(3, 0, 3, 128, 128, "bf16")
    assert tuple(w.shape) == (128, 3, 3, 3, 128)
    # fan-in variance: std close to sqrt(1/(27*128))
    assert abs(float(w.float().std()) - (1.0 / (27 * 128)) ** 0.5) < 2e-3
    b = synth.bias_for(1, 0, 16, "f32")
    assert str(b.dtype) == "torch.float32" and tuple(b.shape) == (16,)


def test_subdivide_children_c_order():
    base = np.array([[1, 2, 3]])
    rng = np.random.default_rng(0)
    kids = synth.subdivide_keep(base, 1, 1.1, rng)  # keep all
    assert kids.tolist() == [[2 + i, 4 + j, 6 + k] for i in (0, 1) for j in (0, 1) for k in (0, 1)]


def test_config5_parent_level_count():
    # two subdivisions of the 9,962-voxel shell, two items: 2 x 9,962 x 64
    c = synth.coords_for("5_parent")
    assert c.shape == (2 * 9962 * 64, 4)
    # the shell spans 4 .. 60 of the 64^3 grid, so its children span 16 .. 243 of 256^3
    assert c[:, 1:].min() == 16 and c[:, 1:].max() == 243

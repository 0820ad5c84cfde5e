"""Pins of the structure-op oracle (subdivide, downsample, upsample) against things other than
itself (CPU only).

* hand-worked golden examples under tests/golden/;
* dense-volume closed forms: 2x max pooling and mean pooling of a dense zero/-inf volume with
  torch CPU max_pool3d / avg_pool3d, read at the occupied coarse cells;
* set identities: the children of a dense G^3 box are the dense (2G)^3 box; downsample undoes
  subdivide; a full mask gives subdivide's child set in the bit-reversed order;
* planted mistakes in the oracle must fail the pins.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import structure_ref as st

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def random_sites(rng, batch, lo, hi, occupancy):
    """Random active sites with spatial coordinates in [lo, hi) per axis, items concatenated."""
    g = hi - lo
    rows = []
    for b in range(batch):
        zyx = np.argwhere(rng.random((g, g, g)) < occupancy) + lo
        rows.append(np.concatenate([np.full((len(zyx), 1), b), zyx], axis=1))
    return np.concatenate(rows, axis=0).astype(np.int32)


def dense_pool(coords, feats, batch, lo, hi, mode):
    """2x pooling through a dense volume: returns (cells [M,4] in C order per item, values)."""
    g = hi - lo
    c = torch.from_numpy(coords.astype(np.int64))
    cin = feats.shape[1]
    fill = -np.inf if mode == "max" else 0.0
    vol = torch.full((batch, cin, g, g, g), fill, dtype=torch.float64)
    occ = torch.zeros((batch, 1, g, g, g), dtype=torch.float64)
    idx = (c[:, 0], slice(None), c[:, 1] - lo, c[:, 2] - lo, c[:, 3] - lo)
    vol[idx] = torch.from_numpy(feats)
    occ[c[:, 0], 0, c[:, 1] - lo, c[:, 2] - lo, c[:, 3] - lo] = 1.0
    count = torch.nn.functional.avg_pool3d(occ, 2) * 8.0
    if mode == "max":
        pooled = torch.nn.functional.max_pool3d(vol, 2)
    else:
        pooled = torch.nn.functional.avg_pool3d(vol, 2) * 8.0 / count.clamp(min=1.0)
    cells = []
    vals = []
    for b in range(batch):
        zyx = np.argwhere(count[b, 0].numpy() > 0)
        for z, y, x in zyx:
            cells.append((b, z + lo // 2, y + lo // 2, x + lo // 2))
            vals.append(pooled[b, :, z, y, x].numpy())
    return np.array(cells, dtype=np.int32).reshape(-1, 4), np.array(vals).reshape(len(cells), cin)


# ----------------------------------------------------------------- golden examples

def test_golden_subdivide():
    g = load("subdivide_example.json")
    child, cf, parent = st.subdivide(np.array(g["coords_bzyx"]), np.array(g["feats"]))
    assert child.tolist() == g["expected_children_bzyx"]
    assert parent.tolist() == g["expected_parent"]
    assert cf[0].tolist() == g["expected_child_feats_first_and_last"][0]
    assert cf[-1].tolist() == g["expected_child_feats_first_and_last"][1]
    assert (cf == np.array(g["feats"])[parent]).all()


def test_golden_masked_upsample():
    g = load("masked_upsample_example.json")
    child, cf, parent = st.upsample_masked(np.array(g["coords_bzyx"]), np.array(g["mask"]),
                                           np.array(g["feats"]))
    assert child.tolist() == g["expected_children_bzyx"]
    assert parent.tolist() == g["expected_parent"]
    assert cf.tolist() == g["expected_child_feats"]
    assert child.tolist() != g["c_order_decode_would_give"]


def test_golden_downsample():
    g = load("downsample_example.json")
    coords = np.array(g["coords_bzyx"])
    feats = np.array(g["feats"])
    coarse, mx, parent = st.downsample(coords, feats, "max")
    assert coarse.tolist() == g["expected_coarse_bzyx"]
    assert parent.tolist() == g["expected_parent"]
    assert mx.tolist() == g["expected_max"]
    _, mean, _ = st.downsample(coords, feats, "mean")
    np.testing.assert_allclose(mean * 3.0, np.array(g["expected_mean_times_3"]), rtol=0, atol=1e-12)


def test_downsample_needs_explicit_mode():
    c = np.array([[0, 0, 0, 0]])
    with pytest.raises(ValueError):
        st.downsample(c, np.ones((1, 2)))
    with pytest.raises(ValueError):
        st.downsample(c, np.ones((1, 2)), "avg")


# ----------------------------------------------------------------- dense-volume closed forms

@pytest.mark.parametrize("mode", ["max", "mean"])
@pytest.mark.parametrize("seed,occ", [(1, 0.15), (2, 0.5), (3, 1.0)])
def test_downsample_matches_dense_pooling(mode, seed, occ):
    rng = np.random.default_rng(seed)
    lo, hi = -6, 6  # negative and positive odd coordinates; the dense box starts at an even lo
    coords = random_sites(rng, 2, lo, hi, occ)
    feats = rng.standard_normal((len(coords), 5))
    cells, vals = dense_pool(coords, feats, 2, lo, hi, mode)
    coarse, pooled, parent = st.downsample(coords, feats, mode)
    assert coarse.tolist() == cells.tolist()
    np.testing.assert_allclose(pooled, vals, rtol=0, atol=1e-12)
    # every fine row's parent cell contains it
    assert ((coords[:, 1:] - 2 * coarse[parent][:, 1:]) >= 0).all()
    assert ((coords[:, 1:] - 2 * coarse[parent][:, 1:]) <= 1).all()
    assert (coords[:, 0] == coarse[parent][:, 0]).all()


def test_downsample_row_order_free():
    rng = np.random.default_rng(7)
    coords = random_sites(rng, 2, -4, 6, 0.4)
    feats = rng.standard_normal((len(coords), 3))
    perm = rng.permutation(len(coords))
    a = st.downsample(coords, feats, "mean")
    b = st.downsample(coords[perm], feats[perm], "mean")
    assert a[0].tolist() == b[0].tolist()
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)
    assert (a[2][perm] == b[2]).all()


# ----------------------------------------------------------------- set identities

def test_subdivide_of_box_is_doubled_box():
    g = 3
    box = np.argwhere(np.ones((g, g, g), dtype=bool))
    coords = np.concatenate([np.zeros((len(box), 1), dtype=int), box], axis=1)
    child, _, parent = st.subdivide(coords)
    want = np.argwhere(np.ones((2 * g, 2 * g, 2 * g), dtype=bool))
    assert sorted(map(tuple, child[:, 1:].tolist())) == sorted(map(tuple, want.tolist()))
    assert len(set(map(tuple, child.tolist()))) == len(child)
    assert ((child[:, 1:] >> 1) == coords[parent][:, 1:]).all()


@pytest.mark.parametrize("mode", ["max", "mean"])
def test_downsample_undoes_subdivide(mode):
    rng = np.random.default_rng(11)
    coords = random_sites(rng, 3, -5, 5, 0.3)
    feats = rng.standard_normal((len(coords), 4))
    child, cf, _ = st.subdivide(coords, feats)
    coarse, pooled, parent = st.downsample(child, cf, mode)
    order = np.lexsort(coords.T[::-1])
    assert coarse.tolist() == coords[order].tolist()
    np.testing.assert_allclose(pooled, feats[order], rtol=0, atol=1e-12)
    np.testing.assert_allclose(st.upsample_cached(parent, pooled), cf, rtol=0, atol=1e-12)


def test_full_mask_is_subdivide_in_bit_reversed_order():
    rng = np.random.default_rng(5)
    coords = random_sites(rng, 2, -3, 3, 0.3)
    sub, _, _ = st.subdivide(coords)
    msk, _, _ = st.upsample_masked(coords, np.ones((len(coords), 8), dtype=np.uint8))
    assert sorted(map(tuple, sub.tolist())) == sorted(map(tuple, msk.tolist()))
    rev = [int(f"{s:03b}"[::-1], 2) for s in range(8)]
    for i in range(len(coords)):
        for s in range(8):
            assert msk[8 * i + s].tolist() == sub[8 * i + rev[s]].tolist()
    assert msk.tolist() != sub.tolist()


def test_empty_mask_row_emits_nothing():
    coords = np.array([[0, 0, 0, 0], [0, 4, 4, 4]])
    mask = np.array([[0] * 8, [0, 0, 0, 1, 0, 0, 0, 0]])
    child, _, parent = st.upsample_masked(coords, mask)
    assert parent.tolist() == [1]
    assert child.tolist() == [[0, 9, 9, 8]]


# ----------------------------------------------------------------- planted mistakes

def test_planted_truncating_division_fails(monkeypatch):
    def trunc_cell(row):
        b, z, y, x = row
        return (b, int(z / 2), int(y / 2), int(x / 2))

    monkeypatch.setattr(st, "coarse_cell", trunc_cell)
    with pytest.raises(AssertionError):
        test_golden_downsample()
    with pytest.raises(AssertionError):
        test_downsample_matches_dense_pooling("max", 2, 0.5)


def test_planted_mean_over_eight_fails(monkeypatch):
    real = st.downsample

    def mean8(coords, feats=None, mode=None):
        coarse, out, parent = real(coords, feats, "max" if mode == "max" else "mean")
        if mode == "mean":
            counts = np.bincount(parent, minlength=len(coarse))
            out = out * counts[:, None] / 8.0
        return coarse, out, parent

    monkeypatch.setattr(st, "downsample", mean8)
    with pytest.raises(AssertionError):
        test_downsample_matches_dense_pooling("mean", 1, 0.15)


def test_planted_c_order_masked_decode_fails(monkeypatch):
    monkeypatch.setattr(st, "masked_offset", st.subdivide_offset)
    with pytest.raises(AssertionError):
        test_golden_masked_upsample()


def test_planted_axis0_fastest_subdivide_fails(monkeypatch):
    monkeypatch.setattr(st, "subdivide_offset", lambda s: (s & 1, (s >> 1) & 1, (s >> 2) & 1))
    with pytest.raises(AssertionError):
        test_golden_subdivide()

"""Pins of the CPU oracle against things other than itself (CPU only).

* closed form: submanifold conv == dense zero-padded conv3d (torch CPU, float64)
  evaluated at the active sites;
* brute force: an O(N^2) scan for every (voxel, tap) rulebook entry;
* dense-box closed form for the rulebook and the pair count (3G - 2)^3;
* a hand-worked orientation example stored under tests/golden/;
* invariants (identity kernel, k=1 == linear layer, lone voxel, translation,
  row permutation, batch isolation, rulebook symmetry, flip-kernel mirror);
* planted mistakes in the oracle must fail the closed-form check.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import submconv_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def random_sites(rng, batch, grid, occupancy):
    rows = []
    for b in range(batch):
        mask = rng.random((grid, grid, grid)) < occupancy
        zyx = np.argwhere(mask)
        rows.append(np.concatenate([np.full((len(zyx), 1), b), zyx], axis=1))
    c = np.concatenate(rows, axis=0).astype(np.int32)
    return c


def dense_conv_at_sites(coords, feats, weight, bias, batch, grid):
    """Scatter into a dense zero volume, run torch conv3d (cross-correlation, padding 1), read the sites."""
    cin = feats.shape[1]
    vol = torch.zeros((batch, cin, grid, grid, grid), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    vol[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(feats)
    w = torch.from_numpy(weight).permute(0, 4, 1, 2, 3).contiguous()  # KRSC -> [O, I, kz, ky, kx]
    b = None if bias is None else torch.from_numpy(bias)
    dense = torch.nn.functional.conv3d(vol, w, b, padding=1)
    return dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()


def brute_rulebook(coords):
    c = np.asarray(coords, dtype=np.int64)
    n = len(c)
    out = np.full((n, 27), -1, dtype=np.int32)
    offs = [(dz, dy, dx) for dz in (-1, 0, 1) for dy in (-1, 0, 1) for dx in (-1, 0, 1)]
    for i in range(n):
        for k, (dz, dy, dx) in enumerate(offs):
            target = c[i] + np.array([0, dz, dy, dx])
            hit = np.nonzero((c == target).all(axis=1))[0]
            assert len(hit) <= 1
            if len(hit):
                out[i, k] = hit[0]
    return out


def rel(a, b):
    return oracle.normwise_rel_error(a, b)


# ----------------------------------------------------------------- closed form

DENSE_CASES = [
    # (grid, batch, occupancy, cin, cout, seed)
    (4, 2, 1.0, 3, 5, 0),
    (6, 2, 0.5, 3, 5, 1),
    (8, 1, 0.1, 16, 16, 2),
    (10, 2, 0.1, 3, 5, 3),
    (7, 2, 0.3, 16, 16, 4),
]


@pytest.mark.parametrize("grid,batch,occ,cin,cout,seed", DENSE_CASES)
def test_conv3_equals_dense_conv3d_at_active_sites(grid, batch, occ, cin, cout, seed):
    rng = np.random.default_rng(seed)
    coords = random_sites(rng, batch, grid, occ)
    f = rng.standard_normal((len(coords), cin))
    w = rng.standard_normal((cout, 3, 3, 3, cin))
    b = rng.standard_normal(cout)
    want = dense_conv_at_sites(coords, f, w, b, batch, grid)
    got_naive = ref.conv3(coords, f, w, b)
    got_rb = ref.conv3_rulebook(ref.rulebook(coords), f, w, b)
    assert rel(got_naive, want) < 1e-12
    assert rel(got_rb, want) < 1e-12
    # Shuffled row order must give the same per-site result.
    perm = rng.permutation(len(coords))
    got_perm = ref.conv3(coords[perm], f[perm], w, b)
    assert rel(got_perm, want[perm]) < 1e-12


def test_conv3_without_bias_equals_dense():
    rng = np.random.default_rng(11)
    coords = random_sites(rng, 1, 6, 0.4)
    f = rng.standard_normal((len(coords), 4))
    w = rng.standard_normal((6, 3, 3, 3, 4))
    want = dense_conv_at_sites(coords, f, w, None, 1, 6)
    assert rel(ref.conv3(coords, f, w, None), want) < 1e-12


# ----------------------------------------------------------------- planted mistakes

def _dense_case():
    rng = np.random.default_rng(5)
    coords = random_sites(rng, 2, 6, 0.5)
    f = rng.standard_normal((len(coords), 3))
    w = rng.standard_normal((5, 3, 3, 3, 3))
    b = rng.standard_normal(5)
    return coords, f, w, b, dense_conv_at_sites(coords, f, w, b, 2, 6)


def test_closed_form_catches_swapped_axis_pairing():
    # Pairing coordinate z with kernel axis kx (and x with kz) is the same as
    # swapping the weight's kz and kx axes.
    coords, f, w, b, want = _dense_case()
    assert rel(ref.conv3(coords, f, np.ascontiguousarray(np.swapaxes(w, 1, 3)), b), want) > 1e-2


def test_closed_form_catches_mirrored_orientation():
    coords, f, w, b, want = _dense_case()
    assert rel(ref.conv3(coords, f, w, b, orientation=-1), want) > 1e-2


def test_closed_form_catches_dropped_bias():
    coords, f, w, b, want = _dense_case()
    assert rel(ref.conv3(coords, f, w, None), want) > 1e-2


def test_closed_form_catches_transposed_weight():
    rng = np.random.default_rng(6)
    coords = random_sites(rng, 1, 6, 0.5)
    f = rng.standard_normal((len(coords), 4))
    w = rng.standard_normal((4, 3, 3, 3, 4))
    want = dense_conv_at_sites(coords, f, w, None, 1, 6)
    wt = np.ascontiguousarray(np.swapaxes(w, 0, 4))
    assert rel(ref.conv3(coords, f, wt, None), want) > 1e-2


def test_closed_form_catches_wrong_tap_order(monkeypatch):
    coords, f, w, b, want = _dense_case()
    good = ref.tap_offset
    monkeypatch.setattr(ref, "tap_offset", lambda k: good(26 - k) if k in (12, 14) else good(k))
    assert rel(ref.conv3_rulebook(ref.rulebook(coords), f, w, b), want) > 1e-2


# ----------------------------------------------------------------- rulebook

@pytest.mark.parametrize("seed", range(6))
def test_rulebook_equals_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 160))
    # Small random sets with negative coordinates, several batch items, clustered so neighbours occur.
    pts = set()
    while len(pts) < n:
        b = int(rng.integers(0, 3))
        z, y, x = (int(v) for v in rng.integers(-4, 3, 3))
        pts.add((b, z - 1000 * (seed % 2), y, x + 7))
    coords = np.array(sorted(pts, key=lambda _: rng.random()), dtype=np.int32)
    want = brute_rulebook(coords)
    assert np.array_equal(ref.rulebook(coords), want)
    assert np.array_equal(ref.rulebook_sorted(coords), want)


@pytest.mark.parametrize("grid", [1, 2, 5, 9])
def test_dense_box_rulebook_closed_form_small(grid):
    coords = np.argwhere(np.ones((grid,) * 3, dtype=bool)).astype(np.int32)
    coords = np.concatenate([np.zeros((len(coords), 1), np.int32), coords], axis=1)
    want = dense_box_closed_form(grid)
    assert np.array_equal(ref.rulebook(coords), want)
    assert np.array_equal(ref.rulebook_sorted(coords), want)
    assert int((want >= 0).sum()) == (3 * grid - 2) ** 3


def dense_box_closed_form(g):
    z, y, x = np.meshgrid(np.arange(g), np.arange(g), np.arange(g), indexing="ij")
    z, y, x = z.ravel(), y.ravel(), x.ravel()
    out = np.empty((g ** 3, 27), dtype=np.int32)
    k = 0
    for dz in (-1, 0, 1):
        for dy in (-1, 0, 1):
            for dx in (-1, 0, 1):
                zz, yy, xx = z + dz, y + dy, x + dx
                ok = (zz >= 0) & (zz < g) & (yy >= 0) & (yy < g) & (xx >= 0) & (xx < g)
                out[:, k] = np.where(ok, (zz * g + yy) * g + xx, -1)
                k += 1
    return out


@pytest.mark.slow
def test_dense_box_128_rulebook_closed_form():
    import synth
    coords = synth.coords_for("3b")
    nbr = ref.rulebook_sorted(coords)
    assert np.array_equal(nbr, dense_box_closed_form(128))
    assert int((nbr >= 0).sum()) == 382 ** 3 == 55_742_968


def test_duplicate_coordinate_raises():
    coords = np.array([[0, 1, 2, 3], [0, 1, 2, 4], [0, 1, 2, 3]], dtype=np.int32)
    with pytest.raises(oracle.DuplicateCoordinate):
        ref.rulebook(coords)
    with pytest.raises(oracle.DuplicateCoordinate):
        ref.rulebook_sorted(coords)
    with pytest.raises(oracle.DuplicateCoordinate):
        ref.conv3(coords, np.zeros((3, 1)), np.zeros((1, 3, 3, 3, 1)))


# ----------------------------------------------------------------- golden (hand-worked)

def _golden():
    with open(os.path.join(GOLDEN, "orientation_example.json")) as fh:
        g = json.load(fh)
    coords = np.array(g["coords_bzyx"], dtype=np.int32)
    w = np.zeros((1, 3, 3, 3, 1))
    for e in g["weights_nonzero"]:
        w[tuple(e["krsc_index"])] = e["value"]
        dz, dy, dx = e["dzdydx"]
        assert tuple(e["krsc_index"]) == (0, dz + 1, dy + 1, dx + 1, 0)
    return g, coords, np.array(g["feats"]), w, np.array(g["bias"])


def test_golden_orientation_example():
    g, coords, f, w, b = _golden()
    assert np.array_equal(ref.conv3(coords, f, w, b), np.array(g["expected_out_c_plus_d"]))
    assert np.array_equal(ref.conv3(coords, f, w, b, orientation=-1), np.array(g["expected_out_c_minus_d"]))
    assert np.array_equal(ref.conv3_rulebook(ref.rulebook(coords), f, w, b), np.array(g["expected_out_c_plus_d"]))


def test_golden_rulebook():
    g, coords, _, _, _ = _golden()
    want = np.full((4, 27), -1, dtype=np.int32)
    for r, name in enumerate(g["row_names"]):
        for k, j in g["expected_rulebook_nonneg"][name].items():
            want[r, int(k)] = j
    assert np.array_equal(ref.rulebook(coords), want)
    assert np.array_equal(ref.rulebook_sorted(coords), want)


# ----------------------------------------------------------------- invariants

def _shell_case(seed=7, cin=5, cout=6):
    import synth
    coords = synth.coords_for("1")
    rng = np.random.default_rng(seed)
    return coords, rng.standard_normal((len(coords), cin)), rng.standard_normal((cout, 3, 3, 3, cin)), rng.standard_normal(cout)


def test_identity_kernel_returns_input_exactly():
    coords, f, _, _ = _shell_case(cin=4, cout=4)
    w = np.zeros((4, 3, 3, 3, 4))
    w[:, 1, 1, 1, :] = np.eye(4)
    assert np.array_equal(ref.conv3(coords, f, w), f)
    assert np.array_equal(ref.conv3_rulebook(ref.rulebook(coords), f, w), f)


def test_k1_is_a_linear_layer():
    coords, f, _, _ = _shell_case()
    rng = np.random.default_rng(3)
    w1 = rng.standard_normal((6, 1, 1, 1, 5))
    b = rng.standard_normal(6)
    lin = torch.nn.functional.linear(torch.from_numpy(f), torch.from_numpy(w1[:, 0, 0, 0, :]), torch.from_numpy(b)).numpy()
    assert rel(ref.conv1(f, w1, b), lin) < 1e-14
    # ... and equals the k=3 path with only the centre tap populated.
    w3 = np.zeros((6, 3, 3, 3, 5))
    w3[:, 1, 1, 1, :] = w1[:, 0, 0, 0, :]
    assert rel(ref.conv3(coords, f, w3, b), ref.conv1(f, w1, b)) < 1e-14


def test_lone_voxel_sees_only_centre():
    coords = np.array([[0, 5, 5, 5], [0, 9, 9, 9], [1, 5, 5, 5]], dtype=np.int32)
    nbr = ref.rulebook(coords)
    for i in range(3):
        assert nbr[i].tolist() == [-1] * 13 + [i] + [-1] * 13
    rng = np.random.default_rng(9)
    f = rng.standard_normal((3, 2))
    w = rng.standard_normal((3, 3, 3, 3, 2))
    b = rng.standard_normal(3)
    want = b[None, :] + f @ w[:, 1, 1, 1, :].T
    assert rel(ref.conv3(coords, f, w, b), want) < 1e-14


def test_translation_invariance():
    coords, f, w, b = _shell_case()
    moved = coords + np.array([0, -1000, 37, 2_000_000], dtype=np.int32)
    assert np.array_equal(ref.rulebook(moved), ref.rulebook(coords))
    assert np.array_equal(ref.rulebook_sorted(moved), ref.rulebook(coords))
    assert np.array_equal(ref.conv3(moved, f, w, b), ref.conv3(coords, f, w, b))


def test_row_permutation_relabels():
    coords, f, w, b = _shell_case()
    rng = np.random.default_rng(1)
    perm = rng.permutation(len(coords))
    inv = np.argsort(perm)
    nbr = ref.rulebook(coords)
    nbr_p = ref.rulebook(coords[perm])
    relabel = np.where(nbr[perm] >= 0, inv[np.maximum(nbr[perm], 0)], -1)
    assert np.array_equal(nbr_p, relabel)
    assert rel(ref.conv3(coords[perm], f[perm], w, b), ref.conv3(coords, f, w, b)[perm]) < 1e-14


def test_batch_isolation():
    coords, f, w, b = _shell_case()
    second = coords.copy()
    second[:, 0] = 1
    both = np.concatenate([coords, second])
    out = ref.conv3(both, np.concatenate([f, f]), w, b)
    single = ref.conv3(coords, f, w, b)
    n = len(coords)
    assert np.array_equal(out[:n], single)
    assert np.array_equal(out[n:], single)
    nbr = ref.rulebook(both)
    assert (nbr[:n][nbr[:n] >= 0] < n).all() and (nbr[n:][nbr[n:] >= 0] >= n).all()


def test_rulebook_symmetry_and_centre():
    import synth
    coords = synth.coords_for("2a")
    nbr = ref.rulebook_sorted(coords)
    n = len(coords)
    assert np.array_equal(nbr[:, 13], np.arange(n))
    i, k = np.nonzero(nbr >= 0)
    j = nbr[i, k]
    assert np.array_equal(nbr[j, 26 - k], i)


def test_flip_kernel_mirror():
    coords, f, w, b = _shell_case()
    flipped = np.ascontiguousarray(w[:, ::-1, ::-1, ::-1, :])
    assert rel(ref.conv3(coords, f, w, b, orientation=-1), ref.conv3(coords, f, flipped, b)) < 1e-14


def test_normwise_error_definition():
    assert oracle.normwise_rel_error([1.0, -4.0], [1.0, -4.0]) == 0.0
    assert oracle.normwise_rel_error([1.5, -4.0], [1.0, -4.0]) == pytest.approx(0.125)
    assert oracle.normwise_rel_error(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


def test_elementwise_error_definition():
    ref = np.array([10.0, -0.5, 0.05, 0.0])
    y = np.array([10.5, -0.45, 1.0, 3.0])
    # floor 1e-2 keeps |ref| >= 0.1: entries 0 and 1 -> max(0.05, 0.1)
    assert oracle.elementwise_rel_error(y, ref) == pytest.approx(0.1)
    # floor 1e-3 also keeps 0.05 (|1.0 - 0.05| / 0.05 = 19)
    assert oracle.elementwise_rel_error(y, ref, floor=1e-3) == pytest.approx(19.0)
    assert oracle.elementwise_rel_error(np.zeros(3), np.zeros(3)) == 0.0


def test_componentwise_ratio_definition_and_float32_bound():
    assert oracle.componentwise_ratio([1.0, 0.5], [1.0, 0.25], [2.0, 1.0]) == pytest.approx(0.25)
    assert oracle.componentwise_ratio([0.0, 1.0], [0.0, 1.0], [0.0, 3.0]) == 0.0
    assert oracle.componentwise_ratio([1e-30, 1.0], [0.0, 1.0], [0.0, 3.0]) == np.inf
    # A float32 evaluation of the convolution's sums (products and a left-to-right sum, each
    # rounded to nearest) stays within gamma_K = K u / (1 - K u) of |b| + sum |W||f|, u = 2^-24,
    # K = 27 cin + 1 terms, entry by entry (the standard error bound of recursive summation);
    # the same evaluation with one sign of the magnitude flipped breaks the bound somewhere.
    coords = np.array([[0, z, y, x] for z in range(4) for y in range(4) for x in range(4) if (x + y + z) % 3], np.int32)
    rng = np.random.default_rng(21)
    cin, cout = 16, 8
    f = rng.standard_normal((len(coords), cin))
    w = rng.standard_normal((cout, 3, 3, 3, cin))
    b = rng.standard_normal(cout)
    nbr = oracle.rulebook(coords)
    ref = oracle.conv3_rulebook(nbr, f, w, b)
    mag = oracle.conv3_rulebook(nbr, np.abs(f), np.abs(w), np.abs(b))
    f32, w32 = f.astype(np.float32), w.astype(np.float32).reshape(cout, 27, cin)
    y = np.empty_like(ref)
    for i in range(len(coords)):
        for o in range(cout):
            acc = np.float32(b[o])
            for k in range(27):
                j = nbr[i, k]
                if j >= 0:
                    for c in range(cin):
                        acc = np.float32(acc + np.float32(w32[o, k, c] * f32[j, c]))
            y[i, o] = acc
    # the inputs were rounded to float32 too: compare against the sum of the rounded inputs
    ref32 = oracle.conv3_rulebook(nbr, f32, w32.reshape(cout, 3, 3, 3, cin), b.astype(np.float32))
    mag32 = oracle.conv3_rulebook(nbr, np.abs(f32), np.abs(w32).reshape(cout, 3, 3, 3, cin), np.abs(b.astype(np.float32)))
    u = 2.0 ** -24
    k_terms = 2 * (27 * cin + 1)  # one rounding per product and one per addition
    gamma = k_terms * u / (1 - k_terms * u)
    ratio = oracle.componentwise_ratio(y, ref32, mag32)
    assert 0.0 < ratio <= gamma
    assert oracle.componentwise_ratio(y, ref32, mag32 * 1e-6) > gamma  # a magnitude far too small fails
    assert np.all(mag >= np.abs(ref))

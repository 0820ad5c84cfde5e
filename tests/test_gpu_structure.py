"""GPU parity of the structure ops (subdivide, child map, downsample, cached and masked upsample)
through the C ABI against the CPU oracle.

Coordinates, parent indices and rulebooks are compared bit for bit; max pooling and every
feature copy are exact, so they are compared bit for bit too; mean pooling sums in float32 and
rounds once, so it is held to the normwise bar of the convolution (1e-5 fp32, 1e-2 fp16 / bf16),
and one test pins its float32 summation order (ascending fine row within a cell) bit for bit.
Multi-million-voxel sets are checked through properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_amd as sc
import synth
from oracle import structure_ref as st

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sc.load_library()


def random_sites(seed, batch, lo, hi, occupancy):
    rng = np.random.default_rng(seed)
    g = hi - lo
    rows = []
    for b in range(batch):
        zyx = np.argwhere(rng.random((g, g, g)) < occupancy) + lo
        rows.append(np.concatenate([np.full((len(zyx), 1), b), zyx], axis=1))
    return np.concatenate(rows, axis=0).astype(np.int32)


def shuffled(c, seed):
    return c[np.random.default_rng(seed).permutation(len(c))]


def dev_coords(c):
    return torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).to(DEV)


def values(n, c, dtype, seed):
    x = np.random.default_rng(seed).standard_normal((n, c))
    return synth.round_to(x, dtype)


def host(t):
    torch.cuda.synchronize()
    return t.cpu()


COORD_CASES = {
    "tiny": lambda: np.array([[0, 1, -1, 3], [1, 0, 0, 0]], dtype=np.int32),
    "random_neg_3b": lambda: random_sites(1, 3, -7, 9, 0.2),
    "shell64_torus": lambda: synth.coords_for("2a"),
    "shuffled_shell16": lambda: shuffled(synth.coords_for("1"), 3),
}


# ----------------------------------------------------------------- subdivide

@pytest.mark.parametrize("case", sorted(COORD_CASES))
def test_subdivide_coords_and_parent(case):
    c = COORD_CASES[case]()
    print(f"subdivide {case}: n={len(c)}", flush=True)
    want, _, parent = st.subdivide(c)
    with sc.sparse_subdivide(dev_coords(c)) as s:
        assert (s.n_coarse, s.n_fine, s.kind) == (len(c), 8 * len(c), sc.SUBM_SUBDIVIDE)
        assert np.array_equal(host(s.fine_coords()).numpy(), want)
        assert np.array_equal(host(s.parent()).numpy(), parent)
        assert np.array_equal(host(s.coarse_coords()).numpy(), c)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("channels", [1, 5, 64, 128])
def test_subdivide_features_exact(dtype, channels):
    c = random_sites(2, 2, -4, 6, 0.3)
    f = values(len(c), channels, dtype, 10 + channels)
    _, want, _ = st.subdivide(c, f.double().numpy())
    with sc.sparse_subdivide(dev_coords(c)) as s:
        got = host(sc.sparse_upsample_forward(s, f.to(DEV)))
    assert got.dtype == TDT[dtype]
    assert np.array_equal(got.double().numpy(), want)


@pytest.mark.parametrize("case", ["random_neg_3b", "shell64_torus", "shuffled_shell16"])
def test_child_map_matches_oracle_rulebook(case):
    c = COORD_CASES[case]()
    print(f"child map {case}: n={len(c)}", flush=True)
    fine, _, _ = st.subdivide(c)
    want = oracle.rulebook_sorted(fine)
    with sc.sparse_indice_map_build(dev_coords(c)) as pm, sc.sparse_subdivide(dev_coords(c)) as s:
        with sc.sparse_indice_map_subdivide(pm, s) as cm:
            assert cm.mode == sc.SUBM_MAP_SUBDIVIDED
            got = host(sc.sparse_indice_map_copy_nbr(cm)).numpy()
            assert np.array_equal(got, want)
            counts = sc.sparse_indice_map_offset_counts(cm)
            assert counts == (want >= 0).sum(axis=0).tolist()
            assert cm.pairs == int((want >= 0).sum())


def test_child_map_drives_the_convolution_bit_exactly():
    c = synth.coords_for("2a")
    cin, cout = 64, 64
    with sc.sparse_subdivide(dev_coords(c)) as s, sc.sparse_indice_map_build(dev_coords(c)) as pm:
        fine = s.fine_coords()
        f = values(s.n_fine, cin, "bf16", 7).to(DEV)
        w = synth.round_to(np.random.default_rng(8).standard_normal((cout, 3, 3, 3, cin)) * 0.03, "bf16").to(DEV)
        with sc.sparse_indice_map_subdivide(pm, s) as cm, sc.sparse_indice_map_build(fine) as bm:
            a = host(sc.subm_conv3d_forward(cm, f, w))
            b = host(sc.subm_conv3d_forward(bm, f, w))
    assert torch.equal(a, b)


def test_subdivide_three_rounds_full_size():
    """Three subdivisions of the 64^3 shell and torus (22,406 -> 11,471,872 children), each child
    map derived from its parent map, checked by properties that hold at any size (the doubled
    parent of every child, every rulebook entry's coordinate difference, symmetry) and, at the
    last level, in full against the oracle: its subdivided coordinates and their rulebook."""
    base = synth.coords_for("2a")
    coords = dev_coords(base)
    pm = sc.sparse_indice_map_build(coords)
    for level in range(3):
        s = sc.sparse_subdivide(coords)
        cm = sc.sparse_indice_map_subdivide(pm, s)
        fine = s.fine_coords()
        par = s.parent().long()
        cpar = coords[par]
        assert torch.equal(fine[:, 0], cpar[:, 0])
        assert torch.equal(fine[:, 1:] >> 1, cpar[:, 1:])
        nbr = sc.sparse_indice_map_copy_nbr(cm).long()
        rows = torch.arange(s.n_fine, device=DEV)
        for k in range(27):
            j = nbr[:, k]
            hit = j >= 0
            d = torch.tensor(oracle.tap_offset(k), device=DEV, dtype=torch.int32)
            assert torch.equal(fine[j[hit]][:, 1:] - fine[rows[hit]][:, 1:], d.expand(int(hit.sum()), 3))
        # symmetry: j is i's neighbour at d exactly when i is j's neighbour at -d
        for k in range(27):
            j = nbr[:, k]
            hit = j >= 0
            assert torch.equal(nbr[j[hit], 26 - k], rows[hit])
        assert int((nbr >= 0).sum()) == cm.pairs
        if level == 2:
            # the last level against the hashing build on the same 11.5 M coordinates
            with sc.sparse_indice_map_build(fine) as bm:
                assert torch.equal(sc.sparse_indice_map_copy_nbr(bm).long(), nbr)
                assert sc.sparse_indice_map_offset_counts(bm) == sc.sparse_indice_map_offset_counts(cm)
            # and against the oracle: three rounds of its subdivision of the base set, then its
            # rulebook of the 11.5 M children (bit for bit, coordinates and rulebook)
            want = base
            for _ in range(3):
                want, _, _ = oracle.structure_ref.subdivide(want)
            assert np.array_equal(fine.cpu().numpy(), want)
            assert np.array_equal(nbr.int().cpu().numpy(), oracle.rulebook_sorted(want))
            print("  level 3 equals the oracle's subdivision and rulebook", flush=True)
        torch.cuda.synchronize()
        print(f"  level {level + 1}: {s.n_fine} children, {cm.pairs} pairs", flush=True)
        pm.free()
        pm, coords = cm, fine
        s.free()
    pm.free()


# ----------------------------------------------------------------- downsample / cached upsample

DOWN_CASES = {
    "tiny_golden": lambda: np.array([[0, 3, 1, -1], [0, 2, 0, -2], [0, -1, 0, 0], [1, 0, 0, 0], [0, 2, 1, -1]],
                                    dtype=np.int32),
    "random_neg_3b": lambda: random_sites(4, 3, -9, 7, 0.25),
    "shuffled_random": lambda: shuffled(random_sites(5, 2, -5, 11, 0.4), 6),
    "shell128": lambda: synth.coords_for("3a"),
    "single": lambda: np.array([[4, -3, 5, 7]], dtype=np.int32),
}


@pytest.mark.parametrize("case", sorted(DOWN_CASES))
def test_downsample_structure(case):
    c = DOWN_CASES[case]()
    print(f"downsample {case}: n={len(c)}", flush=True)
    coarse, _, parent = st.downsample(c)
    with sc.sparse_downsample_build(dev_coords(c)) as s:
        assert (s.n_fine, s.n_coarse, s.kind) == (len(c), len(coarse), sc.SUBM_DOWNSAMPLE)
        assert np.array_equal(host(s.coarse_coords()).numpy(), coarse)
        assert np.array_equal(host(s.parent()).numpy(), parent)
        assert np.array_equal(host(s.fine_coords()).numpy(), c)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("channels", [1, 5, 64, 128])
def test_downsample_features(dtype, channels):
    c = DOWN_CASES["random_neg_3b"]()
    f = values(len(c), channels, dtype, 20 + channels)
    f64 = f.double().numpy()
    _, want_max, parent = st.downsample(c, f64, "max")
    _, want_mean, _ = st.downsample(c, f64, "mean")
    with sc.sparse_downsample_build(dev_coords(c)) as s:
        fd = f.to(DEV)
        got_max = host(sc.sparse_downsample_forward(s, fd, sc.SUBM_POOL_MAX))
        got_mean = host(sc.sparse_downsample_forward(s, fd, sc.SUBM_POOL_MEAN))
        assert np.array_equal(got_max.double().numpy(), want_max)
        err = oracle.normwise_rel_error(got_mean.double().numpy(), want_mean)
        print(f"  mean {dtype} C={channels}: normwise err {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        # the two modes differ on this set (cells with several members)
        assert not torch.equal(got_max, got_mean)
        # cache-paired upsample: every fine row takes its cell's pooled row
        up = host(sc.sparse_upsample_forward(s, got_mean.to(DEV)))
        assert torch.equal(up, got_mean[torch.from_numpy(parent)])


def test_downsample_needs_explicit_mode():
    c = DOWN_CASES["tiny_golden"]()
    with sc.sparse_downsample_build(dev_coords(c)) as s:
        f = torch.ones((len(c), 8), dtype=torch.bfloat16, device=DEV)
        for mode in (0, 3, -1):
            with pytest.raises(sc.SubmError) as e:
                sc.sparse_downsample_forward(s, f, mode)
            assert e.value.name == "SUBM_ERR_INVALID_ARG"


def test_downsample_undoes_subdivide_on_device():
    c = shuffled(synth.coords_for("2a"), 9)
    f = values(len(c), 64, "bf16", 30).to(DEV)
    with sc.sparse_subdivide(dev_coords(c)) as s:
        fine = s.fine_coords()
        ff = sc.sparse_upsample_forward(s, f)
        with sc.sparse_downsample_build(fine) as d:
            order = np.lexsort(c.T[::-1])
            assert np.array_equal(host(d.coarse_coords()).numpy(), c[order])
            for mode in (sc.SUBM_POOL_MAX, sc.SUBM_POOL_MEAN):
                pooled = host(sc.sparse_downsample_forward(d, ff, mode))
                assert torch.equal(pooled, f.cpu()[torch.from_numpy(order)])


def clustered_sites(seed, cells, span):
    """Shuffled fine rows of `cells` random coarse cells (b in [0, 3), z, y, x in [-span, span)),
    each with 1..8 distinct children."""
    rng = np.random.default_rng(seed)
    cc = np.unique(np.concatenate([rng.integers(0, 3, (cells, 1)), rng.integers(-span, span, (cells, 3))], axis=1),
                   axis=0)
    kids = rng.random((len(cc), 8)) < rng.random((len(cc), 1))
    kids[np.arange(len(cc)), rng.integers(0, 8, len(cc))] = True
    ci, s = np.nonzero(kids)
    off = np.stack([(s >> 2) & 1, (s >> 1) & 1, s & 1], axis=1)
    fine = np.concatenate([cc[ci, :1], 2 * cc[ci, 1:] + off], axis=1).astype(np.int32)
    return shuffled(fine, seed + 1)


@pytest.mark.parametrize("span", [40, 3000])  # 23- and 41-bit cell keys: 3 and 5 sort passes
def test_downsample_mean_sums_members_in_ascending_row_order(span):
    # The members of a cell are summed in float32 in ascending fine-row order.  Values spread over
    # 2^-10 .. 2^30 with random signs make each float32 sum depend on that order, so the mean pins
    # that the sort of the cells keeps equal keys in input order (rows shuffled, ~100 k of them,
    # so equal keys meet across many 4096-row sort tiles).
    c = clustered_sites(40 + span, 25000, span)
    n = len(c)
    rng = np.random.default_rng(span)
    f = (rng.choice([-1.0, 1.0], (n, 8)) * rng.random((n, 8)) * 2.0 ** rng.integers(-10, 31, (n, 8))).astype(np.float32)
    coarse, _, parent = st.downsample(c)
    order = np.lexsort((np.arange(n), parent))  # members of each cell in ascending row order
    first = np.searchsorted(parent[order], np.arange(len(coarse)))
    cnt = np.bincount(parent, minlength=len(coarse))
    acc = f[order[first]].copy()
    for k in range(1, 8):
        has = cnt > k
        acc[has] = (acc[has] + f[order[first[has] + k]]).astype(np.float32)
    want = (acc / cnt[:, None].astype(np.float32)).astype(np.float32)
    with sc.sparse_downsample_build(dev_coords(c)) as s:
        assert np.array_equal(host(s.coarse_coords()).numpy(), coarse)
        assert np.array_equal(host(s.parent()).numpy(), parent)
        got = host(sc.sparse_downsample_forward(s, torch.from_numpy(f).to(DEV), sc.SUBM_POOL_MEAN)).numpy()
    print(f"  n={n} cells={len(coarse)} max members={cnt.max()}", flush=True)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_downsample_undoes_subdivide_at_20m_rows():
    # 20.4 M children of the config-5 set: the sort's per-tile digit counts (256 x 4,981 tiles)
    # take the multi-workgroup prefix sum; the cells must come back as the parent set, in order.
    c = synth.coords_for("5")
    order = np.lexsort(c.T[::-1])  # the set is parent-major, not in (b, z, y, x) order
    rank = np.empty(len(c), dtype=np.int64)
    rank[order] = np.arange(len(c))
    coords = dev_coords(c)
    with sc.sparse_subdivide(coords) as s:
        fine = s.fine_coords()
        with sc.sparse_downsample_build(fine) as d:
            assert d.n_coarse == len(c)
            assert torch.equal(d.coarse_coords(), dev_coords(c[order]))
            assert torch.equal(d.parent().long(), torch.from_numpy(rank).to(DEV)[s.parent().long()])
            torch.cuda.synchronize()
            print(f"  {s.n_fine} children -> {d.n_coarse} cells", flush=True)


def test_downsample_full_size_properties():
    """Config-5 coordinate set (2.55 M voxels): the coarse rows are strictly ascending, every fine
    row lies in its parent cell, and the member counts add up."""
    c = synth.coords_for("5")
    coords = dev_coords(c)
    with sc.sparse_downsample_build(coords) as s:
        coarse = s.coarse_coords().long()
        par = s.parent().long()
        key = ((coarse[:, 0] * 65536 + coarse[:, 1]) * 65536 + coarse[:, 2]) * 65536 + coarse[:, 3]
        assert bool((key[1:] > key[:-1]).all())
        fine = coords.long()
        assert torch.equal(fine[:, 0], coarse[par][:, 0])
        assert torch.equal(torch.div(fine[:, 1:], 2, rounding_mode="floor"), coarse[par][:, 1:])
        counts = torch.bincount(par, minlength=s.n_coarse)
        assert int(counts.min()) >= 1 and int(counts.sum()) == len(c)
        # the mean of ones is one in every cell
        ones = torch.ones((len(c), 64), dtype=torch.bfloat16, device=DEV)
        assert bool((sc.sparse_downsample_forward(s, ones, sc.SUBM_POOL_MEAN) == 1).all())
        torch.cuda.synchronize()
        print(f"  {len(c)} voxels -> {s.n_coarse} cells", flush=True)


# ----------------------------------------------------------------- masked upsample

@pytest.mark.parametrize("seed,p", [(1, 0.3), (2, 0.0), (3, 1.0), (4, 0.6)])
def test_masked_upsample(seed, p):
    c = random_sites(seed, 2, -6, 6, 0.3)
    mask = (np.random.default_rng(seed).random((len(c), 8)) < p).astype(np.uint8)
    mask[::7] = 0  # rows with no flagged child
    mask[1::5] *= 3  # any nonzero byte flags
    f = values(len(c), 24, "bf16", 40 + seed)
    want, want_f, parent = st.upsample_masked(c, mask, f.double().numpy())
    with sc.sparse_upsample_masked_build(dev_coords(c), torch.from_numpy(mask).to(DEV)) as s:
        assert (s.n_coarse, s.n_fine, s.kind) == (len(c), len(want), sc.SUBM_UPSAMPLE_MASKED)
        if len(want):
            assert np.array_equal(host(s.fine_coords()).numpy(), want)
            assert np.array_equal(host(s.parent()).numpy(), parent)
            got = host(sc.sparse_upsample_forward(s, f.to(DEV)))
            assert np.array_equal(got.double().numpy(), want_f)
        # pooling the children back: parents without children get 0, the others their value
        back = host(sc.sparse_downsample_forward(s, sc.sparse_upsample_forward(s, f.to(DEV)), sc.SUBM_POOL_MAX))
        has = np.zeros(len(c), dtype=bool)
        has[parent] = True
        assert torch.equal(back[torch.from_numpy(has)], f[torch.from_numpy(has)])
        assert bool((back[torch.from_numpy(~has)] == 0).all())


def test_masked_golden_on_device():
    c = np.array([[0, 1, -1, 3], [2, 0, 0, 0], [1, 5, 5, 5]], dtype=np.int32)
    mask = np.array([[0, 1, 1, 0, 0, 0, 0, 1], [0] * 8, [1, 0, 0, 0, 1, 0, 0, 0]], dtype=np.uint8)
    with sc.sparse_upsample_masked_build(dev_coords(c), torch.from_numpy(mask).to(DEV)) as s:
        got = host(s.fine_coords()).numpy().tolist()
    assert got == [[0, 3, -2, 6], [0, 2, -1, 6], [0, 3, -1, 7], [1, 10, 10, 10], [1, 10, 10, 11]]


# ----------------------------------------------------------------- edge cases and errors

def test_empty_inputs():
    e = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    for build in (sc.sparse_subdivide, sc.sparse_downsample_build):
        with build(e) as s:
            assert (s.n_coarse, s.n_fine) == (0, 0)
            x = torch.empty((0, 8), dtype=torch.bfloat16, device=DEV)
            assert sc.sparse_upsample_forward(s, x).shape == (0, 8)
    with sc.sparse_upsample_masked_build(e, torch.empty((0, 8), dtype=torch.uint8, device=DEV)) as s:
        assert (s.n_coarse, s.n_fine) == (0, 0)
    c = np.array([[0, 0, 0, 0]], dtype=np.int32)
    with sc.sparse_upsample_masked_build(dev_coords(c), torch.zeros((1, 8), dtype=torch.uint8, device=DEV)) as s:
        assert s.n_fine == 0
        out = host(sc.sparse_downsample_forward(s, torch.empty((0, 4), device=DEV), sc.SUBM_POOL_MEAN))
        assert torch.equal(out, torch.zeros((1, 4)))


def test_range_errors():
    big = np.array([[0, 1 << 30, 0, 0]], dtype=np.int32)
    with pytest.raises(sc.SubmError) as e:
        sc.sparse_subdivide(dev_coords(big))
    assert e.value.name == "SUBM_ERR_COORD_RANGE"
    neg_b = np.array([[-1, 0, 0, 0]], dtype=np.int32)
    for build in (sc.sparse_subdivide, sc.sparse_downsample_build):
        with pytest.raises(sc.SubmError) as e:
            build(dev_coords(neg_b))
        assert e.value.name == "SUBM_ERR_COORD_RANGE"
    wide = np.array([[0, 0, 0, 0], [0, 0, 0, 65535]], dtype=np.int32)
    with pytest.raises(sc.SubmError) as e:
        sc.sparse_downsample_build(dev_coords(wide))
    assert e.value.name == "SUBM_ERR_COORD_RANGE"
    ok = np.array([[0, 0, 0, -32767], [0, 0, 0, 32767]], dtype=np.int32)
    with sc.sparse_downsample_build(dev_coords(ok)) as s:
        assert host(s.coarse_coords()).numpy().tolist() == [[0, 0, 0, -16384], [0, 0, 0, 16383]]


def test_child_map_argument_errors():
    c = dev_coords(np.array([[0, 0, 0, 0], [0, 0, 0, 1]], dtype=np.int32))
    with sc.sparse_indice_map_build(c) as pm, sc.sparse_downsample_build(c) as d:
        with pytest.raises(sc.SubmError) as e:
            sc.sparse_indice_map_subdivide(pm, d)
        assert e.value.name == "SUBM_ERR_INVALID_ARG"
    with sc.sparse_indice_map_build(c[:1].contiguous()) as pm, sc.sparse_subdivide(c) as s:
        with pytest.raises(sc.SubmError) as e:
            sc.sparse_indice_map_subdivide(pm, s)
        assert e.value.name == "SUBM_ERR_SHAPE_MISMATCH"


# ----------------------------------------------------------------- seeded random sweep

@pytest.mark.parametrize("seed", range(12))
def test_random_sets_downsample_subdivide_and_child_map(seed):
    # Random sets (1-3 items, random boxes with negative corners and odd sizes, random occupancy,
    # shuffled rows) through downsample (structure, max, mean, cached upsample), subdivide and the
    # child map, against the oracle.
    rng = np.random.default_rng(500 + seed)
    lo = int(rng.integers(-40, 10))
    c = shuffled(random_sites(600 + seed, int(rng.integers(1, 4)), lo, lo + int(rng.integers(3, 18)),
                              float(rng.uniform(0.05, 0.9))), seed)
    dtype = ["f32", "f16", "bf16"][seed % 3]
    ch = int(rng.choice([1, 3, 8, 64, 96]))
    print(f"seed {seed}: n={len(c)} {dtype} C={ch}", flush=True)
    f = values(len(c), ch, dtype, 700 + seed)
    f64 = f.double().numpy()
    coarse, want_max, parent = st.downsample(c, f64, "max")
    _, want_mean, _ = st.downsample(c, f64, "mean")
    with sc.sparse_downsample_build(dev_coords(c)) as s:
        assert np.array_equal(host(s.coarse_coords()).numpy(), coarse)
        assert np.array_equal(host(s.parent()).numpy(), parent)
        fd = f.to(DEV)
        got_max = host(sc.sparse_downsample_forward(s, fd, sc.SUBM_POOL_MAX))
        got_mean = host(sc.sparse_downsample_forward(s, fd, sc.SUBM_POOL_MEAN))
        assert np.array_equal(got_max.double().numpy(), want_max)
        assert oracle.normwise_rel_error(got_mean.double().numpy(), want_mean) <= TOL[dtype]
        up = host(sc.sparse_upsample_forward(s, got_max.to(DEV)))
        assert torch.equal(up, got_max[torch.from_numpy(parent)])
    fine, _, fparent = st.subdivide(c)
    with sc.sparse_indice_map_build(dev_coords(c)) as m, sc.sparse_subdivide(dev_coords(c)) as s:
        assert np.array_equal(host(s.fine_coords()).numpy(), fine)
        assert np.array_equal(host(s.parent()).numpy(), fparent)
        with sc.sparse_indice_map_subdivide(m, s) as cm:
            assert np.array_equal(host(sc.sparse_indice_map_copy_nbr(cm)).numpy(), oracle.rulebook(fine))

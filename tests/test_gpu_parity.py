"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Rulebook: bit-exact.  Features: normwise relative error max|y - ref| / max|ref|
against the float64 oracle on the same rounded inputs, at most 1e-5 for fp32
storage and 1e-2 for fp16 / bf16 storage (fp32 accumulation, one rounding to
the storage dtype at the end: the rounding alone contributes up to 2^-8 for
bf16 and 2^-11 for fp16), plus the componentwise bound and the elementwise
diagnostic of tests/parity_util.py.

Every row of every configuration is compared with the oracle, the
multi-million-voxel ones included (the oracle's sums run in row chunks on the
host's threads); the componentwise bound is taken on sampled rows there (first
and last tiles plus random rows) and on all rows elsewhere.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_amd as sc
import synth
from parity_util import check_features

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sc.load_library()


@functools.lru_cache(maxsize=None)
def coords_of(key):
    return synth.coords_for(key)


@functools.lru_cache(maxsize=None)
def oracle_nbr(key):
    return oracle.rulebook_sorted(coords_of(key))


def to_dev(t):
    return None if t is None else t.to(DEV)


def as64(t):
    return t.double().cpu().numpy()


def gpu_nbr(m):
    out = sc.sparse_indice_map_copy_nbr(m)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def forward(m, f, w, b):
    out = sc.subm_conv3d_forward(m, to_dev(f), to_dev(w), to_dev(b))
    torch.cuda.synchronize()
    return out.cpu()


def check(out, ref, dtype, what=""):
    err = oracle.normwise_rel_error(as64(out), ref)
    print(f"  {what} normwise err {err:.3e} (tol {TOL[dtype]:g})", flush=True)
    assert err <= TOL[dtype], f"{what}: error {err:.3e} above {TOL[dtype]}"


def sample_rows(n, tile=128, count=4096, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(n, 2 * tile)), np.arange(max(0, n - 2 * tile), n),
                           rng.integers(0, n, count)])
    return np.unique(rows)


# ----------------------------------------------------------------- rulebook, all configs

@pytest.mark.parametrize("key", ["1", "2a", "3a", "3b", "4", "5"])
def test_rulebook_bit_exact(key):
    coords = coords_of(key)
    want = oracle_nbr(key)
    if key == "1":
        assert np.array_equal(want, oracle.rulebook(coords))
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        got = gpu_nbr(m)
        assert m.n == len(coords)
        assert np.array_equal(got, want)
        assert m.pairs == int((want >= 0).sum())
        assert sc.sparse_indice_map_offset_counts(m) == (want >= 0).sum(axis=0).tolist()
    print(f"  config {key}: N={len(coords)} pairs={int((want >= 0).sum())}", flush=True)


@pytest.mark.parametrize("key", ["1", "2a", "3a", "3b", "4", "5"])
@pytest.mark.parametrize("mode", ["hash", "grid"])
def test_rulebook_same_from_both_structures(key, mode):
    req = {"hash": sc.SUBM_MAP_HASH, "grid": sc.SUBM_MAP_GRID}[mode]
    with sc.sparse_indice_map_build_ex(torch.from_numpy(coords_of(key)).to(DEV), req) as m:
        assert m.mode == req
        assert np.array_equal(gpu_nbr(m), oracle_nbr(key))
        assert sc.sparse_indice_map_offset_counts(m) == (oracle_nbr(key) >= 0).sum(axis=0).tolist()


def test_automatic_structure_choice():
    # Every workload here has a bounding box within the grid budget; two far-apart voxels do not.
    for key in ("3a", "3b", "4", "5"):
        with sc.sparse_indice_map_build(torch.from_numpy(coords_of(key)).to(DEV)) as m:
            assert m.mode == sc.SUBM_MAP_GRID, key
    far = torch.tensor([[0, 0, 0, 0], [0, 60000, 60000, 60000]], dtype=torch.int32, device=DEV)
    with sc.sparse_indice_map_build(far) as m:
        assert m.mode == sc.SUBM_MAP_HASH
        assert gpu_nbr(m).tolist() == [[-1] * 13 + [0] + [-1] * 13, [-1] * 13 + [1] + [-1] * 13]


# ----------------------------------------------------------------- convolution, all configs

def cfg_tensors(key, layer, cin=None, cout=None):
    c = synth.config(key)
    cin = cin or c.cin
    cout = cout or c.cout
    n = len(coords_of(key))
    f = synth.feats_for(c.number, layer, n, cin, c.dtype)
    w = synth.weight_for(c.number, layer, c.ksize, cin, cout, c.dtype)
    b = synth.bias_for(c.number, layer, cout, c.dtype)
    return f, w, b


def test_config1_tiny_fp32_full():
    coords = coords_of("1")
    f, w, b = cfg_tensors("1", 0)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, b)
    check(out, oracle.conv3(coords, as64(f), as64(w), as64(b)), "f32", "config 1")
    check_features(out, oracle_nbr("1"), as64(f), as64(w), as64(b), "f32", "config 1")


def test_config2_fp16_k3_and_k1_full():
    coords = coords_of("2a")
    f3, w3, b3 = cfg_tensors("2a", 0)
    f1, w1, b1 = cfg_tensors("2b", 1)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out3 = forward(m, f3, w3, b3)
        out1 = forward(m, f1, w1, b1)
    out1_nomap = forward(None, f1, w1, b1)
    check_features(out3, oracle_nbr("2a"), as64(f3), as64(w3), as64(b3), "f16", "config 2a k3")
    ref1 = oracle.conv1(as64(f1), as64(w1), as64(b1))
    check(out1, ref1, "f16", "config 2b k1")
    assert torch.equal(out1, out1_nomap)


def test_config3a_shell_bf16_full():
    coords = coords_of("3a")
    f, w, b = cfg_tensors("3a", 0)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, b)
    check_features(out, oracle_nbr("3a"), as64(f), as64(w), as64(b), "bf16", "config 3a")
    # spot-check the sampled-row path against the dictionary oracle as well
    rows = sample_rows(len(coords), count=256)
    check(out[rows], oracle.conv3(coords, as64(f), as64(w), as64(b), rows=rows), "bf16", "config 3a (dict rows)")


def test_config3b_dense_bf16_full():
    coords = coords_of("3b")
    f, w, b = cfg_tensors("3b", 0)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, b)
    check_features(out, oracle_nbr("3b"), as64(f), as64(w), as64(b), "bf16", "config 3b",
                   mag_rows=sample_rows(len(coords)))


@pytest.mark.parametrize("layer", range(4))
def test_config4_layers_on_a_shared_map_full(layer):
    key = "4"
    c = synth.config(key)
    coords = coords_of(key)
    f = synth.feats_for(c.number, 0, len(coords), c.cin, c.dtype)
    fd = f.to(DEV)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        for lay in range(layer + 1):  # the earlier layers run on the map first, as in the stack
            w = synth.weight_for(c.number, lay, 3, c.cin, c.cout, c.dtype)
            b = synth.bias_for(c.number, lay, c.cout, c.dtype)
            out = sc.subm_conv3d_forward(m, fd, w.to(DEV), b.to(DEV))
        torch.cuda.synchronize()
    check_features(out.cpu(), oracle_nbr(key), as64(f), as64(w), as64(b), c.dtype, f"config 4 layer {layer}",
                   mag_rows=sample_rows(len(coords)))


@pytest.mark.parametrize("layer", range(8))
def test_config5_chained_layers_full(layer):
    key = "5"
    c = synth.config(key)
    coords = coords_of(key)
    x = synth.feats_for(c.number, 0, len(coords), c.cin, c.dtype).to(DEV)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        for lay in range(layer + 1):
            w = synth.weight_for(c.number, lay, 3, c.cin, c.cout, c.dtype)
            b = synth.bias_for(c.number, lay, c.cout, c.dtype)
            x_in = x
            x = sc.subm_conv3d_forward(m, x_in, w.to(DEV), b.to(DEV))
        torch.cuda.synchronize()
    # The oracle consumes the GPU's stored input of this layer (same rounded values).
    check_features(x.cpu(), oracle_nbr(key), as64(x_in), as64(w), as64(b), c.dtype, f"config 5 layer {layer}",
                   mag_rows=sample_rows(len(coords), count=2048))


# ----------------------------------------------------------------- edge cases

def small_case(dtype, cin, cout, key="1", seed=0, ksize=3):
    coords = coords_of(key)
    rng = np.random.default_rng(seed)
    n = len(coords)
    f = synth.round_to(rng.standard_normal((n, cin)), dtype)
    w = synth.round_to(rng.standard_normal((cout, ksize, ksize, ksize, cin)) / np.sqrt(ksize ** 3 * cin), dtype)
    b = synth.round_to(rng.standard_normal(cout) * 0.3, dtype)
    return coords, f, w, b


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cin,cout", [(3, 5), (16, 1), (8, 17), (24, 33), (64, 65), (32, 129), (200, 160), (136, 40)])
def test_channel_shapes_and_tails(dtype, cin, cout):
    coords, f, w, b = small_case(dtype, cin, cout)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, b)
    check(out, oracle.conv3(coords, as64(f), as64(w), as64(b)), dtype, f"{dtype} {cin}->{cout}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cin,cout", [(3, 5), (64, 64), (128, 128), (40, 200)])
def test_k1_matches_linear(dtype, cin, cout):
    coords, f, w, b = small_case(dtype, cin, cout, key="2a", ksize=1)
    out = forward(None, f, w, b)
    check(out, oracle.conv1(as64(f), as64(w), as64(b)), dtype, f"k1 {dtype} {cin}->{cout}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_pointers_take_the_elementwise_path(dtype):
    coords, f, w, b = small_case(dtype, 16, 16)
    n = len(coords)
    big = torch.empty(n * 16 + 1, dtype=TDT[dtype], device=DEV)
    fd = big[1:].view(n, 16)
    fd.copy_(f.to(DEV))
    obig = torch.empty(n * 16 + 1, dtype=TDT[dtype], device=DEV)
    od = obig[1:].view(n, 16)
    assert fd.data_ptr() % 16 != 0 and od.data_ptr() % 16 != 0
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        sc.subm_conv3d_forward(m, fd, w.to(DEV), b.to(DEV), out=od)
        aligned = sc.subm_conv3d_forward(m, f.to(DEV), w.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    check(od.cpu(), oracle.conv3(coords, as64(f), as64(w), as64(b)), dtype, "misaligned")
    assert torch.equal(od.cpu(), aligned.cpu())


def test_no_bias():
    coords, f, w, _ = small_case("bf16", 32, 32)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, None)
    check(out, oracle.conv3(coords, as64(f), as64(w), None), "bf16", "no bias")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_identity_kernel_is_bit_exact(dtype):
    coords, f, _, _ = small_case(dtype, 64, 64, key="2a")
    w = torch.zeros((64, 3, 3, 3, 64), dtype=TDT[dtype])
    w[:, 1, 1, 1, :] = torch.eye(64, dtype=TDT[dtype])
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, None)
    assert torch.equal(out, f)


def test_deterministic_bitwise():
    coords, f, w, b = small_case("bf16", 128, 128, key="2a")
    cd = torch.from_numpy(coords).to(DEV)
    with sc.sparse_indice_map_build(cd) as m1, sc.sparse_indice_map_build(cd) as m2:
        assert np.array_equal(gpu_nbr(m1), gpu_nbr(m2))
        a = forward(m1, f, w, b)
        bb = forward(m2, f, w, b)
    assert torch.equal(a, bb)


def test_empty_input():
    c = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    with sc.sparse_indice_map_build(c) as m:
        assert (m.n, m.pairs) == (0, 0)
        assert sc.sparse_indice_map_copy_nbr(m).shape == (0, 27)
        f = torch.zeros((0, 8), dtype=torch.bfloat16, device=DEV)
        w = torch.zeros((4, 3, 3, 3, 8), dtype=torch.bfloat16, device=DEV)
        out = sc.subm_conv3d_forward(m, f, w)
        assert out.shape == (0, 4)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_single_voxel_sees_only_centre(mode):
    coords = np.array([[3, -7, 100, 2]], dtype=np.int32)
    rng = np.random.default_rng(4)
    f = torch.from_numpy(rng.standard_normal((1, 5)).astype(np.float32))
    w = torch.from_numpy(rng.standard_normal((6, 3, 3, 3, 5)).astype(np.float32))
    b = torch.from_numpy(rng.standard_normal(6).astype(np.float32))
    with sc.sparse_indice_map_build_ex(torch.from_numpy(coords).to(DEV), mode) as m:
        assert gpu_nbr(m).tolist() == [[-1] * 13 + [0] + [-1] * 13]
        out = forward(m, f, w, b)
    check(out, oracle.conv3(coords, as64(f), as64(w), as64(b)), "f32", "single voxel")


@pytest.mark.parametrize("mode", [1, 2])
def test_shuffled_rows_and_batch_isolation(mode):
    base = coords_of("2a")
    rng = np.random.default_rng(8)
    two = np.concatenate([base, base * np.array([0, 1, 1, 1], np.int32) + np.array([1, 0, 0, 0], np.int32)])
    perm = rng.permutation(len(two))
    coords = two[perm]
    with sc.sparse_indice_map_build_ex(torch.from_numpy(coords).to(DEV), mode) as m:
        assert m.mode == mode
        assert np.array_equal(gpu_nbr(m), oracle.rulebook_sorted(coords))
        f = synth.round_to(rng.standard_normal((len(coords), 16)), "f32")
        w = synth.round_to(rng.standard_normal((8, 3, 3, 3, 16)) * 0.05, "f32")
        out = forward(m, f, w, None)
    check(out, oracle.conv3_rulebook(oracle.rulebook_sorted(coords), as64(f), as64(w)), "f32", "shuffled 2-batch")


@pytest.mark.parametrize("mode", [1, 2])
def test_translation_to_large_and_negative_coordinates(mode):
    base = coords_of("1")
    for shift in ([0, -2 ** 31, 5, -7], [0, 2 ** 31 - 20, -2 ** 31, 2 ** 31 - 18], [65533, 0, 0, 0]):
        moved = (base.astype(np.int64) + np.array(shift, np.int64)).astype(np.int32)
        with sc.sparse_indice_map_build_ex(torch.from_numpy(moved).to(DEV), mode) as m:
            assert m.mode == mode
            assert np.array_equal(gpu_nbr(m), oracle_nbr("1")), shift


def test_extent_limits():
    ok = np.array([[0, 0, 0, 0], [0, 0, 0, 1], [0, 65534, 0, 0], [0, 65533, 0, 0]], dtype=np.int32)
    with sc.sparse_indice_map_build(torch.from_numpy(ok).to(DEV)) as m:
        assert np.array_equal(gpu_nbr(m), oracle.rulebook(ok))
    for bad in ([[0, 0, 0, 0], [0, 65535, 0, 0]], [[0, 0, -40000, 0], [0, 0, 30000, 0]],
                [[-1, 0, 0, 0]], [[65535, 0, 0, 0]]):
        with pytest.raises(sc.SubmError) as e:
            sc.sparse_indice_map_build(torch.tensor(bad, dtype=torch.int32, device=DEV))
        assert e.value.name == "SUBM_ERR_COORD_RANGE"


@pytest.mark.parametrize("mode", [1, 2])
def test_duplicates_rejected(mode):
    coords = np.concatenate([coords_of("1"), coords_of("1")[17:18]])
    with pytest.raises(sc.SubmError) as e:
        sc.sparse_indice_map_build_ex(torch.from_numpy(coords).to(DEV), mode)
    assert e.value.name == "SUBM_ERR_DUPLICATE_COORD"


@pytest.mark.parametrize("limit", [None, "3000"])
def test_grid_entries_of_earlier_builds_read_as_absent(monkeypatch, limit):
    # Grid cells keep the entries of earlier builds (told apart by their tags), and the hash table
    # has an area of its own: a subset of a set built after the full set must not see the removed
    # rows, in either structure order; with a tag limit below the set sizes every build refills
    # the grid first.
    if limit is not None:
        monkeypatch.setenv("SUBMCONV_GRID_TAG_LIMIT", limit)
    full = coords_of("2a")
    rng = np.random.default_rng(7)
    seq = [("grid", full), ("grid", full[rng.random(len(full)) < 0.5]), ("hash", full),
           ("grid", full[::3]), ("hash", full[1::2]), ("grid", full[rng.permutation(len(full))]),
           ("grid", full[rng.random(len(full)) < 0.1]), ("grid", coords_of("1"))]
    for step, (mode, c) in enumerate(seq):
        c = np.ascontiguousarray(c)
        req = {"hash": sc.SUBM_MAP_HASH, "grid": sc.SUBM_MAP_GRID}[mode]
        with sc.sparse_indice_map_build_ex(torch.from_numpy(c).to(DEV), req) as m:
            assert m.mode == req
            want = oracle.rulebook_sorted(c)
            assert np.array_equal(gpu_nbr(m), want), f"step {step} ({mode}, {len(c)} rows)"
            assert m.pairs == int((want >= 0).sum())
    dup = np.concatenate([full[::3], full[3:4]])
    with pytest.raises(sc.SubmError) as e:
        sc.sparse_indice_map_build_ex(torch.from_numpy(dup).to(DEV), sc.SUBM_MAP_GRID)
    assert e.value.name == "SUBM_ERR_DUPLICATE_COORD"


def test_shape_mismatch_and_alias_rejected():
    coords, f, w, b = small_case("bf16", 16, 16)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        fd = f.to(DEV)
        with pytest.raises(sc.SubmError) as e:
            sc.subm_conv3d_forward(m, fd[:-1].contiguous(), w.to(DEV), b.to(DEV))
        assert e.value.name == "SUBM_ERR_SHAPE_MISMATCH"
        w1 = torch.zeros((16, 1, 1, 1, 16), dtype=torch.bfloat16, device=DEV)
        with pytest.raises(sc.SubmError) as e:
            sc.subm_conv3d_forward(None, fd, w1, out=fd)
        assert e.value.name == "SUBM_ERR_INVALID_ARG"


# ----------------------------------------------------------------- fast-path tile configurations

TILES = ["r192c128s128", "r192c128s64", "r128c128s64", "r256c128s64", "r384c128s64", "r256c128s128",
         "r192c64s128", "r256c64s64", "r384c64s64", "r128c64s64", "r256c32s64", "r128c32s64",
         "ws256c128s64", "ws192c128s64", "ws256c128s64b", "ws384c64s64", "ws512c64s64",
         "ws192c128s128k", "ws192c128s64k", "ws256c64s128k", "ws192c64s128k"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype,cin,cout", [("bf16", 128, 128), ("f16", 64, 64), ("bf16", 96, 48), ("f16", 200, 136),
                                            ("bf16", 8, 40), ("bf16", 40, 256)])
def test_tile_configs(monkeypatch, tile, dtype, cin, cout):
    monkeypatch.setenv("SUBMCONV_TILE", tile)
    coords, f, w, b = small_case(dtype, cin, cout, key="2a")
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, b)
    check(out, oracle.conv3_rulebook(oracle_nbr("2a"), as64(f), as64(w), as64(b)), dtype,
          f"tile {tile} {dtype} {cin}->{cout}")
    _, f1, w1, b1 = small_case(dtype, cin, cout, key="1", ksize=1)
    out1 = forward(None, f1, w1, b1)
    check(out1, oracle.conv1(as64(f1), as64(w1), as64(b1)), dtype, f"tile {tile} k1")


@pytest.mark.parametrize("tile", [t for t in TILES if "c128" in t])
def test_tile_configs_headline_shell(monkeypatch, tile):
    monkeypatch.setenv("SUBMCONV_TILE", tile)
    coords = coords_of("3a")
    f, w, b = cfg_tensors("3a", 0)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = forward(m, f, w, b)
    check(out, oracle.conv3_rulebook(oracle_nbr("3a"), as64(f), as64(w), as64(b)), "bf16", f"3a tile {tile}")


# ----------------------------------------------------------------- persistent tile walk

# The default 16-bit k = 3 launch above 32 output channels walks several row tiles per workgroup
# (one workgroup per compute unit); SUBMCONV_PERSISTENT=0 selects one tile per workgroup.  Both
# run the same stages in the same order and round once, so their outputs agree bit for bit.
PERSISTENT_CASES = [("bf16", 128, 128, "2a"), ("f16", 64, 64, "2a"), ("bf16", 96, 48, "1"), ("f16", 200, 136, "2a"),
                    ("bf16", 40, 256, "2a"), ("bf16", 64, 40, "2a"), ("bf16", 8, 72, "1"), ("f16", 64, 36, "2a")]


@pytest.mark.parametrize("dtype,cin,cout,key", PERSISTENT_CASES)
def test_persistent_walk_matches_oracle_and_one_tile_launch(monkeypatch, dtype, cin, cout, key):
    monkeypatch.delenv("SUBMCONV_TILE", raising=False)
    monkeypatch.setenv("SUBMCONV_POOL", "0")
    coords, f, w, b = small_case(dtype, cin, cout, key=key, seed=3)
    outs = {}
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        for mode in ("1", "0"):
            monkeypatch.setenv("SUBMCONV_PERSISTENT", mode)
            outs[mode] = forward(m, f, w, b)
    check(outs["1"], oracle.conv3_rulebook(oracle_nbr(key), as64(f), as64(w), as64(b)), dtype,
          f"persistent {dtype} {cin}->{cout} on {key}")
    assert torch.equal(outs["1"], outs["0"])


@pytest.mark.parametrize("key", ["3a", "3b", "4"])
def test_persistent_walk_full_size(monkeypatch, key):
    # 3a: 708 tiles, two or three per workgroup; 3b: 43 per workgroup; 4: the 64-channel tile.
    # (SUBMCONV_POOL=0: 3a and 3b would take the neighbour-pool kernel otherwise.)
    monkeypatch.delenv("SUBMCONV_TILE", raising=False)
    monkeypatch.setenv("SUBMCONV_POOL", "0")
    coords = coords_of(key)
    f, w, b = cfg_tensors(key, 0)
    fd, wd, bd = f.to(DEV), w.to(DEV), b.to(DEV)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        monkeypatch.setenv("SUBMCONV_PERSISTENT", "1")
        y1 = sc.subm_conv3d_forward(m, fd, wd, bd)
        monkeypatch.setenv("SUBMCONV_PERSISTENT", "0")
        y0 = sc.subm_conv3d_forward(m, fd, wd, bd)
        torch.cuda.synchronize()
    assert torch.equal(y1, y0), f"{key}: persistent and one-tile launches differ"
    rows = sample_rows(len(coords), count=1024, seed=5)
    ref = oracle.conv3_rulebook(oracle_nbr(key), as64(f), as64(w), as64(b), rows=rows)
    check(y1.cpu()[rows], ref, synth.config(key).dtype, f"persistent {key}")


# ----------------------------------------------------------------- asynchronous build

@pytest.mark.parametrize("key", ["2a", "3a"])
def test_async_build_matches_the_synchronous_build(key):
    coords = torch.from_numpy(coords_of(key)).to(DEV)
    f, w, b = cfg_tensors(key, 0)
    fd, wd, bd = f.to(DEV), w.to(DEV), b.to(DEV)
    with sc.sparse_indice_map_build(coords) as ms, sc.sparse_indice_map_build(coords, sync=False) as ma:
        ya = sc.subm_conv3d_forward(ma, fd, wd, bd)  # enqueued before the map's status is known
        ma.check()
        ys = sc.subm_conv3d_forward(ms, fd, wd, bd)
        torch.cuda.synchronize()
        assert torch.equal(ya, ys)
        assert np.array_equal(gpu_nbr(ma), oracle_nbr(key))
        assert ma.pairs == ms.pairs
        assert ma.mode == ms.mode


def test_several_async_builds_in_flight():
    keys = ["1", "2a", "3a", "1"]
    maps = [sc.sparse_indice_map_build(torch.from_numpy(coords_of(k)).to(DEV), sync=False) for k in keys]
    try:
        for k, m in zip(keys, maps):
            assert np.array_equal(gpu_nbr(m), oracle_nbr(k)), k
    finally:
        for m in maps:
            m.free()


@pytest.mark.parametrize("mode", [1, 2])
def test_async_build_reports_duplicates_later_and_work_on_it_stays_in_bounds(mode):
    coords = np.concatenate([coords_of("1"), coords_of("1")[17:18]])
    m = sc.sparse_indice_map_build_async(torch.from_numpy(coords).to(DEV), mode)
    try:
        rng = np.random.default_rng(9)
        f = torch.from_numpy(rng.standard_normal((len(coords), 64))).to(torch.bfloat16).to(DEV)
        w = torch.from_numpy(rng.standard_normal((64, 3, 3, 3, 64)) * 0.05).to(torch.bfloat16).to(DEV)
        sc.subm_conv3d_forward(m, f, w)  # a row of the set for every present neighbour: no fault
        torch.cuda.synchronize()
        for call in (m.check, lambda: m.pairs, lambda: gpu_nbr(m),
                     lambda: sc.subm_conv3d_forward_per_offset(m, f, w)):
            with pytest.raises(sc.SubmError) as e:
                call()
            assert e.value.name == "SUBM_ERR_DUPLICATE_COORD"
    finally:
        m.free()


@pytest.mark.parametrize("cout", [16, 64])
def test_async_build_out_of_range_leaves_only_the_bias(cout):
    coords = np.array([[0, 0, 0, 0], [0, 65535, 0, 0], [0, 1, 0, 0]], dtype=np.int32)
    m = sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV), sync=False)
    try:
        rng = np.random.default_rng(10)
        f = torch.from_numpy(rng.standard_normal((3, 32))).to(torch.bfloat16).to(DEV)
        w = torch.from_numpy(rng.standard_normal((cout, 3, 3, 3, 32))).to(torch.bfloat16).to(DEV)
        b = torch.from_numpy(rng.standard_normal(cout)).to(torch.bfloat16).to(DEV)
        y = sc.subm_conv3d_forward(m, f, w, b)  # every rulebook entry is -1
        torch.cuda.synchronize()
        assert torch.equal(y, b.expand(3, cout))
        with pytest.raises(sc.SubmError) as e:
            m.check()
        assert e.value.name == "SUBM_ERR_COORD_RANGE"
    finally:
        m.free()


# ----------------------------------------------------------------- tensors past 31-bit offsets

def test_features_past_31_bit_byte_offsets():
    # Two dense 163^3 boxes with 128 bf16 channels: 2.2 GB of features, past the byte offsets the
    # fast kernels address, so the library takes its 64-bit-indexed kernel.  The rulebook of a
    # dense box has a closed form (checked bit for bit on sampled rows); features on the same rows
    # against the oracle.
    g, cin, cout = 163, 128, 32
    zz, yy, xx = np.meshgrid(np.arange(g), np.arange(g), np.arange(g), indexing="ij")
    one = np.stack([zz.ravel(), yy.ravel(), xx.ravel()], 1)
    coords = np.concatenate([np.concatenate([np.full((len(one), 1), b), one], 1) for b in range(2)]).astype(np.int32)
    n = len(coords)
    assert n * cin * 2 >= 2 ** 31
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    f = torch.randn(n, cin, generator=gen, device=DEV).to(torch.bfloat16)
    rng = np.random.default_rng(12)
    w = torch.from_numpy(rng.standard_normal((cout, 3, 3, 3, cin)) / np.sqrt(27 * cin)).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(cout) * 0.3).to(torch.bfloat16)
    rows = sample_rows(n, count=1024, seed=13)
    rows_d = torch.from_numpy(rows).to(DEV)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        y = sc.subm_conv3d_forward(m, f, w.to(DEV), b.to(DEV))
        nbr_rows = sc.sparse_indice_map_copy_nbr(m)[rows_d].cpu().numpy()
        torch.cuda.synchronize()
    bb, z, yv, x = (coords[rows, a].astype(np.int64) for a in range(4))
    expect = np.full((len(rows), 27), -1, np.int64)
    for k in range(27):
        z2, y2, x2 = z + k // 9 - 1, yv + (k // 3) % 3 - 1, x + k % 3 - 1
        ok = (z2 >= 0) & (z2 < g) & (y2 >= 0) & (y2 < g) & (x2 >= 0) & (x2 < g)
        expect[ok, k] = ((bb[ok] * g + z2[ok]) * g + y2[ok]) * g + x2[ok]
    assert np.array_equal(nbr_rows, expect)
    used = np.unique(expect[expect >= 0])
    fsub = f[torch.from_numpy(used).to(DEV)].cpu()
    local = np.where(expect >= 0, np.searchsorted(used, expect), -1)
    ref = oracle.conv3_rulebook(local, as64(fsub), as64(w), as64(b))
    check(y[rows_d].cpu(), ref, "bf16", "features past 31-bit offsets")
    del f, y
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- builds from two threads

def test_builds_from_two_threads_on_two_streams():
    # The build workspace is shared by every build on the device: builds from two host threads on
    # two streams must still each see only their own coordinate set, synchronous or not.
    import threading
    keys = ("2a", "3a")
    got = {k: [] for k in keys}
    errors = []

    def worker(key):
        try:
            stream = torch.cuda.Stream(device=DEV)
            coords = torch.from_numpy(coords_of(key)).to(DEV)
            torch.cuda.synchronize()
            for rep in range(6):
                with torch.cuda.stream(stream):
                    m = sc.sparse_indice_map_build(coords, stream=stream, sync=rep % 2 == 0)
                    nbr = sc.sparse_indice_map_copy_nbr(m, stream=stream)
                    stream.synchronize()
                    got[key].append(nbr.cpu().numpy())
                    m.free()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in keys]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k in keys:
        assert len(got[k]) == 6
        for nbr in got[k]:
            assert np.array_equal(nbr, oracle_nbr(k)), k


# ----------------------------------------------------------------- freed rulebook memory

def test_freed_rulebook_memory_is_reused_only_in_stream_order():
    # A freed map's rulebook block is kept for the next build on the same stream.  Build, conv and
    # free back to back with no host wait (each build may take the block that the previous step's
    # conv is still reading), over three coordinate sets whose blocks fit each other; every step
    # must see only its own set.  One map is also read on a second stream, so its block goes back
    # to the pool instead.
    base = coords_of("3a")
    keep = np.arange(len(base)) % 6 != 5
    sets = {"3a": base, "reversed": np.ascontiguousarray(base[::-1]), "sixth dropped": np.ascontiguousarray(base[keep])}
    f, w, b = cfg_tensors("3a", 0)
    f_of = {"3a": f, "reversed": f.flip(0), "sixth dropped": f[torch.from_numpy(keep)]}
    w, b = w.to(DEV), b.to(DEV)
    dev_coords, feats, expect_nbr, expect_out = {}, {}, {}, {}
    for name, c in sets.items():
        dev_coords[name] = torch.from_numpy(c).to(DEV)
        feats[name] = f_of[name].contiguous().to(DEV)
        expect_nbr[name] = oracle.rulebook_sorted(c)
        with sc.sparse_indice_map_build(dev_coords[name]) as m:
            assert np.array_equal(gpu_nbr(m), expect_nbr[name]), name
            expect_out[name] = sc.subm_conv3d_forward(m, feats[name], w, b).cpu()
    rows = sample_rows(len(base), count=512, seed=2)
    ref = oracle.conv3_rulebook(expect_nbr["3a"], as64(feats["3a"].cpu()), as64(w.cpu()), as64(b.cpu()), rows=rows)
    check(expect_out["3a"][rows], ref, "bf16", "fresh map, 3a")
    side = torch.cuda.Stream(device=DEV)
    outs, nbrs = [], []
    names = list(sets) * 4
    for step, name in enumerate(names):
        m = sc.sparse_indice_map_build(dev_coords[name], sync=False)
        outs.append((name, sc.subm_conv3d_forward(m, feats[name], w, b)))
        if step == 5:
            side.wait_stream(torch.cuda.current_stream())
            nbrs.append((name, sc.sparse_indice_map_copy_nbr(m, stream=side)))
            torch.cuda.current_stream().wait_stream(side)
        else:
            nbrs.append((name, sc.sparse_indice_map_copy_nbr(m)))
        m.check()
        m.free()
    torch.cuda.synchronize()
    for (name, out), (_, nbr) in zip(outs, nbrs):
        assert np.array_equal(nbr.cpu().numpy(), expect_nbr[name]), name
        assert torch.equal(out.cpu(), expect_out[name]), name


# ----------------------------------------------------------------- seeded random sweep

def random_case(seed):
    # A random set (1-3 batch items, a random box with a negative corner, random occupancy), random
    # channel counts across every dispatch boundary, and a random storage dtype.
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 4))
    dims = rng.integers(4, 24, size=3)
    occ = float(rng.uniform(0.02, 0.6))
    rows = []
    for b in range(batch):
        cells = int(np.prod(dims))
        k = max(1, int(cells * occ))
        pick = rng.choice(cells, size=k, replace=False)
        z, y, x = np.unravel_index(pick, dims)
        rows.append(np.stack([np.full(k, b), z, y, x], axis=1))
    coords = np.concatenate(rows).astype(np.int32)
    coords[:, 1:] += rng.integers(-300, 300, size=3).astype(np.int32)
    coords = coords[rng.permutation(len(coords))]
    dtype = ["f32", "f16", "bf16"][seed % 3]
    cin = int(rng.choice([1, 3, 8, 16, 24, 40, 64, 72, 128, 136]))
    cout = int(rng.choice([1, 5, 16, 17, 32, 33, 48, 64, 65, 96, 128, 136, 256]))
    f = synth.round_to(rng.standard_normal((len(coords), cin)), dtype)
    w = synth.round_to(rng.standard_normal((cout, 3, 3, 3, cin)) / np.sqrt(27 * cin), dtype)
    b = synth.round_to(rng.standard_normal(cout) * 0.3, dtype)
    return np.ascontiguousarray(coords), f, w, b, dtype


@pytest.mark.parametrize("seed", range(24))
def test_random_sets_and_shapes_match_the_oracle(seed):
    coords, f, w, b, dtype = random_case(seed)
    what = f"seed {seed}: n={len(coords)} {dtype} {f.shape[1]}->{w.shape[0]}"
    print(what, flush=True)
    nbr = oracle.rulebook(coords)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        assert np.array_equal(gpu_nbr(m), nbr), what
        out = forward(m, f, w, b)
    check_features(out, nbr, as64(f), as64(w), as64(b), dtype, what)


# ----------------------------------------------------------------- sparse-row order of a reused map

def _order_case(coords, cin, cout, dtype, seed):
    rng = np.random.default_rng(seed)
    n = len(coords)
    f = synth.round_to(rng.standard_normal((n, cin)), dtype)
    w = synth.round_to(rng.standard_normal((cout, 3, 3, 3, cin)) / np.sqrt(27 * cin), dtype)
    b = synth.round_to(rng.standard_normal(cout) * 0.3, dtype)
    return f, w, b


def _calls_on_one_map(coords, f, w, b, calls):
    outs, states = [], []
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        for _ in range(calls):
            outs.append(sc.subm_conv3d_forward(m, to_dev(f), to_dev(w), to_dev(b)))
            torch.cuda.synchronize()
            states.append(sc.sparse_indice_map_row_order_state(m))
    return [o.cpu() for o in outs], states


@pytest.mark.parametrize("dtype,cin,cout", [("bf16", 64, 64), ("f16", 64, 96), ("bf16", 128, 64)])
def test_sparse_row_order_same_bits_as_input_order(monkeypatch, dtype, cin, cout):
    # 300,001 rows of the subdivided 512^3 boxes (about 6.7 of 27 neighbours per row): five sort
    # segments of 65,536 rows, the last one partial, and a partial last tile.
    coords = np.ascontiguousarray(coords_of("5")[:300_001])
    f, w, b = _order_case(coords, cin, cout, dtype, seed=11)
    monkeypatch.setenv("SUBMCONV_ROW_ORDER", "0")
    ref, st0 = _calls_on_one_map(coords, f, w, b, 2)
    assert st0 == [sc.SUBM_ORDER_NONE, sc.SUBM_ORDER_NONE]
    monkeypatch.delenv("SUBMCONV_ROW_ORDER")
    outs, st = _calls_on_one_map(coords, f, w, b, 3)
    print(f"  order states {st}", flush=True)
    assert st == [sc.SUBM_ORDER_NONE, sc.SUBM_ORDER_ON, sc.SUBM_ORDER_ON]
    for o in outs:  # a skipped tap is an absent neighbour: the same bits as the input order
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16))
    check_features(outs[2], oracle.rulebook_sorted(coords), as64(f), as64(w), as64(b), dtype,
                   f"ordered {dtype} {cin}->{cout}", mag_rows=sample_rows(len(coords), count=2048))


def test_sparse_row_order_off_on_dense_maps():
    # 64^3 solid box: 25.4 neighbours per row on average, so the device gate keeps the input order.
    z, y, x = np.nonzero(synth.dense_box(64))
    coords = np.stack([np.zeros_like(z), z, y, x], axis=1).astype(np.int32)
    f, w, b = _order_case(coords, 64, 64, "bf16", seed=12)
    outs, st = _calls_on_one_map(coords, f, w, b, 3)
    assert st == [sc.SUBM_ORDER_NONE, sc.SUBM_ORDER_OFF, sc.SUBM_ORDER_OFF]
    assert torch.equal(outs[1].view(torch.int16), outs[0].view(torch.int16))
    assert torch.equal(outs[2].view(torch.int16), outs[0].view(torch.int16))
    rows = sample_rows(len(coords), count=1024)
    check_features(outs[2][rows], oracle.rulebook_sorted(coords), as64(f), as64(w), as64(b), "bf16",
                   "dense, input order", rows=rows)

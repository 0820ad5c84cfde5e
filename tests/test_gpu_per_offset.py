"""GPU parity of the per-offset convolution (gather -> GEMM -> scatter-add per offset) through the
C ABI against the CPU oracle, to the same normwise bar as the output-stationary kernel (1e-2 for
fp16 / bf16 storage with float32 accumulation).  Full comparison at small sizes; sampled rows at
the full workload sizes; bitwise reproducibility; the limits that return SUBM_ERR_UNSUPPORTED.
"""
import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_amd as sc
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f16": 1e-2, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sc.load_library()


def as64(t):
    return t.double().cpu().numpy()


def check(out, ref, dtype, what):
    err = oracle.normwise_rel_error(as64(out), ref)
    print(f"  {what}: normwise err {err:.3e}", flush=True)
    assert err <= TOL[dtype], f"{what}: {err:.3e}"


def sample_rows(n, count=2048, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(n, 256)), np.arange(max(0, n - 256), n), rng.integers(0, n, count)]))


def small(dtype, cin, cout, coords, seed=0, bias=True):
    rng = np.random.default_rng(seed)
    n = len(coords)
    f = synth.round_to(rng.standard_normal((n, cin)), dtype)
    w = synth.round_to(rng.standard_normal((cout, 3, 3, 3, cin)) / np.sqrt(27 * cin), dtype)
    b = synth.round_to(rng.standard_normal(cout) * 0.3, dtype) if bias else None
    return f, w, b


def run(coords, f, w, b):
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        out = sc.subm_conv3d_forward_per_offset(m, f.to(DEV), w.to(DEV), None if b is None else b.to(DEV))
        torch.cuda.synchronize()
        return out.cpu()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("cin,cout", [(8, 4), (16, 12), (64, 64), (128, 128), (40, 100), (200, 136), (256, 256),
                                      (72, 256)])
def test_shapes_full(dtype, cin, cout):
    coords = synth.coords_for("1")
    f, w, b = small(dtype, cin, cout, coords)
    out = run(coords, f, w, b)
    check(out, oracle.conv3(coords, as64(f), as64(w), as64(b)), dtype, f"{dtype} {cin}->{cout}")


def test_no_bias_shuffled_rows_several_items():
    rng = np.random.default_rng(3)
    rows = []
    for b in range(3):
        zyx = np.argwhere(rng.random((12, 12, 12)) < 0.3) - 6
        rows.append(np.concatenate([np.full((len(zyx), 1), b), zyx], axis=1))
    coords = np.concatenate(rows).astype(np.int32)
    coords = coords[rng.permutation(len(coords))]
    f, w, _ = small("bf16", 32, 48, coords, seed=4, bias=False)
    out = run(coords, f, w, None)
    check(out, oracle.conv3(coords, as64(f), as64(w)), "bf16", "3 items, shuffled, no bias")


def test_lone_voxels_take_the_centre_only():
    coords = np.array([[0, 0, 0, 0], [0, 5, 5, 5], [1, 0, 0, 0]], dtype=np.int32)
    f, w, b = small("bf16", 16, 8, coords, seed=5)
    out = run(coords, f, w, b)
    check(out, oracle.conv3(coords, as64(f), as64(w), as64(b)), "bf16", "lone voxels")


def test_config2a_full_and_matches_fused_kernel():
    coords = synth.coords_for("2a")
    c = synth.config("2a")
    f = synth.feats_for(c.number, 0, len(coords), c.cin, c.dtype)
    w = synth.weight_for(c.number, 0, 3, c.cin, c.cout, c.dtype)
    b = synth.bias_for(c.number, 0, c.cout, c.dtype)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        a = sc.subm_conv3d_forward_per_offset(m, f.to(DEV), w.to(DEV), b.to(DEV))
        a2 = sc.subm_conv3d_forward_per_offset(m, f.to(DEV), w.to(DEV), b.to(DEV))
        fused = sc.subm_conv3d_forward(m, f.to(DEV), w.to(DEV), b.to(DEV))
        torch.cuda.synchronize()
    ref = oracle.conv3_rulebook(oracle.rulebook_sorted(coords), as64(f), as64(w), as64(b))
    check(a.cpu(), ref, c.dtype, "config 2a per-offset")
    assert torch.equal(a, a2), "per-offset path is not bitwise reproducible"
    # the two designs differ only by float32 summation order
    check(a.cpu(), as64(fused), c.dtype, "per-offset vs output-stationary")


@pytest.mark.parametrize("key", ["3a", "5"])
def test_full_size_sampled(key):
    coords = synth.coords_for(key)
    c = synth.config(key)
    f = synth.feats_for(c.number, 0, len(coords), c.cin, c.dtype)
    w = synth.weight_for(c.number, 0, 3, c.cin, c.cout, c.dtype)
    b = synth.bias_for(c.number, 0, c.cout, c.dtype)
    rows = sample_rows(len(coords))
    print(f"config {key}: N={len(coords)}", flush=True)
    out = run(coords, f, w, b)
    ref = oracle.conv3_rulebook(oracle.rulebook_sorted(coords), as64(f), as64(w), as64(b), rows=rows)
    check(out[rows], ref, c.dtype, f"config {key} per-offset (sampled)")


def test_unsupported_shapes_and_dtypes():
    coords = synth.coords_for("1")
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        for dtype, cin, cout in (("f32", 16, 16), ("bf16", 12, 16), ("bf16", 16, 6)):
            f, w, b = small(dtype, cin, cout, coords)
            with pytest.raises(sc.SubmError) as e:
                sc.subm_conv3d_forward_per_offset(m, f.to(DEV), w.to(DEV), b.to(DEV))
            assert e.value.name == "SUBM_ERR_UNSUPPORTED", (dtype, cin, cout)
        f, w, b = small("bf16", 16, 16, coords)
        with pytest.raises(ValueError):
            sc.subm_conv3d_forward_per_offset(m, f.to(DEV), w[:, :1, :1, :1].contiguous().to(DEV))


@pytest.mark.parametrize("seed", range(8))
def test_random_sets_match_the_oracle_and_the_fused_kernel(seed):
    # Random sets (1-3 items, random boxes with negative corners, random occupancy, shuffled rows)
    # and channel counts within the per-offset limits (Cin % 8 == 0, Cout % 4 == 0).
    rng = np.random.default_rng(800 + seed)
    rows = []
    for b in range(int(rng.integers(1, 4))):
        g = int(rng.integers(4, 20))
        zyx = np.argwhere(rng.random((g, g, g)) < rng.uniform(0.05, 0.8)) + int(rng.integers(-50, 50))
        rows.append(np.concatenate([np.full((len(zyx), 1), b), zyx], axis=1))
    coords = np.concatenate(rows).astype(np.int32)
    coords = np.ascontiguousarray(coords[rng.permutation(len(coords))])
    dtype = ["f16", "bf16"][seed % 2]
    cin = int(rng.choice([8, 16, 40, 64, 128]))
    cout = int(rng.choice([4, 12, 36, 64, 100, 128]))
    f, w, b = small(dtype, cin, cout, coords, seed=900 + seed, bias=seed % 3 != 0)
    what = f"seed {seed}: n={len(coords)} {dtype} {cin}->{cout}"
    out = run(coords, f, w, b)
    ref = oracle.conv3_rulebook(oracle.rulebook(coords), as64(f), as64(w), None if b is None else as64(b))
    check(out, ref, dtype, what)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        fused = sc.subm_conv3d_forward(m, f.to(DEV), w.to(DEV), None if b is None else b.to(DEV))
        torch.cuda.synchronize()
    check(out, as64(fused), dtype, what + " vs the output-stationary kernel")

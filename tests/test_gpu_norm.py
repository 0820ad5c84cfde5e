"""GPU parity of the group normalisation + activation through the C ABI against the CPU oracle
(float64), normwise bar 1e-5 for fp32 storage and 1e-2 for fp16 / bf16 storage (float32
arithmetic, one rounding): several channel / group shapes, batch items of very different sizes
including empty and one-row items, in place, full-size multi-item sets, reproducibility.
"""
import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_amd as sc
import synth
from oracle import norm_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
ACT = {"none": sc.SUBM_ACT_NONE, "silu": sc.SUBM_ACT_SILU, "relu": sc.SUBM_ACT_RELU}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sc.load_library()


def inputs(n, c, dtype, seed, shift=0.0):
    rng = np.random.default_rng(seed)
    x = synth.round_to(rng.standard_normal((n, c)) * 2.0 + shift + rng.standard_normal(c), dtype)
    gamma = synth.round_to(1.0 + 0.3 * rng.standard_normal(c), dtype)
    beta = synth.round_to(0.3 * rng.standard_normal(c), dtype)
    return x, gamma, beta


def run(x, offsets, groups, gamma, beta, act, eps=1e-5, out=None):
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    y = sc.sparse_group_norm_act(x, off, groups, gamma, beta, eps, ACT[act], out=out)
    torch.cuda.synchronize()
    return y.cpu()


def check(y, ref, dtype, what):
    err = oracle.normwise_rel_error(y.double().numpy(), ref)
    print(f"  {what}: normwise err {err:.3e}", flush=True)
    assert err <= TOL[dtype], f"{what}: {err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("c,groups", [(64, 32), (128, 32), (256, 32), (96, 32), (64, 8), (512, 1), (1024, 64)])
@pytest.mark.parametrize("act", ["none", "silu", "relu"])
def test_shapes(dtype, c, groups, act):
    if dtype == "f32" and c > 1024:
        pytest.skip("rows above 4 KB are out of range")
    offsets = [0, 300, 300, 301, 1800, 2100]
    x, g, b = inputs(offsets[-1], c, dtype, c + groups)
    y = run(x.to(DEV), offsets, groups, g.to(DEV), b.to(DEV), act)
    ref = norm_ref.group_norm_act(x.double().numpy(), offsets, groups, g.double().numpy(), b.double().numpy(),
                                  1e-5, act)
    check(y, ref, dtype, f"{dtype} C={c} G={groups} {act}")


def test_in_place_and_no_affine_and_reproducible():
    offsets = [0, 1000, 4000]
    x, _, _ = inputs(offsets[-1], 128, "bf16", 3, shift=20.0)  # large mean: the variance needs care
    ref = norm_ref.group_norm_act(x.double().numpy(), offsets, 32, None, None, 1e-5, "silu")
    xd = x.to(DEV)
    a = run(xd, offsets, 32, None, None, "silu")
    b = run(xd, offsets, 32, None, None, "silu")
    assert torch.equal(a, b)
    run(xd, offsets, 32, None, None, "silu", out=xd)  # in place
    assert torch.equal(xd.cpu(), a)
    check(a, ref, "bf16", "in place, no affine, mean 20")


@pytest.mark.parametrize("key", ["4", "5"])
def test_full_size_items(key):
    coords = synth.coords_for(key)
    b = coords[:, 0]
    assert (np.diff(b) >= 0).all()  # items are contiguous row ranges
    offsets = [0] + np.cumsum(np.bincount(b)).tolist()
    c = 64
    x, g, be = inputs(len(coords), c, "bf16", 11)
    print(f"config {key}: N={len(coords)} items={len(offsets) - 1}", flush=True)
    y = run(x.to(DEV), offsets, 32, g.to(DEV), be.to(DEV), "silu")
    ref = norm_ref.group_norm_act(x.double().numpy(), offsets, 32, g.double().numpy(), be.double().numpy(),
                                  1e-5, "silu")
    check(y, ref, "bf16", f"config {key} silu")


def test_many_items_of_one_row():
    n, c = 2000, 64
    offsets = list(range(n + 1))
    x, g, b = inputs(n, c, "f32", 5)
    y = run(x.to(DEV), offsets, 16, g.to(DEV), b.to(DEV), "none")
    ref = norm_ref.group_norm_act(x.double().numpy(), offsets, 16, g.double().numpy(), b.double().numpy(), 1e-5, "none")
    check(y, ref, "f32", "2000 one-row items")


def test_invalid_arguments():
    x = torch.zeros((10, 64), dtype=torch.bfloat16, device=DEV)
    off = torch.tensor([0, 10], dtype=torch.int64, device=DEV)
    with pytest.raises(sc.SubmError) as e:
        sc.sparse_group_norm_act(x, off, 24)
    assert e.value.name == "SUBM_ERR_INVALID_ARG"
    with pytest.raises(ValueError):
        sc.sparse_group_norm_act(x, off.int(), 32)


# ----------------------------------------------------------------- conv + group norm, fused

def multi_item_sites(seed, sizes, lo=-10, hi=10):
    """Items of roughly the given voxel counts (random subsets of a box), rows item by item."""
    rng = np.random.default_rng(seed)
    g = hi - lo
    rows = []
    for b, target in enumerate(sizes):
        occ = min(1.0, target / g ** 3)
        zyx = np.argwhere(rng.random((g, g, g)) < occ) + lo
        rows.append(np.concatenate([np.full((len(zyx), 1), b), zyx], axis=1))
    c = np.ascontiguousarray(np.concatenate(rows, axis=0), dtype=np.int32)
    offsets = [0] + np.cumsum([len(r) for r in rows]).tolist()
    return c, offsets


def conv_norm_oracle(coords, f, w, b, offsets, groups, gamma, beta, act, dtype):
    """conv (float64) -> rounded to the storage dtype -> group norm + act (float64)."""
    conv = oracle.conv3_rulebook(oracle.rulebook_sorted(coords), f.double().numpy(), w.double().numpy(),
                                 None if b is None else b.double().numpy())
    conv = synth.round_to(conv, dtype).double().numpy()
    return norm_ref.group_norm_act(conv, offsets, groups, None if gamma is None else gamma.double().numpy(),
                                   None if beta is None else beta.double().numpy(), 1e-5, act)


FUSED_CASES = [
    # (seed, item sizes, cin, cout, groups, dtype, act): the fast path (cout > 32, groups inside
    # one 64- or 128-channel tile) and shapes that fall back to conv + separate norm
    (1, [3000, 150, 5000, 40, 2600], 64, 128, 32, "bf16", "silu"),
    (2, [4000, 4000, 4000], 64, 64, 32, "f16", "relu"),
    (3, [7, 3, 900, 1, 2, 5000], 32, 256, 64, "bf16", "silu"),
    (4, [2500, 2500], 40, 96, 32, "bf16", "silu"),   # 3 channels per group: fallback
    (5, [2500, 2500], 32, 32, 8, "bf16", "none"),    # 32 output channels: fallback
    (6, [3000, 1000], 16, 64, 4, "f32", "silu"),     # float32: fallback
]


@pytest.mark.parametrize("epilogue", ["0", "1"])
@pytest.mark.parametrize("seed,sizes,cin,cout,groups,dtype,act", FUSED_CASES)
def test_fused_conv_group_norm(seed, sizes, cin, cout, groups, dtype, act, epilogue, monkeypatch):
    # "1": group statistics from the convolution epilogue where the shape allows it; "0": the
    # default conv + separate statistics pass
    monkeypatch.setenv("SUBMCONV_GN_EPILOGUE", epilogue)
    coords, offsets = multi_item_sites(seed, sizes)
    rng = np.random.default_rng(100 + seed)
    n = len(coords)
    f = synth.round_to(rng.standard_normal((n, cin)), dtype)
    w = synth.round_to(rng.standard_normal((cout, 3, 3, 3, cin)) / np.sqrt(27 * cin), dtype)
    b = synth.round_to(rng.standard_normal(cout) * 2.0, dtype)
    gamma = synth.round_to(1.0 + 0.2 * rng.standard_normal(cout), dtype)
    beta = synth.round_to(0.2 * rng.standard_normal(cout), dtype)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    print(f"fused {dtype} n={n} items={len(sizes)} {cin}->{cout} G={groups} {act} epilogue={epilogue}", flush=True)
    with sc.sparse_indice_map_build(torch.from_numpy(coords).to(DEV)) as m:
        fd, wd, bd, gd, bed = (t.to(DEV) for t in (f, w, b, gamma, beta))
        fused = sc.subm_conv3d_forward_group_norm_act(m, fd, wd, bd, off, groups, gd, bed, 1e-5, ACT[act])
        fused2 = sc.subm_conv3d_forward_group_norm_act(m, fd, wd, bd, off, groups, gd, bed, 1e-5, ACT[act])
        conv = sc.subm_conv3d_forward(m, fd, wd, bd)
        split = sc.sparse_group_norm_act(conv, off, groups, gd, bed, 1e-5, ACT[act])
        torch.cuda.synchronize()
    assert torch.equal(fused, fused2), "fused path is not bitwise reproducible"
    ref = conv_norm_oracle(coords, f, w, b, offsets, groups, gamma, beta, act, dtype)
    check(fused.cpu(), ref, dtype, "fused vs oracle")
    check(split.cpu(), ref, dtype, "conv + norm vs oracle")


@pytest.mark.parametrize("seed", range(10))
def test_random_item_splits_and_shapes(seed):
    # Random row counts split into 1-6 items (empty and one-row items included), random channel
    # and group counts (rows a multiple of 16 bytes, the kernel's layout rule), dtypes, activations
    # and means far from zero.
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 6000))
    cuts = np.sort(rng.integers(0, n + 1, size=int(rng.integers(0, 6))))
    offsets = [0] + [int(v) for v in cuts] + [n]
    groups = int(rng.choice([1, 2, 4, 8, 32]))
    c = int(np.lcm(groups, 8)) * int(rng.choice([1, 2, 3, 4, 8]))
    dtype = ["f32", "f16", "bf16"][seed % 3]
    act = ["none", "silu", "relu"][(seed // 3) % 3]
    x, g, b = inputs(n, c, dtype, 400 + seed, shift=float(rng.uniform(-20, 20)))
    y = run(x.to(DEV), offsets, groups, g.to(DEV), b.to(DEV), act)
    ref = norm_ref.group_norm_act(x.double().numpy(), offsets, groups, g.double().numpy(), b.double().numpy(),
                                  1e-5, act)
    check(y, ref, dtype, f"seed {seed}: n={n} items={len(offsets) - 1} C={c} G={groups} {dtype} {act}")

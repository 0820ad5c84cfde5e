"""subm_conv3d_forward_noalloc (static scratch, no device allocation) against subm_conv3d_forward.

Both entry points run the same kernels, so their outputs must agree bit for bit: on the
neighbour-pool path (packed weights in the static array) and on the general path, two calls in a
row with the second smaller (the array keeps the first call's contents), and a call whose
packed weights exceed the array is rejected.  Every call goes through the C ABI.
"""
import functools

import pytest
import torch

import submanifold_sparse_convolution_amd as sc
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sc.load_library()


@pytest.fixture(autouse=True)
def _env(monkeypatch):
    for var in ("SUBMCONV_POOL", "SUBMCONV_TILE", "SUBMCONV_PERSISTENT"):
        monkeypatch.delenv(var, raising=False)


@functools.lru_cache(maxsize=None)
def coords(key):
    return synth.coords_for(key)


def tensors(n, cin, cout, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    f = torch.randn(n, cin, generator=g).to(dtype).to(DEV)
    w = (torch.randn(cout, 3, 3, 3, cin, generator=g) / (27 * cin) ** 0.5).to(dtype).to(DEV)
    b = (torch.randn(cout, generator=g) * 0.3).to(dtype).to(DEV)
    return f, w, b


def both(m, f, w, b):
    ref = sc.subm_conv3d_forward(m, f, w, b)
    got = torch.full_like(ref, float("nan"))
    sc.subm_conv3d_forward_noalloc(m, f, w, b, out=got)
    torch.cuda.synchronize()
    return ref, got


def test_pool_path_two_calls_second_smaller():
    c = torch.from_numpy(coords("3a")).to(DEV)
    n = c.shape[0]
    with sc.sparse_indice_map_build(c) as m:
        f, w, b = tensors(n, 256, 128, seed=1)  # 1,769,472 bytes of packed weights: the whole array
        sc.subm_conv3d_forward(m, f, w, b)  # builds the plan (an allocating call)
        torch.cuda.synchronize()
        assert sc.sparse_indice_map_plan_state(m) == sc.SUBM_PLAN_READY
        ref, got = both(m, f, w, b)
        assert torch.equal(ref, got)
        f2, w2, b2 = tensors(n, 64, 128, seed=2)  # second call: a quarter of the array
        ref2, got2 = both(m, f2, w2, b2)
        assert torch.equal(ref2, got2)
        assert not torch.equal(ref2, torch.zeros_like(ref2))


def test_general_path_and_smaller_set():
    for key, cin, cout in (("3a", 64, 64), ("2a", 32, 48)):  # 64 output channels; a small set
        c = torch.from_numpy(coords(key)).to(DEV)
        with sc.sparse_indice_map_build(c) as m:
            f, w, b = tensors(c.shape[0], cin, cout, seed=3)
            ref, got = both(m, f, w, b)
            assert torch.equal(ref, got), key


def test_no_plan_yet_takes_the_general_kernels(monkeypatch):
    c = torch.from_numpy(coords("3a")).to(DEV)
    with sc.sparse_indice_map_build(c) as m:
        f, w, b = tensors(c.shape[0], 128, 128, seed=4)
        got = torch.empty(c.shape[0], 128, dtype=torch.bfloat16, device=DEV)
        sc.subm_conv3d_forward_noalloc(m, f, w, b, out=got)
        torch.cuda.synchronize()
        assert sc.sparse_indice_map_plan_state(m) == sc.SUBM_PLAN_NONE
        ref = torch.empty_like(got)
        monkeypatch.setenv("SUBMCONV_POOL", "0")
        sc.subm_conv3d_forward(m, f, w, b, out=ref)
        torch.cuda.synchronize()
        assert torch.equal(ref, got)


def test_packed_weights_beyond_the_array_are_rejected():
    c = torch.from_numpy(coords("3a")).to(DEV)
    with sc.sparse_indice_map_build(c) as m:
        f, w, b = tensors(c.shape[0], 288, 128, seed=5)
        sc.subm_conv3d_forward(m, f, w, b)
        torch.cuda.synchronize()
        out = torch.empty(c.shape[0], 128, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(sc.SubmError) as e:
            sc.subm_conv3d_forward_noalloc(m, f, w, b, out=out)
        assert e.value.name == "SUBM_ERR_UNSUPPORTED"
        with pytest.raises(ValueError):
            sc.subm_conv3d_forward_noalloc(m, f, w, b, out=None)

"""Pins of the group-norm + activation oracle against torch CPU library routines (CPU only).

* each batch item laid out as [1, C, rows] through torch.nn.functional.group_norm (float64);
* torch's silu and relu;
* item isolation and an empty item;
* planted mistakes (unbiased variance, statistics over all items, per-channel statistics)
  must fail.
"""
import numpy as np
import pytest
import torch

from oracle import norm_ref as nr


def torch_reference(x, offsets, groups, gamma, beta, eps, act):
    out = np.empty_like(x)
    for lo, hi in zip(offsets, offsets[1:]):
        if hi == lo:
            continue
        t = torch.from_numpy(x[lo:hi].T.copy())[None]  # [1, C, rows]
        y = torch.nn.functional.group_norm(t, groups, torch.from_numpy(gamma), torch.from_numpy(beta), eps)
        if act == "silu":
            y = torch.nn.functional.silu(y)
        elif act == "relu":
            y = torch.nn.functional.relu(y)
        out[lo:hi] = y[0].numpy().T
    return out


@pytest.mark.parametrize("act", ["none", "silu", "relu"])
@pytest.mark.parametrize("c,groups", [(64, 32), (128, 32), (96, 8), (32, 32)])
def test_group_norm_matches_torch(act, c, groups):
    rng = np.random.default_rng(c + groups)
    # an empty item and a one-row item (two rows when a group is one channel: torch refuses a
    # group of a single value)
    offsets = [0, 37, 37, 150, 151 if c > groups else 152, 400]
    x = rng.standard_normal((offsets[-1], c)) * 3.0 + rng.standard_normal(c) * 5.0
    gamma = rng.standard_normal(c)
    beta = rng.standard_normal(c)
    got = nr.group_norm_act(x, offsets, groups, gamma, beta, 1e-5, act)
    want = torch_reference(x, offsets, groups, gamma, beta, 1e-5, act)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


def test_items_are_isolated():
    rng = np.random.default_rng(3)
    offsets = [0, 50, 120]
    x = rng.standard_normal((120, 64))
    a = nr.group_norm_act(x, offsets, 32, act="silu")
    x2 = x.copy()
    x2[50:] *= 10.0
    b = nr.group_norm_act(x2, offsets, 32, act="silu")
    np.testing.assert_array_equal(a[:50], b[:50])


def test_bad_offsets_rejected():
    x = np.zeros((10, 32))
    for off in ([1, 10], [0, 9], [0, 6, 4, 10]):
        with pytest.raises(ValueError):
            nr.group_norm_act(x, off, 32)
    with pytest.raises(ValueError):
        nr.group_norm_act(np.zeros((4, 30)), [0, 4], 32)


def test_planted_unbiased_variance_fails(monkeypatch):
    def unbiased(x, offsets, groups, gamma=None, beta=None, eps=1e-5, act="none"):
        # the same steps with the variance divided by (count - 1)
        x = np.asarray(x, dtype=np.float64)
        out = np.empty_like(x)
        per = x.shape[1] // groups
        for lo, hi in zip(offsets, offsets[1:]):
            item = x[lo:hi].reshape(hi - lo, groups, per)
            m = item.mean(axis=(0, 2))
            cnt = item.shape[0] * per
            var = ((item - m[None, :, None]) ** 2).sum(axis=(0, 2)) / (cnt - 1)
            out[lo:hi] = ((item - m[None, :, None]) / np.sqrt(var[None, :, None] + eps)).reshape(hi - lo, -1)
        return nr.activation(out, act)

    monkeypatch.setattr(nr, "group_norm_act", unbiased)
    with pytest.raises(AssertionError):
        _check("none", 64, 32)


def _check(act, c, groups, offsets=(0, 37, 150, 400)):
    rng = np.random.default_rng(9)
    offsets = list(offsets)
    x = rng.standard_normal((offsets[-1], c)) * 2.0 + 1.0
    gamma = np.ones(c)
    beta = np.zeros(c)
    got = nr.group_norm_act(x, offsets, groups, gamma, beta, 1e-5, act)
    want = torch_reference(x, offsets, groups, gamma, beta, 1e-5, act)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-8)


def test_planted_statistics_over_all_items_fails(monkeypatch):
    real = nr.group_norm_act
    monkeypatch.setattr(nr, "group_norm_act",
                        lambda x, off, g, gamma=None, beta=None, eps=1e-5, act="none":
                        real(x, [0, len(x)], g, gamma, beta, eps, act))
    with pytest.raises(AssertionError):
        _check("none", 64, 32)


def test_planted_per_channel_statistics_fails(monkeypatch):
    real = nr.group_norm_act
    monkeypatch.setattr(nr, "group_norm_act",
                        lambda x, off, g, gamma=None, beta=None, eps=1e-5, act="none":
                        real(x, off, np.asarray(x).shape[1], gamma, beta, eps, act))
    with pytest.raises(AssertionError):
        _check("silu", 64, 32)


def test_planted_missing_sigmoid_fails(monkeypatch):
    real = nr.activation
    monkeypatch.setattr(nr, "activation", lambda y, act: real(y, "relu" if act == "silu" else act))
    with pytest.raises(AssertionError):
        _check("silu", 64, 32)

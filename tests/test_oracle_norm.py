"""Pins of the gated RMSNorm oracle (CPU): finite differences of its own
forward (a check that does not restate the backward's formula), torch's
library RMSNorm and silu on special cases, and invariants of the definition."""
import numpy as np
import pytest
import torch

from oracle import norm


def _case(rows, D, seed, gate=True):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((rows, D))
    z = rng.standard_normal((rows, D)) * 1.5 if gate else None
    w = rng.uniform(0.5, 1.5, D)
    return y, z, w


@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("group", [4, 12])
def test_backward_matches_finite_differences(gate, group):
    rows, D, eps = 3, 12, 1e-3
    y, z, w = _case(rows, D, 7, gate)
    dout = np.random.default_rng(8).standard_normal((rows, D))
    loss = lambda y_, z_, w_: float(np.sum(norm.fwd(y_, z_, w_, group, eps)[0] * dout))
    dy, dz, dw = norm.bwd(dout, y, z, w, group, eps)
    h = 1e-6
    for name, arr, grad in (("y", y, dy), ("z", z, dz), ("w", w, dw)):
        if arr is None:
            assert grad is None
            continue
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args = {"y": (p, z, w), "z": (y, p, w), "w": (y, z, p)}[name]
            argm = {"y": (m, z, w), "z": (y, m, w), "w": (y, z, m)}[name]
            num[idx] = (loss(*args) - loss(*argm)) / (2 * h)
        assert np.max(np.abs(num - grad)) <= 1e-7 * max(1.0, np.max(np.abs(grad))), name


def test_no_gate_whole_row_is_torch_rms_norm():
    y, _, w = _case(5, 64, 3, gate=False)
    out, _ = norm.fwd(y, None, w, 64, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.tensor(y), (64,), torch.tensor(w), eps=1e-5).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_gate_is_torch_silu():
    y, z, w = _case(4, 32, 4)
    out, _ = norm.fwd(y, z, w, 32, 1e-5)
    v = y * torch.nn.functional.silu(torch.tensor(z)).numpy()
    ref = torch.nn.functional.rms_norm(torch.tensor(v), (32,), torch.tensor(w), eps=1e-5).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_groups_are_independent_rms_norms():
    """Each group is normalised on its own: a group's output depends only on
    its own columns, and with w = 1, eps = 0 every group has RMS exactly 1."""
    y, z, _ = _case(6, 48, 5)
    w1 = np.ones(48)
    out, r = norm.fwd(y, z, w1, 16, 0.0)
    rms = np.sqrt(np.mean(out.reshape(6, 3, 16) ** 2, axis=2))
    assert np.allclose(rms, 1.0, atol=1e-13)
    y2 = y.copy()
    y2[:, 16:32] *= 7.0  # change group 1 only (by scale: its normalised output is unchanged)
    out2, r2 = norm.fwd(y2, z, w1, 16, 0.0)
    assert np.allclose(out2, out, atol=1e-13)
    assert np.allclose(r2[:, 1], r[:, 1] / 7.0) and np.allclose(r2[:, [0, 2]], r[:, [0, 2]])

"""The seeded generator hits the recipe's targets (active fraction per
token, outlier fraction, determinism, exact dtype rounding)."""
import numpy as np
import pytest

from unstructured_sparse_feedforward_amd import workloads as wl


def _active_per_token(inp, rows):
    z = inp.x[rows].astype(np.float64) @ inp.w_gate.astype(np.float64).T
    return (z > 0).sum(axis=1)


@pytest.mark.parametrize("w,T", [(wl.SMALL_F32, 128), (wl.GATED_1P5B, 1024),
                                 (wl.NONGATED[108], 512)])
def test_active_fraction(w, T):
    inp = wl.make_inputs(w, seed=0, T=T)
    normal = np.flatnonzero(~inp.outlier)
    n = _active_per_token(inp, normal)
    # mean of T binomials: within 6 standard errors of the target
    se = np.sqrt(w.nnz * (1 - w.nnz / w.F) / len(normal))
    assert abs(n.mean() - w.nnz) < 6 * se + 0.02 * w.nnz
    if inp.outlier.any():
        o = _active_per_token(inp, np.flatnonzero(inp.outlier))
        assert abs(o.mean() / w.F - 0.5) < 0.05


def test_outliers_and_front_bias():
    inp = wl.make_inputs(wl.GATED_1P5B, seed=0)
    assert abs(inp.outlier.mean() - 0.01) < 0.004
    assert np.all(inp.x[inp.outlier, 0] == 0) and np.all(inp.x[~inp.outlier, 0] == 1)
    m = wl.outlier_mask(wl.STACK_LAYER, np.random.default_rng(0))
    pos = np.arange(wl.STACK_LAYER.T) % 2048
    assert abs(m.mean() - 0.02) < 0.006
    assert abs(m[pos < 32].mean() - 0.3) < 0.08


def test_deterministic_and_prefix():
    a = wl.make_inputs(wl.SMALL_F32, seed=3)
    b = wl.make_inputs(wl.SMALL_F32, seed=3, T=64)
    assert np.array_equal(a.x[:64], b.x) and np.array_equal(a.w_gate, b.w_gate)
    c = wl.make_inputs(wl.SMALL_F32, seed=4)
    assert not np.array_equal(a.x, c.x)


def test_bf16_values_exact():
    inp = wl.make_inputs(wl.GATED_1P5B, seed=1, T=16)
    for name in ("x", "w_gate", "w_up", "w_down"):
        a = getattr(inp, name)
        assert np.all((a.view(np.uint32) & 0xFFFF) == 0), name
        bits = inp.bits(name)
        back = (bits.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(back, a)

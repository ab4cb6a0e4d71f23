"""Pins for the CPU oracle.

Each ``check_*`` takes an oracle module and raises AssertionError when the
oracle disagrees with something fixed outside it: hand-worked examples
under tests/golden/, a library routine (torch CPU float64, torch autograd),
an invariant of the format definitions, a special case with a known answer,
or brute force over every input of a tiny size. test_oracle_pins.py runs
them on the oracle; test_oracle_mutants.py runs them on copies of the
oracle with planted mistakes and expects each mutant to fail at least one.
"""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------- TwELL

def check_twell_golden(orc):
    g = _golden("twell_3x8_W4_C2.json")
    tw = orc.pack_twell(np.array(g["z"]), g["W"], g["C"])
    assert np.array_equal(tw["val"], np.array(g["val"]))
    assert np.array_equal(tw["idx"], np.array(g["idx"]))
    assert np.array_equal(tw["cnt"], np.array(g["cnt"]))
    assert np.array_equal(tw["row_flag"], np.array(g["row_flag"]))


def _check_twell_invariants(orc, z, W, C):
    T, F = z.shape
    tw = orc.pack_twell(z, W, C)
    nt = -(-F // W)
    assert tw["val"].shape == (T, nt, C) and tw["cnt"].shape == (T, nt)
    # the counts are the number of positives per tile, uncapped
    assert int(tw["cnt"].sum()) == int((z > 0).sum())
    for t in range(T):
        for b in range(nt):
            n = min(int(tw["cnt"][t, b]), C)
            js = tw["idx"][t, b, :n]
            # stored indices lie in their tile, strictly ascending, positive
            assert np.all((js >= b * W) & (js < min((b + 1) * W, F)))
            assert np.all(np.diff(js) > 0)
            assert np.all(z[t, js] > 0)
            assert np.array_equal(tw["val"][t, b, :n], z[t, js])
            # padding is (0, 0)
            assert np.all(tw["val"][t, b, n:] == 0)
            assert np.all(tw["idx"][t, b, n:] == 0)
    assert np.array_equal(tw["row_flag"], (tw["cnt"] > C).any(axis=1))
    # unpack(pack(Z)) reproduces ReLU(Z) exactly on unflagged rows
    rz = np.where(z > 0, z, 0.0)
    un = orc.unpack_twell(tw, F)
    ok = ~tw["row_flag"]
    assert np.array_equal(un[ok], rz[ok])
    return tw


def check_twell_invariants(orc):
    r = _rng(1)
    for (T, F, W, C, p) in [(7, 64, 16, 3, 0.1), (5, 100, 32, 4, 0.2),
                            (4, 256, 128, 16, 0.05), (3, 40, 8, 8, 0.5)]:
        z = r.standard_normal((T, F)) + np.where(r.random((T, F)) < p, 3.0,
                                                 -3.0)
        _check_twell_invariants(orc, z, W, C)


def check_twell_bruteforce(orc):
    """Every sign pattern of a 1 x 8 row, W = 4, C in {0, 1, 2, 4}."""
    for bits in range(256):
        pos = [(bits >> j) & 1 for j in range(8)]
        z = np.array([[(j + 1.0) if pos[j] else -(j + 1.0) for j in range(8)]])
        for C in (0, 1, 2, 4):
            tw = orc.pack_twell(z, 4, C)
            flag = False
            for b in range(2):
                set_cols = [j for j in range(4 * b, 4 * b + 4) if pos[j]]
                assert tw["cnt"][0, b] == len(set_cols)
                kept = set_cols[:C]
                assert list(tw["idx"][0, b, :len(kept)]) == kept
                assert list(tw["val"][0, b, :len(kept)]) == [j + 1.0 for j in kept]
                flag |= len(set_cols) > C
            assert bool(tw["row_flag"][0]) == flag


def check_twell_special_cases(orc):
    r = _rng(2)
    z = r.standard_normal((6, 96))
    # capacity >= tile width: nothing is flagged and the pack is lossless
    tw = orc.pack_twell(z, 32, 32)
    assert not tw["row_flag"].any()
    assert np.array_equal(orc.unpack_twell(tw, 96), np.where(z > 0, z, 0.0))
    # everything far below zero: all counts 0
    tw = orc.pack_twell(z - 1e9, 32, 4)
    assert (tw["cnt"] == 0).all() and not tw["row_flag"].any()
    # zeros, negative zeros and NaN are inactive
    zz = np.array([[0.0, -0.0, np.nan, 1e-300, -1e-300, 0.0, 0.0, 2.0]])
    tw = orc.pack_twell(zz, 8, 8)
    assert list(tw["idx"][0, 0, :2]) == [3, 7] and tw["cnt"][0, 0] == 2


# --------------------------------------------------------------- Hybrid

def check_hybrid_golden(orc):
    g = _golden("twell_3x8_W4_C2.json")
    tw = orc.pack_twell(np.array(g["z"]), g["W"], g["C"])
    h3 = orc.hybrid_compact(tw, 3)
    e3 = g["hybrid"]["K3"]
    assert np.array_equal(h3["ell_cnt"], e3["ell_cnt"])
    assert np.array_equal(h3["ell_idx"], e3["ell_idx"])
    assert np.array_equal(h3["ell_a"], e3["ell_a"])
    assert np.array_equal(h3["slot"], e3["slot"])
    assert np.array_equal(h3["brow"], e3["brow"])
    h2 = orc.hybrid_compact(tw, 2)
    e2 = g["hybrid"]["K2"]
    assert np.array_equal(h2["ell_cnt"], e2["ell_cnt"])
    assert np.array_equal(h2["slot"], e2["slot"])
    assert np.array_equal(h2["brow"], e2["brow"])
    # backup rows carry the dense A and U rows of their tokens
    z = np.array(g["z"])
    a = np.where(z > 0, z, 0.0)
    u = np.array(g["u"])
    for K, e in ((3, e3), (2, e2)):
        hy = orc.hybrid_compact(tw, K, a, u)
        assert np.array_equal(hy["bk_a"], np.array(e["bk_a"])), K
        assert np.array_equal(hy["bk_u"], np.array(e["bk_u"])), K


def check_hybrid_invariants(orc):
    r = _rng(3)
    T, F, W = 20, 64, 16
    z = r.standard_normal((T, F)) + np.where(r.random((T, F)) < 0.1, 2.0, -2.0)
    z[3] = np.abs(z[3]) + 0.1           # a heavy row
    a = np.where(z > 0, z, 0.0)
    tw = orc.pack_twell(z, W, W)        # lossless TwELL
    nnz = (z > 0).sum(axis=1)
    # K >= F: nothing goes to the backup
    hy = orc.hybrid_compact(tw, F, a)
    assert hy["n_backup"] == 0 and (hy["slot"] == -1).all()
    assert np.array_equal(hy["ell_cnt"], nnz)
    # K = 0: exactly the rows with any positive go to the backup
    hy = orc.hybrid_compact(tw, 0, a)
    assert np.array_equal(hy["slot"] >= 0, nnz > 0)
    for K in (0, 3, 5, 8, 64):
        hy = orc.hybrid_compact(tw, K, a)
        heavy = nnz > K
        assert np.array_equal(hy["slot"] >= 0, heavy)
        # backup slots are 0..n-1 in ascending token order
        assert np.array_equal(hy["brow"], np.flatnonzero(heavy))
        assert np.array_equal(hy["slot"][hy["brow"]], np.arange(heavy.sum()))
        # ELL plus backup rebuild ReLU(Z) exactly
        assert np.array_equal(orc.unpack_hybrid(hy, F), a)
    # a flagged TwELL row goes to the backup even when its count fits K
    tw = orc.pack_twell(z, W, 1)
    hy = orc.hybrid_compact(tw, F, a)
    assert np.array_equal(hy["slot"] >= 0, tw["row_flag"])
    assert np.array_equal(orc.unpack_hybrid(hy, F), a)
    # the backup's u rows are the given U rows of the backup tokens, at the
    # same slots as their A rows (U independent of A here)
    u = r.standard_normal((T, F))
    for K in (0, 5):
        hy = orc.hybrid_compact(orc.pack_twell(z, W, W), K, a, u)
        for s_, t in enumerate(np.flatnonzero(nnz > K)):
            assert np.array_equal(hy["bk_u"][s_], u[t])
            assert np.array_equal(hy["bk_a"][s_], a[t])


# --------------------------------------------------------------- dense layer

def check_ffn_golden(orc):
    g = _golden("ffn_1x2x2_integers.json")
    y, it = orc.dense_ffn(np.array(g["x"]), np.array(g["w_gate"]),
                          np.array(g["w_up"]), np.array(g["w_down"]))
    assert np.array_equal(y, np.array(g["y"]))
    assert np.array_equal(it["z"], np.array(g["z"]))
    assert np.array_equal(it["h"], np.array(g["h"]))


def _rand_layer(r, T, d, F, gated=True):
    x = r.standard_normal((T, d))
    wg = r.standard_normal((d, F))
    wu = r.standard_normal((d, F)) if gated else None
    wd = r.standard_normal((F, d))
    return x, wg, wu, wd


def check_ffn_vs_torch(orc):
    r = _rng(4)
    for gated in (True, False):
        x, wg, wu, wd = _rand_layer(r, 9, 7, 13, gated)
        y, _ = orc.dense_ffn(x, wg, wu, wd)
        tx = torch.from_numpy(x)
        h = torch.relu(tx @ torch.from_numpy(wg))
        if gated:
            h = h * (tx @ torch.from_numpy(wu))
        ref = (h @ torch.from_numpy(wd)).numpy()
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def check_gated_reduces_to_nongated(orc):
    """W_u[:, j] = e_0 with x[:, 0] = 1 makes U = 1, so the gated layer
    equals the non-gated one with W_1 = W_g, W_2 = W_d exactly."""
    r = _rng(5)
    x, wg, _, wd = _rand_layer(r, 6, 5, 12, False)
    x[:, 0] = 1.0
    wu = np.zeros((5, 12))
    wu[0, :] = 1.0
    yg, _ = orc.dense_ffn(x, wg, wu, wd)
    yn, _ = orc.dense_ffn(x, wg, None, wd)
    assert np.array_equal(yg, yn)


def check_bf16_rounding(orc):
    r = _rng(6)
    v = r.standard_normal(4096).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(orc.round_bf16(v), ref)
    # ties go to even
    assert orc.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert orc.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert orc.round_bf16(np.array([-(1 + 2.0 ** -8)]))[0] == -1.0


def check_bf16_hidden_golden(orc):
    """Hand-worked standard bf16 layer: H rounded once, ties to even."""
    g = _golden("ffn_bf16_hidden_1x2x3.json")
    y = orc.dense_ffn_bf16_hidden(np.array(g["x"]), np.array(g["w_gate"]),
                                  np.array(g["w_up"]), np.array(g["w_down"]))
    assert np.array_equal(y, np.array(g["y"]))


def check_bf16_hidden_vs_torch(orc):
    """Integer inputs keep every H exact in float32, so torch's own bf16
    conversion of H (float32 -> bfloat16, round to nearest even) is exact
    to compare against; H spans values well above 256, where bf16 drops
    bits. Gated and non-gated."""
    r = _rng(14)
    for gated in (True, False):
        x = r.integers(-4, 5, (9, 6)).astype(np.float64)
        wg = r.integers(-4, 5, (6, 16)).astype(np.float64)
        wu = r.integers(-9, 10, (6, 16)).astype(np.float64) if gated else None
        wd = r.integers(-3, 4, (16, 6)).astype(np.float64)
        y = orc.dense_ffn_bf16_hidden(x, wg, wu, wd)
        tx = torch.from_numpy(x)
        h = torch.relu(tx @ torch.from_numpy(wg))
        if gated:
            h = h * (tx @ torch.from_numpy(wu))
        assert float(h.abs().max()) > 512 or not gated
        hb = h.float().to(torch.bfloat16).double()
        ref = (hb @ torch.from_numpy(wd)).numpy()
        assert np.array_equal(y, ref)
        # at least one H was changed by the rounding
        assert gated is False or bool((hb != h).any())


def check_bf16_store_golden(orc):
    """Hand-worked layer with bf16 stored activations, forward and backward."""
    g = _golden("ffn_bf16_store_1x2x2.json")
    args = [np.array(g[k]) for k in ("x", "w_gate", "w_up", "w_down")]
    assert np.array_equal(orc.dense_ffn_bf16_store(*args), np.array(g["y"]))
    gr = orc.backward_bf16_store(*args, np.array(g["dy"]))
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(gr[k], np.array(g[k])), k


def _ste_bf16(t):
    """torch: the value rounded to bf16 in the forward, the identity in the
    backward (exact for values that float32 holds exactly)."""
    return t + (t.float().to(torch.bfloat16).double() - t).detach()


def check_bf16_store_vs_autograd(orc):
    """Integer inputs keep every A, U and product exact in float32, so
    torch's own bf16 conversion rounds them as the storage does; torch
    autograd through the rounding-as-identity gives the gradients. A and U
    span values above 256, where bf16 drops bits."""
    r = _rng(16)
    for gated in (True, False):
        for l1 in (0.0, 0.5):
            x = r.integers(-4, 5, (7, 6)).astype(np.float64)
            wg = r.integers(-60, 61, (6, 16)).astype(np.float64)
            wu = r.integers(-60, 61, (6, 16)).astype(np.float64) if gated else None
            wd = r.integers(-3, 4, (16, 6)).astype(np.float64)
            dy = r.integers(-2, 3, (7, 6)).astype(np.float64)
            tx = torch.tensor(x, requires_grad=True)
            twg = torch.tensor(wg, requires_grad=True)
            twd = torch.tensor(wd, requires_grad=True)
            z = tx @ twg
            assert float(z.detach().abs().max()) > 256
            a = _ste_bf16(torch.relu(z))
            if gated:
                twu = torch.tensor(wu, requires_grad=True)
                h = a * _ste_bf16(tx @ twu)
            else:
                h = a
            y = h @ twd
            assert np.array_equal(orc.dense_ffn_bf16_store(x, wg, wu, wd), y.detach().numpy())
            # the L1 term acts on the activation as the layer computes it
            loss = (y * torch.from_numpy(dy)).sum() + l1 * torch.relu(z).sum()
            loss.backward()
            gr = orc.backward_bf16_store(x, wg, wu, wd, dy, l1_coeff=l1)
            assert np.allclose(gr["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-9)
            assert np.allclose(gr["dw_gate"], twg.grad.numpy(), rtol=1e-12, atol=1e-9)
            assert np.allclose(gr["dw_down"], twd.grad.numpy(), rtol=1e-12, atol=1e-9)
            if gated:
                assert np.allclose(gr["dw_up"], twu.grad.numpy(), rtol=1e-12, atol=1e-9)
            # a given active set (a third of the entries flipped): A = Z * M
            m = (x @ wg > 0) ^ (r.random((7, 16)) < 0.33)
            tx.grad = twg.grad = twd.grad = None
            zm = (tx @ twg) * torch.from_numpy(m.astype(np.float64))
            a = _ste_bf16(zm)
            h = a * _ste_bf16(tx @ twu) if gated else a
            ((h @ twd) * torch.from_numpy(dy)).sum().add(l1 * zm.sum()).backward()
            gm = orc.backward_bf16_store(x, wg, wu, wd, dy, l1_coeff=l1, mask=m)
            assert np.allclose(gm["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-9)
            assert np.allclose(gm["dw_gate"], twg.grad.numpy(), rtol=1e-12, atol=1e-9)
            assert np.allclose(gm["dw_down"], twd.grad.numpy(), rtol=1e-12, atol=1e-9)


def check_bf16_store_exact_values(orc):
    """When every A and U is a bf16 value already, the storage changes
    nothing: the plain layer and its backward come back exactly."""
    r = _rng(17)
    x = r.integers(-3, 4, (6, 5)).astype(np.float64)
    wg = r.integers(-2, 3, (5, 9)).astype(np.float64)
    wu = r.integers(-2, 3, (5, 9)).astype(np.float64)
    wd = r.integers(-2, 3, (9, 5)).astype(np.float64)
    dy = r.integers(-2, 3, (6, 5)).astype(np.float64)
    y, _ = orc.dense_ffn(x, wg, wu, wd)
    assert np.array_equal(orc.dense_ffn_bf16_store(x, wg, wu, wd), y)
    a, b = orc.backward_bf16_store(x, wg, wu, wd, dy, 0.25), orc.backward(x, wg, wu, wd, dy, 0.25)
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(a[k], b[k]), k


def check_dense_train_golden(orc):
    """Hand-worked standard bf16 dense training step."""
    g = _golden("ffn_dense_train_bf16_1x2x2.json")
    r = orc.dense_train_bf16(*(np.array(g[k]) for k in ("x", "w_gate", "w_up", "w_down", "dy")))
    for k in ("y", "dx", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(r[k], np.array(g[k])), k


class _RoundBoth(torch.autograd.Function):
    """bf16 rounding of the value in the forward and of the gradient in the
    backward (exact for values float32 holds exactly)."""

    @staticmethod
    def forward(ctx, t):
        return t.float().to(torch.bfloat16).double()

    @staticmethod
    def backward(ctx, g):
        return g.float().to(torch.bfloat16).double()


def check_dense_train_vs_autograd(orc):
    """The step as torch autograd sees it: the GEMM outputs rounded in
    value and in gradient (so the gradients entering the weight GEMMs are
    bf16), H rounded in value only, on integer inputs that float32 holds
    exactly; values pass 256, where bf16 drops bits."""
    r = _rng(18)
    for gated in (True, False):
        for l1 in (0.0, 0.5):
            x = r.integers(-4, 5, (7, 6)).astype(np.float64)
            wg = r.integers(-60, 61, (6, 16)).astype(np.float64)
            wu = r.integers(-60, 61, (6, 16)).astype(np.float64) if gated else None
            wd = r.integers(-3, 4, (16, 6)).astype(np.float64)
            dy = r.integers(-9, 10, (7, 6)).astype(np.float64)
            tx = torch.tensor(x, requires_grad=True)
            twg = torch.tensor(wg, requires_grad=True)
            twd = torch.tensor(wd, requires_grad=True)
            zs = _RoundBoth.apply(tx @ twg)
            a = torch.relu(zs)
            if gated:
                twu = torch.tensor(wu, requires_grad=True)
                h = _ste_bf16(a * _RoundBoth.apply(tx @ twu))
            else:
                h = a
            y = h @ twd
            (y * torch.from_numpy(dy)).sum().add(l1 * a.sum()).backward()
            got = orc.dense_train_bf16(x, wg, wu, wd, dy, l1_coeff=l1)
            assert float(zs.detach().abs().max()) > 256
            assert np.array_equal(got["y"], y.detach().numpy())
            assert np.allclose(got["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-9)
            assert np.allclose(got["dw_gate"], twg.grad.numpy(), rtol=1e-12, atol=1e-9)
            assert np.allclose(got["dw_down"], twd.grad.numpy(), rtol=1e-12, atol=1e-9)
            if gated:
                assert np.allclose(got["dw_up"], twu.grad.numpy(), rtol=1e-12, atol=1e-9)


def check_dense_train_exact_values(orc):
    """With every Z, U, H, dZ and dU a bf16 value already, the step is the
    plain layer and its backward exactly."""
    r = _rng(19)
    x = r.integers(-2, 3, (6, 4)).astype(np.float64)
    wg = r.integers(-2, 3, (4, 9)).astype(np.float64)
    wu = r.integers(-2, 3, (4, 9)).astype(np.float64)
    wd = r.integers(-1, 2, (9, 4)).astype(np.float64)
    dy = r.integers(-1, 2, (6, 4)).astype(np.float64)
    got = orc.dense_train_bf16(x, wg, wu, wd, dy, 0.5)
    y, _ = orc.dense_ffn(x, wg, wu, wd)
    ref = orc.backward(x, wg, wu, wd, dy, 0.5)
    assert np.array_equal(got["y"], y)
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(got[k], ref[k]), k


# --------------------------------------------------------------- sparse layer

def check_sparse_equals_dense(orc):
    r = _rng(7)
    for trial in range(12):
        T = int(r.integers(1, 9))
        d = int(r.integers(1, 9))
        F = int(r.integers(1, 17))
        W = int(r.integers(1, 9))
        C = int(r.integers(0, 5))
        gated = bool(trial % 2)
        x, wg, wu, wd = _rand_layer(r, T, d, F, gated)
        y, _ = orc.sparse_ffn(x, wg, wu, wd, W, C)
        yd, _ = orc.dense_ffn(x, wg, wu, wd)
        assert np.allclose(y, yd, rtol=1e-12, atol=1e-12)


def check_sparse_exact_integers(orc):
    """Small integer inputs make every sum exact, so the sparse and dense
    orders of summation give identical results."""
    r = _rng(8)
    for gated in (True, False):
        x = r.integers(-3, 4, (8, 6)).astype(np.float64)
        wg = r.integers(-2, 3, (6, 16)).astype(np.float64)
        wu = r.integers(-2, 3, (6, 16)).astype(np.float64) if gated else None
        wd = r.integers(-2, 3, (16, 6)).astype(np.float64)
        y, tw = orc.sparse_ffn(x, wg, wu, wd, 8, 8)
        yd, _ = orc.dense_ffn(x, wg, wu, wd)
        assert not tw["row_flag"].any()
        assert np.array_equal(y, yd)


def check_forced_backup(orc):
    """C = 0 flags every row with a positive, so every such row is dense."""
    r = _rng(9)
    x, wg, wu, wd = _rand_layer(r, 7, 4, 10)
    y, tw = orc.sparse_ffn(x, wg, wu, wd, 4, 0)
    yd, it = orc.dense_ffn(x, wg, wu, wd)
    assert np.array_equal(tw["row_flag"], (it["z"] > 0).any(axis=1))
    assert np.array_equal(y, yd)


# --------------------------------------------------------------- backward

def check_backward_golden(orc):
    g = _golden("ffn_1x2x2_integers.json")
    gr = orc.backward(np.array(g["x"]), np.array(g["w_gate"]),
                      np.array(g["w_up"]), np.array(g["w_down"]),
                      np.array(g["dy"]))
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(gr[k], np.array(g[k])), k


def check_backward_vs_autograd(orc):
    r = _rng(10)
    for gated in (True, False):
        for l1 in (0.0, 0.37):
            x, wg, wu, wd = _rand_layer(r, 6, 5, 11, gated)
            dy = r.standard_normal((6, 5))
            gr = orc.backward(x, wg, wu, wd, dy, l1_coeff=l1)
            tx = torch.tensor(x, requires_grad=True)
            twg = torch.tensor(wg, requires_grad=True)
            twd = torch.tensor(wd, requires_grad=True)
            a = torch.relu(tx @ twg)
            if gated:
                twu = torch.tensor(wu, requires_grad=True)
                h = a * (tx @ twu)
            else:
                h = a
            loss = ((h @ twd) * torch.from_numpy(dy)).sum() + l1 * a.sum()
            loss.backward()
            assert np.allclose(gr["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-12)
            assert np.allclose(gr["dw_gate"], twg.grad.numpy(), rtol=1e-12, atol=1e-12)
            assert np.allclose(gr["dw_down"], twd.grad.numpy(), rtol=1e-12, atol=1e-12)
            if gated:
                assert np.allclose(gr["dw_up"], twu.grad.numpy(), rtol=1e-12, atol=1e-12)


def check_backward_given_mask_vs_autograd(orc):
    """A fixed active set M: the layer with A = Z * M (M constant) under
    torch autograd; M = 1[Z > 0] reproduces the plain backward exactly."""
    r = _rng(15)
    for gated in (True, False):
        x, wg, wu, wd = _rand_layer(r, 6, 5, 11, gated)
        dy = r.standard_normal((6, 5))
        z = x @ wg
        assert np.array_equal(orc.backward(x, wg, wu, wd, dy, 0.2, mask=z > 0)["dx"],
                              orc.backward(x, wg, wu, wd, dy, 0.2)["dx"])
        # a mask that disagrees with Z > 0 on a third of the entries
        m = (z > 0) ^ (r.random(z.shape) < 0.33)
        gr = orc.backward(x, wg, wu, wd, dy, l1_coeff=0.2, mask=m)
        tx = torch.tensor(x, requires_grad=True)
        twg = torch.tensor(wg, requires_grad=True)
        twd = torch.tensor(wd, requires_grad=True)
        a = (tx @ twg) * torch.from_numpy(m.astype(np.float64))
        if gated:
            twu = torch.tensor(wu, requires_grad=True)
            h = a * (tx @ twu)
        else:
            h = a
        loss = ((h @ twd) * torch.from_numpy(dy)).sum() + 0.2 * a.sum()
        loss.backward()
        assert np.allclose(gr["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(gr["dw_gate"], twg.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(gr["dw_down"], twd.grad.numpy(), rtol=1e-12, atol=1e-12)
        if gated:
            assert np.allclose(gr["dw_up"], twu.grad.numpy(), rtol=1e-12, atol=1e-12)


def check_backward_finite_differences(orc):
    # first seeded draw whose pre-activations all keep clear of the kink
    for seed in range(11, 200):
        r = _rng(seed)
        x, wg, wu, wd = _rand_layer(r, 4, 3, 7)
        dy = r.standard_normal((4, 3))
        if np.abs(x @ wg).min() > 1e-2:
            break
    gr = orc.backward(x, wg, wu, wd, dy)
    f = lambda xx, g_, u_, d_: float((orc.dense_ffn(xx, g_, u_, d_)[0] * dy).sum())
    eps = 1e-6
    for name, arr, pos in (("dx", x, 0), ("dw_gate", wg, 1), ("dw_up", wu, 2),
                           ("dw_down", wd, 3)):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            args = [x, wg, wu, wd]
            p, m = arr.copy(), arr.copy()
            p[i] += eps
            m[i] -= eps
            args[pos] = p
            fp = f(*args)
            args[pos] = m
            fm = f(*args)
            num[i] = (fp - fm) / (2 * eps)
        assert np.allclose(gr[name], num, rtol=1e-6, atol=1e-6), name


def check_backward_sparse_equals_dense(orc):
    r = _rng(12)
    for gated in (True, False):
        x, wg, wu, wd = _rand_layer(r, 9, 6, 16, gated)
        wg[0, :] -= 1.0
        dy = r.standard_normal((9, 6))
        z = x @ wg
        tw = orc.pack_twell(z, 8, 2)
        for K in (0, 3, 100):
            hy = orc.hybrid_compact(tw, K)
            gs = orc.backward_sparse(x, wg, wu, wd, dy, hy, l1_coeff=0.1)
            gd = orc.backward(x, wg, wu, wd, dy, l1_coeff=0.1)
            for k in ("dx", "dw_gate", "dw_down") + (("dw_up",) if gated else ()):
                assert np.allclose(gs[k], gd[k], rtol=1e-12, atol=1e-12), k


def check_dead_neurons_zero_grad(orc):
    r = _rng(13)
    x, wg, wu, wd = _rand_layer(r, 5, 4, 9)
    wg[:, 2] = 0.0
    wg[0, 2] = -1.0
    x[:, 0] = 1.0
    dy = r.standard_normal((5, 4))
    gr = orc.backward(x, wg, wu, wd, dy)   # neuron 2 is never active
    assert np.all(gr["dw_gate"][:, 2] == 0)
    assert np.all(gr["dw_up"][:, 2] == 0)
    assert np.all(gr["dw_down"][2] == 0)


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]


def run_all(orc):
    failures = []
    for c in ALL_CHECKS:
        try:
            c(orc)
        except Exception as e:   # noqa: BLE001 - any failure counts
            failures.append((c.__name__, repr(e)))
    return failures



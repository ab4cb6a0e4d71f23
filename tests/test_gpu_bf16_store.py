"""The layer with bf16 stored activations (desc.store_dtype = SFFN_BF16)
against the oracle that rounds A and U to bf16 where they are stored.

TwELL values, ELL a and u, and backup rows' a and u are bf16; the layer
computes with the stored values (H = bf16(a) bf16(u)) and the backward
reads them. Bars: TwELL and Hybrid bit-exact against the oracle packer's
values rounded to bf16 when the pack gets the oracle's pre-activations;
outputs and gradients within the bf16 bound of the mirrored oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close_bf16, assert_twell_equal, dev, layer, math_weights, to_np,
                      twell_np)
from test_gpu_hybrid import _plant_near_zero, hybrid_np
from unstructured_sparse_feedforward_amd import SparseFFN
from unstructured_sparse_feedforward_amd import binding as B
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _print(*a):
    print(*a, flush=True)


def _rb(v):
    return oracle.round_bf16(np.asarray(v, dtype=np.float64))


def _args(inp):
    return [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]


@pytest.mark.parametrize("T,F,C,seed", [(33, 256, 1, 1), (257, 5632, 8, 3), (1000, 8192, 48, 5)])
def test_pack_bf16_store_bitexact(T, F, C, seed):
    _print(f"pack bf16 store T={T} F={F} C={C}")
    r = np.random.default_rng(seed)
    z = (r.standard_normal((T, F)) * 300 - 600).astype(np.float32)   # values bf16 must round
    heavy = r.random(T) < 0.05
    z[heavy] = np.abs(z[heavy]) * np.where(r.random((heavy.sum(), F)) < 0.5, 1, -1)
    ffn = SparseFFN(512, F, gated=True, twell_cap=C, dtype=BF, store_dtype=BF)
    tw = twell_np(ffn.pack_twell(torch.from_numpy(z).cuda()))
    ref = oracle.pack_twell(z.astype(np.float64), 128, C)
    ref["val"] = _rb(ref["val"])
    assert_twell_equal(tw, ref)


@pytest.mark.parametrize("w,T", [(wl.GATED_1P5B, 1024), (wl.NONGATED[108], 333)])
def test_fused_twell_bf16_store_matches_pack_of_own_z(w, T):
    inp = wl.make_inputs(w, seed=12, T=T)
    ffn = layer(inp, store_dtype=BF)
    args = _args(inp)
    tw_f = ffn.new_twell(T)
    assert tw_f["val"].dtype == BF
    ffn.forward(*args, tw=tw_f)
    tw_p = ffn.pack_twell(ffn.gate_preact(args[0], args[1]))
    a, b = twell_np(tw_f), twell_np(tw_p)
    assert_twell_equal(a, b)
    assert a["n_flagged"] == b["n_flagged"]


def test_hybrid_compact_bf16_store_bitexact():
    T, F, C, K = 300, 1024, 16, 8
    r = np.random.default_rng(0)
    z = (r.standard_normal((T, F)) * 300 - 800).astype(np.float32)
    heavy = r.random(T) < 0.05
    z[heavy] = (r.standard_normal((heavy.sum(), F)) * 300).astype(np.float32)
    ffn = SparseFFN(512, F, gated=True, twell_cap=C, ell_cap=K, dtype=BF, store_dtype=BF)
    zd = torch.from_numpy(z).cuda()
    hy = hybrid_np(ffn.hybrid_compact(ffn.pack_twell(zd), T, z=zd))
    a = np.where(z > 0, z, 0).astype(np.float64)
    ref = oracle.hybrid_compact(oracle.pack_twell(z.astype(np.float64), 128, C), K, a_dense=a)
    assert hy["n_backup"] == ref["n_backup"] > 0
    assert np.array_equal(hy["ell_cnt"], ref["ell_cnt"])
    m = np.arange(K)[None, :] < ref["ell_cnt"][:, None]
    assert np.array_equal(hy["ell_idx"][m], ref["ell_idx"][m])
    assert np.array_equal(hy["ell_a"][m].astype(np.float64), _rb(ref["ell_a"][m]))
    assert np.array_equal(hy["bk_a"][:ref["n_backup"]].astype(np.float64), _rb(ref["bk_a"]))


def _y_store(inp, rows=None):
    wg, wu, wd = math_weights(inp)
    x = inp.x.astype(np.float64)
    return oracle.dense_ffn_bf16_store(x if rows is None else x[rows], wg, wu, wd)


@pytest.mark.parametrize("w,T", [(wl.GATED_1P5B, 1024), (wl.GATED_1P5B_NNZ15, 1024),
                                 (wl.NONGATED[29], 512), (wl.NONGATED[108], 256),
                                 (wl.stack_layer(5), 400)])
def test_forward_bf16_store(w, T):
    _print(f"forward bf16 store {w.name} T={T}")
    inp = wl.make_inputs(w, seed=16, T=T)
    ffn = layer(inp, store_dtype=BF)
    tw = ffn.new_twell(T)
    y = ffn.forward(*_args(inp), tw=tw).cpu().numpy()
    _print("  flagged rows:", twell_np(tw)["n_flagged"])
    assert_close_bf16(y, _y_store(inp), "y")


def test_forward_bf16_store_full_size_sampled_rows():
    """The gated workload at its full size with bf16 storage, in the launch
    configuration the benchmark times; 384 sampled rows (all flagged rows
    among them) against the mirrored oracle."""
    w = wl.GATED_1P5B
    inp = wl.make_inputs(w, seed=0)
    ffn = layer(inp, store_dtype=BF)
    tw = ffn.new_twell(w.T)
    y = ffn.forward(*_args(inp), tw=tw).cpu().numpy()
    g = twell_np(tw)
    flagged = g["flagged"][:g["n_flagged"]]
    r = np.random.default_rng(0)
    rows = np.unique(np.concatenate([flagged, r.choice(w.T, 384 - len(flagged), replace=False)]))
    assert_close_bf16(y[rows], _y_store(inp, rows), "sampled rows")


def _gpu_mask(hy, T, F):
    m = np.zeros((T, F), dtype=bool)
    for t in range(T):
        if hy["slot"][t] >= 0:
            m[t] = hy["bk_a"][hy["slot"][t]] > 0
        else:
            m[t, hy["ell_idx"][t, :hy["ell_cnt"][t]]] = True
    return m


@pytest.mark.parametrize("w,T,seed,l1,plant", [
    (wl.TRAIN_HYBRID, 256, 47, 0.0, False),
    (wl.TRAIN_HYBRID, 512, 57, 0.05, False),
    (wl.TRAIN_HYBRID, 256, 71, 0.0, True),
    (wl.TRAIN_HYBRID.replace(gated=False, F=8192, nnz=40, name="train_nongated"), 256, 55, 0.0,
     False),
])
def test_training_bf16_store(w, T, seed, l1, plant):
    """Training forward and backward with bf16 storage against the mirrored
    oracle, evaluated on the GPU's own active set (as the Hybrid stores it;
    with planted near-zero pre-activations the sets differ on some
    entries)."""
    _print(f"training bf16 store {w.name} T={T} l1={l1} plant={plant}")
    inp = wl.make_inputs(w, seed=seed, T=T)
    if plant:
        r = np.random.default_rng(5)
        _plant_near_zero(inp, list(zip(r.choice(T, 96), r.choice(w.F, 96, replace=False))))
    ffn = SparseFFN(w.d, w.F, gated=w.gated, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=BF, store_dtype=BF)
    args = _args(inp)
    y, hyd = ffn.forward_train(*args)
    assert hyd["ell_a"].dtype == BF and hyd["bk_a"].dtype == BF
    assert ffn.hybrid_check(hyd) == B.SFFN_OK
    dx, dwg, dwu, dwd = ffn.backward(*args, hyd, dev(inp, "dy"), l1_coeff=l1)
    hy = hybrid_np(hyd)
    _print("  backup rows:", hy["n_backup"])
    wg, wu, wd = math_weights(inp)
    x64 = inp.x.astype(np.float64)
    mask = _gpu_mask(hy, T, w.F)
    z = x64 @ wg
    assert np.all(np.abs(z[mask != (z > 0)]) < 1e-3)
    assert_close_bf16(y.cpu().numpy(), _y_store(inp), "y")
    ref = oracle.backward_bf16_store(x64, wg, wu, wd, inp.dy.astype(np.float64), l1_coeff=l1,
                                     mask=mask)
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")
    if w.gated:
        assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    # the saved activations are the rounded values
    rows, ks = np.nonzero(np.arange(w.ell_cap)[None, :] < hy["ell_cnt"][:, None])
    js = hy["ell_idx"][rows, ks]
    assert np.abs(hy["ell_a"][rows, ks] - _rb(z[rows, js])).max() <= 2.0 ** -7 * np.abs(
        z[rows, js]).max()


def test_training_bf16_store_full_size_sampled():
    """The training step at its full size (T = 8192, d = 2048, F = 5632,
    K = 64, 5% outliers) with bf16 storage; sampled rows of dx and y and
    sampled neurons of dW against the mirrored oracle (rows and neurons
    with a pre-activation within 2e-5 of 0 left out)."""
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=11)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dense_rows=w.dense_rows, dtype=BF, store_dtype=BF)
    args = _args(inp)
    y, hyd = ffn.forward_train(*args)
    assert ffn.hybrid_check(hyd) == B.SFFN_OK
    dx, dwg, dwu, dwd = ffn.backward(*args, hyd, dev(inp, "dy"))
    torch.cuda.synchronize()
    slot = hyd["slot"].cpu().numpy()[:w.T]
    nb = int(hyd["n_backup"][0].item())
    wg, wu, wd = math_weights(inp)
    x64, dy64 = inp.x.astype(np.float64), inp.dy.astype(np.float64)
    rng = np.random.default_rng(0)
    rows = np.sort(np.concatenate([rng.choice(np.flatnonzero(slot < 0), 96, replace=False),
                                   rng.choice(np.flatnonzero(slot >= 0), min(nb, 32),
                                              replace=False)]))
    rows = rows[np.abs(x64[rows] @ wg).min(axis=1) > 2e-5]
    assert rows.size > 100
    ref = oracle.backward_bf16_store(x64[rows], wg, wu, wd, dy64[rows])
    assert_close_bf16(y.cpu().numpy()[rows],
                      oracle.dense_ffn_bf16_store(x64[rows], wg, wu, wd), "y rows")
    assert_close_bf16(dx.cpu().numpy()[rows], ref["dx"], "dx rows")
    J = np.sort(rng.choice(w.F, 96, replace=False))
    J = J[np.abs(x64 @ wg[:, J]).min(axis=0) > 2e-5]
    assert J.size > 64
    refJ = oracle.backward_bf16_store(x64, wg[:, J], wu[:, J], wd[J], dy64)
    assert_close_bf16(dwg.cpu().numpy()[J], refJ["dw_gate"].T, "dw_gate neurons")
    assert_close_bf16(dwu.cpu().numpy()[J], refJ["dw_up"].T, "dw_up neurons")
    assert_close_bf16(dwd.cpu().numpy()[J], refJ["dw_down"], "dw_down neurons")

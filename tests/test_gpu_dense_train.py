"""The same library's dense bf16 training step (the sparse step's
comparator) against the oracle's standard bf16 dense training step, which
rounds Z, U, H, dZ and dU to bf16 at the same points."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close_bf16, dev, math_weights
from unstructured_sparse_feedforward_amd import SparseFFN
from unstructured_sparse_feedforward_amd import binding as B
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _check(got, ref, rows=None, what=""):
    y, dx, dwg, dwu, dwd = got
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    assert_close_bf16(sel(y.cpu().numpy()), ref["y"], what + "y")
    assert_close_bf16(sel(dx.cpu().numpy()), ref["dx"], what + "dx")


@pytest.mark.parametrize("w,T,seed,l1", [
    (wl.TRAIN_HYBRID, 256, 47, 0.0),
    (wl.TRAIN_HYBRID, 320, 57, 0.05),
    (wl.TRAIN_HYBRID.replace(gated=False, F=8192, nnz=40, name="train_nongated"), 256, 55, 0.0),
])
def test_dense_training_step(w, T, seed, l1):
    _print(f"dense training {w.name} T={T} l1={l1}")
    inp = wl.make_inputs(w, seed=seed, T=T)
    wg, wu, wd = math_weights(inp)
    x64 = inp.x.astype(np.float64)
    assert np.abs(x64 @ wg).min() > 2e-5
    ffn = SparseFFN(w.d, w.F, gated=w.gated, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y, act = ffn.forward_train_dense(*args)
    dx, dwg, dwu, dwd = ffn.backward_dense(*args, act, dev(inp, "dy"), l1_coeff=l1)
    ref = oracle.dense_train_bf16(x64, wg, wu, wd, inp.dy.astype(np.float64), l1_coeff=l1)
    assert_close_bf16(y.cpu().numpy(), ref["y"], "y")
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")
    if w.gated:
        assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    # the saved Z_s are the bf16 pre-activations
    F = w.F
    zs = act[:T * F].view(T, F).float().cpu().numpy()
    # one bf16 step (2^-7 of the value) where fp32 and fp64 round differently
    assert np.abs(zs - oracle.round_bf16(x64 @ wg)).max() <= 2.0 ** -7 * np.abs(x64 @ wg).max()


def test_dense_training_full_size_sampled():
    """The dense training step at the training workload's full size
    (T = 8192, d = 2048, F = 5632) in the configuration the benchmark
    times: sampled rows of y and dx, sampled neurons of every dW."""
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=11)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y, act = ffn.forward_train_dense(*args)
    dx, dwg, dwu, dwd = ffn.backward_dense(*args, act, dev(inp, "dy"))
    torch.cuda.synchronize()
    wg, wu, wd = math_weights(inp)
    x64, dy64 = inp.x.astype(np.float64), inp.dy.astype(np.float64)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(w.T, 128, replace=False))
    rows = rows[np.abs(x64[rows] @ wg).min(axis=1) > 2e-5]
    ref = oracle.dense_train_bf16(x64[rows], wg, wu, wd, dy64[rows])
    assert_close_bf16(y.cpu().numpy()[rows], ref["y"], "y rows")
    assert_close_bf16(dx.cpu().numpy()[rows], ref["dx"], "dx rows")
    J = np.sort(rng.choice(w.F, 96, replace=False))
    J = J[np.abs(x64 @ wg[:, J]).min(axis=0) > 2e-5]
    assert J.size > 64
    refJ = oracle.dense_train_bf16(x64, wg[:, J], wu[:, J], wd[J], dy64)
    assert_close_bf16(dwg.cpu().numpy()[J], refJ["dw_gate"].T, "dw_gate neurons")
    assert_close_bf16(dwu.cpu().numpy()[J], refJ["dw_up"].T, "dw_up neurons")
    assert_close_bf16(dwd.cpu().numpy()[J], refJ["dw_down"], "dw_down neurons")


def test_dense_training_needs_t_multiple_of_64():
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=47, T=100)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    with pytest.raises(B.SffnError) as ei:
        ffn.forward_train_dense(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")))
    assert ei.value.status == B.SFFN_E_UNSUPPORTED

"""The dense path's row capacity and the ELL capacity at inference.

The workspace holds the dense path's rows up to desc.dense_rows; a call
that routes more rows leaves the dense path's rows invalid (the ELL rows
are unaffected) and sffn_check reports SFFN_E_CAPACITY (once; the report
is cleared by the check). The
binding's checked calls then rebuild the handle with a T-row capacity and
repeat the call, so their results are complete. At inference, rows with
more active neurons than the ELL capacity K take the dense path too (the
Hybrid's routing rule) and the layer's output does not change.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close_bf16, dev, layer, math_weights, twell_np
from unstructured_sparse_feedforward_amd import SparseFFN
from unstructured_sparse_feedforward_amd import binding as B
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _args(inp):
    return [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]


def _y_ref(inp, rows=None):
    wg, wu, wd = math_weights(inp)
    x = inp.x.astype(np.float64)
    y, _ = oracle.dense_ffn(x if rows is None else x[rows], wg, wu, wd)
    return y


def test_inference_capacity_reported_and_recovered():
    w = wl.GATED_1P5B.replace(outlier_frac=0.2)
    inp = wl.make_inputs(w, seed=31, T=600)
    _print("inference capacity: dense_rows=32, about 120 flagged rows")
    ffn = layer(inp, dense_rows=32)
    args = _args(inp)
    tw = ffn.new_twell(600)
    y = ffn.forward(*args, tw=tw, check=False)
    assert ffn.lib.sffn_check(ffn.h, B._stream()) == B.SFFN_E_CAPACITY
    # the report is cleared by the check
    assert ffn.lib.sffn_check(ffn.h, B._stream()) == B.SFFN_OK
    g = twell_np(tw)
    flagged = g["flagged"][:g["n_flagged"]]
    assert len(flagged) > 64
    # the rows on the ELL path are unaffected (the dense path's rows are
    # not valid after an overflow)
    y = y.cpu().numpy()
    done = np.setdiff1d(np.arange(600), flagged)
    assert_close_bf16(y[done], _y_ref(inp, done), "ELL rows")
    # the checked call rebuilds the handle with a T-row capacity and repeats
    y2 = ffn.forward(*args, tw=tw)
    assert ffn.dense_rows == 0
    assert_close_bf16(y2.cpu().numpy(), _y_ref(inp), "y after the fallback")


@pytest.mark.parametrize("K", [24, 40])
def test_inference_ell_cap_routes_rows_dense(K):
    """An ELL capacity near the mean count (29) sends many rows with more
    positives than K to the dense path; the output is the layer's all the
    same and equal to the K = n_t * C run within the bound."""
    w = wl.GATED_1P5B
    inp = wl.make_inputs(w, seed=32, T=700)
    _print(f"inference ELL capacity K={K}")
    args = _args(inp)
    ffn = layer(inp, ell_cap=K, dense_rows=1024)
    y = ffn.forward(*args).cpu().numpy()
    assert_close_bf16(y, _y_ref(inp), "y")
    y_full = layer(inp, ell_cap=0, dense_rows=1024).forward(*args).cpu().numpy()
    assert_close_bf16(y, y_full.astype(np.float64), "y against K = n_t * C")


def test_training_capacity_reported_and_recovered():
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=47, T=256)
    _print("training capacity: dense_rows=4")
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dense_rows=4, dtype=torch.bfloat16)
    args = _args(inp)
    _, hy = ffn.forward_train(*args, check=False)
    assert hy["max_backup"] == 4
    assert ffn.hybrid_check(hy) == B.SFFN_E_CAPACITY
    assert ffn.lib.sffn_check(ffn.h, B._stream()) == B.SFFN_E_CAPACITY
    nb = int(hy["n_backup"][0].item())
    assert nb > 4
    # checked: a T-row capacity and a T-row Hybrid, then the full step
    y, hy = ffn.forward_train(*args)
    assert ffn.dense_rows == 0 and hy["max_backup"] == 256
    assert ffn.hybrid_check(hy) == B.SFFN_OK
    assert_close_bf16(y.cpu().numpy(), _y_ref(inp), "y")
    dx, dwg, dwu, dwd = ffn.backward(*args, hy, dev(inp, "dy"))
    wg, wu, wd = math_weights(inp)
    ref = oracle.backward(inp.x.astype(np.float64), wg, wu, wd, inp.dy.astype(np.float64))
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")


def test_caller_hybrid_too_small_raises():
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=47, T=256)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    hy = ffn.new_hybrid(256, max_backup=2)
    with pytest.raises(B.SffnError) as ei:
        ffn.forward_train(*_args(inp), hy=hy)
    assert ei.value.status == B.SFFN_E_CAPACITY


def test_workspace_follows_the_sparse_work():
    """Workspace bytes at the benchmark shapes: the inference workspace
    (T = 8192, d = 2048, F = 5632, C = 8, K = 64, 512 dense rows) is about
    the size of the dense layer's bf16 hidden tensor (the dense layer's
    workspace is that tensor and its transposed W_d), and no region grows
    as T x F."""
    w = wl.GATED_1P5B
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dense_rows=w.dense_rows, dtype=torch.bfloat16)
    sp = ffn.workspace_bytes(w.T, B.SFFN_OP_FORWARD_SPARSE)
    de = ffn.workspace_bytes(w.T, B.SFFN_OP_FORWARD_DENSE)
    _print(f"inference workspace: sparse {sp / 1e6:.1f} MB, dense {de / 1e6:.1f} MB")
    assert de == w.T * w.F * 2 + w.F * w.d * 2
    assert sp <= 120e6
    # doubling T adds per-token regions only (no T x F region)
    sp2 = ffn.workspace_bytes(2 * w.T, B.SFFN_OP_FORWARD_SPARSE)
    assert sp2 - sp < 0.5 * w.T * w.F * 4
    t = wl.TRAIN_HYBRID
    tr = SparseFFN(t.d, t.F, gated=True, twell_cap=t.twell_cap, ell_cap=t.ell_cap,
                   dense_rows=t.dense_rows, dtype=torch.bfloat16)
    f = tr.workspace_bytes(t.T, B.SFFN_OP_FORWARD_TRAIN)
    b = tr.workspace_bytes(t.T, B.SFFN_OP_BACKWARD)
    _print(f"training workspace: forward {f / 1e6:.1f} MB, backward {b / 1e6:.1f} MB")
    assert f <= 150e6 and b <= 300e6

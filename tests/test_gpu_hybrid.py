"""Hybrid format and training forward on the GPU against the CPU oracle.

The compaction is checked bit for bit on a TwELL the GPU packs from a host
pre-activation tensor (the same tensor the oracle packs); the training
forward is checked against the oracle's dense layer, Hybrid routing and
saved activations.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close_bf16, assert_close_f32, dev, math_weights, rel_fro, to_np,
                      twell_np)
from unstructured_sparse_feedforward_amd import SparseFFN
from unstructured_sparse_feedforward_amd import binding as B
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def hybrid_np(hy):
    torch.cuda.synchronize()
    out = {k: (to_np(v) if isinstance(v, torch.Tensor) else v) for k, v in hy.items()}
    out["ell_idx"] = out["ell_idx"].view(np.uint16).astype(np.int64)
    out["n_backup"] = int(out["n_backup"][0])
    return out


def _z(T, F, seed, heavy_frac=0.05, shift=-2.6):
    r = np.random.default_rng(seed)
    z = (r.standard_normal((T, F)) + shift).astype(np.float32)
    heavy = r.random(T) < heavy_frac
    z[heavy] = r.standard_normal((heavy.sum(), F)).astype(np.float32)
    z[r.random((T, F)) < 0.002] = 0.0
    return z


@pytest.mark.parametrize("T,F,C,K,seed", [(300, 1024, 16, 8, 0), (129, 5632, 16, 64, 1),
                                          (64, 512, 4, 64, 2), (1000, 2048, 8, 12, 3)])
def test_hybrid_compact_bitexact(T, F, C, K, seed):
    _print(f"hybrid T={T} F={F} C={C} K={K}")
    z = _z(T, F, seed)
    ffn = SparseFFN(512, F, gated=True, twell_cap=C, ell_cap=K, dtype=torch.bfloat16)
    zd = torch.from_numpy(z).cuda()
    tw = ffn.pack_twell(zd)
    hy = hybrid_np(ffn.hybrid_compact(tw, T, z=zd))
    ref_tw = oracle.pack_twell(z.astype(np.float64), 128, C)
    a = np.where(z > 0, z, 0).astype(np.float64)
    ref = oracle.hybrid_compact(ref_tw, K, a_dense=a)
    assert hy["n_backup"] == ref["n_backup"]
    assert np.array_equal(hy["slot"][:T], ref["slot"])
    assert np.array_equal(hy["brow"][:ref["n_backup"]], ref["brow"])
    assert np.array_equal(hy["ell_cnt"], ref["ell_cnt"])
    m = np.arange(K)[None, :] < ref["ell_cnt"][:, None]
    assert np.array_equal(hy["ell_idx"][m], ref["ell_idx"][m])
    assert np.array_equal(hy["ell_a"][m].astype(np.float64), ref["ell_a"][m])
    assert np.array_equal(hy["bk_a"][:ref["n_backup"]].astype(np.float64), ref["bk_a"])
    assert ffn.hybrid_check(ffn.hybrid_compact(tw, T, z=zd)) == B.SFFN_OK


def test_hybrid_capacity_overflow_is_reported():
    T, F, C, K = 256, 1024, 16, 8
    z = _z(T, F, 4, heavy_frac=0.2)
    ffn = SparseFFN(512, F, gated=True, twell_cap=C, ell_cap=K, dtype=torch.bfloat16)
    zd = torch.from_numpy(z).cuda()
    tw = ffn.pack_twell(zd)
    ref = oracle.hybrid_compact(oracle.pack_twell(z.astype(np.float64), 128, C), K)
    cap = ref["n_backup"] // 2
    hyd = ffn.hybrid_compact(tw, T, z=zd, max_backup=cap)
    hy = hybrid_np(hyd)
    # the true count is reported, the first cap backup rows are listed
    assert hy["n_backup"] == ref["n_backup"] > cap
    assert np.array_equal(hy["brow"][:cap], ref["brow"][:cap])
    assert ffn.hybrid_check(hyd) == B.SFFN_E_CAPACITY


@pytest.mark.parametrize("w,T,seed", [(wl.TRAIN_HYBRID, 300, 5), (wl.TRAIN_HYBRID, 1024, 6),
                                      (wl.TRAIN_HYBRID.replace(gated=False, F=8192, nnz=40,
                                                               name="train_nongated"), 200, 7)])
def test_forward_train(w, T, seed):
    _print(f"forward_train {w.name} T={T}")
    inp = wl.make_inputs(w, seed=seed, T=T)
    ffn = SparseFFN(w.d, w.F, gated=w.gated, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    y, hyd = ffn.forward_train(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")))
    assert ffn.hybrid_check(hyd) == B.SFFN_OK
    hy = hybrid_np(hyd)
    wg, wu, wd = math_weights(inp)
    x64 = inp.x.astype(np.float64)
    yr, it = oracle.dense_ffn(x64, wg, wu, wd)
    assert_close_bf16(y.cpu().numpy(), yr, "y")
    # routing against the oracle's Hybrid of the oracle's own pre-activations;
    # a row may differ only if one of its pre-activations is within 1e-4 of 0
    ref = oracle.hybrid_compact(oracle.pack_twell(it["z"], 128, w.twell_cap), w.ell_cap)
    near = (np.abs(it["z"]) < 1e-4).any(axis=1)
    same = ~near
    assert np.array_equal((hy["slot"][:T] >= 0)[same], (ref["slot"] >= 0)[same])
    assert np.array_equal(hy["ell_cnt"][same], ref["ell_cnt"][same])
    _print("  backup rows:", hy["n_backup"], " ELL slots:", int(hy["ell_cnt"].sum()))
    # saved activations: a and u of every ELL slot, ReLU(z) and u rows of backup rows
    rows, ks = np.nonzero(np.arange(w.ell_cap)[None, :] < hy["ell_cnt"][:, None])
    js = hy["ell_idx"][rows, ks]
    assert rel_fro(hy["ell_a"][rows, ks], it["a"][rows, js]) < 1e-5
    assert np.all(it["z"][rows, js] > -1e-4)
    if w.gated:
        assert rel_fro(hy["ell_u"][rows, ks], it["u"][rows, js]) < 1e-5
    nb = hy["n_backup"]
    br = hy["brow"][:nb]
    assert np.array_equal(np.flatnonzero(hy["slot"][:T] >= 0), br)
    assert rel_fro(hy["bk_a"][:nb], it["a"][br]) < 1e-5
    if w.gated:
        assert rel_fro(hy["bk_u"][:nb], it["u"][br]) < 1e-5


def test_forward_train_equals_inference_y():
    """With K >= n_t * C the training forward routes exactly the rows the
    inference forward sends down its dense path, and both give the same y
    bit for bit (the same kernels in the same order)."""
    w = wl.GATED_1P5B
    inp = wl.make_inputs(w, seed=8, T=512)
    K = (w.F // 128) * w.twell_cap
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=K, dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y_inf = ffn.forward(*args, mode="sparse").clone()
    y_tr, hyd = ffn.forward_train(*args)
    torch.cuda.synchronize()
    assert torch.equal(y_inf.view(torch.int32), y_tr.view(torch.int32))


# --------------------------------------------------------------- backward

def _grads_ref(inp, l1):
    wg, wu, wd = math_weights(inp)
    return oracle.backward(inp.x.astype(np.float64), wg, wu, wd, inp.dy.astype(np.float64),
                           l1_coeff=l1)


# seeds whose pre-activations all keep |z| > 2e-5, so the ReLU mask of the
# GPU's fp32 pre-activations is the oracle's
@pytest.mark.parametrize("w,T,seed,l1", [
    (wl.TRAIN_HYBRID, 256, 47, 0.0),
    (wl.TRAIN_HYBRID, 512, 57, 0.0),
    # 264 rows: a last block of 8 slot units in the neuron-major grouping
    (wl.TRAIN_HYBRID, 264, 102, 0.0),
    (wl.TRAIN_HYBRID, 256, 47, 0.05),
    (wl.TRAIN_HYBRID.replace(gated=False, F=8192, nnz=40, name="train_nongated"), 256, 55, 0.0),
])
def test_backward(w, T, seed, l1):
    _print(f"backward {w.name} T={T} l1={l1}")
    inp = wl.make_inputs(w, seed=seed, T=T)
    wg, _, _ = math_weights(inp)
    assert np.abs(inp.x.astype(np.float64) @ wg).min() > 2e-5
    ffn = SparseFFN(w.d, w.F, gated=w.gated, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    _, hy = ffn.forward_train(*args)
    assert ffn.hybrid_check(hy) == B.SFFN_OK
    _print("  backup rows:", int(hy["n_backup"][0].item()))
    dx, dwg, dwu, dwd = ffn.backward(*args, hy, dev(inp, "dy"), l1_coeff=l1)
    ref = _grads_ref(inp, l1)
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    # dW is neuron-major [F, d]: the transpose of the math d x F matrices
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")
    if w.gated:
        assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    # neurons never active in the batch have exactly zero weight gradients
    dead = ~((inp.x.astype(np.float64) @ wg) > 0).any(axis=0)
    if dead.any():
        assert np.all(dwg.cpu().numpy()[dead] == 0) and np.all(dwd.cpu().numpy()[dead] == 0)


def test_backward_deterministic():
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=47, T=256)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    _, hy = ffn.forward_train(*args)
    dy = dev(inp, "dy")
    g1 = [t.clone() for t in ffn.backward(*args, hy, dy)]
    g2 = ffn.backward(*args, hy, dy)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_backward_same_with_kernel_timing_and_side_stream():
    """With backup rows the backward forks the ELL rows' dx sums and the
    neuron-major grouping to a second stream and joins it before the dW
    sums. With per-kernel timing on (events recorded on both streams) and
    on a non-default caller stream, every gradient is the same bit for bit
    as a plain run on the default stream."""
    w = wl.TRAIN_HYBRID
    inp = wl.make_inputs(w, seed=61, T=512)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    _, hy = ffn.forward_train(*args)
    assert int(hy["n_backup"][0].item()) > 0
    dy = dev(inp, "dy")
    g1 = [t.clone() for t in ffn.backward(*args, hy, dy)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ffn.profile(True)
        g2 = [t.clone() for t in ffn.backward(*args, hy, dy)]
        prof = ffn.profile_read()
        ffn.profile(False)
    torch.cuda.synchronize()
    assert prof["bwd_dx"][1] >= 1 and prof["bwd_transpose"][1] == 1
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_backward_all_rows_backup():
    """K = 1 sends every row with more than one positive to the dense
    backup: the gradients come from the dense GEMM path alone."""
    w = wl.TRAIN_HYBRID.replace(ell_cap=1)
    inp = wl.make_inputs(w, seed=47, T=256)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=1, dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    _, hy = ffn.forward_train(*args)
    nb = int(hy["n_backup"][0].item())
    assert nb > 200
    dx, dwg, dwu, dwd = ffn.backward(*args, hy, dev(inp, "dy"))
    ref = _grads_ref(inp, 0.0)
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")


def test_backward_wide_ell_rows():
    """With TwELL capacity C = 128 (no tile can overflow) and K = 3000 the
    outlier rows (about half of the 5632 neurons active) stay in the ELL:
    rows of up to 47 units of 64 slots, so that the neuron-major grouping
    orders slots across several units of a row and across blocks of units."""
    w = wl.TRAIN_HYBRID.replace(twell_cap=128, ell_cap=3000)
    _print("backward wide ELL rows K=3000")
    inp = wl.make_inputs(w, seed=53, T=256)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    _, hy = ffn.forward_train(*args)
    assert ffn.hybrid_check(hy) == B.SFFN_OK
    assert int(hy["ell_cnt"].max().item()) > 64
    dx, dwg, dwu, dwd = ffn.backward(*args, hy, dev(inp, "dy"))
    ref = _grads_ref(inp, 0.0)
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")


@pytest.mark.parametrize("max_backup", [None, 0])
def test_backward_no_backup_rows(max_backup):
    """No outlier tokens and K = 64 keep every row on the ELL path. With
    backup buffers (None: T rows) their dW products are zero and the ELL
    sums add to them; without (0 rows) the ELL sums are stored alone."""
    w = wl.TRAIN_HYBRID.replace(outlier_frac=0.0)
    _print(f"backward no backup rows max_backup={max_backup}")
    inp = wl.make_inputs(w, seed=47, T=256)
    wg, _, _ = math_weights(inp)
    assert np.abs(inp.x.astype(np.float64) @ wg).min() > 2e-5
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    _, hy = ffn.forward_train(*args, max_backup=max_backup)
    assert ffn.hybrid_check(hy) == B.SFFN_OK
    assert int(hy["n_backup"][0].item()) == 0
    # stale values in the outputs must not leak into the result
    outs = tuple(torch.full((n, w.d), 7.0, device="cuda") for n in (256, w.F, w.F, w.F))
    dx, dwg, dwu, dwd = ffn.backward(*args, hy, dev(inp, "dy"), out=outs)
    ref = _grads_ref(inp, 0.0)
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")


def test_training_f32():
    """The fp32 training step (true fp32 GEMMs, no split operands) against
    the oracle at the fp32 bound, on a layer where about half the rows take
    the dense backup path (K = 20 of about 20 active, 5% outliers)."""
    w = wl.SMALL_F32.replace(ell_cap=20, outlier_frac=0.05, train=True)
    _print("training f32")
    inp = wl.make_inputs(w, seed=6)
    wg, wu, wd = math_weights(inp)
    x64 = inp.x.astype(np.float64)
    assert np.abs(x64 @ wg).min() > 1e-4
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.float32)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y, hy = ffn.forward_train(*args)
    assert ffn.hybrid_check(hy) == B.SFFN_OK
    nb = int(hy["n_backup"][0].item())
    _print("  backup rows:", nb)
    assert 20 < nb < w.T - 20
    dx, dwg, dwu, dwd = ffn.backward(*args, hy, dev(inp, "dy"), l1_coeff=0.01)
    yr, _ = oracle.dense_ffn(x64, wg, wu, wd)
    ref = _grads_ref(inp, 0.01)
    assert_close_f32(y.cpu().numpy(), yr, "y")
    assert_close_f32(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_f32(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_f32(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    assert_close_f32(dwd.cpu().numpy(), ref["dw_down"], "dw_down")


def test_training_full_size_sampled():
    """The training step at its full size (T = 8192, d = 2048, F = 5632,
    K = 64, 5% outlier tokens) in the launch configuration the benchmark
    times. dx rows depend only on their own token, so the oracle's
    backward on the sampled rows gives them exactly; dW columns of a
    neuron set J depend only on J's weights, so the oracle's backward of
    the layer restricted to J gives them exactly. Rows and neurons with a
    pre-activation within 2e-5 of 0 are left out of the sample."""
    w = wl.TRAIN_HYBRID
    _print(f"training full size {w.name}")
    inp = wl.make_inputs(w, seed=11)
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y, hyd = ffn.forward_train(*args)
    assert ffn.hybrid_check(hyd) == B.SFFN_OK
    dx, dwg, dwu, dwd = ffn.backward(*args, hyd, dev(inp, "dy"))
    torch.cuda.synchronize()
    slot = hyd["slot"].cpu().numpy()[:w.T]
    nb = int(hyd["n_backup"][0].item())
    _print("  backup rows:", nb)
    assert 0 < nb < w.T // 4
    wg, wu, wd = math_weights(inp)
    x64, dy64 = inp.x.astype(np.float64), inp.dy.astype(np.float64)
    rng = np.random.default_rng(0)
    # rows: ELL rows and backup rows, with all their |z| > 2e-5
    ell_rows = rng.choice(np.flatnonzero(slot < 0), 96, replace=False)
    bk_rows = rng.choice(np.flatnonzero(slot >= 0), min(nb, 32), replace=False)
    rows = np.sort(np.concatenate([ell_rows, bk_rows]))
    rows = rows[np.abs(x64[rows] @ wg).min(axis=1) > 2e-5]
    assert rows.size > 100
    ref = oracle.backward(x64[rows], wg, wu, wd, dy64[rows])
    yr, _ = oracle.dense_ffn(x64[rows], wg, wu, wd)
    assert_close_bf16(y.cpu().numpy()[rows], yr, "y rows")
    assert_close_bf16(dx.cpu().numpy()[rows], ref["dx"], "dx rows")
    # neurons: a random set whose pre-activations over all T tokens keep |z| > 2e-5
    J = np.sort(rng.choice(w.F, 96, replace=False))
    J = J[np.abs(x64 @ wg[:, J]).min(axis=0) > 2e-5]
    assert J.size > 64
    refJ = oracle.backward(x64, wg[:, J], wu[:, J], wd[J], dy64)
    assert_close_bf16(dwg.cpu().numpy()[J], refJ["dw_gate"].T, "dw_gate neurons")
    assert_close_bf16(dwu.cpu().numpy()[J], refJ["dw_up"].T, "dw_up neurons")
    assert_close_bf16(dwd.cpu().numpy()[J], refJ["dw_down"], "dw_down neurons")


def _plant_near_zero(inp, pairs):
    """Make z[t, j] = x_t . W_g[:, j] vanish up to about 1e-10 for the
    given (t, j) pairs (distinct j): the column's entries at the four
    largest |x_t[k]| are cleared, then set one by one to the bf16 value
    nearest to -(x_t . w without entry k) / x_t[k]; each step leaves at
    most 2^-9 of the residual, so four steps bring it from O(1) to about
    1e-10. The GPU's float32 sum of the same products errs by about 1e-7,
    so the sign of such an entry, and with it the ReLU mask, is a coin
    toss."""
    x = inp.x.astype(np.float64)
    for t, j in pairs:
        w = inp.w_gate[j].astype(np.float64)
        ks = np.argsort(-np.abs(x[t]))[:4]
        w[ks] = 0.0
        for k in ks:
            rest = x[t] @ w - x[t, k] * w[k]
            w[k] = float(wl.round_bf16(np.array([-rest / x[t, k]], dtype=np.float32))[0])
        inp.w_gate[j] = w.astype(np.float32)


def test_backward_mask_disagreement():
    """Pre-activations planted within 1e-10 of zero make the GPU's ReLU mask
    (decided on its float32 z) differ from the oracle's (float64) on some
    entries. The masks may differ only where |z| < 1e-3, and the gradients
    match the oracle's backward evaluated on the GPU's own mask (as saved
    in the Hybrid: ELL slots and positive entries of the backup rows)."""
    w = wl.TRAIN_HYBRID
    T = 256
    inp = wl.make_inputs(w, seed=71, T=T)
    r = np.random.default_rng(5)
    pairs = list(zip(r.choice(T, 96), r.choice(w.F, 96, replace=False)))
    _plant_near_zero(inp, pairs)
    wg, wu, wd = math_weights(inp)
    x64 = inp.x.astype(np.float64)
    z = x64 @ wg
    assert max(abs(z[t, j]) for t, j in pairs) < 1e-8
    ffn = SparseFFN(w.d, w.F, gated=True, twell_cap=w.twell_cap, ell_cap=w.ell_cap,
                    dtype=torch.bfloat16)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y, hyd = ffn.forward_train(*args)
    dx, dwg, dwu, dwd = ffn.backward(*args, hyd, dev(inp, "dy"))
    hy = hybrid_np(hyd)
    mask = np.zeros((T, w.F), dtype=bool)
    for t in range(T):
        if hy["slot"][t] >= 0:
            mask[t] = hy["bk_a"][hy["slot"][t]] > 0
        else:
            mask[t, hy["ell_idx"][t, :hy["ell_cnt"][t]]] = True
    diff = mask != (z > 0)
    _print(f"  mask disagreements: {int(diff.sum())} (of {len(pairs)} planted)")
    assert np.all(np.abs(z[diff]) < 1e-3)
    assert diff.sum() >= 4
    ref = oracle.backward(x64, wg, wu, wd, inp.dy.astype(np.float64), mask=mask)
    assert_close_bf16(y.cpu().numpy(), oracle.dense_ffn(x64, wg, wu, wd)[0], "y")
    assert_close_bf16(dx.cpu().numpy(), ref["dx"], "dx")
    assert_close_bf16(dwg.cpu().numpy(), ref["dw_gate"].T, "dw_gate")
    assert_close_bf16(dwu.cpu().numpy(), ref["dw_up"].T, "dw_up")
    assert_close_bf16(dwd.cpu().numpy(), ref["dw_down"], "dw_down")

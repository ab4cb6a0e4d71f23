"""HIP path against the CPU oracle, through the C ABI.

Inputs come from the seeded generator and are fed identically to both
sides. Bars: TwELL indices, counts, flags and the flagged list bit-exact
when the pack kernel gets the same pre-activations as the oracle packer;
in the fused gate path, active-set mismatches only where the oracle's
|pre-activation| < 1e-3; outputs within relative Frobenius 1e-3 and
max-abs 1e-2 * max|y| for bf16 inputs (fp32 accumulation) and relative
1e-5 for fp32 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close_bf16, assert_close_f32, assert_twell_equal, dev, layer,
                      math_weights, rel_fro, twell_np)
from unstructured_sparse_feedforward_amd import SparseFFN
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


# --------------------------------------------------------------- stand-alone pack

@pytest.mark.parametrize("T,F,C,seed", [(1, 128, 8, 0), (33, 256, 1, 1), (100, 1024, 16, 2),
                                        (257, 5632, 8, 3), (64, 1024, 128, 4),
                                        (1000, 8192, 48, 5)])
def test_pack_bitexact(T, F, C, seed):
    _print(f"pack T={T} F={F} C={C}")
    r = np.random.default_rng(seed)
    # pre-activations with a few percent positive, a sprinkling of exact
    # zeros and negative zeros, and some heavy rows that overflow C
    z = (r.standard_normal((T, F)) - 2.0).astype(np.float32)
    z[r.random((T, F)) < 0.01] = 0.0
    z[r.random((T, F)) < 0.01] = -0.0
    heavy = r.random(T) < 0.05
    z[heavy] = np.abs(z[heavy]) * np.where(r.random((heavy.sum(), F)) < 0.5, 1, -1)
    ffn = SparseFFN(512, F, gated=True, twell_cap=C, dtype=torch.bfloat16)
    tw = twell_np(ffn.pack_twell(torch.from_numpy(z).cuda()))
    ref = oracle.pack_twell(z.astype(np.float64), 128, C)
    # counts, flags and every defined slot bit-exact (slots past the count
    # are unspecified)
    assert_twell_equal(tw, ref)
    flagged = np.flatnonzero(ref["row_flag"])
    assert tw["n_flagged"] == len(flagged)
    assert np.array_equal(tw["flagged"][:len(flagged)], flagged)


# --------------------------------------------------------------- gate GEMM

@pytest.mark.parametrize("w,T", [(wl.SMALL_F32, 128), (wl.SMALL_F32, 77),
                                 (wl.GATED_1P5B, 300), (wl.NONGATED[29], 129)])
def test_gate_preact(w, T):
    _print(f"gate {w.name} T={T}")
    inp = wl.make_inputs(w, seed=11, T=T)
    ffn = layer(inp)
    z = ffn.gate_preact(dev(inp, "x"), dev(inp, "w_gate")).cpu().numpy()
    wg, _, _ = math_weights(inp)
    ref = inp.x.astype(np.float64) @ wg
    # fp32 and bf16 operands: exact products, fp32 accumulation over d
    assert rel_fro(z, ref) <= (1e-6 if w.dtype == "f32" else 1e-5)
    # element-wise: d fp32 additions of partial sums of size O(1) each
    # round by at most 2^-24 of the partial sum, far below 1e-4
    assert np.abs(z - ref).max() <= 1e-4


# --------------------------------------------------------------- fused TwELL

G2048 = wl.GATED_1P5B.replace(F=2048, nnz=12, name="g2048")


@pytest.mark.parametrize("w,T", [(wl.SMALL_F32, 128), (wl.GATED_1P5B, 1024),
                                 (wl.NONGATED[108], 333),
                                 # the full gated shape, and a narrower layer with fewer,
                                 # more and ragged 256-row tiles than CUs
                                 (wl.GATED_1P5B, 8192), (G2048, 6144), (G2048, 6100),
                                 (G2048, 14336),
                                 # capacities with many stored entries per lane (the
                                 # epilogue stores them four at a time), and C = 1
                                 (wl.NONGATED[911], 512),
                                 (wl.GATED_1P5B.replace(twell_cap=128, name="c128"), 700),
                                 (wl.GATED_1P5B.replace(twell_cap=1, nnz=400, name="c1"), 260)])
def test_fused_twell_matches_pack_of_own_z(w, T):
    """The gate GEMM's TwELL epilogue equals the stand-alone pack of the
    same kernel's pre-activations, bit for bit (GPU against GPU)."""
    _print(f"fused-vs-pack {w.name} T={T}")
    inp = wl.make_inputs(w, seed=12, T=T)
    ffn = layer(inp)
    x, wg, wu, wd = (dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down"))
    tw_f = ffn.new_twell(T)
    ffn.forward(x, wg, wu, wd, mode="sparse", tw=tw_f)
    z = ffn.gate_preact(x, wg)
    tw_p = ffn.pack_twell(z)
    a, b = twell_np(tw_f), twell_np(tw_p)
    assert_twell_equal(a, b)
    assert a["n_flagged"] == b["n_flagged"]
    assert np.array_equal(a["flagged"][:a["n_flagged"]], b["flagged"][:b["n_flagged"]])


@pytest.mark.parametrize("w,T", [(wl.SMALL_F32, 128), (wl.GATED_1P5B, 1024)])
def test_fused_twell_vs_oracle(w, T):
    _print(f"fused-vs-oracle {w.name} T={T}")
    inp = wl.make_inputs(w, seed=13, T=T)
    ffn = layer(inp)
    x, wg, wu, wd = (dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down"))
    tw = ffn.new_twell(T)
    ffn.forward(x, wg, wu, wd, mode="sparse", tw=tw)
    g = twell_np(tw)
    mg, _, _ = math_weights(inp)
    z = inp.x.astype(np.float64) @ mg
    ref = oracle.pack_twell(z, 128, w.twell_cap)
    # active sets: GPU unpacked vs oracle, on rows neither side flagged
    ok = ~(ref["row_flag"] | g["row_flag"].astype(bool))
    act_g = oracle.unpack_twell(g, w.F)[ok] > 0
    act_o = z[ok] > 0
    diff = act_g != act_o
    assert np.all(np.abs(z[ok][diff]) < 1e-3), "active-set mismatch away from zero"
    # counts may differ only by the near-zero mismatches
    cdiff = np.abs(g["cnt"] - ref["cnt"]).sum()
    near = (np.abs(z) < 1e-3).sum()
    assert cdiff <= near
    # stored values are the pre-activations
    both = act_g & act_o
    vg = oracle.unpack_twell(g, w.F)[ok][both]
    assert np.abs(vg - z[ok][both]).max() <= 1e-4


# --------------------------------------------------------------- forward

def _oracle_y(inp):
    wg, wu, wd = math_weights(inp)
    y, _ = oracle.dense_ffn(inp.x.astype(np.float64), wg, wu, wd)
    return y


@pytest.mark.parametrize("w,T", [(wl.SMALL_F32, 128), (wl.SMALL_F32, 1),
                                 (wl.SMALL_F32, 97)])
def test_forward_sparse_f32(w, T):
    _print(f"forward f32 {w.name} T={T}")
    inp = wl.make_inputs(w, seed=14, T=T)
    ffn = layer(inp)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")), mode="sparse")
    assert_close_f32(y.cpu().numpy(), _oracle_y(inp), "y")


def test_forward_sparse_f32_with_flagged_rows():
    w = wl.SMALL_F32.replace(outlier_frac=0.1)
    inp = wl.make_inputs(w, seed=15)
    ffn = layer(inp)
    tw = ffn.new_twell(w.T)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")), mode="sparse",
                    tw=tw)
    g = twell_np(tw)
    assert g["n_flagged"] > 0
    assert_close_f32(y.cpu().numpy(), _oracle_y(inp), "y")


@pytest.mark.parametrize("w,T", [(wl.GATED_1P5B, 1024), (wl.GATED_1P5B, 131),
                                 (wl.NONGATED[29], 512), (wl.NONGATED[108], 256),
                                 (wl.NONGATED[911], 200), (wl.stack_layer(5), 400),
                                 (wl.TRAIN_HYBRID, 300)])
def test_forward_sparse_bf16(w, T):
    _print(f"forward bf16 {w.name} T={T}")
    inp = wl.make_inputs(w, seed=16, T=T)
    ffn = layer(inp)
    tw = ffn.new_twell(T)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")), mode="sparse",
                    tw=tw)
    _print("  flagged rows:", twell_np(tw)["n_flagged"])
    assert_close_bf16(y.cpu().numpy(), _oracle_y(inp), "y")


@pytest.mark.parametrize("w,T", [(wl.SMALL_F32, 128), (wl.GATED_1P5B, 512),
                                 (wl.NONGATED[29], 300)])
def test_forward_dense(w, T):
    _print(f"forward dense {w.name} T={T}")
    inp = wl.make_inputs(w, seed=17, T=T)
    ffn = layer(inp)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")),
                    mode="dense").cpu().numpy()
    wg, wu, wd = math_weights(inp)
    x64 = inp.x.astype(np.float64)
    if w.dtype == "bf16":
        # a standard bf16 layer rounds the hidden activations once to bf16
        assert_close_bf16(y, oracle.dense_ffn_bf16_hidden(x64, wg, wu, wd), "y dense")
    else:
        assert_close_f32(y, _oracle_y(inp), "y dense")


def test_forward_exact_integers():
    """Sparse ternary inputs keep every sum an exact small integer, so the
    GPU output equals the oracle's bit for bit, on the sparse path and on
    the dense path of flagged rows (whose hidden values fit a bf16 hi+lo
    split exactly)."""
    T, d, F = 160, 512, 256
    r = np.random.default_rng(21)
    x = r.choice([-1.0, 0.0, 1.0], size=(T, d), p=[0.1, 0.8, 0.1]).astype(np.float32)
    x[:, 0] = 1.0
    x[::7, 0] = 0.0                      # heavy rows: overflow C
    wg = r.choice([-1.0, 0.0, 1.0], size=(F, d)).astype(np.float32)
    wg[:, 0] = -16.0
    wu = r.choice([-1.0, 0.0, 1.0], size=(F, d)).astype(np.float32)
    wd = r.choice([-1.0, 0.0, 1.0], size=(F, d)).astype(np.float32)
    y_ref, it = oracle.dense_ffn(x.astype(np.float64), wg.T.astype(np.float64),
                                 wu.T.astype(np.float64), wd.astype(np.float64))
    assert np.abs(it["h"]).max() < 2 ** 16 and np.abs(y_ref).max() < 2 ** 24
    ffn = SparseFFN(d, F, gated=True, twell_cap=16, dtype=torch.bfloat16)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    tw = ffn.new_twell(T)
    y = ffn.forward(bf(x), bf(wg), bf(wu), bf(wd), mode="sparse", tw=tw).cpu().numpy()
    g = twell_np(tw)
    assert g["n_flagged"] > 0 and g["n_flagged"] < T
    assert np.array_equal(y.astype(np.float64), y_ref)
    # the dense mode rounds H once to bf16 (a standard bf16 layer); with
    # integer H both sides round the same exact values
    yd = ffn.forward(bf(x), bf(wg), bf(wu), bf(wd), mode="dense").cpu().numpy()
    yd_ref = oracle.dense_ffn_bf16_hidden(x.astype(np.float64), wg.T.astype(np.float64),
                                          wu.T.astype(np.float64), wd.astype(np.float64))
    assert np.array_equal(yd.astype(np.float64), yd_ref)


def test_forward_deterministic():
    inp = wl.make_inputs(wl.GATED_1P5B, seed=18, T=700)
    ffn = layer(inp)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    tw1, tw2 = ffn.new_twell(700), ffn.new_twell(700)
    y1 = ffn.forward(*args, mode="sparse", tw=tw1).clone()
    y2 = ffn.forward(*args, mode="sparse", tw=tw2).clone()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    a, b = twell_np(tw1), twell_np(tw2)
    assert_twell_equal(a, b)


def test_forward_same_with_kernel_timing():
    """Per-kernel timing brackets every launch with events on the caller's
    stream; y is the same bit for bit as without it."""
    inp = wl.make_inputs(wl.GATED_1P5B, seed=23, T=1500)
    ffn = layer(inp)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    tw = ffn.new_twell(1500)
    y1 = ffn.forward(*args, mode="sparse", tw=tw).clone()
    assert twell_np(tw)["n_flagged"] > 0
    ffn.profile(True)
    y2 = ffn.forward(*args, mode="sparse").clone()
    prof = ffn.profile_read()
    ffn.profile(False)
    assert prof["flagged_gateup"][1] == 1 and prof["sparse_down"][1] == 1
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_empty_batch_is_noop():
    inp = wl.make_inputs(wl.SMALL_F32, seed=19, T=4)
    ffn = layer(inp)
    x = dev(inp, "x")[:0]
    y = torch.full((0, 256), 7.0, device="cuda")
    ffn.forward(x, dev(inp, "w_gate"), dev(inp, "w_up"), dev(inp, "w_down"), y=y)
    ffn.check()


def test_all_rows_flagged():
    """C = 1 with many positives per tile sends every row down the dense path."""
    w = wl.GATED_1P5B.replace(nnz=400, twell_cap=1)
    inp = wl.make_inputs(w, seed=20, T=260)
    ffn = layer(inp)
    tw = ffn.new_twell(260)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")), tw=tw)
    assert twell_np(tw)["n_flagged"] == 260
    assert_close_bf16(y.cpu().numpy(), _oracle_y(inp), "y")


def test_no_active_neurons():
    w = wl.GATED_1P5B.replace(nnz=1e-9, outlier_frac=0.0)
    inp = wl.make_inputs(w, seed=22, T=128)
    ffn = layer(inp)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")))
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("d,F,T", [(512, 1024, 200), (1024, 2048, 150), (4096, 1024, 70)])
def test_forward_bf16_model_dims(d, F, T):
    """Every supported bf16 model width (the d slices: 2 x 256, 4 x 256,
    8 x 512 for up; 256-column slices for down), with outlier rows."""
    w = wl.GATED_1P5B.replace(d=d, F=F, nnz=F * 0.01, outlier_frac=0.05,
                              name=f"gated_d{d}_F{F}")
    _print(f"forward bf16 d={d} F={F} T={T}")
    inp = wl.make_inputs(w, seed=24, T=T)
    ffn = layer(inp)
    tw = ffn.new_twell(T)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")), tw=tw)
    assert twell_np(tw)["n_flagged"] > 0
    assert_close_bf16(y.cpu().numpy(), _oracle_y(inp), "y")


# --------------------------------------------------------------- full size

def test_full_size_sampled_rows():
    """The gated workload at its full size (T = 8192, d = 2048, F = 5632,
    bf16, ~29 active per token, 1% outliers) in the launch configuration
    the benchmark times; 384 sampled rows (all flagged rows among them) are
    checked against the oracle row by row."""
    w = wl.GATED_1P5B
    inp = wl.make_inputs(w, seed=0)
    ffn = layer(inp)
    tw = ffn.new_twell(w.T)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")), tw=tw)
    y = y.cpu().numpy()
    g = twell_np(tw)
    flagged = g["flagged"][:g["n_flagged"]]
    r = np.random.default_rng(0)
    rows = np.unique(np.concatenate([flagged, r.choice(w.T, 384 - len(flagged), replace=False)]))
    wg, wu, wd = math_weights(inp)
    y_ref, _ = oracle.dense_ffn(inp.x[rows].astype(np.float64), wg, wu, wd)
    assert_close_bf16(y[rows], y_ref, "sampled rows")
    # every outlier token is flagged; a normal token overflows C = 8 only
    # with probability ~3e-8 per tile
    assert set(np.flatnonzero(inp.outlier)) <= set(flagged.tolist())
    assert len(flagged) - inp.outlier.sum() <= 2


def test_full_size_nongated_sampled_rows():
    """The non-gated workload at its full size (T = 16384, d = 2048,
    F = 8192, bf16, ~29 active per token, no outliers) in the launch
    configuration the benchmark times; 256 sampled rows against the oracle."""
    w = wl.NONGATED[29]
    inp = wl.make_inputs(w, seed=0)
    ffn = layer(inp)
    y = ffn.forward(*(dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down"))).cpu().numpy()
    rows = np.sort(np.random.default_rng(1).choice(w.T, 256, replace=False))
    wg, _, wd = math_weights(inp)
    y_ref, _ = oracle.dense_ffn(inp.x[rows].astype(np.float64), wg, None, wd)
    assert_close_bf16(y[rows], y_ref, "sampled rows")


# --------------------------------------------------------------- one-kernel up/down

@pytest.mark.parametrize("w,T", [(wl.GATED_1P5B, 1024), (wl.NONGATED[108], 512),
                                 (wl.GATED_1P5B.replace(d=512, F=1024, nnz=10, name="g512"), 300)])
def test_fused_updown_variant(w, T):
    """desc.updown = 1 (the up/down projection as one kernel without d
    slices) against the oracle and against the sliced path."""
    _print(f"fused up/down {w.name} T={T}")
    inp = wl.make_inputs(w, seed=25, T=T)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    y = layer(inp, fused_updown=True).forward(*args).cpu().numpy()
    assert_close_bf16(y, _oracle_y(inp), "y")
    y_sl = layer(inp).forward(*args).cpu().numpy()
    assert_close_bf16(y, y_sl.astype(np.float64), "y against the sliced path")

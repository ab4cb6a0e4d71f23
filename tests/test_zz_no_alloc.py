"""sffn_forward_noalloc (the static-scratch forward) against sffn_forward.

Both entry points run the same kernels; the one without a workspace
argument uses the library's static device scratch. Two calls in a row,
the second with a smaller batch (so the scratch holds the first call's
contents), in sparse and dense mode, must give the same y and TwELL as
sffn_forward bit for bit, and therefore the same parity with the oracle.
A batch whose workspace exceeds the scratch is refused before anything
is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close_bf16, assert_twell_equal, dev, layer, math_weights, twell_np
from unstructured_sparse_feedforward_amd import binding as B
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20


def _print(*a):
    print(*a, flush=True)


def _call(ffn, args, T, y, tw, mode):
    s = ctypes.byref(ffn._tw_struct(tw)) if tw is not None else None
    return ffn.lib.sffn_forward_noalloc(ffn.h, *(a.data_ptr() for a in args), T, y.data_ptr(),
                                        s, mode, B._stream())


@pytest.mark.parametrize("mode", [B.SFFN_SPARSE, B.SFFN_DENSE])
def test_noalloc_matches_forward_two_calls(mode):
    w = wl.GATED_1P5B
    inp = wl.make_inputs(w, seed=81)
    ffn = layer(inp)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    for T in (w.T, 1000):
        _print(f"noalloc mode={mode} T={T}")
        a = [args[0][:T]] + args[1:]
        tw_ref = ffn.new_twell(T) if mode == B.SFFN_SPARSE else None
        y_ref = ffn.forward(*a, mode="sparse" if mode == B.SFFN_SPARSE else "dense",
                            tw=tw_ref)
        tw = ffn.new_twell(T) if mode == B.SFFN_SPARSE else None
        y = torch.full((T, w.d), 7.0, device="cuda")
        assert _call(ffn, a, T, y, tw, mode) == B.SFFN_OK
        ffn.check()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
        if tw is not None:
            g, r = twell_np(tw), twell_np(tw_ref)
            assert_twell_equal(g, r)
            assert g["n_flagged"] == r["n_flagged"] > 0
        # and the oracle on sampled rows
        rows = np.sort(np.random.default_rng(T).choice(T, 64, replace=False))
        wg, wu, wd = math_weights(inp)
        x64 = inp.x[rows].astype(np.float64)
        ref = (oracle.dense_ffn(x64, wg, wu, wd)[0] if mode == B.SFFN_SPARSE
               else oracle.dense_ffn_bf16_hidden(x64, wg, wu, wd))
        assert_close_bf16(y.cpu().numpy()[rows], ref, "sampled rows")


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    w = wl.GATED_1P5B
    inp = wl.make_inputs(w, seed=82, T=64)
    ffn = layer(inp)
    lo, hi = 1, 1 << 20
    while lo < hi:        # the largest T whose workspace fits the scratch
        mid = (lo + hi + 1) // 2
        if ffn.workspace_bytes(mid, B.SFFN_OP_FORWARD_SPARSE) <= SCRATCH:
            lo = mid
        else:
            hi = mid - 1
    _print(f"largest sparse batch on the static scratch: T = {lo}")
    assert 8192 <= lo
    T = lo + 1
    x = torch.zeros((T, w.d), dtype=torch.bfloat16, device="cuda")
    args = [x] + [dev(inp, k) for k in ("w_gate", "w_up", "w_down")]
    y = torch.full((T, w.d), 7.0, device="cuda")
    assert _call(ffn, args, T, y, None, B.SFFN_SPARSE) == B.SFFN_E_ARG
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())

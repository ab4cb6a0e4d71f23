"""C ABI argument checks that need a handle (and so a GPU): misaligned
pointers and workspaces are rejected on the host with SFFN_E_ARG before
anything is enqueued (outputs keep their contents), and the backward of an
empty batch stores zero weight gradients."""
import ctypes

import pytest
import torch

from unstructured_sparse_feedforward_amd import SparseFFN
from unstructured_sparse_feedforward_amd import binding as B

pytestmark = pytest.mark.gpu

T, D, F = 64, 512, 1024


@pytest.fixture(scope="module")
def env():
    ffn = SparseFFN(D, F, gated=True, twell_cap=8, ell_cap=16, dtype=torch.bfloat16)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    # one spare element in front so that p + 2 (or + 4) stays inside
    x = torch.zeros(T * D + 8, **bf)
    w = [torch.zeros(F * D + 8, **bf) for _ in range(3)]
    dy = torch.zeros(T * D + 8, **bf)
    y = torch.full((T * D + 8,), 7.0, **f32)
    dx = torch.full((T * D + 8,), 7.0, **f32)
    dws = [torch.full((F * D + 8,), 7.0, **f32) for _ in range(3)]
    z = torch.zeros(T * F + 8, **f32)
    tw = ffn.new_twell(T)
    hy = ffn.new_hybrid(T)
    ws = torch.empty(ffn.workspace_bytes(T, B.SFFN_OP_BACKWARD) + 1024, dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    return dict(ffn=ffn, x=x, w=w, dy=dy, y=y, dx=dx, dws=dws, z=z, tw=tw, hy=hy, ws=ws)


def _ws(e, off=0):
    p = (e["ws"].data_ptr() + 255) // 256 * 256 + off
    return p, e["ws"].numel() - 512


def _fwd(e, x_off=0, w_off=(0, 0, 0), y_off=0, ws_off=0, tw=None):
    ffn = e["ffn"]
    p, n = _ws(e, ws_off)
    ts = ctypes.byref(tw) if tw is not None else None
    return ffn.lib.sffn_forward(ffn.h, e["x"].data_ptr() + x_off,
                                *(t.data_ptr() + o for t, o in zip(e["w"], w_off)), T,
                                e["y"].data_ptr() + y_off, ts, B.SFFN_SPARSE, p, n, B._stream())


@pytest.mark.parametrize("case", ["x", "w_gate", "w_up", "w_down", "y", "ws", "tw"])
def test_forward_rejects_misaligned(env, case):
    kws = dict(x=dict(x_off=2), w_gate=dict(w_off=(2, 0, 0)), w_up=dict(w_off=(0, 2, 0)),
               w_down=dict(w_off=(0, 0, 2)), y=dict(y_off=4), ws=dict(ws_off=16))
    if case == "tw":
        s = SparseFFN._tw_struct(env["tw"])
        s.val = s.val + 4
        kw = dict(tw=s)
    else:
        kw = kws[case]
    assert _fwd(env, **kw) == B.SFFN_E_ARG
    torch.cuda.synchronize()
    assert bool((env["y"] == 7.0).all())
    # the same call with aligned pointers is accepted
    assert _fwd(env) == B.SFFN_OK
    torch.cuda.synchronize()
    env["y"].fill_(7.0)


def test_pack_and_gate_reject_misaligned(env):
    ffn = env["ffn"]
    p, n = _ws(env)
    s = SparseFFN._tw_struct(env["tw"])
    z = env["z"].data_ptr()
    assert ffn.lib.sffn_pack_twell(ffn.h, z + 4, T, ctypes.byref(s), p, n,
                                   B._stream()) == B.SFFN_E_ARG
    s.idx = s.idx + 2
    assert ffn.lib.sffn_pack_twell(ffn.h, z, T, ctypes.byref(s), p, n,
                                   B._stream()) == B.SFFN_E_ARG
    assert ffn.lib.sffn_gate_preact(ffn.h, env["x"].data_ptr(), env["w"][0].data_ptr(), T,
                                    z + 4, B._stream()) == B.SFFN_E_ARG


@pytest.mark.parametrize("field", ["ell_a", "ell_idx", "slot", "bk_a", "n_backup"])
def test_hybrid_calls_reject_misaligned(env, field):
    ffn = env["ffn"]
    p, n = _ws(env)
    ts = SparseFFN._tw_struct(env["tw"])
    hs = SparseFFN._hy_struct(env["hy"])
    setattr(hs, field, getattr(hs, field) + 4)
    assert ffn.lib.sffn_hybrid_compact(ffn.h, ctypes.byref(ts), None, T, ctypes.byref(hs), p, n,
                                       B._stream()) == B.SFFN_E_ARG
    x, (wg, wu, wd) = env["x"].data_ptr(), (t.data_ptr() for t in env["w"])
    assert ffn.lib.sffn_forward_train(ffn.h, x, wg, wu, wd, T, env["y"].data_ptr(), None,
                                      ctypes.byref(hs), p, n, B._stream()) == B.SFFN_E_ARG


@pytest.mark.parametrize("case", ["dx", "dw_gate", "dw_up", "dw_down", "dy", "x"])
def test_backward_rejects_misaligned(env, case):
    ffn = env["ffn"]
    p, n = _ws(env)
    hs = SparseFFN._hy_struct(env["hy"])
    off = {k: 0 for k in ("dx", "dw_gate", "dw_up", "dw_down", "dy", "x")}
    off[case] = 4 if case.startswith("d") and case != "dy" else 2
    wg, wu, wd = (t.data_ptr() for t in env["w"])
    g0, g1, g2 = (t.data_ptr() for t in env["dws"])
    st = ffn.lib.sffn_backward(ffn.h, env["x"].data_ptr() + off["x"], wg, wu, wd,
                               ctypes.byref(hs), env["dy"].data_ptr() + off["dy"], T,
                               env["dx"].data_ptr() + off["dx"], g0 + off["dw_gate"],
                               g1 + off["dw_up"], g2 + off["dw_down"], 0.0, p, n, B._stream())
    assert st == B.SFFN_E_ARG
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in env["dws"])


def test_backward_empty_batch_zeroes_weight_gradients(env):
    ffn = env["ffn"]
    hs = SparseFFN._hy_struct(env["hy"])
    wg, wu, wd = (t.data_ptr() for t in env["w"])
    g = [torch.full((F, D), 7.0, device="cuda") for _ in range(3)]
    st = ffn.lib.sffn_backward(ffn.h, env["x"].data_ptr(), wg, wu, wd, ctypes.byref(hs),
                               env["dy"].data_ptr(), 0, env["dx"].data_ptr(),
                               *(t.data_ptr() for t in g), 0.0, None, 0, B._stream())
    assert st == B.SFFN_OK
    torch.cuda.synchronize()
    assert all(int(torch.count_nonzero(t).item()) == 0 for t in g)
    assert bool((env["dx"] == 7.0).all())


def test_probe_rates_run():
    """libsffn_probe.so measures finite, positive rates and rejects bad
    arguments on the host."""
    import math
    import os
    path = os.path.join(os.path.dirname(B.LIB_PATH), "libsffn_probe.so")
    lib = ctypes.CDLL(path)
    lib.sffn_probe_rates.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.sffn_probe_rates.restype = ctypes.c_int
    out = (ctypes.c_double * 5)()
    assert lib.sffn_probe_rates(0, out, 5) != 0
    assert lib.sffn_probe_rates(8, out, 4) != 0
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert lib.sffn_probe_rates(n_cu, out, 5) == 0
    torch.cuda.synchronize()
    for v in out:
        assert math.isfinite(v) and v > 0.0

"""Helpers shared by the GPU tests: device copies of the seeded inputs,
the oracle's view of the same inputs, and error measures."""
import numpy as np
import torch

from unstructured_sparse_feedforward_amd import SparseFFN


def dev(inp, name):
    """Device tensor of one input, in the workload's storage dtype."""
    a = getattr(inp, name)
    if a is None:
        return None
    if inp.wl.dtype == "bf16":
        return torch.from_numpy(inp.bits(name).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def math_weights(inp):
    """float64 weights in the paper's math orientation: W_g, W_u are d x F and
    W_d is F x d."""
    wg = inp.w_gate.astype(np.float64).T
    wu = None if inp.w_up is None else inp.w_up.astype(np.float64).T
    wd = inp.w_down.astype(np.float64)
    return wg, wu, wd


def layer(inp, **kw):
    """The workload's layer handle, with its ELL and dense-row capacities
    (as the benchmark builds it) unless overridden."""
    w = inp.wl
    return SparseFFN(w.d, w.F, gated=w.gated, twell_cap=kw.get("C", w.twell_cap),
                     tile=w.tile, ell_cap=kw.get("ell_cap", w.ell_cap),
                     dense_rows=kw.get("dense_rows", w.dense_rows),
                     dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                     store_dtype=kw.get("store_dtype", torch.float32),
                     fused_updown=kw.get("fused_updown", False))


def rel_fro(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    n = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (n if n > 0 else 1.0)


def assert_close_bf16(got, ref, what=""):
    """Bound for bf16 inputs with fp32 accumulation: relative Frobenius
    error <= 1e-3 and max-abs error <= 1e-2 * max|ref|."""
    r = rel_fro(got, ref)
    mx = np.abs(np.asarray(got, np.float64) - ref).max() if np.size(ref) else 0.0
    assert r <= 1e-3, f"{what}: relative Frobenius error {r:.3e} > 1e-3"
    assert mx <= 1e-2 * max(np.abs(ref).max(), 1e-30), f"{what}: max-abs {mx:.3e}"


def assert_close_f32(got, ref, what=""):
    """Bound for fp32 inputs: relative Frobenius error <= 1e-5."""
    r = rel_fro(got, ref)
    assert r <= 1e-5, f"{what}: relative Frobenius error {r:.3e} > 1e-5"


def to_np(v):
    """Host copy; bf16 tensors come back as float32 values."""
    return v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()


def twell_np(tw):
    torch.cuda.synchronize()
    out = {k: to_np(v) for k, v in tw.items()}
    out["idx"] = out["idx"].view(np.uint16).astype(np.int64)
    out["n_flagged"] = int(out["n_flagged"][0])
    return out


def valid_slots(tw):
    """Mask [T, n_t, C] of the slots a TwELL defines (s < min(cnt, C));
    the others are unspecified."""
    C = tw["val"].shape[2]
    n = np.minimum(tw["cnt"], C)
    return np.arange(C)[None, None, :] < n[:, :, None]


def assert_twell_equal(a, b, flags=True):
    """Counts equal, and values and indices equal on every defined slot."""
    assert np.array_equal(a["cnt"], b["cnt"]), "cnt"
    m = valid_slots(a)
    assert np.array_equal(a["idx"][m], b["idx"][m]), "idx"
    assert np.array_equal(np.asarray(a["val"], np.float64)[m], np.asarray(b["val"], np.float64)[m]), "val"
    if flags:
        assert np.array_equal(np.asarray(a["row_flag"]).astype(bool),
                              np.asarray(b["row_flag"]).astype(bool)), "row_flag"

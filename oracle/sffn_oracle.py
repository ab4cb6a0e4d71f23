"""CPU oracle for the activation-sparse ReLU feedforward layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry and the
benchmark's CPU-baseline leg may import this module. The product path
(the HIP library and its Python binding) never calls it, and it shares no
code with that path.

Everything is plain numpy in float64, written from "Sparser, Faster,
Lighter Transformer Language Models" (Cetin et al.):

  * the feedforward layer, gated h_g = ReLU(x W_g), y = (h_g * (x W_u)) W_d,
    and the non-gated ReLU(x W_1) W_2 (gist.science explainer,
    "2. Methodology" B: inference kernels; appendix Table 2 for the gated and
    non-gated shapes);
  * TwELL, the tile-wise ELLPACK format: the columns of each row are cut
    into 1-D tiles and each tile keeps its non-zero values and their indices
    in a small ELL list (explainer, "2. Methodology" A; wispaper blog,
    "1. TwELL: Tile-wise ELLPACK");
  * the Hybrid training format: rows with few non-zeros go to a compact
    ELL matrix, heavy rows to a dense backup (explainer "2. Methodology" A,
    "Hybrid Format for Training"; wispaper blog "2. The Hybrid Training
    Algorithm");
  * the backward pass restricted to active entries (explainer
    "2. Methodology" B, training kernels: backpropagation).

Weights use the paper's math orientation: w_gate and w_up are d x F,
w_down is F x d. Readings where the descriptions leave a step open:

  * active means strictly Z > 0 (ReLU); zero, -0.0 and NaN are inactive;
  * slots inside a tile are in ascending column order, padded with
    (0.0, 0); the count is the true (uncapped) number of positives;
  * a row whose tile count exceeds the capacity C is flagged and the
    layer's output for that row is the dense one;
  * Hybrid sends a row to the dense backup iff its total count exceeds
    the ELL capacity K or any of its TwELL tiles overflowed; backup rows
    take slots in ascending token order.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# dense layer (the plain definition)
# ---------------------------------------------------------------------------

def relu(z):
    """ReLU with 'active' meaning strictly positive."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z > 0, z, 0.0)


def dense_ffn(x, w_gate, w_up, w_down):
    """Gated ReLU feedforward: y = (ReLU(x W_g) * (x W_u)) W_d.

    Returns y and the intermediates (Z = x W_g, A = ReLU(Z), U = x W_u,
    H = A * U), all float64. With ``w_up=None`` the layer is the
    non-gated ReLU(x W_1) W_2 and U is None.
    """
    x = np.asarray(x, dtype=np.float64)
    z = x @ np.asarray(w_gate, dtype=np.float64)
    a = relu(z)
    if w_up is None:
        u = None
        h = a
    else:
        u = x @ np.asarray(w_up, dtype=np.float64)
        h = a * u
    y = h @ np.asarray(w_down, dtype=np.float64)
    return y, dict(z=z, a=a, u=u, h=h)


def round_bf16(v):
    """float64 -> nearest bfloat16 (ties to even), returned as float64.

    Used only to mirror the one rounding point of a standard bf16 dense
    feedforward (the hidden activations are stored in bf16 between the
    two GEMMs)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    m, e = np.frexp(v[nz])            # v = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: scale the mantissa to [128, 256)
    s = m * 256.0
    r = np.round(s)                   # numpy rounds half to even
    out[nz] = np.ldexp(r, e - 8)
    return out


def dense_ffn_bf16_hidden(x, w_gate, w_up, w_down):
    """Standard bf16 dense layer: as :func:`dense_ffn`, but the hidden
    activations H are rounded once to bf16 before the down projection."""
    _, it = dense_ffn(x, w_gate, w_up, w_down)
    hb = round_bf16(it["h"])
    return hb @ np.asarray(w_down, dtype=np.float64)


def dense_ffn_bf16_store(x, w_gate, w_up, w_down):
    """The layer whose stored activations are bfloat16: the gate activations
    A = ReLU(x W_g) and the up values U = x W_u are each rounded once to
    bf16 (the values the TwELL/Hybrid formats hold when they store 16-bit
    activations, halving their bytes) and the layer computes with the
    stored values: H = bf16(A) * bf16(U), y = H W_d (non-gated:
    y = bf16(A) W_2). Z, the products and y stay exact."""
    _, it = dense_ffn(x, w_gate, w_up, w_down)
    a_s = round_bf16(it["a"])
    h = a_s if it["u"] is None else a_s * round_bf16(it["u"])
    return h @ np.asarray(w_down, dtype=np.float64)


def backward_bf16_store(x, w_gate, w_up, w_down, dy, l1_coeff=0.0, mask=None):
    """Gradients of :func:`dense_ffn_bf16_store`, with the roundings passed
    through unchanged (their derivative taken as 1): the backward reads the
    stored values. With A_s = bf16(Z * M), U_s = bf16(U) and M = 1[Z > 0]
    (or the given mask): dH = dy W_d^T; dU = dH * A_s;
    dZ = dH * U_s * M + l1 * M; dx = dZ W_g^T + dU W_u^T; dW_g = x^T dZ;
    dW_u = x^T dU; dW_d = (A_s * U_s)^T dy. Non-gated: dZ = dH * M + l1 * M,
    dx = dZ W_1^T, dW_1 = x^T dZ, dW_2 = A_s^T dy."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wd = np.asarray(w_down, dtype=np.float64)
    _, it = dense_ffn(x, w_gate, w_up, w_down)
    if mask is None:
        m = (it["z"] > 0).astype(np.float64)
    else:
        m = np.asarray(mask, dtype=bool).astype(np.float64)
    a_s = round_bf16(it["z"] * m)
    dh = dy @ wd.T
    if w_up is None:
        dz = dh * m + l1_coeff * m
        return dict(dx=dz @ wg.T, dw_gate=x.T @ dz, dw_up=None, dw_down=a_s.T @ dy)
    wu = np.asarray(w_up, dtype=np.float64)
    u_s = round_bf16(it["u"])
    du = dh * a_s
    dz = dh * u_s * m + l1_coeff * m
    return dict(dx=dz @ wg.T + du @ wu.T, dw_gate=x.T @ dz, dw_up=x.T @ du,
                dw_down=(a_s * u_s).T @ dy)


def dense_train_bf16(x, w_gate, w_up, w_down, dy, l1_coeff=0.0):
    """A standard bf16 dense training step of the layer (the comparator of
    the sparse step): the two GEMMs' outputs are bf16, Z_s = bf16(x W_g)
    and U_s = bf16(x W_u); H = bf16(ReLU(Z_s) * U_s); y = H W_d. Backward
    with M = 1[Z_s > 0]: dH = dy W_d^T; the gradients that enter GEMMs are
    bf16, dZ = bf16(dH * U_s * M + l1 * M) and dU = bf16(dH * ReLU(Z_s));
    dx = dZ W_g^T + dU W_u^T; dW_g = x^T dZ; dW_u = x^T dU; dW_d = H^T dy.
    Non-gated: H = ReLU(Z_s), dZ = bf16(dH * M + l1 * M), dW_2 = H^T dy.
    Returns dict(y, dx, dw_gate, dw_up, dw_down)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wd = np.asarray(w_down, dtype=np.float64)
    z_s = round_bf16(x @ wg)
    m = (z_s > 0).astype(np.float64)
    a_s = z_s * m
    dh = dy @ wd.T
    if w_up is None:
        h = a_s
        dz = round_bf16(dh * m + l1_coeff * m)
        return dict(y=h @ wd, dx=dz @ wg.T, dw_gate=x.T @ dz, dw_up=None, dw_down=h.T @ dy)
    wu = np.asarray(w_up, dtype=np.float64)
    u_s = round_bf16(x @ wu)
    h = round_bf16(a_s * u_s)
    dz = round_bf16(dh * u_s * m + l1_coeff * m)
    du = round_bf16(dh * a_s)
    return dict(y=h @ wd, dx=dz @ wg.T + du @ wu.T, dw_gate=x.T @ dz, dw_up=x.T @ du,
                dw_down=h.T @ dy)


# ---------------------------------------------------------------------------
# TwELL
# ---------------------------------------------------------------------------

def pack_twell(z, W, C):
    """Pack ReLU(Z) into TwELL.

    For each row t and each tile b (columns [b*W, min((b+1)*W, F))), list
    the columns j of the tile with Z[t, j] > 0 in ascending order; keep the
    first C of them as (value, global column index); record the true count.
    A row is flagged when any of its tiles holds more than C positives.

    Returns dict(val [T, nt, C] float64, idx [T, nt, C] int64,
    cnt [T, nt] int64, row_flag [T] bool).
    """
    z = np.asarray(z, dtype=np.float64)
    T, F = z.shape
    nt = -(-F // W)
    val = np.zeros((T, nt, C), dtype=np.float64)
    idx = np.zeros((T, nt, C), dtype=np.int64)
    cnt = np.zeros((T, nt), dtype=np.int64)
    for t in range(T):
        for b in range(nt):
            lo, hi = b * W, min((b + 1) * W, F)
            cols = lo + np.flatnonzero(z[t, lo:hi] > 0)   # ascending
            cnt[t, b] = len(cols)
            keep = cols[:C]
            val[t, b, :len(keep)] = z[t, keep]
            idx[t, b, :len(keep)] = keep
    row_flag = (cnt > C).any(axis=1)
    return dict(val=val, idx=idx, cnt=cnt, row_flag=row_flag)


def unpack_twell(tw, F):
    """Dense [T, F] matrix holding the stored TwELL entries."""
    val, idx, cnt = tw["val"], tw["idx"], tw["cnt"]
    T, nt, C = val.shape
    out = np.zeros((T, F), dtype=np.float64)
    for t in range(T):
        for b in range(nt):
            for s in range(min(int(cnt[t, b]), C)):
                out[t, idx[t, b, s]] = val[t, b, s]
    return out


def active_pairs(tw):
    """Per row, the stored (neuron, value) pairs in ascending neuron order."""
    val, idx, cnt = tw["val"], tw["idx"], tw["cnt"]
    T, nt, C = val.shape
    rows = []
    for t in range(T):
        js, vs = [], []
        for b in range(nt):
            n = min(int(cnt[t, b]), C)
            js.extend(idx[t, b, :n].tolist())
            vs.extend(val[t, b, :n].tolist())
        rows.append((np.asarray(js, dtype=np.int64),
                     np.asarray(vs, dtype=np.float64)))
    return rows


def sparse_ffn(x, w_gate, w_up, w_down, W, C):
    """The layer computed the sparse way: gate, TwELL pack, then up/down
    projections only over each row's stored active neurons (dot product
    with the up column, scalar times the down row). Flagged rows take the
    dense result. Equal to :func:`dense_ffn` up to summation order."""
    x = np.asarray(x, dtype=np.float64)
    w_down = np.asarray(w_down, dtype=np.float64)
    z = x @ np.asarray(w_gate, dtype=np.float64)
    tw = pack_twell(z, W, C)
    y_dense, _ = dense_ffn(x, w_gate, w_up, w_down)
    T, d = x.shape[0], w_down.shape[1]
    y = np.zeros((T, d), dtype=np.float64)
    wu = None if w_up is None else np.asarray(w_up, dtype=np.float64)
    for t, (js, vs) in enumerate(active_pairs(tw)):
        if tw["row_flag"][t]:
            y[t] = y_dense[t]
            continue
        for j, a in zip(js, vs):
            h = a if wu is None else a * float(x[t] @ wu[:, j])
            y[t] += h * w_down[j]
    return y, tw


# ---------------------------------------------------------------------------
# Hybrid (training format)
# ---------------------------------------------------------------------------

def hybrid_compact(tw, K, a_dense=None, u_dense=None):
    """TwELL -> Hybrid.

    nnz_t = sum of the row's tile counts. A row goes to the dense backup
    iff nnz_t > K or the row is flagged; otherwise its tile lists are
    concatenated (ascending neuron) into an ELL row of K slots, padded with
    (0.0, 0). Backup rows get slots 0, 1, ... in ascending token order;
    ``slot[t]`` is that slot or -1 for ELL rows. If ``a_dense`` (and
    ``u_dense``) are given, the backup rows' dense A (and U) rows are
    returned as bk_a (bk_u).
    """
    cnt, row_flag = tw["cnt"], tw["row_flag"]
    T = cnt.shape[0]
    nnz = cnt.sum(axis=1)
    pairs = active_pairs(tw)
    ell_a = np.zeros((T, K), dtype=np.float64)
    ell_idx = np.zeros((T, K), dtype=np.int64)
    ell_cnt = np.zeros(T, dtype=np.int64)
    slot = np.full(T, -1, dtype=np.int64)
    brow = []
    for t in range(T):
        if nnz[t] > K or row_flag[t]:
            slot[t] = len(brow)
            brow.append(t)
            continue
        js, vs = pairs[t]
        ell_cnt[t] = len(js)
        ell_idx[t, :len(js)] = js
        ell_a[t, :len(js)] = vs
    brow = np.asarray(brow, dtype=np.int64)
    out = dict(ell_a=ell_a, ell_idx=ell_idx, ell_cnt=ell_cnt, slot=slot,
               brow=brow, n_backup=len(brow), nnz=nnz)
    if a_dense is not None:
        out["bk_a"] = np.asarray(a_dense, dtype=np.float64)[brow]
    if u_dense is not None:
        out["bk_u"] = np.asarray(u_dense, dtype=np.float64)[brow]
    return out


def unpack_hybrid(hy, F, a_dense_rows=None):
    """Dense [T, F] matrix from a Hybrid (ELL rows + backup rows)."""
    T, K = hy["ell_a"].shape
    out = np.zeros((T, F), dtype=np.float64)
    for t in range(T):
        if hy["slot"][t] >= 0:
            out[t] = hy["bk_a"][hy["slot"][t]]
        else:
            for s in range(int(hy["ell_cnt"][t])):
                out[t, hy["ell_idx"][t, s]] = hy["ell_a"][t, s]
    return out


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def backward(x, w_gate, w_up, w_down, dy, l1_coeff=0.0, mask=None):
    """Gradients of the gated layer for upstream dy (matrix calculus).

    M = 1[Z > 0];  dH = dy W_d^T;  dU = dH * A;  dZ = dH * U * M + l1 * M
    dx = dZ W_g^T + dU W_u^T;  dW_g = x^T dZ;  dW_u = x^T dU;  dW_d = H^T dy.
    Non-gated (w_up None): dA = dy W_2^T; dZ = dA * M + l1 * M;
    dx = dZ W_1^T; dW_1 = x^T dZ; dW_2 = A^T dy.
    The l1 term is the derivative of l1 * sum(A) through the ReLU mask.

    ``mask`` (boolean [T, F]) fixes the active set M instead of Z > 0; then
    A = Z * M and H = A * U. It serves a caller whose active set was decided
    by a lower-precision Z: entries with Z within that precision of zero
    may be active on one side and not on the other, and the gradients are
    then compared on the same set.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wd = np.asarray(w_down, dtype=np.float64)
    _, it = dense_ffn(x, w_gate, w_up, w_down)
    if mask is None:
        m = (it["z"] > 0).astype(np.float64)
        a = it["a"]
    else:
        m = np.asarray(mask, dtype=bool).astype(np.float64)
        a = it["z"] * m
    dh = dy @ wd.T
    if w_up is None:
        dz = dh * m + l1_coeff * m
        dx = dz @ wg.T
        return dict(dx=dx, dw_gate=x.T @ dz, dw_up=None,
                    dw_down=a.T @ dy)
    wu = np.asarray(w_up, dtype=np.float64)
    du = dh * a
    dz = dh * it["u"] * m + l1_coeff * m
    dx = dz @ wg.T + du @ wu.T
    return dict(dx=dx, dw_gate=x.T @ dz, dw_up=x.T @ du,
                dw_down=(a * it["u"]).T @ dy)


def backward_sparse(x, w_gate, w_up, w_down, dy, hy, l1_coeff=0.0):
    """The same gradients computed from a Hybrid, looping only over the
    stored active pairs of ELL rows and densely over backup rows."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wu = None if w_up is None else np.asarray(w_up, dtype=np.float64)
    wd = np.asarray(w_down, dtype=np.float64)
    T, d = x.shape
    F = wg.shape[1]
    dx = np.zeros((T, d))
    dwg = np.zeros((d, F))
    dwu = None if wu is None else np.zeros((d, F))
    dwd = np.zeros((F, d))
    for t in range(T):
        if hy["slot"][t] >= 0:
            z = x[t] @ wg
            msk = z > 0
            js = np.flatnonzero(msk)
            avals = z[js]
        else:
            n = int(hy["ell_cnt"][t])
            js = hy["ell_idx"][t, :n]
            avals = hy["ell_a"][t, :n]
        for j, a in zip(js, avals):
            dh = float(dy[t] @ wd[j])
            if wu is None:
                h = a
                dz = dh + l1_coeff
            else:
                u = float(x[t] @ wu[:, j])
                h = a * u
                du = dh * a
                dz = dh * u + l1_coeff
                dx[t] += du * wu[:, j]
                dwu[:, j] += du * x[t]
            dx[t] += dz * wg[:, j]
            dwg[:, j] += dz * x[t]
            dwd[j] += h * dy[t]
    return dict(dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd)

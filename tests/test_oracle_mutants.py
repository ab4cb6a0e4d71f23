"""Planted mistakes in copies of the oracle must each break some pin.

Each mutant is the oracle's source with one textual change (a flipped
comparison, a dropped term, a wrong operand), loaded as a separate module
on the CPU; the real oracle is never modified."""
import os
import types

import pytest

from oracle_pins import run_all

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "sffn_oracle.py")

MUTATIONS = [
    ("pack: >= instead of >", "cols = lo + np.flatnonzero(z[t, lo:hi] > 0)",
     "cols = lo + np.flatnonzero(z[t, lo:hi] >= 0)"),
    ("pack: keeps the last C", "keep = cols[:C]", "keep = cols[-C:] if C else cols[:0]"),
    ("pack: flag at cnt == C", "row_flag = (cnt > C).any(axis=1)",
     "row_flag = (cnt >= C).any(axis=1)"),
    ("pack: capped count", "cnt[t, b] = len(cols)", "cnt[t, b] = min(len(cols), C)"),
    ("dense: ReLU dropped", "h = a * u\n    y = h @", "h = z * u\n    y = h @"),
    ("dense: up projection dropped", "h = a * u\n    y = h @", "h = a\n    y = h @"),
    ("relu: leaky", "return np.where(z > 0, z, 0.0)",
     "return np.where(z > 0, z, 0.01 * z)"),
    ("sparse: up projection dropped", "h = a if wu is None else a * float(x[t] @ wu[:, j])",
     "h = a"),
    ("hybrid: >= K", "if nnz[t] > K or row_flag[t]:", "if nnz[t] >= K or row_flag[t]:"),
    ("hybrid: flag ignored", "if nnz[t] > K or row_flag[t]:", "if nnz[t] > K:"),
    ("backward: dU W_u^T dropped", "dx = dz @ wg.T + du @ wu.T", "dx = dz @ wg.T"),
    ("backward: mask dropped", 'dz = dh * it["u"] * m + l1_coeff * m',
     'dz = dh * it["u"] + l1_coeff * m'),
    ("backward: dW_d uses A", 'dw_down=(a * it["u"]).T @ dy)', 'dw_down=a.T @ dy)'),
    ("backward: transposed dW_g", "return dict(dx=dx, dw_gate=x.T @ dz, dw_up=x.T @ du,",
     "return dict(dx=dx, dw_gate=(dz.T @ x).T[:, ::-1].copy(), dw_up=x.T @ du,"),
    ("bf16: 7 significant bits", "s = m * 256.0", "s = m * 128.0"),
    ("bf16: ties away", "r = np.round(s)", "r = np.floor(s + 0.5)"),
    ("bf16 layer: no rounding", 'hb = round_bf16(it["h"])', 'hb = it["h"]'),
    ("bf16 layer: rounds y", 'hb = round_bf16(it["h"])\n    return hb @ np.asarray(w_down, dtype=np.float64)',
     'return round_bf16(it["h"] @ np.asarray(w_down, dtype=np.float64))'),
    ("bf16 layer: rounds A instead of H", 'hb = round_bf16(it["h"])',
     'hb = round_bf16(it["a"]) * (1.0 if it["u"] is None else it["u"])'),
    ("bf16 layer: rounds A and U before the product", 'hb = round_bf16(it["h"])',
     'hb = round_bf16(it["a"]) * (1.0 if it["u"] is None else round_bf16(it["u"]))'),
    ("bf16 layer: rounds before the ReLU", 'hb = round_bf16(it["h"])',
     'hb = relu(round_bf16(it["z"])) * (1.0 if it["u"] is None else it["u"])'),
    ("backward: given mask ignored",
     'm = np.asarray(mask, dtype=bool).astype(np.float64)\n        a = it["z"] * m',
     'm = (it["z"] > 0).astype(np.float64)\n        a = it["z"] * m'),
    ("bf16 store: given mask ignored",
     'm = np.asarray(mask, dtype=bool).astype(np.float64)\n    a_s = round_bf16',
     'm = (it["z"] > 0).astype(np.float64)\n    a_s = round_bf16'),
    ("backward: given mask not applied to A", 'a = it["z"] * m', 'a = it["a"]'),
    ("bf16 store: U not rounded in the forward", 'h = a_s if it["u"] is None else a_s * round_bf16(it["u"])',
     'h = a_s if it["u"] is None else a_s * it["u"]'),
    ("bf16 store: A not rounded in the forward", 'a_s = round_bf16(it["a"])\n    h = a_s', 'a_s = it["a"]\n    h = a_s'),
    ("bf16 store: y rounded instead", 'return h @ np.asarray(w_down, dtype=np.float64)\n\n\ndef backward_bf16_store',
     'return round_bf16(h @ np.asarray(w_down, dtype=np.float64))\n\n\ndef backward_bf16_store'),
    ("bf16 store: backward reads the unrounded U", "u_s = round_bf16(it[\"u\"])", 'u_s = it["u"]'),
    ("bf16 store: backward reads the unrounded A", "a_s = round_bf16(it[\"z\"] * m)", 'a_s = it["z"] * m'),
    ("bf16 store: dW_d from the unrounded H", "dw_down=(a_s * u_s).T @ dy)", 'dw_down=it["h"].T @ dy)'),
    ("dense train: dZ not rounded", "dz = round_bf16(dh * u_s * m + l1_coeff * m)",
     "dz = dh * u_s * m + l1_coeff * m"),
    ("dense train: dU not rounded", "du = round_bf16(dh * a_s)\n    return dict(y=h @ wd",
     "du = dh * a_s\n    return dict(y=h @ wd"),
    ("dense train: H not rounded", "h = round_bf16(a_s * u_s)", "h = a_s * u_s"),
    ("dense train: U not rounded", "u_s = round_bf16(x @ wu)", "u_s = x @ wu"),
    ("dense train: Z not rounded", "z_s = round_bf16(x @ wg)", "z_s = x @ wg"),
    ("hybrid: bk_u from A", 'out["bk_u"] = np.asarray(u_dense, dtype=np.float64)[brow]',
     'out["bk_u"] = np.asarray(a_dense, dtype=np.float64)[brow]'),
    ("hybrid: bk_u rows of the ELL rows", 'out["bk_u"] = np.asarray(u_dense, dtype=np.float64)[brow]',
     'out["bk_u"] = np.asarray(u_dense, dtype=np.float64)[np.flatnonzero(slot < 0)[:len(brow)]]'),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation target not found or not unique: {old}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    failures = run_all(mod)
    assert failures, f"mutant '{name}' passed every pin"

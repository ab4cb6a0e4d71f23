"""The 18-layer stack chained with residual connections and RMS
normalisation, each layer in the mode the library picks from its own
TwELL: per layer, sampled rows of its output against the oracle on the
input the GPU gave it (the standard bf16 layer's oracle for layers run
dense), and the per-layer active counts against the ramp the synthetic
layers are calibrated for."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close_bf16, math_weights
from unstructured_sparse_feedforward_amd import workloads as wl
from unstructured_sparse_feedforward_amd.stack import FFNStack

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _bf(a):
    return torch.from_numpy((a.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).view(
        torch.bfloat16).cuda()


def test_chained_stack_per_layer_parity():
    T = 2048            # one sequence of the stack workload
    Ws = [wl.stack_layer(i).replace(T=T) for i in range(len(wl.STACK_RAMP))]
    inps = [wl.make_inputs(W, seed=3, layer=i) for i, W in enumerate(Ws)]
    weights = [tuple(_bf(getattr(inp, k)) for k in ("w_gate", "w_up", "w_down")) for inp in inps]
    stack = FFNStack(weights, Ws, T)
    outlier = inps[0].outlier
    keep = torch.from_numpy((~outlier).astype(np.float32)).to(torch.bfloat16).cuda()
    h0 = torch.from_numpy(inps[0].x).cuda()
    info = stack.choose_modes(h0, keep)
    rec = []
    stack.forward(h0, keep, record=rec)
    stack.check()
    modes = [m for m, _, _ in info]
    _print("modes:", modes)
    _print("mean active:", [round(m, 1) for _, m, _ in info])
    assert "sparse" in modes
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.flatnonzero(outlier)[:8],
                                     rng.choice(T, 40, replace=False)]))
    for l, ((x, y, mode), inp, (_, mean, _)) in enumerate(zip(rec, inps, info)):
        # the synthetic layers stay calibrated through the chain
        assert 0.75 * wl.STACK_RAMP[l] < mean < 1.25 * wl.STACK_RAMP[l], (l, mean)
        xr = x[rows].float().cpu().numpy().astype(np.float64)
        wg, wu, wd = math_weights(inp)
        ref = (oracle.dense_ffn(xr, wg, wu, wd)[0] if mode == "sparse"
               else oracle.dense_ffn_bf16_hidden(xr, wg, wu, wd))
        assert_close_bf16(y.cpu().numpy()[rows], ref, f"layer {l} ({mode})")

"""A stack of feedforward layers chained as in an MLP-only pre-norm
Transformer (no attention): h_{l+1} = h_l + FFN_l(x_l) with x_l the RMS
normalisation of h_l, so that every layer's input keeps unit scale and the
layer's gate threshold stays calibrated (the pages' models are such stacks,
with the activation sparsity varying from layer to layer: listing page,
Figure 6 and Figures 10-11).

Column 0 of every layer's input is the synthetic layers' bias input (1 for
normal tokens, 0 for the outlier tokens, whose gate then has no threshold);
the normalisation runs over the other d - 1 columns. The residual add and
the normalisation between the layers are torch operations (plumbing around
the library's layers); every layer runs through libsffn's sparse or dense
forward, in the mode the library chooses from the layer's own TwELL
(sffn_choose_mode).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from .binding import SparseFFN


class FFNStack:
    """``weights``: per layer (w_gate, w_up or None, w_down) device bf16
    tensors, neuron-major [F, d]; ``workloads``: the per-layer Workload
    records (shapes, TwELL and ELL capacities)."""

    def __init__(self, weights: Sequence[Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]],
                 workloads: Sequence, T: int, store_dtype: torch.dtype = torch.float32):
        self.weights = list(weights)
        self.ffns = [SparseFFN(W.d, W.F, gated=W.gated, twell_cap=W.twell_cap, tile=W.tile,
                               ell_cap=W.ell_cap, dense_rows=W.dense_rows, dtype=torch.bfloat16,
                               store_dtype=store_dtype) for W in workloads]
        d = workloads[0].d
        self.T = T
        self.tw = [f.new_twell(T) for f in self.ffns]
        self.modes: List[str] = ["sparse"] * len(self.ffns)
        self.x = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty((T, d), dtype=torch.float32, device="cuda")
        self.h = torch.empty((T, d), dtype=torch.float32, device="cuda")

    @staticmethod
    def layer_input(h: torch.Tensor, keep: torch.Tensor, out: torch.Tensor) -> None:
        """out = bf16 RMS normalisation of columns 1.. of h; out[:, 0] = keep."""
        hs = h[:, 1:]
        r = torch.rsqrt(hs.square().mean(dim=1, keepdim=True) + 1e-6)
        out[:, 1:] = (hs * r).to(torch.bfloat16)
        out[:, 0] = keep

    def forward(self, h0: torch.Tensor, keep: torch.Tensor, record: Optional[list] = None):
        """Runs the stack on the residual stream h0 [T, d] float32; returns
        the final residual stream. With a list ``record``, each layer's
        (input, output, mode) is appended (copies)."""
        h = self.h
        h.copy_(h0)
        for l, (ffn, w) in enumerate(zip(self.ffns, self.weights)):
            self.layer_input(h, keep, self.x)
            mode = self.modes[l]
            ffn.forward(self.x, *w, mode=mode, tw=self.tw[l] if mode == "sparse" else None,
                        y=self.y, check=False)
            if record is not None:
                record.append((self.x.clone(), self.y.clone(), mode))
            h.add_(self.y)
        return h

    def choose_modes(self, h0: torch.Tensor, keep: torch.Tensor):
        """One pass with every layer sparse, then each layer's mode from its
        own TwELL (sffn_choose_mode). Returns per layer (mode, mean active
        neurons per token over its non-overflowing rows, crossover)."""
        self.modes = ["sparse"] * len(self.ffns)
        self.forward(h0, keep)
        self.check()
        info = [f.choose_mode(tw, self.T) for f, tw in zip(self.ffns, self.tw)]
        self.modes = [m for m, _, _ in info]
        return info

    def check(self):
        for f in self.ffns:
            f.check()

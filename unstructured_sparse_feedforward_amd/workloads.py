"""Seeded synthetic workloads for the activation-sparse ReLU feedforward layer.

This module only draws and rounds random inputs. It holds none of the
layer's arithmetic (no ReLU, no products, no packing), so the CPU oracle
and the GPU path can both be fed from it without sharing any computation.

Shapes follow the hyperparameter table of "Sparser, Faster, Lighter
Transformer Language Models" (appendix Table 2: hidden size 2048,
intermediate 5632 gated / 8192 non-gated). The per-token active counts
follow its Tables 3 and 5 (911 with plain ReLU, 108 with sparsity warm-up,
29 with L1 = 2e-5). The outlier tokens stand in for the paper's
observation (Figure 2, Figure 7) that a few high-information tokens and
early positions activate many more neurons.

Recipe (identical for every workload):
  * numpy PCG64 streams from ``SeedSequence([seed, layer])`` spawned into
    x, W_gate, W_up, W_down, outlier mask and dy streams;
  * x ~ N(0, 1) with x[:, 0] = 1 on normal tokens and 0 on outlier tokens;
  * W ~ N(0, std = 1/sqrt(fan_in)) with fan_in = d for W_gate/W_up and
    F for W_down; weights are stored neuron-major [F, d];
  * W_gate[:, 0] = -tau with tau = sqrt((d-1)/d) * Phi^-1(1 - nnz/F), so a
    normal token's pre-activation is N(-tau, (d-1)/d) and about nnz of its
    F pre-activations are positive; an outlier token's is N(0, (d-1)/d),
    i.e. about half positive;
  * dy ~ N(0, 1) for training workloads;
  * values are drawn in float64, rounded to float32 (RNE) and, for bf16
    workloads, rounded once more from float32 to bfloat16 (RNE).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
from numpy.random import Generator, PCG64, SeedSequence
from scipy.special import ndtri


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer's shape and sparsity recipe."""

    name: str
    T: int
    d: int
    F: int
    gated: bool
    dtype: str            # "f32" or "bf16": storage type of x, W and dy
    nnz: float            # target active neurons per normal token
    twell_cap: int        # TwELL capacity C per (row, tile)
    tile: int = 128       # TwELL tile width W
    outlier_frac: float = 0.0
    front_positions: int = 0      # first positions of each sequence ...
    front_prob: float = 0.0       # ... are outliers with this probability
    seq_len: int = 0              # sequence length for the front bias
    ell_cap: int = 0              # ELL capacity K of the sparse path: rows with more
                                  # active neurons take the dense path (training: the
                                  # Hybrid's K; 0 at inference = n_t * C)
    dense_rows: int = 1024        # rows the dense path holds per call (0 = every row)
    train: bool = False           # draw dy as well

    @property
    def tau(self) -> float:
        p = self.nnz / self.F
        return math.sqrt((self.d - 1) / self.d) * float(ndtri(1.0 - p))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Names say what they are; sizes are in the fields.
SMALL_F32 = Workload("gated_T128_d256_F1024_f32", T=128, d=256, F=1024,
                     gated=True, dtype="f32", nnz=0.02 * 1024, twell_cap=16)
# ELL capacities sit several standard deviations above the per-token
# count (29 +- 5.4 here), so that in practice only the outlier tokens take
# the dense path; the dense-row capacities hold several times the expected
# number of such tokens.
GATED_1P5B = Workload("gated_T8192_d2048_F5632_bf16_nnz29", T=8192, d=2048,
                      F=5632, gated=True, dtype="bf16", nnz=29, twell_cap=8,
                      outlier_frac=0.01, ell_cap=64, dense_rows=512)
# A stronger L1 than 2e-5 leaves fewer active neurons (listing Table 4,
# L1 = 3e-5; the pages print no count for it): half the 2e-5 count.
GATED_1P5B_NNZ15 = GATED_1P5B.replace(name="gated_T8192_d2048_F5632_bf16_nnz15", nnz=15)
NONGATED = {n: Workload(f"nongated_T16384_d2048_F8192_bf16_nnz{n}", T=16384,
                        d=2048, F=8192, gated=False, dtype="bf16", nnz=n,
                        twell_cap=c, ell_cap=k, dense_rows=256)
            for n, c, k in ((29, 8, 64), (108, 16, 192), (911, 48, 1280))}
# 18-layer stack: per-layer target active counts ramp 15 -> 120 (layer 5)
# -> 20 (layer 17); 2% outliers with a front-of-sequence bias.
STACK_RAMP = [15, 36, 57, 78, 99, 120, 112, 103, 95, 87, 78, 70, 62, 53,
              45, 37, 28, 20]
STACK_LAYER = Workload("stack18_T16384_d2048_F5632_bf16", T=16384, d=2048,
                       F=5632, gated=True, dtype="bf16", nnz=66.4,
                       twell_cap=16, outlier_frac=0.02, front_positions=32,
                       front_prob=0.3, seq_len=2048, ell_cap=256, dense_rows=1024)
TRAIN_HYBRID = Workload("train_T8192_d2048_F5632_bf16_nnz29_K64", T=8192,
                        d=2048, F=5632, gated=True, dtype="bf16", nnz=29,
                        twell_cap=16, outlier_frac=0.05, ell_cap=64,
                        dense_rows=512, train=True)


def stack_layer(i: int) -> Workload:
    return STACK_LAYER.replace(name=f"{STACK_LAYER.name}_layer{i}",
                               nnz=STACK_RAMP[i])


@dataclasses.dataclass
class Inputs:
    """Rounded inputs. Float arrays hold values exactly representable in
    ``dtype``; ``*_bits`` give the raw bf16 bit patterns (uint16) for
    bf16 workloads."""

    wl: Workload
    x: np.ndarray            # [T, d] float32
    w_gate: np.ndarray       # [F, d] float32 (neuron-major)
    w_up: Optional[np.ndarray]   # [F, d] float32 or None (non-gated)
    w_down: np.ndarray       # [F, d] float32 (row j = neuron j's outputs)
    outlier: np.ndarray      # [T] bool
    dy: Optional[np.ndarray] = None  # [T, d] float32

    def bits(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.wl.dtype != "bf16":
            raise ValueError("bits() is for bf16 workloads")
        return (a.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def round_bf16(a32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 round-to-nearest-even, returned as float32."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2**32
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _to_dtype(a64: np.ndarray, dtype: str) -> np.ndarray:
    a = round_f32(a64)
    return round_bf16(a) if dtype == "bf16" else a


def outlier_mask(wl: Workload, rng: Generator) -> np.ndarray:
    u = rng.random(wl.T)
    if wl.front_positions and wl.seq_len:
        pos = np.arange(wl.T) % wl.seq_len
        front = pos < wl.front_positions
        # the rest of each sequence is drawn so the expected fraction
        # stays at outlier_frac overall
        n_front = wl.front_positions / wl.seq_len
        p_rest = (wl.outlier_frac - n_front * wl.front_prob) / (1 - n_front)
        return np.where(front, u < wl.front_prob, u < p_rest)
    return u < wl.outlier_frac


def make_inputs(wl: Workload, seed: int, layer: int = 0,
                T: Optional[int] = None) -> Inputs:
    """Draw one layer's inputs. ``T`` overrides the token count (the
    first T rows of the same recipe with a smaller batch)."""
    if T is not None:
        wl = wl.replace(T=T)
    ss = SeedSequence([seed, layer])
    r_x, r_g, r_u, r_d, r_m, r_dy = [Generator(PCG64(s)) for s in ss.spawn(6)]
    T_, d, F = wl.T, wl.d, wl.F
    mask = outlier_mask(wl, r_m)
    x = r_x.standard_normal((T_, d))
    x[:, 0] = np.where(mask, 0.0, 1.0)
    wg = r_g.standard_normal((F, d)) / math.sqrt(d)
    wg[:, 0] = -wl.tau
    wu = r_u.standard_normal((F, d)) / math.sqrt(d) if wl.gated else None
    wd = r_d.standard_normal((F, d)) / math.sqrt(F)
    dy = r_dy.standard_normal((T_, d)) if wl.train else None
    cv = lambda a: None if a is None else _to_dtype(a, wl.dtype)
    return Inputs(wl=wl, x=cv(x), w_gate=cv(wg), w_up=cv(wu),
                  w_down=cv(wd), outlier=mask, dy=cv(dy))

"""Thin Python binding of libsffn.so (the C ABI in include/sffn.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels. PyTorch supplies device memory and the current stream. There
is no fallback: if libsffn.so is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsffn.so")

SFFN_OK = 0
SFFN_E_ARG = -1
SFFN_E_UNSUPPORTED = -2
SFFN_E_HIP = -3
SFFN_E_CAPACITY = -4

SFFN_F32 = 0
SFFN_BF16 = 1
SFFN_SPARSE = 0
SFFN_DENSE = 1
SFFN_OP_PACK = 0
SFFN_OP_FORWARD_SPARSE = 1
SFFN_OP_FORWARD_DENSE = 2
SFFN_OP_HYBRID = 3
SFFN_OP_FORWARD_TRAIN = 4
SFFN_OP_BACKWARD = 5
SFFN_OP_TRAIN_DENSE = 6
SFFN_OP_BACKWARD_DENSE = 7

# every symbol include/sffn.h declares
EXPORTS = ("sffn_create", "sffn_destroy", "sffn_last_error", "sffn_status_string",
           "sffn_workspace_bytes", "sffn_pack_twell", "sffn_gate_preact",
           "sffn_forward", "sffn_check", "sffn_profile_enable", "sffn_profile_read",
           "sffn_kernel_name", "sffn_hybrid_compact", "sffn_forward_train",
           "sffn_hybrid_check", "sffn_backward", "sffn_forward_noalloc",
           "sffn_choose_mode", "sffn_train_dense_act_bytes", "sffn_forward_train_dense",
           "sffn_backward_dense")
SFFN_K_COUNT = 24


class SffnDesc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("gated", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("twell_cap", ctypes.c_int32), ("ell_cap", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("dense_rows", ctypes.c_int32),
                ("store_dtype", ctypes.c_int32), ("dense_above", ctypes.c_float),
                ("updown", ctypes.c_int32)]


class SffnTwell(ctypes.Structure):
    _fields_ = [("val", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("cnt", ctypes.c_void_p), ("row_flag", ctypes.c_void_p),
                ("flagged", ctypes.c_void_p), ("n_flagged", ctypes.c_void_p)]


class SffnHybrid(ctypes.Structure):
    _fields_ = [("ell_a", ctypes.c_void_p), ("ell_u", ctypes.c_void_p),
                ("ell_idx", ctypes.c_void_p), ("ell_cnt", ctypes.c_void_p),
                ("slot", ctypes.c_void_p), ("brow", ctypes.c_void_p),
                ("n_backup", ctypes.c_void_p), ("bk_a", ctypes.c_void_p),
                ("bk_u", ctypes.c_void_p), ("max_backup", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsffn.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run unstructured_sparse_feedforward_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.sffn_create.argtypes = [ctypes.POINTER(SffnDesc), ctypes.POINTER(vp)]
    lib.sffn_create.restype = i32
    lib.sffn_destroy.argtypes = [vp]
    lib.sffn_destroy.restype = None
    lib.sffn_last_error.argtypes = [vp]
    lib.sffn_last_error.restype = ctypes.c_char_p
    lib.sffn_status_string.argtypes = [i32]
    lib.sffn_status_string.restype = ctypes.c_char_p
    lib.sffn_workspace_bytes.argtypes = [vp, i64, i32, ctypes.POINTER(sz)]
    lib.sffn_workspace_bytes.restype = i32
    lib.sffn_pack_twell.argtypes = [vp, vp, i64, ctypes.POINTER(SffnTwell), vp, sz, vp]
    lib.sffn_pack_twell.restype = i32
    lib.sffn_gate_preact.argtypes = [vp, vp, vp, i64, vp, vp]
    lib.sffn_gate_preact.restype = i32
    lib.sffn_forward.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.POINTER(SffnTwell), i32,
                                 vp, sz, vp]
    lib.sffn_forward.restype = i32
    lib.sffn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, vp,
                                         ctypes.POINTER(SffnTwell), i32, vp]
    lib.sffn_forward_noalloc.restype = i32
    lib.sffn_choose_mode.argtypes = [vp, ctypes.POINTER(SffnTwell), i64, ctypes.POINTER(i32),
                                     ctypes.POINTER(ctypes.c_float),
                                     ctypes.POINTER(ctypes.c_float), vp]
    lib.sffn_choose_mode.restype = i32
    lib.sffn_train_dense_act_bytes.argtypes = [vp, i64, ctypes.POINTER(sz)]
    lib.sffn_train_dense_act_bytes.restype = i32
    lib.sffn_forward_train_dense.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
    lib.sffn_forward_train_dense.restype = i32
    lib.sffn_backward_dense.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp,
                                        ctypes.c_float, vp, sz, vp]
    lib.sffn_backward_dense.restype = i32
    lib.sffn_check.argtypes = [vp, vp]
    lib.sffn_check.restype = i32
    lib.sffn_profile_enable.argtypes = [vp, i32]
    lib.sffn_profile_enable.restype = i32
    lib.sffn_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(i32), i32]
    lib.sffn_profile_read.restype = i32
    lib.sffn_kernel_name.argtypes = [i32]
    lib.sffn_kernel_name.restype = ctypes.c_char_p
    lib.sffn_hybrid_compact.argtypes = [vp, ctypes.POINTER(SffnTwell), vp, i64,
                                        ctypes.POINTER(SffnHybrid), vp, sz, vp]
    lib.sffn_hybrid_compact.restype = i32
    lib.sffn_forward_train.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.POINTER(SffnTwell),
                                       ctypes.POINTER(SffnHybrid), vp, sz, vp]
    lib.sffn_forward_train.restype = i32
    lib.sffn_hybrid_check.argtypes = [vp, ctypes.POINTER(SffnHybrid), vp]
    lib.sffn_hybrid_check.restype = i32
    lib.sffn_backward.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(SffnHybrid), vp, i64,
                                  vp, vp, vp, vp, ctypes.c_float, vp, sz, vp]
    lib.sffn_backward.restype = i32
    _lib = lib
    return lib


class SffnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


DEFAULT_DENSE_ROWS = 1024


class SparseFFN:
    """One feedforward layer's handle.

    Weights are passed to each call (neuron-major [F, d] for w_gate, w_up
    and w_down); x is [T, d]; outputs are float32.

    ``ell_cap`` is the ELL capacity K of the sparse path (rows with more
    active neurons, or with an overflowing TwELL tile, take the dense
    path; 0 at inference = n_t * C). ``dense_rows`` is the most rows one
    call computes on the dense path; the workspace holds that many dense
    rows (0 = every row, a T x F workspace). When a call routes more rows
    than that, the dense path's rows are not valid (the ELL rows are) and
    ``sffn_check`` reports SFFN_E_CAPACITY. The calls here check by default
    (``check=True``, one stream synchronisation per call): on that report
    the handle is rebuilt with ``dense_rows = 0`` and the call is repeated,
    so results are always complete. ``check=False`` skips the
    synchronisation; the caller then runs :meth:`check` itself before
    trusting the results.
    """

    def __init__(self, d: int, d_ff: int, gated: bool = True, twell_cap: int = 8,
                 tile: int = 128, ell_cap: int = 0, dtype: torch.dtype = torch.bfloat16,
                 dense_rows: int = DEFAULT_DENSE_ROWS,
                 store_dtype: torch.dtype = torch.float32, dense_above: float = 0.0,
                 fused_updown: bool = False):
        self.lib = load_library()
        self.d, self.d_ff, self.gated = d, d_ff, gated
        self.tile, self.twell_cap, self.ell_cap = tile, twell_cap, ell_cap
        self.dtype = dtype
        # dtype of the stored activations (TwELL values, Hybrid a and u)
        self.store_dtype = store_dtype
        self.dense_above = dense_above
        # the inference up/down as one fused kernel instead of the sliced
        # three launches
        self.fused_updown = fused_updown
        self.n_t = d_ff // tile
        self.h = None
        self._ws: Dict[str, torch.Tensor] = {}
        self._create(dense_rows)

    def _create(self, dense_rows: int):
        self.close()
        self.dense_rows = dense_rows
        self.desc = SffnDesc(self.d, self.d_ff, int(self.gated), self.tile, self.twell_cap,
                             self.ell_cap,
                             SFFN_BF16 if self.dtype == torch.bfloat16 else SFFN_F32,
                             dense_rows,
                             SFFN_BF16 if self.store_dtype == torch.bfloat16 else SFFN_F32,
                             self.dense_above, 1 if self.fused_updown else 0)
        h = ctypes.c_void_p()
        st = self.lib.sffn_create(ctypes.byref(self.desc), ctypes.byref(h))
        if st != SFFN_OK:
            raise SffnError(st, f"sffn_create: {self.lib.sffn_status_string(st).decode()}")
        self.h = h

    def _grow(self) -> bool:
        """After a capacity report: rebuild with a T-row dense capacity.
        Returns False when the capacity was already unbounded."""
        if self.dense_rows == 0:
            return False
        self._create(0)
        return True

    def close(self):
        if getattr(self, "h", None):
            self.lib.sffn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int, what: str):
        if st != SFFN_OK:
            err = self.lib.sffn_last_error(self.h).decode()
            raise SffnError(st, f"{what}: {self.lib.sffn_status_string(st).decode()} {err}")

    def _capacity_ok(self) -> bool:
        """sffn_check: False on a capacity report, raise on other errors."""
        st = self.lib.sffn_check(self.h, _stream())
        if st == SFFN_E_CAPACITY:
            return False
        self._check(st, "sffn_check")
        return True

    def workspace_bytes(self, T: int, op: int) -> int:
        n = ctypes.c_size_t()
        self._check(self.lib.sffn_workspace_bytes(self.h, T, op, ctypes.byref(n)),
                    "sffn_workspace_bytes")
        return n.value

    def workspace(self, T: int, op: int, device=None):
        """A 256-byte aligned device buffer of the needed size; returns
        (pointer, bytes). One buffer serves every operation of the handle
        (grown to the largest need): the calls run one after the other on
        the stream, and no call's workspace outlives it."""
        n = self.workspace_bytes(T, op)
        buf = self._ws.get("ws")
        if buf is None or buf.numel() < n + 256:
            self._ws.pop("ws", None)
            buf = torch.empty(n + 256, dtype=torch.uint8, device=device or "cuda")
            self._ws["ws"] = buf
        p = buf.data_ptr()
        return (p + 255) // 256 * 256, n

    def new_twell(self, T: int, device="cuda") -> Dict[str, torch.Tensor]:
        C, nt = self.twell_cap, self.n_t
        return dict(
            val=torch.empty((T, nt, C), dtype=self.store_dtype, device=device),
            idx=torch.empty((T, nt, C), dtype=torch.int16, device=device),  # uint16 bits
            cnt=torch.empty((T, nt), dtype=torch.int32, device=device),
            row_flag=torch.empty((T,), dtype=torch.uint8, device=device),
            flagged=torch.empty((max(T, 1),), dtype=torch.int32, device=device),
            n_flagged=torch.zeros((4,), dtype=torch.int32, device=device),
        )

    @staticmethod
    def _tw_struct(tw: Dict[str, torch.Tensor]) -> SffnTwell:
        return SffnTwell(*(tw[k].data_ptr() for k in
                           ("val", "idx", "cnt", "row_flag", "flagged", "n_flagged")))

    def pack_twell(self, z: torch.Tensor, tw: Optional[Dict[str, torch.Tensor]] = None):
        T = z.shape[0]
        tw = tw if tw is not None else self.new_twell(T, z.device)
        ws, n = self.workspace(T, SFFN_OP_PACK, z.device)
        s = self._tw_struct(tw)
        self._check(self.lib.sffn_pack_twell(self.h, _ptr(z), T, ctypes.byref(s), ws, n,
                                             _stream()), "sffn_pack_twell")
        return tw

    def gate_preact(self, x: torch.Tensor, w_gate: torch.Tensor,
                    z: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0]
        if z is None:
            z = torch.empty((T, self.d_ff), dtype=torch.float32, device=x.device)
        self._check(self.lib.sffn_gate_preact(self.h, _ptr(x), _ptr(w_gate), T, _ptr(z),
                                              _stream()), "sffn_gate_preact")
        return z

    def forward(self, x: torch.Tensor, w_gate: torch.Tensor, w_up: Optional[torch.Tensor],
                w_down: torch.Tensor, mode: str = "sparse",
                tw: Optional[Dict[str, torch.Tensor]] = None,
                y: Optional[torch.Tensor] = None, check: bool = True) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.d), dtype=torch.float32, device=x.device)
        m = SFFN_SPARSE if mode == "sparse" else SFFN_DENSE
        op = SFFN_OP_FORWARD_SPARSE if m == SFFN_SPARSE else SFFN_OP_FORWARD_DENSE
        while True:
            ws, n = self.workspace(T, op, x.device)
            s = ctypes.byref(self._tw_struct(tw)) if tw is not None else None
            self._check(self.lib.sffn_forward(self.h, _ptr(x), _ptr(w_gate), _ptr(w_up),
                                              _ptr(w_down), T, _ptr(y), s, m, ws, n,
                                              _stream()), "sffn_forward")
            if not check or self._capacity_ok() or not self._grow():
                return y

    def forward_noalloc(self, x: torch.Tensor, w_gate: torch.Tensor,
                        w_up: Optional[torch.Tensor], w_down: torch.Tensor, y: torch.Tensor,
                        mode: str = "sparse",
                        tw: Optional[Dict[str, torch.Tensor]] = None) -> torch.Tensor:
        """sffn_forward_noalloc: as :meth:`forward` with the library's static
        scratch as workspace; y (and tw) are the caller's. Nothing is
        allocated and nothing is checked (run :meth:`check` afterwards)."""
        m = SFFN_SPARSE if mode == "sparse" else SFFN_DENSE
        s = ctypes.byref(self._tw_struct(tw)) if tw is not None else None
        self._check(self.lib.sffn_forward_noalloc(self.h, _ptr(x), _ptr(w_gate), _ptr(w_up),
                                                  _ptr(w_down), x.shape[0], _ptr(y), s, m,
                                                  _stream()), "sffn_forward_noalloc")
        return y

    def choose_mode(self, tw: Dict[str, torch.Tensor], T: int):
        """sffn_choose_mode: ("sparse" or "dense", mean active neurons per
        token, crossover) from the layer's TwELL of T rows."""
        m = ctypes.c_int32()
        mean, cross = ctypes.c_float(), ctypes.c_float()
        s = self._tw_struct(tw)
        self._check(self.lib.sffn_choose_mode(self.h, ctypes.byref(s), T, ctypes.byref(m),
                                              ctypes.byref(mean), ctypes.byref(cross),
                                              _stream()), "sffn_choose_mode")
        return ("dense" if m.value == SFFN_DENSE else "sparse"), mean.value, cross.value

    def check(self):
        """sffn_check: raises SffnError (SFFN_E_CAPACITY when a call since the
        last check routed more rows to the dense path than it holds)."""
        self._check(self.lib.sffn_check(self.h, _stream()), "sffn_check")

    # ------------------------------------------------------------ Hybrid

    def new_hybrid(self, T: int, max_backup: Optional[int] = None,
                   device="cuda") -> Dict[str, torch.Tensor]:
        """Hybrid buffers; ``max_backup`` defaults to the handle's dense-row
        capacity (T when that is unbounded)."""
        K, F = self.ell_cap, self.d_ff
        if max_backup is None:
            max_backup = min(T, self.dense_rows) if self.dense_rows > 0 else T
        R = max_backup
        f32 = dict(dtype=self.store_dtype, device=device)
        return dict(
            ell_a=torch.empty((T, K), **f32),
            ell_u=torch.empty((T, K), **f32) if self.gated else None,
            ell_idx=torch.empty((T, K), dtype=torch.int16, device=device),  # uint16 bits
            ell_cnt=torch.empty((T,), dtype=torch.int32, device=device),
            slot=torch.empty((max(T, 1),), dtype=torch.int32, device=device),
            brow=torch.empty((max(R, 1),), dtype=torch.int32, device=device),
            n_backup=torch.zeros((4,), dtype=torch.int32, device=device),
            bk_a=torch.empty((max(R, 1), F), **f32),
            bk_u=torch.empty((max(R, 1), F), **f32) if self.gated else None,
            max_backup=R,
        )

    @staticmethod
    def _hy_struct(hy) -> SffnHybrid:
        p = lambda k: None if hy[k] is None else hy[k].data_ptr()
        return SffnHybrid(p("ell_a"), p("ell_u"), p("ell_idx"), p("ell_cnt"), p("slot"),
                          p("brow"), p("n_backup"), p("bk_a"), p("bk_u"), hy["max_backup"])

    def hybrid_compact(self, tw: Dict[str, torch.Tensor], T: int,
                       hy: Optional[Dict[str, torch.Tensor]] = None,
                       z: Optional[torch.Tensor] = None, max_backup: Optional[int] = None):
        hy = hy if hy is not None else self.new_hybrid(T, max_backup)
        ws, n = self.workspace(T, SFFN_OP_HYBRID)
        ts, hs = self._tw_struct(tw), self._hy_struct(hy)
        self._check(self.lib.sffn_hybrid_compact(self.h, ctypes.byref(ts), _ptr(z), T,
                                                 ctypes.byref(hs), ws, n, _stream()),
                    "sffn_hybrid_compact")
        return hy

    def forward_train(self, x, w_gate, w_up, w_down, hy=None, tw=None, y=None,
                      max_backup: Optional[int] = None, check: bool = True):
        """Training forward; returns (y, Hybrid). With ``check`` a capacity
        report (more backup rows than max_backup or dense_rows) rebuilds the
        handle with a T-row capacity, gives a caller-less Hybrid T backup
        rows, and repeats the call; a caller's Hybrid that is too small
        raises SffnError(SFFN_E_CAPACITY)."""
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.d), dtype=torch.float32, device=x.device)
        own = hy is None
        hy = hy if hy is not None else self.new_hybrid(T, max_backup, x.device)
        while True:
            ws, n = self.workspace(T, SFFN_OP_FORWARD_TRAIN, x.device)
            ts = ctypes.byref(self._tw_struct(tw)) if tw is not None else None
            hs = self._hy_struct(hy)
            self._check(self.lib.sffn_forward_train(self.h, _ptr(x), _ptr(w_gate), _ptr(w_up),
                                                    _ptr(w_down), T, _ptr(y), ts,
                                                    ctypes.byref(hs), ws, n, _stream()),
                        "sffn_forward_train")
            if not check or self._capacity_ok():
                return y, hy
            if not own and hy["max_backup"] < T:
                self._check(SFFN_E_CAPACITY, "sffn_forward_train: the Hybrid's max_backup")
            if not self._grow() and not own:
                self._check(SFFN_E_CAPACITY, "sffn_forward_train")
            if own:
                hy = self.new_hybrid(T, T, x.device)

    def backward(self, x, w_gate, w_up, w_down, hy, dy, l1_coeff: float = 0.0, out=None):
        """Gradients (dx [T, d], dw_gate, dw_up, dw_down [F, d]; float32) of
        the step whose Hybrid ``hy`` sffn_forward_train saved. ``out`` may
        pass the four output tensors (dw_up None when non-gated) to reuse."""
        T = x.shape[0]
        f32 = dict(dtype=torch.float32, device=x.device)
        if out is not None:
            dx, dwg, dwu, dwd = out
        else:
            dx = torch.empty((T, self.d), **f32)
            dwg = torch.empty((self.d_ff, self.d), **f32)
            dwu = torch.empty((self.d_ff, self.d), **f32) if self.gated else None
            dwd = torch.empty((self.d_ff, self.d), **f32)
        ws, n = self.workspace(T, SFFN_OP_BACKWARD, x.device)
        hs = self._hy_struct(hy)
        self._check(self.lib.sffn_backward(self.h, _ptr(x), _ptr(w_gate), _ptr(w_up),
                                           _ptr(w_down), ctypes.byref(hs), _ptr(dy), T,
                                           _ptr(dx), _ptr(dwg), _ptr(dwu), _ptr(dwd),
                                           float(l1_coeff), ws, n, _stream()), "sffn_backward")
        return dx, dwg, dwu, dwd

    # ------------------------------------------------------------ dense training

    def forward_train_dense(self, x, w_gate, w_up, w_down, y=None, act=None):
        """The same library's dense bf16 training forward; returns (y, act)
        with act the saved bf16 activations (Z_s, U_s, H^T)."""
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.d), dtype=torch.float32, device=x.device)
        if act is None:
            n = ctypes.c_size_t()
            self._check(self.lib.sffn_train_dense_act_bytes(self.h, T, ctypes.byref(n)),
                        "sffn_train_dense_act_bytes")
            act = torch.empty(n.value // 2, dtype=torch.bfloat16, device=x.device)
        ws, nb = self.workspace(T, SFFN_OP_TRAIN_DENSE, x.device)
        self._check(self.lib.sffn_forward_train_dense(self.h, _ptr(x), _ptr(w_gate), _ptr(w_up),
                                                      _ptr(w_down), T, _ptr(y), _ptr(act), ws,
                                                      nb, _stream()), "sffn_forward_train_dense")
        return y, act

    def backward_dense(self, x, w_gate, w_up, w_down, act, dy, l1_coeff: float = 0.0,
                       out=None):
        """Gradients of the dense training step (dx, dw_gate, dw_up, dw_down)."""
        T = x.shape[0]
        f32 = dict(dtype=torch.float32, device=x.device)
        if out is not None:
            dx, dwg, dwu, dwd = out
        else:
            dx = torch.empty((T, self.d), **f32)
            dwg = torch.empty((self.d_ff, self.d), **f32)
            dwu = torch.empty((self.d_ff, self.d), **f32) if self.gated else None
            dwd = torch.empty((self.d_ff, self.d), **f32)
        ws, nb = self.workspace(T, SFFN_OP_BACKWARD_DENSE, x.device)
        self._check(self.lib.sffn_backward_dense(self.h, _ptr(x), _ptr(w_gate), _ptr(w_up),
                                                 _ptr(w_down), _ptr(act), _ptr(dy), T, _ptr(dx),
                                                 _ptr(dwg), _ptr(dwu), _ptr(dwd),
                                                 float(l1_coeff), ws, nb, _stream()),
                    "sffn_backward_dense")
        return dx, dwg, dwu, dwd

    def hybrid_check(self, hy) -> int:
        """SFFN_OK, or SFFN_E_CAPACITY when the backup rows exceed capacity."""
        hs = self._hy_struct(hy)
        return self.lib.sffn_hybrid_check(self.h, ctypes.byref(hs), _stream())

    def profile(self, enable: bool = True):
        """Bracket every kernel launch with HIP events on the call's stream."""
        self._check(self.lib.sffn_profile_enable(self.h, int(enable)), "sffn_profile_enable")

    def profile_read(self) -> Dict[str, tuple]:
        """{kernel name: (total ms, launches)} since the last read."""
        n = SFFN_K_COUNT
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int32 * n)()
        self._check(self.lib.sffn_profile_read(self.h, ms, cnt, n), "sffn_profile_read")
        return {self.lib.sffn_kernel_name(k).decode(): (ms[k], cnt[k])
                for k in range(n) if cnt[k]}

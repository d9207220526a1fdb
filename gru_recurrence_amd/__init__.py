"""gru_recurrence_amd -- Python binding of librnn355 (multi-head LSTM / GRU
recurrence with block-diagonal R on MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``librnn355.so`` behind the C ABI declared in ``include/rnn355.h``.  torch
supplies device memory (inputs, outputs, workspace) and the current stream.
There is no fallback: if the library is missing, ``load()`` raises.

Shapes (H = NH*Dh, G = 4 for the LSTM, 3 for the GRU, N = NH*G*Dh):
  x [T,B,Din], W [Din,N], R [NH,Dh,G*Dh] in torch.bfloat16 or torch.float32,
  b [N] float32, h0/c0 [B,H] float32; outputs float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librnn355.so")

RNN_OK, RNN_ERR_INVALID_ARG, RNN_ERR_UNSUPPORTED, RNN_ERR_WORKSPACE, RNN_ERR_HIP, \
    RNN_ERR_BARRIER_TIMEOUT = range(6)
RNN_F32, RNN_BF16 = 0, 1
OP_FWD_LSTM, OP_FWD_GRU, OP_BWD_LSTM, OP_BWD_GRU, OP_REC_LSTM, OP_REC_GRU = range(6)

EXPORTS = ("rnn_status_str", "rnn_workspace_size", "rnn_plan_describe", "rnn_input_proj",
           "rnn_input_proj_t",
           "rnn_rec_lstm", "rnn_rec_lstm_noalloc", "rnn_rec_gru", "rnn_fwd_lstm", "rnn_fwd_gru", "rnn_bwd_lstm",
           "rnn_bwd_gru", "rnn_workspace_size_stack", "rnn_fwd_lstm_stack", "rnn_fwd_gru_stack",
           "rnn_workspace_size_chunked", "rnn_fwd_lstm_chunked", "rnn_fwd_gru_chunked",
           "rnn_bwd_lstm_ckpt", "rnn_bwd_gru_ckpt", "rnn_plan_search", "rnn_workspace_status")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("B", ctypes.c_int), ("Din", ctypes.c_int),
                ("NH", ctypes.c_int), ("Dh", ctypes.c_int)]


class PlanCandidate(ctypes.Structure):
    """One assignment of the recurrence plan's variables (rnn_plan_candidate)."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "family", "rows_per_wg", "wg_per_head", "blocks_per_wg", "k_splits",
        "kchunks_per_wave", "row_slots", "frags_agpr", "frags_vgpr", "frags_lds", "waves",
        "grid", "r_vgpr", "wg_per_cu", "xcd_local")] + [("lds_bytes", ctypes.c_longlong),
                                                          ("feasible", ctypes.c_int),
                              ("violated", ctypes.c_int), ("ns_per_step", ctypes.c_double),
                              ("ns_total", ctypes.c_double)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class RnnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s" % (what, status_str(status)))


_lib = None


def load(path: Optional[str] = None):
    """Load librnn355.so (built in-tree by gru_recurrence_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError("librnn355.so not built at %s: run "
                          "`python -m gru_recurrence_amd.build`" % p)
    lib = ctypes.CDLL(p)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    lib.rnn_status_str.restype = ctypes.c_char_p
    lib.rnn_status_str.argtypes = [I]
    lib.rnn_workspace_size.restype = S
    lib.rnn_workspace_size.argtypes = [I, D, I]
    lib.rnn_plan_describe.argtypes = [I, D, I, ctypes.c_char_p, S]
    lib.rnn_input_proj.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.rnn_input_proj_t.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.rnn_rec_lstm.argtypes = [D, I, P, P, P, P, P, P, P, P, P, S, P]
    lib.rnn_rec_gru.argtypes = [D, I, P, P, P, P, P, P, S, P]
    lib.rnn_rec_lstm_noalloc.argtypes = [D, I, P, P, P, P, P, P, P, P, P, P]
    lib.rnn_fwd_lstm.argtypes = [D, I, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.rnn_fwd_gru.argtypes = [D, I, P, P, P, P, P, P, P, P, S, P]
    lib.rnn_bwd_lstm.argtypes = [D, I] + [P] * 17 + [P, S, P]
    lib.rnn_bwd_gru.argtypes = [D, I] + [P] * 13 + [P, S, P]
    lib.rnn_workspace_status.argtypes = [P, S, P]
    lib.rnn_workspace_size_stack.restype = S
    lib.rnn_workspace_size_stack.argtypes = [I, D, I, I]
    lib.rnn_fwd_lstm_stack.argtypes = [D, I, I, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.rnn_fwd_gru_stack.argtypes = [D, I, I, P, P, P, P, P, P, P, P, S, P]
    lib.rnn_workspace_size_chunked.restype = S
    lib.rnn_workspace_size_chunked.argtypes = [I, D, I, I]
    lib.rnn_fwd_lstm_chunked.argtypes = [D, I, I] + [P] * 13 + [S, P]
    lib.rnn_fwd_gru_chunked.argtypes = [D, I, I] + [P] * 9 + [S, P]
    lib.rnn_bwd_lstm_ckpt.argtypes = [D, I, I] + [P] * 18 + [S, P]
    lib.rnn_bwd_gru_ckpt.argtypes = [D, I, I] + [P] * 14 + [S, P]
    lib.rnn_plan_search.argtypes = [I, D, I, I, ctypes.POINTER(PlanCandidate), I,
                                    ctypes.POINTER(I), ctypes.POINTER(I)]
    for f in ("rnn_plan_describe", "rnn_input_proj", "rnn_input_proj_t", "rnn_rec_lstm", "rnn_rec_gru",
              "rnn_fwd_lstm", "rnn_fwd_gru", "rnn_bwd_lstm", "rnn_bwd_gru",
              "rnn_fwd_lstm_stack", "rnn_fwd_gru_stack", "rnn_fwd_lstm_chunked",
              "rnn_fwd_gru_chunked", "rnn_bwd_lstm_ckpt", "rnn_bwd_gru_ckpt",
              "rnn_plan_search", "rnn_workspace_status"):
        getattr(lib, f).restype = I
    _lib = lib
    return lib


def status_str(s: int) -> str:
    return load().rnn_status_str(int(s)).decode()


def _check(s: int, what: str):
    if s != RNN_OK:
        raise RnnError(s, what)


# ----------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RNN_BF16
    if t.dtype == torch.float32:
        return RNN_F32
    raise TypeError("x/W/R must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t, name, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    torch = _torch()
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    del torch
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dims_of(x, R) -> Dims:
    T, B, Din = x.shape
    NH, Dh = R.shape[0], R.shape[1]
    return Dims(T, B, Din, NH, Dh)


def workspace_size(op: int, dims: Dims, dtype_code: int) -> int:
    return int(load().rnn_workspace_size(op, ctypes.byref(dims), dtype_code))


def plan_describe(op: int, dims: Dims, dtype_code: int) -> str:
    buf = ctypes.create_string_buffer(256)
    s = load().rnn_plan_describe(op, ctypes.byref(dims), dtype_code, buf, 256)
    _check(s, "rnn_plan_describe")
    return buf.value.decode()


def _workspace(op, d, dt, device, ws=None):
    torch = _torch()
    need = workspace_size(op, d, dt)
    if need == 0:
        raise RnnError(RNN_ERR_UNSUPPORTED, "rnn_workspace_size")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws


def _common(x, W, R, G):
    torch = _torch()
    dt = _dtype_code(x)
    tdt = x.dtype
    d = dims_of(x, R)
    N = d.NH * G * d.Dh
    _ptr(x, "x", tdt)
    _ptr(W, "W", tdt, (d.Din, N))
    _ptr(R, "R", tdt, (d.NH, d.Dh, G * d.Dh))
    del torch
    return d, dt, N


def input_proj(x, W, b=None, out=None, stream=None):
    """gx = x W + b over all T*B rows (float32 [T,B,N])."""
    torch = _torch()
    T, B, Din = x.shape
    N = W.shape[1]
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty((T, B, N), dtype=torch.float32, device=x.device)
    s = load().rnn_input_proj(T * B, Din, N, dt, _ptr(x, "x", x.dtype), _ptr(W, "W", x.dtype),
                              _ptr(b, "b", torch.float32, (N,), optional=True),
                              _ptr(out, "gx", torch.float32, (T, B, N)), _stream(stream))
    _check(s, "rnn_input_proj")
    return out


def input_proj_t(x, Wt, b=None, out=None, stream=None):
    """gx = x Wt^T + b with the weights given transposed, Wt [N, Din] (bf16,
    Din % 32 == 0): the fused forward's contraction (float32 [T,B,N])."""
    torch = _torch()
    T, B, Din = x.shape
    N = Wt.shape[0]
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty((T, B, N), dtype=torch.float32, device=x.device)
    s = load().rnn_input_proj_t(T * B, Din, N, dt, _ptr(x, "x", x.dtype),
                                _ptr(Wt, "Wt", x.dtype, (N, Din)),
                                _ptr(b, "b", torch.float32, (N,), optional=True),
                                _ptr(out, "gx", torch.float32, (T, B, N)), _stream(stream))
    _check(s, "rnn_input_proj_t")
    return out


def lstm_fwd(x, W, R, b=None, h0=None, c0=None, *, with_seq: bool = True, ws=None,
             out=None, stream=None):
    """Multi-head LSTM forward.  Returns (h_seq, c_seq, hT, cT); the
    sequences are None when with_seq is False."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 4)
    H = d.NH * d.Dh
    dev = x.device
    f32 = torch.float32
    if out is None:
        out = {}
    h_seq = out.get("h_seq") if with_seq else None
    c_seq = out.get("c_seq") if with_seq else None
    if with_seq and h_seq is None:
        h_seq = torch.empty((d.T, d.B, H), dtype=f32, device=dev)
    if with_seq and c_seq is None:
        c_seq = torch.empty((d.T, d.B, H), dtype=f32, device=dev)
    hT = out.get("hT")
    cT = out.get("cT")
    hT = torch.empty((d.B, H), dtype=f32, device=dev) if hT is None else hT
    cT = torch.empty((d.B, H), dtype=f32, device=dev) if cT is None else cT
    ws = _workspace(OP_FWD_LSTM, d, dt, dev, ws)
    s = load().rnn_fwd_lstm(ctypes.byref(d), dt, _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
                            _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
                            _ptr(c0, "c0", f32, (d.B, H), True),
                            _ptr(h_seq, "h_seq", f32, None, True),
                            _ptr(c_seq, "c_seq", f32, None, True),
                            _ptr(hT, "hT", f32), _ptr(cT, "cT", f32),
                            _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_fwd_lstm")
    return h_seq, c_seq, hT, cT


def gru_fwd(x, W, R, b=None, h0=None, *, with_seq: bool = True, ws=None, out=None,
            stream=None):
    """Multi-head GRU forward (reset-after).  Returns (h_seq, hT)."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 3)
    H = d.NH * d.Dh
    dev = x.device
    f32 = torch.float32
    if out is None:
        out = {}
    h_seq = out.get("h_seq") if with_seq else None
    if with_seq and h_seq is None:
        h_seq = torch.empty((d.T, d.B, H), dtype=f32, device=dev)
    hT = out.get("hT")
    hT = torch.empty((d.B, H), dtype=f32, device=dev) if hT is None else hT
    ws = _workspace(OP_FWD_GRU, d, dt, dev, ws)
    s = load().rnn_fwd_gru(ctypes.byref(d), dt, _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
                           _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
                           _ptr(h_seq, "h_seq", f32, None, True), _ptr(hT, "hT", f32),
                           _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_fwd_gru")
    return h_seq, hT


def workspace_size_stack(op: int, dims: Dims, L: int, dtype_code: int) -> int:
    return int(load().rnn_workspace_size_stack(op, ctypes.byref(dims), int(L), dtype_code))


def _stack(cell, x, Ws, Rs, bs, h0, c0, with_seq, ws, out, stream):
    torch = _torch()
    L = len(Ws)
    if len(Rs) != L or (bs is not None and len(bs) != L):
        raise ValueError("Ws, Rs and bs need one entry per layer")
    G = 4 if cell == "lstm" else 3
    d, dt, N = _common(x, Ws[0], Rs[0], G)
    H = d.NH * d.Dh
    f32 = torch.float32
    dev = x.device
    for layer in range(1, L):
        if tuple(Ws[layer].shape) != (H, N) or Ws[layer].dtype != Ws[0].dtype:
            raise ValueError("W[%d] must be [%d, %d] %s" % (layer, H, N, Ws[0].dtype))
        if tuple(Rs[layer].shape) != tuple(Rs[0].shape) or Rs[layer].dtype != Rs[0].dtype:
            raise ValueError("R[%d] must match R[0]" % layer)
    P = ctypes.c_void_p
    Wp = (P * L)(*[_ptr(w, "W[%d]" % i) for i, w in enumerate(Ws)])
    Rp = (P * L)(*[_ptr(r, "R[%d]" % i) for i, r in enumerate(Rs)])
    bp = None if bs is None else (P * L)(*[_ptr(v, "b[%d]" % i, f32, (N,), True)
                                          for i, v in enumerate(bs)])
    out = {} if out is None else out
    h_seq = out.get("h_seq") if with_seq else None
    if with_seq and h_seq is None:
        h_seq = torch.empty((d.T, d.B, H), dtype=f32, device=dev)
    hT = out.get("hT")
    hT = torch.empty((L, d.B, H), dtype=f32, device=dev) if hT is None else hT
    op = OP_FWD_LSTM if cell == "lstm" else OP_FWD_GRU
    need = workspace_size_stack(op, d, L, dt)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if cell == "lstm":
        c_seq = out.get("c_seq") if with_seq else None
        if with_seq and c_seq is None:
            c_seq = torch.empty((d.T, d.B, H), dtype=f32, device=dev)
        cT = out.get("cT")
        cT = torch.empty((L, d.B, H), dtype=f32, device=dev) if cT is None else cT
        s = load().rnn_fwd_lstm_stack(ctypes.byref(d), L, dt, _ptr(x, "x"), Wp, Rp, bp,
                                      _ptr(h0, "h0", f32, (L, d.B, H), True),
                                      _ptr(c0, "c0", f32, (L, d.B, H), True),
                                      _ptr(h_seq, "h_seq", f32, None, True),
                                      _ptr(c_seq, "c_seq", f32, None, True),
                                      _ptr(hT, "hT", f32, (L, d.B, H)),
                                      _ptr(cT, "cT", f32, (L, d.B, H)),
                                      _ptr(ws, "ws"), ws.numel(), _stream(stream))
        _check(s, "rnn_fwd_lstm_stack")
        return h_seq, c_seq, hT, cT
    s = load().rnn_fwd_gru_stack(ctypes.byref(d), L, dt, _ptr(x, "x"), Wp, Rp, bp,
                                 _ptr(h0, "h0", f32, (L, d.B, H), True),
                                 _ptr(h_seq, "h_seq", f32, None, True),
                                 _ptr(hT, "hT", f32, (L, d.B, H)),
                                 _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_fwd_gru_stack")
    return h_seq, hT


def lstm_stack_fwd(x, Ws, Rs, bs=None, h0=None, c0=None, *, with_seq: bool = True, ws=None,
                   out=None, stream=None):
    """Stacked multi-head LSTM: Ws, Rs, bs are per-layer lists (Ws[0] [Din,N],
    Ws[l>0] [H,N]); h0, c0 [L,B,H].  Returns (h_seq, c_seq) of the last layer
    and hT, cT [L,B,H] of every layer."""
    return _stack("lstm", x, Ws, Rs, bs, h0, c0, with_seq, ws, out, stream)


def gru_stack_fwd(x, Ws, Rs, bs=None, h0=None, *, with_seq: bool = True, ws=None, out=None,
                  stream=None):
    """Stacked multi-head GRU.  Returns (h_seq of the last layer, hT [L,B,H])."""
    return _stack("gru", x, Ws, Rs, bs, h0, None, with_seq, ws, out, stream)


def rec_lstm(gx, R, h0=None, c0=None, *, with_seq=True, ws=None, out=None, stream=None):
    """The LSTM recurrence alone on a precomputed gx [T,B,N]."""
    torch = _torch()
    T, B, N = gx.shape
    NH, Dh = R.shape[0], R.shape[1]
    d = Dims(T, B, 1, NH, Dh)
    dt = _dtype_code(R)
    H = NH * Dh
    f32 = torch.float32
    dev = gx.device
    out = out or {}
    h_seq = out.get("h_seq") if with_seq else None
    c_seq = out.get("c_seq") if with_seq else None
    if with_seq and h_seq is None:
        h_seq = torch.empty((T, B, H), dtype=f32, device=dev)
    if with_seq and c_seq is None:
        c_seq = torch.empty((T, B, H), dtype=f32, device=dev)
    hT = out.get("hT") if out.get("hT") is not None else torch.empty((B, H), dtype=f32, device=dev)
    cT = out.get("cT") if out.get("cT") is not None else torch.empty((B, H), dtype=f32, device=dev)
    ws = _workspace(OP_REC_LSTM, d, dt, dev, ws)
    s = load().rnn_rec_lstm(ctypes.byref(d), dt, _ptr(gx, "gx", f32, (T, B, NH * 4 * Dh)),
                            _ptr(R, "R", None, (NH, Dh, 4 * Dh)),
                            _ptr(h0, "h0", f32, (B, H), True), _ptr(c0, "c0", f32, (B, H), True),
                            _ptr(h_seq, "h_seq", f32, None, True),
                            _ptr(c_seq, "c_seq", f32, None, True),
                            _ptr(hT, "hT", f32), _ptr(cT, "cT", f32),
                            _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_rec_lstm")
    return h_seq, c_seq, hT, cT


def rec_lstm_noalloc(gx, R, h0=None, c0=None, *, with_seq=True, out=None, status=None,
                     stream=None):
    """rec_lstm through rnn_rec_lstm_noalloc: no workspace (the library's
    own device scratch).  Outputs are allocated here unless given in `out`;
    `status` (a 4-byte int32 device tensor) receives the device status word."""
    torch = _torch()
    T, B, N = gx.shape
    NH, Dh = R.shape[0], R.shape[1]
    d = Dims(T, B, 1, NH, Dh)
    dt = _dtype_code(R)
    H = NH * Dh
    f32 = torch.float32
    dev = gx.device
    out = out or {}
    h_seq = out.get("h_seq") if with_seq else None
    c_seq = out.get("c_seq") if with_seq else None
    if with_seq and h_seq is None:
        h_seq = torch.empty((T, B, H), dtype=f32, device=dev)
    if with_seq and c_seq is None:
        c_seq = torch.empty((T, B, H), dtype=f32, device=dev)
    hT = out.get("hT") if out.get("hT") is not None else torch.empty((B, H), dtype=f32, device=dev)
    cT = out.get("cT") if out.get("cT") is not None else torch.empty((B, H), dtype=f32, device=dev)
    s = load().rnn_rec_lstm_noalloc(ctypes.byref(d), dt,
                                    _ptr(gx, "gx", f32, (T, B, NH * 4 * Dh)),
                                    _ptr(R, "R", None, (NH, Dh, 4 * Dh)),
                                    _ptr(h0, "h0", f32, (B, H), True),
                                    _ptr(c0, "c0", f32, (B, H), True),
                                    _ptr(h_seq, "h_seq", f32, None, True),
                                    _ptr(c_seq, "c_seq", f32, None, True),
                                    _ptr(hT, "hT", f32), _ptr(cT, "cT", f32),
                                    _ptr(status, "status", torch.int32, (1,), True),
                                    _stream(stream))
    _check(s, "rnn_rec_lstm_noalloc")
    return h_seq, c_seq, hT, cT


def rec_gru(gx, R, h0=None, *, with_seq=True, ws=None, out=None, stream=None):
    """The GRU recurrence alone on a precomputed gx [T,B,N]."""
    torch = _torch()
    T, B, N = gx.shape
    NH, Dh = R.shape[0], R.shape[1]
    d = Dims(T, B, 1, NH, Dh)
    dt = _dtype_code(R)
    H = NH * Dh
    f32 = torch.float32
    dev = gx.device
    out = out or {}
    h_seq = out.get("h_seq") if with_seq else None
    if with_seq and h_seq is None:
        h_seq = torch.empty((T, B, H), dtype=f32, device=dev)
    hT = out.get("hT") if out.get("hT") is not None else torch.empty((B, H), dtype=f32, device=dev)
    ws = _workspace(OP_REC_GRU, d, dt, dev, ws)
    s = load().rnn_rec_gru(ctypes.byref(d), dt, _ptr(gx, "gx", f32, (T, B, NH * 3 * Dh)),
                           _ptr(R, "R", None, (NH, Dh, 3 * Dh)),
                           _ptr(h0, "h0", f32, (B, H), True),
                           _ptr(h_seq, "h_seq", f32, None, True), _ptr(hT, "hT", f32),
                           _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_rec_gru")
    return h_seq, hT


def lstm_bwd(x, W, R, b, h0, c0, h_seq, c_seq, dh_seq, dhT=None, dcT=None, *, ws=None,
             out=None, stream=None):
    """Multi-head LSTM BPTT.  Returns dict dx, dW, dR, db, dh0, dc0 (taken
    from ``out`` where given, else allocated)."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 4)
    H = d.NH * d.Dh
    dev = x.device
    f32 = torch.float32
    shapes = dict(dx=(d.T, d.B, d.Din), dW=(d.Din, N), dR=(d.NH, d.Dh, 4 * d.Dh), db=(N,),
                  dh0=(d.B, H), dc0=(d.B, H))
    out = out or {}
    g = {k: out[k] if out.get(k) is not None else torch.empty(v, dtype=f32, device=dev)
         for k, v in shapes.items()}
    ws = _workspace(OP_BWD_LSTM, d, dt, dev, ws)
    seq = (d.T, d.B, H)
    s = load().rnn_bwd_lstm(ctypes.byref(d), dt, _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
                            _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
                            _ptr(c0, "c0", f32, (d.B, H), True),
                            _ptr(h_seq, "h_seq", f32, seq), _ptr(c_seq, "c_seq", f32, seq),
                            _ptr(dh_seq, "dh_seq", f32, seq),
                            _ptr(dhT, "dhT", f32, (d.B, H), True),
                            _ptr(dcT, "dcT", f32, (d.B, H), True),
                            _ptr(g["dx"], "dx", f32, shapes["dx"]), _ptr(g["dW"], "dW", f32, shapes["dW"]),
                            _ptr(g["dR"], "dR", f32, shapes["dR"]), _ptr(g["db"], "db", f32, shapes["db"]),
                            _ptr(g["dh0"], "dh0", f32, shapes["dh0"]),
                            _ptr(g["dc0"], "dc0", f32, shapes["dc0"]),
                            _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_bwd_lstm")
    return g


def gru_bwd(x, W, R, b, h0, h_seq, dh_seq, dhT=None, *, ws=None, out=None, stream=None):
    """Multi-head GRU BPTT.  Returns dict dx, dW, dR, db, dh0 (taken from
    ``out`` where given, else allocated)."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 3)
    H = d.NH * d.Dh
    dev = x.device
    f32 = torch.float32
    shapes = dict(dx=(d.T, d.B, d.Din), dW=(d.Din, N), dR=(d.NH, d.Dh, 3 * d.Dh), db=(N,),
                  dh0=(d.B, H))
    out = out or {}
    g = {k: out[k] if out.get(k) is not None else torch.empty(v, dtype=f32, device=dev)
         for k, v in shapes.items()}
    ws = _workspace(OP_BWD_GRU, d, dt, dev, ws)
    seq = (d.T, d.B, H)
    s = load().rnn_bwd_gru(ctypes.byref(d), dt, _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
                           _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
                           _ptr(h_seq, "h_seq", f32, seq), _ptr(dh_seq, "dh_seq", f32, seq),
                           _ptr(dhT, "dhT", f32, (d.B, H), True),
                           _ptr(g["dx"], "dx", f32, shapes["dx"]), _ptr(g["dW"], "dW", f32, shapes["dW"]),
                           _ptr(g["dR"], "dR", f32, shapes["dR"]), _ptr(g["db"], "db", f32, shapes["db"]),
                           _ptr(g["dh0"], "dh0", f32, shapes["dh0"]),
                           _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_bwd_gru")
    return g


def plan_search(op: int, dims: Dims, dtype_code: int, num_cu: int = 0):
    """Every candidate plan of the recurrence (list of dicts) and the index
    of the chosen one (-1 if none is feasible)."""
    buf = (PlanCandidate * 512)()
    n, best = ctypes.c_int(0), ctypes.c_int(-1)
    s = load().rnn_plan_search(op, ctypes.byref(dims), dtype_code, int(num_cu), buf, 512,
                               ctypes.byref(n), ctypes.byref(best))
    if s not in (RNN_OK, RNN_ERR_UNSUPPORTED):
        _check(s, "rnn_plan_search")
    return [buf[i].as_dict() for i in range(n.value)], best.value


def workspace_size_chunked(op: int, dims: Dims, chunk: int, dtype_code: int) -> int:
    return int(load().rnn_workspace_size_chunked(op, ctypes.byref(dims), int(chunk), dtype_code))


def _chunk_ws(op, d, chunk, dt, dev, ws):
    torch = _torch()
    need = workspace_size_chunked(op, d, chunk, dt)
    if need == 0:
        raise RnnError(RNN_ERR_INVALID_ARG, "rnn_workspace_size_chunked")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    return ws


def lstm_fwd_chunked(x, W, R, b=None, h0=None, c0=None, *, chunk: int, with_seq: bool = True,
                     ckpt: bool = True, ws=None, out=None, stream=None):
    """The LSTM forward in chunks of `chunk` steps (workspace independent of
    T).  Returns (h_seq, c_seq, hT, cT, h_ckpt, c_ckpt); the checkpoints are
    [ceil(T/chunk), B, H] (None unless ckpt)."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 4)
    H = d.NH * d.Dh
    dev, f32 = x.device, torch.float32
    out = out or {}
    nck = (d.T + chunk - 1) // chunk

    def get(k, shape, want=True):
        if not want:
            return None
        v = out.get(k)
        return torch.empty(shape, dtype=f32, device=dev) if v is None else v
    h_seq, c_seq = get("h_seq", (d.T, d.B, H), with_seq), get("c_seq", (d.T, d.B, H), with_seq)
    hT, cT = get("hT", (d.B, H)), get("cT", (d.B, H))
    h_ck, c_ck = get("h_ckpt", (nck, d.B, H), ckpt), get("c_ckpt", (nck, d.B, H), ckpt)
    ws = _chunk_ws(OP_FWD_LSTM, d, chunk, dt, dev, ws)
    s = load().rnn_fwd_lstm_chunked(
        ctypes.byref(d), dt, int(chunk), _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
        _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
        _ptr(c0, "c0", f32, (d.B, H), True), _ptr(h_seq, "h_seq", f32, None, True),
        _ptr(c_seq, "c_seq", f32, None, True), _ptr(hT, "hT", f32, (d.B, H)),
        _ptr(cT, "cT", f32, (d.B, H)), _ptr(h_ck, "h_ckpt", f32, (nck, d.B, H), True),
        _ptr(c_ck, "c_ckpt", f32, (nck, d.B, H), True), _ptr(ws, "ws"), ws.numel(),
        _stream(stream))
    _check(s, "rnn_fwd_lstm_chunked")
    return h_seq, c_seq, hT, cT, h_ck, c_ck


def gru_fwd_chunked(x, W, R, b=None, h0=None, *, chunk: int, with_seq: bool = True,
                    ckpt: bool = True, ws=None, out=None, stream=None):
    """The GRU forward in chunks.  Returns (h_seq, hT, h_ckpt)."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 3)
    H = d.NH * d.Dh
    dev, f32 = x.device, torch.float32
    out = out or {}
    nck = (d.T + chunk - 1) // chunk

    def get(k, shape, want=True):
        if not want:
            return None
        v = out.get(k)
        return torch.empty(shape, dtype=f32, device=dev) if v is None else v
    h_seq, hT = get("h_seq", (d.T, d.B, H), with_seq), get("hT", (d.B, H))
    h_ck = get("h_ckpt", (nck, d.B, H), ckpt)
    ws = _chunk_ws(OP_FWD_GRU, d, chunk, dt, dev, ws)
    s = load().rnn_fwd_gru_chunked(
        ctypes.byref(d), dt, int(chunk), _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
        _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
        _ptr(h_seq, "h_seq", f32, None, True), _ptr(hT, "hT", f32, (d.B, H)),
        _ptr(h_ck, "h_ckpt", f32, (nck, d.B, H), True), _ptr(ws, "ws"), ws.numel(),
        _stream(stream))
    _check(s, "rnn_fwd_gru_chunked")
    return h_seq, hT, h_ck


def lstm_bwd_ckpt(x, W, R, b, h0, c0, h_ckpt, c_ckpt, dh_seq, dhT=None, dcT=None, *,
                  chunk: int, ws=None, out=None, stream=None):
    """LSTM BPTT from the checkpoints of lstm_fwd_chunked (same chunk).
    Returns dict dx, dW, dR, db, dh0, dc0."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 4)
    H = d.NH * d.Dh
    dev, f32 = x.device, torch.float32
    nck = (d.T + chunk - 1) // chunk
    shapes = dict(dx=(d.T, d.B, d.Din), dW=(d.Din, N), dR=(d.NH, d.Dh, 4 * d.Dh), db=(N,),
                  dh0=(d.B, H), dc0=(d.B, H))
    out = out or {}
    g = {k: out[k] if out.get(k) is not None else torch.empty(v, dtype=f32, device=dev)
         for k, v in shapes.items()}
    ws = _chunk_ws(OP_BWD_LSTM, d, chunk, dt, dev, ws)
    s = load().rnn_bwd_lstm_ckpt(
        ctypes.byref(d), dt, int(chunk), _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
        _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
        _ptr(c0, "c0", f32, (d.B, H), True), _ptr(h_ckpt, "h_ckpt", f32, (nck, d.B, H), True),
        _ptr(c_ckpt, "c_ckpt", f32, (nck, d.B, H), True),
        _ptr(dh_seq, "dh_seq", f32, (d.T, d.B, H)), _ptr(dhT, "dhT", f32, (d.B, H), True),
        _ptr(dcT, "dcT", f32, (d.B, H), True),
        *[_ptr(g[k], k, f32, shapes[k]) for k in ("dx", "dW", "dR", "db", "dh0", "dc0")],
        _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_bwd_lstm_ckpt")
    return g


def gru_bwd_ckpt(x, W, R, b, h0, h_ckpt, dh_seq, dhT=None, *, chunk: int, ws=None, out=None,
                 stream=None):
    """GRU BPTT from the checkpoints of gru_fwd_chunked (same chunk).
    Returns dict dx, dW, dR, db, dh0."""
    torch = _torch()
    d, dt, N = _common(x, W, R, 3)
    H = d.NH * d.Dh
    dev, f32 = x.device, torch.float32
    nck = (d.T + chunk - 1) // chunk
    shapes = dict(dx=(d.T, d.B, d.Din), dW=(d.Din, N), dR=(d.NH, d.Dh, 3 * d.Dh), db=(N,),
                  dh0=(d.B, H))
    out = out or {}
    g = {k: out[k] if out.get(k) is not None else torch.empty(v, dtype=f32, device=dev)
         for k, v in shapes.items()}
    ws = _chunk_ws(OP_BWD_GRU, d, chunk, dt, dev, ws)
    s = load().rnn_bwd_gru_ckpt(
        ctypes.byref(d), dt, int(chunk), _ptr(x, "x"), _ptr(W, "W"), _ptr(R, "R"),
        _ptr(b, "b", f32, (N,), True), _ptr(h0, "h0", f32, (d.B, H), True),
        _ptr(h_ckpt, "h_ckpt", f32, (nck, d.B, H), True),
        _ptr(dh_seq, "dh_seq", f32, (d.T, d.B, H)), _ptr(dhT, "dhT", f32, (d.B, H), True),
        *[_ptr(g[k], k, f32, shapes[k]) for k in ("dx", "dW", "dR", "db", "dh0")],
        _ptr(ws, "ws"), ws.numel(), _stream(stream))
    _check(s, "rnn_bwd_gru_ckpt")
    return g


def workspace_status(ws, stream=None) -> int:
    """Synchronise and report a recorded step-wait timeout (RNN_OK if none)."""
    return int(load().rnn_workspace_status(_ptr(ws, "ws"), ws.numel(), _stream(stream)))

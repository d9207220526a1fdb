"""Python face of the CPU oracle (``oracle.c``): plain double-precision
multi-head LSTM / GRU forward and backpropagation through time.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library ``gru_recurrence_amd`` and never imports it.

All arrays are float64 numpy arrays in the layouts stated in ``oracle.c``;
inputs may be any float dtype and are widened exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (OpenMP over chains)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        lib.oracle_num_threads.restype = I
        lib.oracle_lstm_fwd.argtypes = [I] * 5 + [P] * 6 + [P] + [P] * 4
        lib.oracle_gru_fwd.argtypes = [I] * 5 + [P] * 5 + [P] + [P] * 2
        lib.oracle_lstm_bptt.argtypes = [I] * 5 + [P] * 6 + [P] * 3 + [P] + [P] * 4
        lib.oracle_gru_bptt.argtypes = [I] * 5 + [P] * 5 + [P] * 2 + [P] + [P] * 4
        lib.oracle_param_grads.argtypes = [I] * 6 + [P] * 6 + [P] * 4
        lib.oracle_param_grad_entries.argtypes = [I] * 7 + [L, P] + [P] * 6 + [P]
        lib.oracle_input_proj.argtypes = [L, I, I, P, P, P, L, P, P]
        for f in (lib.oracle_input_proj, lib.oracle_lstm_fwd, lib.oracle_gru_fwd, lib.oracle_lstm_bptt,
                  lib.oracle_gru_bptt, lib.oracle_param_grads,
                  lib.oracle_param_grad_entries):
            f.restype = I
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _d(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mask(mask, B, NH):
    if mask is None:
        return None
    m = np.ascontiguousarray(mask, dtype=np.uint8).reshape(B, NH)
    return m


def _nan(shape):
    return np.full(shape, np.nan, dtype=np.float64)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def input_proj(x, W, b=None, rows=None):
    """gx = x W + b for x [M,K] (or [T,B,K], flattened), W [K,N]; optionally
    only at the given flat row indices.  Returns [len(rows) or M, N]."""
    x = _d(x)
    x = x.reshape(-1, x.shape[-1])
    W, b = _d(W), _d(b)
    M, K = x.shape
    N = W.shape[1]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int_)
    out = np.zeros((M if r is None else r.size, N))
    rc = _load().oracle_input_proj(M, K, N, _p(x), _p(W), _p(b), 0 if r is None else r.size,
                                   _p(r), _p(out))
    _check(rc, "input_proj")
    return out


def lstm_fwd(x, W, R, b, h0=None, c0=None, *, NH: int, Dh: int, chain_mask=None):
    """Multi-head LSTM forward.  Returns dict h_seq, c_seq [T,B,H], hT, cT [B,H].
    Chains outside ``chain_mask`` ([B,NH] bool) are left NaN."""
    x, W, R, b, h0, c0 = map(_d, (x, W, R, b, h0, c0))
    T, B, Din = x.shape
    H = NH * Dh
    out = dict(h_seq=_nan((T, B, H)), c_seq=_nan((T, B, H)),
               hT=_nan((B, H)), cT=_nan((B, H)))
    m = _mask(chain_mask, B, NH)
    rc = _load().oracle_lstm_fwd(T, B, Din, NH, Dh, _p(x), _p(W), _p(R), _p(b),
                                 _p(h0), _p(c0), _p(m), _p(out["h_seq"]),
                                 _p(out["c_seq"]), _p(out["hT"]), _p(out["cT"]))
    _check(rc, "lstm_fwd")
    return out


def gru_fwd(x, W, R, b, h0=None, *, NH: int, Dh: int, chain_mask=None):
    """Multi-head GRU forward.  Returns dict h_seq [T,B,H], hT [B,H]."""
    x, W, R, b, h0 = map(_d, (x, W, R, b, h0))
    T, B, Din = x.shape
    H = NH * Dh
    out = dict(h_seq=_nan((T, B, H)), hT=_nan((B, H)))
    m = _mask(chain_mask, B, NH)
    rc = _load().oracle_gru_fwd(T, B, Din, NH, Dh, _p(x), _p(W), _p(R), _p(b),
                                _p(h0), _p(m), _p(out["h_seq"]), _p(out["hT"]))
    _check(rc, "gru_fwd")
    return out


def round_bf16(a):
    """Round to bfloat16 (nearest, ties to even) and widen back to float64:
    first to float32 (numpy rounds to nearest even), then the float32 bit
    pattern to its top 16 bits with the same rule.  NaN is not expected."""
    f = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _stack(cell, x, Ws, Rs, bs, h0s, c0s, NH, Dh, bf16_between, chain_mask):
    L = len(Ws)
    inp = _d(x)
    hT, cT, last = [], [], None
    for layer in range(L):
        h0 = None if h0s is None else h0s[layer]
        if cell == "lstm":
            c0 = None if c0s is None else c0s[layer]
            r = lstm_fwd(inp, Ws[layer], Rs[layer], bs[layer], h0, c0, NH=NH, Dh=Dh,
                         chain_mask=chain_mask)
            cT.append(r["cT"])
        else:
            r = gru_fwd(inp, Ws[layer], Rs[layer], bs[layer], h0, NH=NH, Dh=Dh,
                        chain_mask=chain_mask)
        hT.append(r["hT"])
        last = r
        if layer + 1 < L:
            inp = round_bf16(r["h_seq"]) if bf16_between else r["h_seq"]
    out = dict(h_seq=last["h_seq"], hT=np.stack(hT))
    if cell == "lstm":
        out["c_seq"] = last["c_seq"]
        out["cT"] = np.stack(cT)
    return out


def lstm_stack_fwd(x, Ws, Rs, bs, h0=None, c0=None, *, NH: int, Dh: int,
                   bf16_between: bool = False, chain_mask=None):
    """Stacked multi-head LSTM: layer l > 0 takes layer l-1's sequence h_1..h_T
    as its input (Ws[l] is [NH*Dh][NH*4*Dh]); every layer has its own W, R, b
    and initial state (h0, c0: [L][B][H] or None).  With bf16_between the
    layer input is rounded to bfloat16 as the first layer's x is in a bf16
    run.  Returns the last layer's h_seq, c_seq and every layer's hT, cT
    ([L][B][H]).  A chain_mask must keep whole batch rows (all heads), since a
    layer's input row depends on every head of the layer below.
    Inter-layer parallelism of multi-layer RNNs: blog.hotdry.top 2025-09-21,
    the list of framework-level optimisations, first item."""
    return _stack("lstm", x, Ws, Rs, bs, h0, c0, NH, Dh, bf16_between, chain_mask)


def gru_stack_fwd(x, Ws, Rs, bs, h0=None, *, NH: int, Dh: int, bf16_between: bool = False,
                  chain_mask=None):
    """Stacked multi-head GRU, as lstm_stack_fwd (no cell state)."""
    return _stack("gru", x, Ws, Rs, bs, h0, None, NH, Dh, bf16_between, chain_mask)


def param_grads(x, W, h0, h_seq, dG, dS, *, NH: int, Dh: int, G: int,
                want=("dx", "dW", "dR", "db")):
    """dx, dW, dR, db from the per-step gate gradients (see oracle.c)."""
    x, W, h0, h_seq, dG, dS = map(_d, (x, W, h0, h_seq, dG, dS))
    T, B, Din = x.shape
    N = NH * G * Dh
    res = {}
    res["dx"] = np.zeros((T, B, Din)) if "dx" in want else None
    res["dW"] = np.zeros((Din, N)) if "dW" in want else None
    res["dR"] = np.zeros((NH, Dh, G * Dh)) if "dR" in want else None
    res["db"] = np.zeros((N,)) if "db" in want else None
    rc = _load().oracle_param_grads(T, B, Din, NH, Dh, G, _p(x), _p(W), _p(h0),
                                    _p(h_seq), _p(dG), _p(dS), _p(res["dx"]),
                                    _p(res["dW"]), _p(res["dR"]), _p(res["db"]))
    _check(rc, "param_grads")
    return {k: v for k, v in res.items() if v is not None}


def param_grad_entries(kind: str, idx, x, W, h0, h_seq, dG, dS, *,
                       NH: int, Dh: int, G: int):
    """Entries of db ('db': idx rows (c,)), dW ('dW': (k,c)), dx ('dx': (m,k),
    m = t*B+b) or dR ('dR': (n,mm,c)) without forming the whole gradient."""
    kinds = {"db": 0, "dW": 1, "dx": 2, "dR": 3}
    x, W, h0, h_seq, dG, dS = map(_d, (x, W, h0, h_seq, dG, dS))
    T, B, _ = x.shape
    idx = np.asarray(idx, dtype=np.int64)
    if idx.ndim == 1:
        idx = idx[:, None]
    full = np.zeros((idx.shape[0], 3), dtype=np.int64)
    full[:, :idx.shape[1]] = idx
    full = np.ascontiguousarray(full).astype(np.int_)
    out = np.zeros(idx.shape[0])
    rc = _load().oracle_param_grad_entries(T, B, x.shape[2], NH, Dh, G, kinds[kind],
                                           idx.shape[0], _p(full), _p(x), _p(W),
                                           _p(h0), _p(h_seq), _p(dG), _p(dS), _p(out))
    _check(rc, "param_grad_entries")
    return out


def lstm_bwd(x, W, R, b, h0, c0, dh_seq, dhT=None, dcT=None, *, NH: int, Dh: int,
             chain_mask=None, grads=("dx", "dW", "dR", "db")):
    """LSTM BPTT.  Returns dict dA [T,B,N], dh0, dc0 [B,H], h_seq (the
    oracle's own forward) and the parameter gradients named in ``grads``."""
    x, W, R, b, h0, c0, dh_seq, dhT, dcT = map(_d, (x, W, R, b, h0, c0, dh_seq, dhT, dcT))
    T, B, Din = x.shape
    H, N = NH * Dh, NH * 4 * Dh
    dA = np.zeros((T, B, N))
    dh0, dc0 = _nan((B, H)), _nan((B, H))
    h_seq = _nan((T, B, H))
    m = _mask(chain_mask, B, NH)
    rc = _load().oracle_lstm_bptt(T, B, Din, NH, Dh, _p(x), _p(W), _p(R), _p(b),
                                  _p(h0), _p(c0), _p(dh_seq), _p(dhT), _p(dcT), _p(m),
                                  _p(dA), _p(dh0), _p(dc0), _p(h_seq))
    _check(rc, "lstm_bptt")
    out = dict(dA=dA, dh0=dh0, dc0=dc0, h_seq=h_seq)
    if grads:
        out.update(param_grads(x, W, h0, h_seq, dA, dA, NH=NH, Dh=Dh, G=4, want=grads))
    return out


def gru_bwd(x, W, R, b, h0, dh_seq, dhT=None, *, NH: int, Dh: int,
            chain_mask=None, grads=("dx", "dW", "dR", "db")):
    """GRU BPTT.  Returns dict dGx, dS [T,B,N], dh0 [B,H], h_seq and the
    parameter gradients named in ``grads``."""
    x, W, R, b, h0, dh_seq, dhT = map(_d, (x, W, R, b, h0, dh_seq, dhT))
    T, B, Din = x.shape
    H, N = NH * Dh, NH * 3 * Dh
    dGx, dS = np.zeros((T, B, N)), np.zeros((T, B, N))
    dh0 = _nan((B, H))
    h_seq = _nan((T, B, H))
    m = _mask(chain_mask, B, NH)
    rc = _load().oracle_gru_bptt(T, B, Din, NH, Dh, _p(x), _p(W), _p(R), _p(b),
                                 _p(h0), _p(dh_seq), _p(dhT), _p(m), _p(dGx), _p(dS),
                                 _p(dh0), _p(h_seq))
    _check(rc, "gru_bptt")
    out = dict(dGx=dGx, dS=dS, dh0=dh0, h_seq=h_seq)
    if grads:
        out.update(param_grads(x, W, h0, h_seq, dGx, dS, NH=NH, Dh=Dh, G=3, want=grads))
    return out

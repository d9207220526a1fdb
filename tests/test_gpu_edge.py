"""The method's special cases on the GPU, in every plan family of the
forward recurrence (one CU per chain with R in VGPRs, with one and with four
batch rows per workgroup; the projection overlapped in the same launch; R
split over one CU's registers and LDS; several CUs per head exchanging h_t
through memory and through one XCD's L2; the float32 LDS kernel).

* Saturated LSTM gates (forget bias +40, input bias -40): sigma(40+-few)
  rounds to 1 and sigma(-40+-few) is ~1e-17, so c_t = c0 at every step and
  |h_t| <= |tanh(c0)| (closed form), and the result matches the oracle.
* Saturated GRU update gate (update bias +40): h_t = h0 at every step.
* Constant gates (W = R = 0): the gates are the activated biases, so
  LSTM  c_t = f^t c0 + i z (1 - f^t) / (1 - f),  h_t = o tanh(c_t)
  GRU   h_t = n + u^t (h0 - n),  n = tanh(b_n), u = sigma(b_z)
  (closed forms evaluated here in float64).
* Head-permutation equivariance: permuting the heads of R, of W's and b's
  column blocks and of h0 / c0 permutes the outputs the same way, bitwise
  (heads are independent: blog.hotdry.top 2025-09-21, the paragraph on
  head-wise splitting; FlashRNN card, abstract).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402

ENV_KEYS = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_WIDE", "RNN355_MC_XCD",
            "RNN355_PIPELINE", "RNN355_SPIN_LIMIT", "RNN355_MC_ROWLANES")

# name: (cell set, Dh, NH, B, T, dtype, environment, expected plan substrings)
FAMILIES = {
    "one_cu": (("lstm", "gru"), 128, 3, 3, 29, "bf16", {}, ("mfma_resident_R", "rows_per_wg=1 ")),
    "one_cu_rows4": (("lstm", "gru"), 64, 3, 5, 29, "bf16", {"RNN355_REC_BT": "4"},
                     ("mfma_resident_R", "rows_per_wg=4 ")),
    "pipelined": (("lstm", "gru"), 128, 3, 4, 96, "bf16", {"RNN355_PIPELINE": "1"},
                  ("mfma_resident_R", "input_proj=pipelined")),
    "split_R": (("lstm", "gru"), 256, 3, 1, 23, "bf16", {}, ("mfma_split_R",)),
    "multi_cu_memory": (("lstm", "gru"), 256, 3, 1, 23, "bf16", {"RNN355_REC_WIDE": "0"},
                        ("mfma_multi_cu", "exchange=memory")),
    "multi_cu_xcd_l2": (("lstm", "gru"), 256, 2, 8, 21, "bf16",
                        {"RNN355_REC_WIDE": "0", "RNN355_REC_BT": "2"},
                        ("mfma_multi_cu", "exchange=xcd_l2")),
    "multi_cu_dh384": (("lstm",), 384, 2, 2, 19, "bf16", {}, ("mfma_multi_cu",)),
    "lds_f32": (("lstm", "gru"), 32, 3, 3, 29, "f32", {}, ("lds_simple",)),
}
CASES = [(f, cell) for f, spec in FAMILIES.items() for cell in spec[0]]
IDS = ["%s-%s" % c for c in CASES]


@pytest.fixture(autouse=True)
def _clean_env():
    old = {k: os.environ.pop(k, None) for k in ENV_KEYS}
    yield
    for k in ENV_KEYS:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def _setup(family, cell):
    _, Dh, NH, B, T, dtype, env, expect = FAMILIES[family]
    os.environ.update(env)
    Din = 32 if dtype == "f32" else 64
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    p = g.plan_describe(op, g.Dims(T, B, Din, NH, Dh),
                        g.RNN_F32 if dtype == "f32" else g.RNN_BF16)
    print("  plan:", p, flush=True)
    for s in expect:
        assert s in p, (s, p)
    return d, dtype


def _run(c):
    if c.cell == "lstm":
        h_seq, c_seq, hT, cT = g.lstm_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"),
                                          dev(c, "h0"), dev(c, "c0"))
        torch.cuda.synchronize()
        return dict(h_seq=host(h_seq), c_seq=host(c_seq), hT=host(hT), cT=host(cT))
    h_seq, hT = g.gru_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0"))
    torch.cuda.synchronize()
    return dict(h_seq=host(h_seq), hT=host(hT))


def _oracle(c):
    d = c.dims
    if c.cell == "lstm":
        return oracle.lstm_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                               c.f64("c0"), NH=d.NH, Dh=d.Dh)
    return oracle.gru_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          NH=d.NH, Dh=d.Dh)


def _tol(dtype):
    return 1e-5 if dtype == "f32" else 2e-2


def _bias(cell, d, per_gate, seed):
    """[NH][G][Dh] bias: gate g set to per_gate[g] (a number) or, where
    per_gate[g] is None, to N(0, 1) draws."""
    G = synth.gates_of(cell)
    b = synth.normal(seed, d.NH * G * d.Dh, 1.0).reshape(d.NH, G, d.Dh)
    for gi, v in enumerate(per_gate):
        if v is not None:
            b[:, gi, :] = v
    return b.reshape(-1)


@pytest.mark.parametrize("family,cell", CASES, ids=IDS)
def test_saturated_gates_hold_the_state(family, cell):
    d, dtype = _setup(family, cell)
    if cell == "lstm":
        bias = _bias(cell, d, (-40.0, 40.0, None, None), 9500)
    else:
        bias = _bias(cell, d, (None, 40.0, None), 9501)
    c = synth.make_case(cell, d, dtype, 9600 + d.Dh, bias=bias, h0_var=0.2, c0_var=0.2)
    got = _run(c)
    for k, y in got.items():
        assert np.isfinite(y).all(), k
    if cell == "lstm":
        c0 = c.vals["c0"].astype(np.float64)
        dev_c = np.max(np.abs(got["c_seq"] - c0[None]))
        print("  max |c_t - c0| = %.3e (max |c0| %.3e)" % (dev_c, np.max(np.abs(c0))), flush=True)
        assert dev_c <= 1e-6 * np.max(np.abs(c0))
        bound = np.abs(np.tanh(c0))[None] + 1e-6
        assert np.all(np.abs(got["h_seq"]) <= bound)
    else:
        # h_t = u (h_{t-1} - n) + n with u = 1 exactly: each step may round
        # h_{t-1} - n and the sum once, so the drift is a few ulp per step
        h0 = c.vals["h0"].astype(np.float64)
        dev_h = np.max(np.abs(got["h_seq"] - h0[None]))
        print("  max |h_t - h0| = %.3e" % dev_h, flush=True)
        assert dev_h <= 2.0 * d.T * 2.0 ** -23 * (np.max(np.abs(h0)) + 1.0)
    ref = _oracle(c)
    for k in got:
        check(k, got[k], ref[k], _tol(dtype))


def _sigm(a):
    return 1.0 / (1.0 + np.exp(-a))


@pytest.mark.parametrize("family,cell", CASES, ids=IDS)
def test_constant_gates_closed_form(family, cell):
    d, dtype = _setup(family, cell)
    G = synth.gates_of(cell)
    bias = _bias(cell, d, (None,) * G, 9700 + d.Dh)
    c = synth.make_case(cell, d, dtype, 9800 + d.Dh, w_var=0.0, r_var=0.0, bias=bias,
                        h0_var=0.3, c0_var=0.3)
    assert not np.any(c.vals["W"]) and not np.any(c.vals["R"])
    got = _run(c)
    T, B, H = d.T, d.B, d.H
    bb = bias.astype(np.float32).astype(np.float64).reshape(d.NH, G, d.Dh)
    t = np.arange(1, T + 1, dtype=np.float64)[:, None, None]
    if cell == "lstm":
        ig, fg = _sigm(bb[:, 0]).reshape(H), _sigm(bb[:, 1]).reshape(H)
        zg, og = np.tanh(bb[:, 2]).reshape(H), _sigm(bb[:, 3]).reshape(H)
        c0 = c.vals["c0"].astype(np.float64)[None]
        ft = fg[None, None] ** t
        c_seq = ft * c0 + ig * zg * (1.0 - ft) / (1.0 - fg)
        want = dict(c_seq=c_seq, h_seq=og * np.tanh(c_seq))
        want["hT"], want["cT"] = want["h_seq"][-1], want["c_seq"][-1]
    else:
        u, n = _sigm(bb[:, 1]).reshape(H), np.tanh(bb[:, 2]).reshape(H)
        h0 = c.vals["h0"].astype(np.float64)[None]
        want = dict(h_seq=n + u[None, None] ** t * (h0 - n))
        want["hT"] = want["h_seq"][-1]
    for k in got:
        check(k, got[k], want[k], 1e-4)


def _permute_heads(c, perm):
    """A copy of case c with head m of every per-head input taken from head
    perm[m] of c."""
    d, G = c.dims, c.G
    GD = G * d.Dh
    p = synth.Case(c.cell, d, c.dtype)

    def cols(a):          # [..., NH*G*Dh] head-major column blocks
        sh = a.shape
        return a.reshape(sh[:-1] + (d.NH, GD))[..., perm, :].reshape(sh)

    def units(a):         # [..., NH*Dh]
        sh = a.shape
        return a.reshape(sh[:-1] + (d.NH, d.Dh))[..., perm, :].reshape(sh)

    p.vals["x"] = c.vals["x"]
    p.vals["W"], p.vals["R"], p.vals["b"] = cols(c.vals["W"]), c.vals["R"][perm], cols(c.vals["b"])
    for k in ("h0", "c0"):
        if k in c.vals:
            p.vals[k] = units(c.vals[k])
    for k, v in c.bits.items():
        p.bits[k] = cols(v) if k == "W" else v[perm] if k == "R" else v
    return p


@pytest.mark.parametrize("family,cell", CASES, ids=IDS)
def test_head_permutation_equivariance_bitwise(family, cell):
    d, dtype = _setup(family, cell)
    c = synth.make_case(cell, d, dtype, 9900 + d.Dh, bias=_bias(cell, d, (None,) * synth.gates_of(cell), 9950),
                        h0_var=0.2, c0_var=0.2)
    perm = np.roll(np.arange(d.NH), 1)          # head m takes old head m-1
    perm = perm[::-1].copy() if d.NH > 2 else perm
    base = _run(c)
    got = _run(_permute_heads(c, perm))
    for k, y in base.items():
        sh = y.shape
        want = y.reshape(sh[:-1] + (d.NH, d.Dh))[..., perm, :].reshape(sh)
        assert np.array_equal(got[k], want), k
    ref = _oracle(c)
    for k in base:
        check(k, base[k], ref[k], _tol(dtype))


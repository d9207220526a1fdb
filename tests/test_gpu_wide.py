"""GPU parity of the Dh = 256 forward recurrence on one compute unit per
(head, batch row), with R split over AGPRs, VGPRs and LDS, against the
oracle (normwise error <= 2e-2 for bf16 calls), plus the invariants it
shares with the other kernels: run-to-run bitwise equality, resume through
(hT, cT), the recurrence-only entry point equal to the full forward, and
head / batch independence."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402

TOL_BF16 = 2e-2


@pytest.fixture(autouse=True)
def _clean_env():
    keys = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_WIDE", "RNN355_PIPELINE")
    old = {k: os.environ.pop(k, None) for k in keys}
    yield
    for k in keys:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def run(c, **kw):
    if c.cell == "lstm":
        h_seq, c_seq, hT, cT = g.lstm_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"),
                                          dev(c, "h0"), dev(c, "c0"), **kw)
        torch.cuda.synchronize()
        return dict(h_seq=host(h_seq), c_seq=host(c_seq), hT=host(hT), cT=host(cT))
    h_seq, hT = g.gru_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0"), **kw)
    torch.cuda.synchronize()
    return dict(h_seq=host(h_seq), hT=host(hT))


def want(c):
    d = c.dims
    if c.cell == "lstm":
        return oracle.lstm_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                               c.f64("c0"), NH=d.NH, Dh=d.Dh)
    return oracle.gru_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          NH=d.NH, Dh=d.Dh)


def plan(c):
    d = c.dims
    op = g.OP_FWD_LSTM if c.cell == "lstm" else g.OP_FWD_GRU
    return g.plan_describe(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16)


@pytest.mark.parametrize("cell,T,B,NH,Din", [
    ("lstm", 23, 3, 2, 64),    # odd T: a last group of one step
    ("lstm", 1, 1, 1, 32),     # a single step
    ("lstm", 40, 5, 3, 96),    # Din not a multiple of 32: register-staged projection
    ("gru", 23, 3, 2, 64),
    ("gru", 2, 2, 1, 32),      # one full group
    ("gru", 37, 4, 3, 64),
])
def test_split_r_forward(cell, T, B, NH, Din):
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=256)
    c = synth.make_case(cell, d, "bf16", 9600 + T + B + NH,
                        bias="forget+1" if cell == "lstm" else "zero", h0_var=0.2, c0_var=0.2)
    p = plan(c)
    print("  plan:", p, flush=True)
    assert "split_R" in p
    got, ref = run(c), want(c)
    for key in got:
        check(key, got[key], ref[key], TOL_BF16)


def test_split_r_bitwise_repeatable_resume_and_rec_entry():
    d = synth.Dims(T=30, B=3, Din=64, NH=2, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 9700, bias="forget+1", h0_var=0.1, c0_var=0.1)
    a, b = run(c), run(c)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    x, W, R, bb = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b")
    h1, c1, hT1, cT1 = g.lstm_fwd(x[:13].contiguous(), W, R, bb, dev(c, "h0"), dev(c, "c0"))
    h2, c2, hT2, cT2 = g.lstm_fwd(x[13:].contiguous(), W, R, bb, hT1, cT1)
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate([host(h1), host(h2)]), a["h_seq"])
    assert np.array_equal(host(cT2), a["cT"])
    gx = g.input_proj(x, W, bb)
    h, cs, hT, cT = g.rec_lstm(gx, R, dev(c, "h0"), dev(c, "c0"))
    torch.cuda.synchronize()
    assert np.array_equal(host(h), a["h_seq"])
    assert np.array_equal(host(cs), a["c_seq"])
    assert np.array_equal(host(cT), a["cT"])


def test_split_r_gru_rec_entry_and_independence():
    d = synth.Dims(T=19, B=3, Din=32, NH=3, Dh=256)
    c = synth.make_case("gru", d, "bf16", 9800, h0_var=0.1)
    base = run(c)
    gx = g.input_proj(dev(c, "x"), dev(c, "W"), dev(c, "b"))
    h, hT = g.rec_gru(gx, dev(c, "R"), dev(c, "h0"))
    torch.cuda.synchronize()
    assert np.array_equal(host(h), base["h_seq"])
    c.vals["h0"][:, 256:512] += 0.5      # head 1 state
    c.vals["h0"][2] -= 0.5               # batch row 2
    pert = run(c)
    keep = np.r_[0:256, 512:768]
    assert np.array_equal(pert["h_seq"][:, :2][..., keep], base["h_seq"][:, :2][..., keep])
    assert not np.array_equal(pert["h_seq"][:, 2], base["h_seq"][:, 2])


def test_split_r_without_sequence_outputs():
    d = synth.Dims(T=9, B=2, Din=32, NH=1, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 9900, bias="forget+1")
    full = run(c)
    _, _, hT, cT = g.lstm_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"),
                              with_seq=False)
    torch.cuda.synchronize()
    assert np.array_equal(host(hT), full["hT"])
    assert np.array_equal(host(cT), full["cT"])

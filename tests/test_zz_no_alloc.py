"""The allocation-free recurrence (rnn_rec_lstm_noalloc, scratch in a device
array of the library) against the workspace entry point rnn_rec_lstm,
through the C ABI: two calls in a row on one GPU, the second with a smaller
input, in each plan family whose kernels use scratch (one CU per chain;
several CUs per head exchanging h_t through one XCD's L2 or through memory;
R split over one CU with R^T staged in scratch).  The kernels are the same,
so the outputs must be the same bits; one case is also held to the oracle."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402

KEYS = ("RNN355_REC_WIDE", "RNN355_SPIN_LIMIT", "RNN355_MC_XCD")


@pytest.fixture(autouse=True)
def _clean_env():
    old = {k: os.environ.pop(k, None) for k in KEYS}
    yield
    for k in KEYS:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def _inputs(d, seed):
    c = synth.make_case("lstm", d, "bf16", seed, bias="forget+1", h0_var=0.2, c0_var=0.2)
    gx = g.input_proj(dev(c, "x"), dev(c, "W"), dev(c, "b"))
    return c, gx, dev(c, "R"), dev(c, "h0"), dev(c, "c0")


def _both(d, seed, expect):
    c, gx, R, h0, c0 = _inputs(d, seed)
    p = g.plan_describe(g.OP_REC_LSTM, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16)
    print("  plan (T=%d B=%d NH=%d Dh=%d): %s" % (d.T, d.B, d.NH, d.Dh, p), flush=True)
    assert expect in p, p
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    a = g.rec_lstm_noalloc(gx, R, h0, c0, status=status)
    a = [t.clone() for t in a]
    b = g.rec_lstm(gx, R, h0, c0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for name, x, y in zip(("h_seq", "c_seq", "hT", "cT"), a, b):
        assert torch.equal(x, y), name
    return c, a


@pytest.mark.parametrize("family,big,small", [
    ("mfma_resident_R", synth.Dims(T=256, B=16, Din=64, NH=6, Dh=128),
     synth.Dims(T=100, B=5, Din=64, NH=2, Dh=128)),
    ("exchange=xcd_l2", synth.Dims(T=64, B=16, Din=64, NH=1, Dh=768),
     synth.Dims(T=20, B=16, Din=32, NH=1, Dh=768)),
    ("exchange=memory", synth.Dims(T=40, B=3, Din=64, NH=3, Dh=256),
     synth.Dims(T=9, B=1, Din=32, NH=2, Dh=256)),
    ("mfma_split_R", synth.Dims(T=40, B=1, Din=64, NH=3, Dh=256),
     synth.Dims(T=11, B=2, Din=32, NH=1, Dh=256)),
])
def test_noalloc_matches_workspace_entry_twice(family, big, small):
    if family == "exchange=memory":
        os.environ["RNN355_REC_WIDE"] = "0"
    c, a = _both(big, 12000 + big.Dh, family)
    _both(small, 12100 + small.Dh, family)
    if family == "mfma_resident_R":
        ref = oracle.lstm_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                              c.f64("c0"), NH=big.NH, Dh=big.Dh)
        for name, y in zip(("h_seq", "c_seq", "hT", "cT"), a):
            check(name, host(y), ref[name], 2e-2)


def test_noalloc_reports_a_step_wait_timeout_then_clears_it():
    """A spin limit of one poll (set from the host) makes the multi-CU step
    waits give up; the kernel ends normally and the status output says so.
    The next call starts from a cleared status word."""
    os.environ["RNN355_REC_WIDE"] = "0"
    d = synth.Dims(T=64, B=2, Din=32, NH=1, Dh=256)
    c, gx, R, h0, c0 = _inputs(d, 12300)
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    os.environ["RNN355_SPIN_LIMIT"] = "1"
    g.rec_lstm_noalloc(gx, R, h0, c0, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    os.environ.pop("RNN355_SPIN_LIMIT")
    a = g.rec_lstm_noalloc(gx, R, h0, c0, status=status)
    b = g.rec_lstm(gx, R, h0, c0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(a[0], b[0]) and torch.equal(a[3], b[3])


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    d = g.Dims(8, 2, 1, 64, 256)
    gx = torch.zeros((8, 2, 64 * 4 * 256), dtype=torch.float32, device="cuda")
    R = torch.zeros((64, 256, 4 * 256), dtype=torch.bfloat16, device="cuda")
    assert g.workspace_size(g.OP_REC_LSTM, d, g.RNN_BF16) > (8 << 20)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        g.rec_lstm_noalloc(gx, R)

"""GPU parity of plans the constraint search picks where a fixed rule did
not: many one-row workgroups sharing CUs, 48 workgroups per head, the LDS
kernel at two rows per workgroup.  Each case checks the plan it ran and the
results against the oracle."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402


@pytest.fixture(autouse=True)
def _clean_env():
    keys = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_KCW", "RNN355_REC_WIDE")
    old = {k: os.environ.pop(k, None) for k in keys}
    yield
    for k, v in old.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


@pytest.mark.parametrize("cell,B,NH,Dh,dtype,want", [
    ("lstm", 64, 12, 64, "bf16", "rows_per_wg=1 wg=768"),   # three workgroups per CU
    ("gru", 33, 12, 32, "bf16", "rows_per_wg=1 wg=396"),
    ("lstm", 1, 1, 768, "bf16", "wg_per_head_row_tile=48"),
    ("lstm", 2, 1, 384, "bf16", "wg_per_head_row_tile=24"),
    ("gru", 16, 6, 384, "bf16", "rows_per_wg=6"),
    ("lstm", 4, 4, 32, "f32", "lds_simple rows_per_wg=2"),
])
def test_searched_plan_parity(cell, B, NH, Dh, dtype, want):
    d = synth.Dims(T=12, B=B, Din=64, NH=NH, Dh=Dh)
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    dt = g.RNN_BF16 if dtype == "bf16" else g.RNN_F32
    plan = g.plan_describe(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), dt)
    print("  plan:", plan, flush=True)
    assert want in plan
    c = synth.make_case(cell, d, dtype, 6600 + B + Dh, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2)
    t = [dev(c, k) for k in ("x", "W", "R", "b", "h0")]
    if cell == "lstm":
        h, cs, hT, cT = g.lstm_fwd(*t, dev(c, "c0"))
        got = dict(h_seq=host(h), c_seq=host(cs), hT=host(hT), cT=host(cT))
        ref = oracle.lstm_fwd(*[c.f64(k) for k in ("x", "W", "R", "b", "h0", "c0")], NH=NH, Dh=Dh)
    else:
        h, hT = g.gru_fwd(*t)
        got = dict(h_seq=host(h), hT=host(hT))
        ref = oracle.gru_fwd(*[c.f64(k) for k in ("x", "W", "R", "b", "h0")], NH=NH, Dh=Dh)
    tol = 1e-5 if dtype == "f32" else 2e-2
    for k in got:
        check(k, got[k], ref[k], tol)

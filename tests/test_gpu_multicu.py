"""GPU parity of the multi-CU forward recurrence (heads of Dh >= 256 split
over several workgroups that swap h_t through global memory every step)
against the oracle, plus its time-out path forced from the host.  At Dh =
256 the plan prefers the one-CU kernel with split R; RNN355_REC_WIDE=0
selects the multi-CU kernel there."""
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
    keys = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_SPIN_LIMIT", "RNN355_REC_WIDE",
            "RNN355_MC_XCD", "RNN355_MC_ROWLANES")
    old = {k: os.environ.pop(k, None) for k in keys}
    os.environ["RNN355_REC_WIDE"] = "0"
    yield
    for k in keys:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def run(c, ws=None):
    if c.cell == "lstm":
        h_seq, c_seq, hT, cT = g.lstm_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"),
                                          dev(c, "h0"), dev(c, "c0"), ws=ws)
        torch.cuda.synchronize()
        return dict(h_seq=host(h_seq), c_seq=host(c_seq), hT=host(hT), cT=host(cT))
    h_seq, hT = g.gru_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0"), ws=ws)
    torch.cuda.synchronize()
    return dict(h_seq=host(h_seq), hT=host(hT))


def want(c, mask=None):
    d = c.dims
    if c.cell == "lstm":
        return oracle.lstm_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                               c.f64("c0"), NH=d.NH, Dh=d.Dh, chain_mask=mask)
    return oracle.gru_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          NH=d.NH, Dh=d.Dh, chain_mask=mask)


def plan(c):
    d = c.dims
    op = g.OP_FWD_LSTM if c.cell == "lstm" else g.OP_FWD_GRU
    return g.plan_describe(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16)


@pytest.mark.parametrize("cell,Dh,NH,B,bt,k", [
    ("lstm", 256, 2, 3, None, None),   # 2 workgroups per head, one row each
    ("lstm", 256, 2, 5, 2, None),      # two row slots, ragged batch
    ("lstm", 256, 1, 6, 4, 4),         # four row slots, 4 workgroups per head
    ("gru", 256, 2, 3, None, None),
    ("gru", 256, 1, 7, 4, None),
    ("lstm", 384, 1, 2, None, None),   # k split over 3 waves (LDS reduction)
    ("gru", 384, 1, 3, 2, None),
    ("lstm", 768, 1, 2, None, None),   # 24 workgroups per head
])
def test_multicu_forward(cell, Dh, NH, B, bt, k):
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    if k is not None:
        os.environ["RNN355_REC_K"] = str(k)
    d = synth.Dims(T=23, B=B, Din=64, NH=NH, Dh=Dh)
    c = synth.make_case(cell, d, "bf16", 8000 + Dh + B, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2)
    p = plan(c)
    print("  plan:", p, flush=True)
    assert "multi_cu" in p
    got, ref = run(c), want(c)
    for key in got:
        check(key, got[key], ref[key], TOL_BF16)


# groups (heads x batch tiles) a multiple of 8: the members of a group are
# numbered so that they run on one XCD and exchange h_t through its L2 when
# every member finds itself there; RNN355_MC_XCD=0 keeps the exchange
# through memory.  Same sums either way: the outputs must be the same bits.
@pytest.mark.parametrize("cell,Dh,NH,B,bt", [
    ("lstm", 256, 2, 8, 2),     # 8 groups of 2 workgroups
    ("gru", 256, 4, 4, 2),      # 8 groups, GRU
    ("lstm", 384, 1, 16, 2),    # 8 groups, k split over waves
    ("lstm", 768, 1, 16, None), # the Dh = 768 plan: 8 groups of 24
])
def test_multicu_xcd_grouped_exchange(cell, Dh, NH, B, bt):
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=21, B=B, Din=64, NH=NH, Dh=Dh)
    c = synth.make_case(cell, d, "bf16", 8300 + Dh + B, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2)
    p = plan(c)
    print("  plan:", p, flush=True)
    assert "multi_cu" in p
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    need = g.workspace_size(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    got = run(c, ws=ws)
    assert g.workspace_status(ws) == g.RNN_OK
    os.environ["RNN355_MC_XCD"] = "0"
    mem = run(c, ws=ws)
    assert g.workspace_status(ws) == g.RNN_OK
    for key in got:
        assert np.array_equal(got[key], mem[key]), key
    ref = want(c)
    for key in got:
        check(key, got[key], ref[key], TOL_BF16)


# 2..16 batch rows per workgroup: by default the gate wave transposes the
# MFMA tile so that each cell update pass covers four rows (row 4p + q in lane
# group q); RNN355_MC_ROWLANES=0 runs one pass per register slot.  The
# sums and the cell arithmetic are the same, so the outputs are the same bits.
@pytest.mark.parametrize("cell,Dh,NH,B,bt", [
    ("lstm", 256, 2, 5, 2),     # ragged: the last tile holds one row
    ("lstm", 256, 1, 7, 4),     # four rows, ragged (3 in the last tile)
    ("gru", 256, 2, 6, 3),
    ("gru", 384, 1, 4, 4),      # k split over waves
    ("lstm", 768, 1, 16, None), # the Dh = 768 plan (two rows per tile)
    ("lstm", 384, 2, 13, 6),    # two passes (rows 0-3, 4-5), ragged (tiles 6, 6, 1)
    ("gru", 256, 1, 16, 8),     # two passes, 8 k-chunks per wave
    ("lstm", 256, 1, 11, 12),   # four passes, one ragged tile of 11 rows
    ("lstm", 512, 1, 16, 16),   # four passes, a full 16-row tile
])
def test_multicu_rows_in_lane_groups_bitwise(cell, Dh, NH, B, bt):
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=17, B=B, Din=64, NH=NH, Dh=Dh)
    c = synth.make_case(cell, d, "bf16", 8700 + Dh + B, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2)
    p = plan(c)
    print("  plan:", p, flush=True)
    assert "multi_cu" in p and "rows_per_wg=1 " not in p
    got = run(c)
    os.environ["RNN355_MC_ROWLANES"] = "0"
    slots = run(c)
    for key in got:
        assert np.array_equal(got[key], slots[key]), key
    ref = want(c)
    for key in got:
        check(key, got[key], ref[key], TOL_BF16)


def test_multicu_run_to_run_bitwise():
    d = synth.Dims(T=17, B=2, Din=32, NH=1, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 8100, bias="forget+1")
    a, b = run(c), run(c)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_step_wait_timeout_is_reported():
    """A spin limit of one poll (set from the host) makes the first step wait
    give up: every workgroup stops, the kernel ends normally and the
    workspace reports the time-out; the next call clears it."""
    d = synth.Dims(T=64, B=2, Din=32, NH=1, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 8200, bias="forget+1")
    need = g.workspace_size(g.OP_FWD_LSTM, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    os.environ["RNN355_SPIN_LIMIT"] = "1"
    run(c, ws=ws)
    assert g.workspace_status(ws) == g.RNN_ERR_BARRIER_TIMEOUT
    os.environ.pop("RNN355_SPIN_LIMIT")
    got = run(c, ws=ws)
    assert g.workspace_status(ws) == g.RNN_OK
    assert nerr(got["h_seq"], want(c)["h_seq"]) <= TOL_BF16


_ORACLE = {}


def _workload_oracle(name, c):
    """The oracle's whole forward of a full-size workload (every chain),
    computed once per test session."""
    if name not in _ORACLE:
        _ORACLE[name] = want(c)
    return _ORACLE[name]


# Full-size workloads in the plans they run by default (multi-CU, h through
# one XCD's L2), with the exchange through memory (RNN355_MC_XCD=0), and at
# Dh = 256 in the split-R plan the default takes where groups cannot share
# an L2.  Every chain and every output is compared with the oracle.
@pytest.mark.parametrize("name", [
    "lstm_1h_b16_dh768",
    "lstm_1h_b16_dh768/memory",
    "lstm_fwdbwd_b16_nh4_dh256",
    "lstm_fwdbwd_b16_nh4_dh256/memory",
    "lstm_fwdbwd_b16_nh4_dh256/split_R",
])
def test_large_head_workloads_full_size_every_chain(name):
    name, _, variant = name.partition("/")
    os.environ.pop("RNN355_REC_WIDE")
    if variant == "memory":
        os.environ["RNN355_MC_XCD"] = "0"
        os.environ["RNN355_REC_WIDE"] = "0"
    elif variant == "split_R":
        os.environ["RNN355_MC_XCD"] = "0"
    w = synth.WORKLOADS[name]
    c = synth.workload_case(w)
    p = plan(c)
    print("  plan:", p, flush=True)
    assert ("split_R" if variant == "split_R" else
            "exchange=memory" if variant == "memory" else "exchange=xcd_l2") in p
    need = g.workspace_size(g.OP_FWD_LSTM, g.Dims(*(getattr(w.dims, k) for k in
                                                      ("T", "B", "Din", "NH", "Dh"))), g.RNN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    got = run(c, ws=ws)
    assert g.workspace_status(ws) == g.RNN_OK
    ref = _workload_oracle(name, c)
    for key in ("h_seq", "c_seq", "hT", "cT"):
        check(key, got[key], ref[key], TOL_BF16)

"""GPU parity of the LSTM and GRU backward (BPTT) against the oracle.

The GPU backward runs on the GPU forward's h_seq / c_seq; the oracle runs
its own forward.  Bar: normwise 2e-2 on every gradient (bf16 operands, f32
accumulation; dA is rounded to bf16 only as the operand of the dx, dW, dR
contractions)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402

TOL = 2e-2


@pytest.fixture(autouse=True)
def _clean_env():
    keys = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_WIDE", "RNN355_MC_XCD",
            "RNN355_BWD_WIDE2", "RNN355_SPIN_LIMIT", "RNN355_BWD_OVERLAP")
    old = {k: os.environ.pop(k, None) for k in keys}
    yield
    for k in keys:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def gpu_bwd(c, final=False):
    x, W, R, b = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b")
    h0, c0 = dev(c, "h0"), dev(c, "c0")
    h_seq, c_seq, _, _ = g.lstm_fwd(x, W, R, b, h0, c0)
    grads = g.lstm_bwd(x, W, R, b, h0, c0, h_seq, c_seq, dev(c, "dH"),
                       dev(c, "dhT") if final else None, dev(c, "dcT") if final else None)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in grads.items()}


# bt "x": RNN355_REC_WIDE=0, the exchange-based sweep at Dh = 256 (the
# default there is one workgroup per (head, row) with R split over
# registers and LDS)
@pytest.mark.parametrize("Dh,B,bt,final", [
    (16, 3, None, True),      # two gate-column chunks per head (two per wave)
    (32, 3, None, False),     # one workgroup per head, dA through LDS
    (64, 5, 2, True),         # two row slots, ragged, final-state gradients
    (128, 3, 4, False),       # four row slots
    (128, 2, None, True),
    (256, 3, None, True),     # split R, one workgroup per (head, row)
    (256, 5, None, False),
    (256, 3, "x", True),      # several workgroups per head, dA as tagged words
    (256, 5, "x4", False),
])
def test_lstm_backward_small(Dh, B, bt, final):
    if isinstance(bt, str):
        os.environ["RNN355_REC_WIDE"] = "0"
        bt = int(bt[1:]) if len(bt) > 1 else None
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=19, B=B, Din=64, NH=2, Dh=Dh)
    c = synth.make_case("lstm", d, "bf16", 9000 + Dh + B, bias="forget+1", h0_var=0.2,
                        c0_var=0.2, backward=True, final_grads=final)
    got = gpu_bwd(c, final)
    ref = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          c.f64("c0"), c.f64("dH"), c.f64("dhT") if final else None,
                          c.f64("dcT") if final else None, NH=d.NH, Dh=d.Dh)
    for k in ("dx", "dW", "dR", "db", "dh0", "dc0"):
        check(k, got[k], ref[k], TOL)


@pytest.mark.parametrize("wide", ["1", "0"])
def test_lstm_backward_bitwise_repeatable(wide):
    os.environ["RNN355_REC_WIDE"] = wide
    d = synth.Dims(T=11, B=2, Din=32, NH=2, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 9100, bias="forget+1", backward=True)
    a, b = gpu_bwd(c), gpu_bwd(c)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def _head_param_grads(ref, c, n, G, want):
    """dW and/or dR of head n alone, by the oracle's parameter-gradient sums
    on that head's slices (the sums over t and b never mix heads)."""
    d = c.dims
    GD, sl = G * d.Dh, slice(n * d.Dh, (n + 1) * d.Dh)
    dG = (ref["dA"] if G == 4 else ref["dGx"])[..., n * GD:(n + 1) * GD]
    dS = (ref["dA"] if G == 4 else ref["dS"])[..., n * GD:(n + 1) * GD]
    return oracle.param_grads(c.f64("x"), c.f64("W")[:, n * GD:(n + 1) * GD],
                              c.f64("h0")[:, sl], ref["h_seq"][..., sl], dG, dS,
                              NH=1, Dh=d.Dh, G=G, want=want)


def _full_size_backward_checks(got, ref, c, G, heads_dW, n_t=64, seed=5):
    """Every chain's dh0 (and dc0), all of db and dR, dW of the given heads,
    dx of every batch row and input column at n_t sampled steps."""
    d = c.dims
    GD = G * d.Dh
    for k in ("dh0", "dc0") if G == 4 else ("dh0",):
        check(k, got[k], ref[k], TOL)
    dG = ref["dA"] if G == 4 else ref["dGx"]
    dS = ref["dA"] if G == 4 else ref["dS"]
    full = oracle.param_grads(c.f64("x"), c.f64("W"), c.f64("h0"), ref["h_seq"], dG, dS,
                              NH=d.NH, Dh=d.Dh, G=G, want=("db", "dR"))
    check("db", got["db"], full["db"], TOL)
    check("dR", got["dR"], full["dR"], TOL)
    for n in heads_dW:
        hd = _head_param_grads(ref, c, n, G, ("dW",))
        check("dW[h%d]" % n, got["dW"][:, n * GD:(n + 1) * GD], hd["dW"], TOL)
    rng = np.random.default_rng(seed)
    tt = np.sort(rng.choice(d.T, size=min(n_t, d.T), replace=False))
    tt[0], tt[-1] = 0, d.T - 1
    m = (tt[:, None] * d.B + np.arange(d.B)[None, :]).reshape(-1)
    idx = np.stack([np.repeat(m, d.Din), np.tile(np.arange(d.Din), m.size)], 1)
    args = (c.f64("x"), c.f64("W"), c.f64("h0"), ref["h_seq"], dG, dS)
    dx_ref = oracle.param_grad_entries("dx", idx, *args, NH=d.NH, Dh=d.Dh, G=G)
    check("dx[%dt]" % tt.size, got["dx"][tt].reshape(-1), dx_ref, TOL)


def test_backward_workload_full_size():
    """LSTM forward+BPTT, B=16, NH=4, Dh=256, T=1024, Din=1024 at full size,
    in the default plan.  The oracle runs BPTT on all 64 chains; compared:
    dh0 and dc0 of every chain, all of db and dR, dW of two whole heads, dx of
    every batch row at 64 steps (the first and last among them)."""
    w = synth.WORKLOADS["lstm_fwdbwd_b16_nh4_dh256"]
    c = synth.workload_case(w)
    d = w.dims
    got = gpu_bwd(c)
    ref = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          c.f64("c0"), c.f64("dH"), NH=d.NH, Dh=d.Dh, grads=())
    _full_size_backward_checks(got, ref, c, 4, heads_dW=(1, 3))


@pytest.mark.parametrize("cell,T,B,NH,Dh,Din,final", [
    ("lstm", 1030, 8, 2, 256, 128, True),  # two CUs per (head, row); chunks 3 x 258 + 256
    ("gru", 512, 4, 3, 128, 64, True),     # four chunks of 128
    ("lstm", 600, 5, 2, 64, 96, False),    # four chunks of 150
])
def test_backward_chunked_sweep_matches_one_piece(cell, T, B, NH, Dh, Din, final):
    """The backward whose sweep runs in time chunks, each chunk's dx, dW, dR
    and db computed on two other streams beside the next chunk's sweep, against
    the same call with the sweep in one piece (RNN355_BWD_OVERLAP=0): dx,
    dh0 and dc0 bitwise (the carries pass between chunks as float32), dW, dR
    and db to float32 rounding (the chunks' sums are added in chunk order)."""
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    c = synth.make_case(cell, d, "bf16", 9300 + T + Dh, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2, backward=True, final_grads=final)
    run = gpu_bwd if cell == "lstm" else gpu_bwd_gru
    op = g.OP_BWD_LSTM if cell == "lstm" else g.OP_BWD_GRU
    gd = g.Dims(T, B, Din, NH, Dh)
    plan = g.plan_describe(op, gd, g.RNN_BF16)
    print("  plan:", plan, flush=True)
    assert " chunks=1 " not in plan
    chunked = run(c, final)
    os.environ["RNN355_BWD_OVERLAP"] = "0"
    assert " chunks=1 " in g.plan_describe(op, gd, g.RNN_BF16)
    whole = run(c, final)
    for k in ("dx", "dh0") + (("dc0",) if cell == "lstm" else ()):
        assert np.array_equal(chunked[k], whole[k]), k
    for k in ("dW", "dR", "db"):
        e = nerr(chunked[k], whole[k])
        print("  %s: %.2e" % (k, e), flush=True)
        assert e <= 1e-5, k


def gpu_bwd_gru(c, final=False):
    x, W, R, b = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b")
    h0 = dev(c, "h0")
    h_seq, _ = g.gru_fwd(x, W, R, b, h0)
    grads = g.gru_bwd(x, W, R, b, h0, h_seq, dev(c, "dH"), dev(c, "dhT") if final else None)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in grads.items()}


@pytest.mark.parametrize("Dh,B,bt,final", [
    (32, 3, None, True),      # three gate-column chunks per head (three per wave)
    (64, 3, None, False),     # one workgroup per (head, row): 6 chunks per wave, dS through LDS
    (64, 5, 2, True),         # two row slots, ragged, final-state gradient
    (128, 2, None, True),     # 12 chunks per wave, one workgroup
    (128, 5, 4, False),       # four row slots
    (256, 3, None, True),     # split R, one workgroup per (head, row)
    (256, 5, None, False),
    (256, 3, "x", True),      # two k-splits, four workgroups per head: dS as tagged words
    (256, 5, "x2", False),
])
def test_gru_backward_small(Dh, B, bt, final):
    if isinstance(bt, str):
        os.environ["RNN355_REC_WIDE"] = "0"
        bt = int(bt[1:]) if len(bt) > 1 else None
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=17, B=B, Din=64, NH=2, Dh=Dh)
    c = synth.make_case("gru", d, "bf16", 9500 + Dh + B,
                        bias=synth.normal(9400 + Dh, d.NH * 3 * Dh, 0.25), h0_var=0.3,
                        backward=True, final_grads=final)
    got = gpu_bwd_gru(c, final)
    ref = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                         c.f64("dH"), c.f64("dhT") if final else None, NH=d.NH, Dh=d.Dh)
    for k in ("dx", "dW", "dR", "db", "dh0"):
        check(k, got[k], ref[k], TOL)


@pytest.mark.parametrize("wide", ["1", "0"])
def test_gru_backward_bitwise_repeatable(wide):
    os.environ["RNN355_REC_WIDE"] = wide
    d = synth.Dims(T=13, B=3, Din=32, NH=2, Dh=256)
    c = synth.make_case("gru", d, "bf16", 9600, h0_var=0.2, backward=True)
    a, b = gpu_bwd_gru(c), gpu_bwd_gru(c)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_gru_backward_small_batch_workload_shape_full():
    """GRU BPTT at the shape of the small-batch GRU workload (B=4, NH=12,
    Dh=64, T=2048, Din=768; dL/dh_t ~ N(0,1) for all t).  The oracle runs
    BPTT on all 48 chains; compared: dh0 of every chain, all of db and dR, dW
    of two whole heads, dx of every batch row at 64 steps."""
    w = synth.WORKLOADS["gru_mh_b4_nh12_dh64"]
    d = w.dims
    c = synth.make_case("gru", d, "bf16", 9000, h0_var=0.1, backward=True)
    got = gpu_bwd_gru(c)
    ref = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                         c.f64("dH"), NH=d.NH, Dh=d.Dh, grads=())
    _full_size_backward_checks(got, ref, c, 3, heads_dW=(0, 5))


# 8 (head, row) groups of four workgroups in the exchange-based sweep
# (RNN355_REC_WIDE=0): numbered so that each group runs on one XCD and swaps
# dA through its L2 (each launch checks the placement); RNN355_MC_XCD=0 swaps
# through memory.  Same sums either way: the gradients must be the same bits.
@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_backward_xcd_grouped_exchange(cell):
    os.environ["RNN355_REC_WIDE"] = "0"
    d = synth.Dims(T=15, B=4, Din=64, NH=2, Dh=256)
    lstm = cell == "lstm"
    c = synth.make_case(cell, d, "bf16", 9700 + (0 if lstm else 1),
                        bias="forget+1" if lstm else "zero", h0_var=0.2, c0_var=0.2,
                        backward=True, final_grads=True)
    x, W, R, b, h0 = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0")
    op = g.OP_BWD_LSTM if lstm else g.OP_BWD_GRU
    ws = torch.empty(g.workspace_size(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16),
                     dtype=torch.uint8, device="cuda")

    def once():
        if lstm:
            c0 = dev(c, "c0")
            h_seq, c_seq, _, _ = g.lstm_fwd(x, W, R, b, h0, c0)
            grads = g.lstm_bwd(x, W, R, b, h0, c0, h_seq, c_seq, dev(c, "dH"), dev(c, "dhT"),
                               dev(c, "dcT"), ws=ws)
        else:
            h_seq, _ = g.gru_fwd(x, W, R, b, h0)
            grads = g.gru_bwd(x, W, R, b, h0, h_seq, dev(c, "dH"), dev(c, "dhT"), ws=ws)
        torch.cuda.synchronize()
        assert g.workspace_status(ws) == g.RNN_OK
        return {k: host(v) for k, v in grads.items()}

    got = once()
    os.environ["RNN355_MC_XCD"] = "0"
    mem = once()
    for k in got:
        assert np.array_equal(got[k], mem[k]), k
    if lstm:
        ref = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                              c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"),
                              NH=d.NH, Dh=d.Dh)
    else:
        ref = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                             c.f64("dH"), c.f64("dhT"), NH=d.NH, Dh=d.Dh)
    for k in got:
        check(k, got[k], ref[k], TOL)


def _bwd_with_ws(c, ws, final=True):
    lstm = c.cell == "lstm"
    x, W, R, b, h0 = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0")
    if lstm:
        c0 = dev(c, "c0")
        h_seq, c_seq, _, _ = g.lstm_fwd(x, W, R, b, h0, c0)
        grads = g.lstm_bwd(x, W, R, b, h0, c0, h_seq, c_seq, dev(c, "dH"),
                           dev(c, "dhT") if final else None, dev(c, "dcT") if final else None,
                           ws=ws)
    else:
        h_seq, _ = g.gru_fwd(x, W, R, b, h0)
        grads = g.gru_bwd(x, W, R, b, h0, h_seq, dev(c, "dH"), dev(c, "dhT") if final else None,
                          ws=ws)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in grads.items()}


# Dh = 256 with (heads x rows) a multiple of 8: the sweep runs on two CUs per
# (head, row), each holding half of R in AGPRs and swapping partial carries
# (RNN355_BWD_WIDE2=0: one CU with R split over AGPRs, VGPRs and LDS).  The
# two sum the carries in different orders, so they agree to rounding.
@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_backward_two_cu_split_r(cell):
    d = synth.Dims(T=17, B=4, Din=64, NH=2, Dh=256)
    lstm = cell == "lstm"
    c = synth.make_case(cell, d, "bf16", 9800 + (0 if lstm else 1),
                        bias="forget+1" if lstm else "zero", h0_var=0.2, c0_var=0.2,
                        backward=True, final_grads=True)
    op = g.OP_BWD_LSTM if lstm else g.OP_BWD_GRU
    ws = torch.empty(g.workspace_size(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16),
                     dtype=torch.uint8, device="cuda")
    got = _bwd_with_ws(c, ws)
    assert g.workspace_status(ws) == g.RNN_OK
    again = _bwd_with_ws(c, ws)
    for k in got:
        assert np.array_equal(got[k], again[k]), k
    if lstm:
        ref = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                              c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"),
                              NH=d.NH, Dh=d.Dh)
    else:
        ref = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                             c.f64("dH"), c.f64("dhT"), NH=d.NH, Dh=d.Dh)
    for k in got:
        check(k, got[k], ref[k], TOL)
    os.environ["RNN355_BWD_WIDE2"] = "0"
    one = _bwd_with_ws(c, ws)
    for k in got:
        e = nerr(got[k], one[k])
        print("  %-4s two-CU vs one-CU nerr=%.3e" % (k, e), flush=True)
        assert e <= 1e-2, (k, e)


def test_chunked_backward_timeout_is_reported():
    """The sweep in four chunks with a spin limit of one poll: every chunk's
    launch ends normally, the status word the first sweep set survives the
    later chunks' launches, and the next call (no limit) clears it."""
    d = synth.Dims(T=512, B=4, Din=32, NH=2, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 9910, bias="forget+1", backward=True,
                        final_grads=True)
    ws = torch.empty(g.workspace_size(g.OP_BWD_LSTM, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh),
                                      g.RNN_BF16), dtype=torch.uint8, device="cuda")
    os.environ["RNN355_SPIN_LIMIT"] = "1"
    _bwd_with_ws(c, ws)
    assert g.workspace_status(ws) == g.RNN_ERR_BARRIER_TIMEOUT
    os.environ.pop("RNN355_SPIN_LIMIT")
    got = _bwd_with_ws(c, ws)
    assert g.workspace_status(ws) == g.RNN_OK
    ref = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"), NH=d.NH, Dh=d.Dh)
    for k in ("dx", "dW", "dR", "db", "dh0", "dc0"):
        check(k, got[k], ref[k], TOL)


def test_backward_two_cu_timeout_is_reported():
    """A spin limit of one poll (set from the host) makes the first swap of
    partial carries give up: both CUs stop, the kernel ends normally and the
    workspace reports the time-out; the next call clears it."""
    d = synth.Dims(T=24, B=4, Din=32, NH=2, Dh=256)
    c = synth.make_case("lstm", d, "bf16", 9900, bias="forget+1", backward=True,
                        final_grads=True)
    ws = torch.empty(g.workspace_size(g.OP_BWD_LSTM, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh),
                                      g.RNN_BF16), dtype=torch.uint8, device="cuda")
    os.environ["RNN355_SPIN_LIMIT"] = "1"
    _bwd_with_ws(c, ws)
    assert g.workspace_status(ws) == g.RNN_ERR_BARRIER_TIMEOUT
    os.environ.pop("RNN355_SPIN_LIMIT")
    got = _bwd_with_ws(c, ws)
    assert g.workspace_status(ws) == g.RNN_OK
    ref = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"), NH=d.NH, Dh=d.Dh)
    assert nerr(got["dh0"], ref["dh0"]) <= TOL


TOL_F32 = 1e-5


def _bwd_any(c, final):
    x, W, R, b = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b")
    h0 = dev(c, "h0")
    if c.cell == "lstm":
        c0 = dev(c, "c0")
        h_seq, c_seq, _, _ = g.lstm_fwd(x, W, R, b, h0, c0)
        grads = g.lstm_bwd(x, W, R, b, h0, c0, h_seq, c_seq, dev(c, "dH"),
                           dev(c, "dhT") if final else None, dev(c, "dcT") if final else None)
    else:
        h_seq, _ = g.gru_fwd(x, W, R, b, h0)
        grads = g.gru_bwd(x, W, R, b, h0, h_seq, dev(c, "dH"), dev(c, "dhT") if final else None)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in grads.items()}


def _bwd_oracle(c, final):
    d = c.dims
    if c.cell == "lstm":
        return oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                               c.f64("c0"), c.f64("dH"), c.f64("dhT") if final else None,
                               c.f64("dcT") if final else None, NH=d.NH, Dh=d.Dh)
    return oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          c.f64("dH"), c.f64("dhT") if final else None, NH=d.NH, Dh=d.Dh)


@pytest.mark.parametrize("cell,T,B,NH,Dh,Din,final", [
    ("lstm", 64, 2, 1, 32, 32, False),   # the shape of the float32 tiny LSTM workload
    ("lstm", 19, 3, 2, 24, 20, True),    # several heads, ragged sizes, final-state gradients
    ("lstm", 9, 11, 3, 48, 16, True),    # three heads, two row tiles of the sweep
    ("gru", 64, 2, 1, 32, 32, False),
    ("gru", 23, 5, 2, 40, 12, True),
])
def test_backward_f32(cell, T, B, NH, Dh, Din, final):
    """float32 BPTT (every intermediate float32) against the oracle at the
    float32 bar, normwise 1e-5 on every gradient."""
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    bias = "forget+1" if cell == "lstm" else synth.normal(9800 + Dh, NH * 3 * Dh, 0.25)
    c = synth.make_case(cell, d, "f32", 9900 + T + Dh, bias=bias, h0_var=0.2,
                        c0_var=0.2 if cell == "lstm" else 0.0, backward=True, final_grads=final)
    got = _bwd_any(c, final)
    ref = _bwd_oracle(c, final)
    keys = ("dx", "dW", "dR", "db", "dh0", "dc0") if cell == "lstm" else ("dx", "dW", "dR", "db", "dh0")
    for k in keys:
        check(k, got[k], ref[k], TOL_F32)


@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_backward_f32_from_checkpoints_matches_one_piece(cell):
    """float32 BPTT from chunk checkpoints (segments recomputed, then their
    BPTT with the carries of the later segment): dx and the initial-state
    gradients are the bits of the one-piece call; dW, dR, db are sums over
    segments (float32 order differs)."""
    d = synth.Dims(T=40, B=3, Din=16, NH=2, Dh=32)
    lstm = cell == "lstm"
    c = synth.make_case(cell, d, "f32", 9990, bias="forget+1" if lstm else "zero", h0_var=0.2,
                        c0_var=0.2 if lstm else 0.0, backward=True)
    x, W, R, b, h0 = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0")
    chunk = 16
    if lstm:
        c0 = dev(c, "c0")
        fc = g.lstm_fwd_chunked(x, W, R, b, h0, c0, chunk=chunk, with_seq=False, ckpt=True)
        ck = g.lstm_bwd_ckpt(x, W, R, b, h0, c0, fc[4], fc[5], dev(c, "dH"), chunk=chunk)
    else:
        fc = g.gru_fwd_chunked(x, W, R, b, h0, chunk=chunk, with_seq=False, ckpt=True)
        ck = g.gru_bwd_ckpt(x, W, R, b, h0, fc[2], dev(c, "dH"), chunk=chunk)
    torch.cuda.synchronize()
    ck = {k: host(v) for k, v in ck.items()}
    one = _bwd_any(c, False)
    for k in ("dx", "dh0") + (("dc0",) if lstm else ()):
        assert np.array_equal(ck[k], one[k]), k
    ref = _bwd_oracle(c, False)
    for k in ck:
        check(k, ck[k], ref[k], TOL_F32)

"""GPU parity of stacked layers (rnn_fwd_lstm_stack / rnn_fwd_gru_stack)
against the stacked oracle: layer l > 0 reads layer l-1's h sequence,
rounded to bf16 in bf16 runs.  Bar: normwise 2e-2 (bf16) / 1e-5 (f32) on
the last layer's sequences and every layer's final states."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402


@pytest.fixture
def overlap_env():
    old = {k: os.environ.pop(k, None) for k in ("RNN355_STACK_OVERLAP", "RNN355_SPIN_LIMIT")}
    yield
    for k, v in old.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


def run(cs, **kw):
    Ws = [dev(c, "W") for c in cs]
    Rs = [dev(c, "R") for c in cs]
    bs = [dev(c, "b") for c in cs]
    L, c0 = len(cs), cs[0]
    h0 = torch.stack([dev(c, "h0") for c in cs])
    if c0.cell == "lstm":
        cst = torch.stack([dev(c, "c0") for c in cs])
        h_seq, c_seq, hT, cT = g.lstm_stack_fwd(dev(c0, "x"), Ws, Rs, bs, h0, cst, **kw)
        torch.cuda.synchronize()
        out = dict(hT=host(hT), cT=host(cT))
        if h_seq is not None:
            out.update(h_seq=host(h_seq), c_seq=host(c_seq))
        return out
    h_seq, hT = g.gru_stack_fwd(dev(c0, "x"), Ws, Rs, bs, h0, **kw)
    torch.cuda.synchronize()
    out = dict(hT=host(hT))
    if h_seq is not None:
        out["h_seq"] = host(h_seq)
    return out


def want(cs, mask=None):
    c0 = cs[0]
    d = c0.dims
    args = (c0.f64("x"), [c.f64("W") for c in cs], [c.f64("R") for c in cs],
            [c.f64("b") for c in cs], np.stack([c.f64("h0") for c in cs]))
    kw = dict(NH=d.NH, Dh=d.Dh, bf16_between=c0.dtype == "bf16", chain_mask=mask)
    if c0.cell == "lstm":
        return oracle.lstm_stack_fwd(*args, np.stack([c.f64("c0") for c in cs]), **kw)
    return oracle.gru_stack_fwd(*args, **kw)


@pytest.mark.parametrize("cell,L,NH,Dh,dtype,Din", [
    ("lstm", 2, 2, 64, "bf16", 64),
    ("lstm", 3, 2, 128, "bf16", 96),    # Din != H: the second layer's W is [H][N]
    ("lstm", 2, 1, 256, "bf16", 64),    # split-R recurrence in every layer
    ("lstm", 2, 2, 32, "f32", 48),      # f32: no rounding between layers
    ("gru", 2, 3, 64, "bf16", 64),
    ("gru", 3, 1, 256, "bf16", 32),
    ("gru", 2, 1, 32, "f32", 40),
])
def test_stack_forward(cell, L, NH, Dh, dtype, Din):
    d = synth.Dims(T=21, B=3, Din=Din, NH=NH, Dh=Dh)
    cs = synth.make_stack_case(cell, d, L, dtype, 9900 + 10 * L + Dh,
                               bias="forget+1" if cell == "lstm" else "zero",
                               h0_var=0.2, c0_var=0.2)
    got, ref = run(cs), want(cs)
    tol = 1e-5 if dtype == "f32" else 2e-2
    for k in got:
        check(k, got[k], ref[k], tol)


def test_one_layer_stack_is_the_forward_bitwise():
    d = synth.Dims(T=17, B=2, Din=32, NH=2, Dh=64)
    cs = synth.make_stack_case("lstm", d, 1, "bf16", 9950, bias="forget+1", h0_var=0.1, c0_var=0.1)
    s = run(cs)
    c = cs[0]
    h, cseq, hT, cT = g.lstm_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0"),
                                 dev(c, "c0"))
    torch.cuda.synchronize()
    assert np.array_equal(s["h_seq"], host(h))
    assert np.array_equal(s["cT"][0], host(cT))


def test_stack_final_states_only():
    d = synth.Dims(T=9, B=2, Din=32, NH=1, Dh=64)
    cs = synth.make_stack_case("gru", d, 2, "bf16", 9960, h0_var=0.1)
    a, b = run(cs), run(cs, with_seq=False)
    assert np.array_equal(a["hT"], b["hT"]) and "h_seq" not in b


@pytest.mark.parametrize("overlap", ["1", "0"])
def test_two_layer_headline_stack_full_size_sampled_rows(overlap_env, overlap):
    """Two stacked layers at the headline shape (B=16, NH=6, Dh=128, T=1024,
    Din=768); the oracle computes whole batch rows 0 and 9 (every head)."""
    os.environ["RNN355_STACK_OVERLAP"] = overlap
    w = synth.WORKLOADS["lstm_stack2_b16_nh6_dh128"]
    cs = synth.workload_stack_case(w)
    got = run(cs)
    rows = [0, 9]
    mask = np.zeros((w.dims.B, w.dims.NH), bool)
    mask[rows] = True
    ref = want(cs, mask)
    for k in ("h_seq", "c_seq"):
        e = nerr(got[k][:, rows], ref[k][:, rows])
        print("  %-6s nerr=%.3e" % (k, e), flush=True)
        assert e <= 2e-2, (k, e)
    for k in ("hT", "cT"):
        e = nerr(got[k][:, rows], ref[k][:, rows])
        print("  %-6s nerr=%.3e" % (k, e), flush=True)
        assert e <= 2e-2, (k, e)


@pytest.mark.parametrize("cell,L,T,B,NH,Din", [
    ("lstm", 2, 21, 3, 2, 96),      # one row panel
    ("lstm", 3, 100, 5, 1, 64),     # two panels, ragged; the third layer runs alone
    ("lstm", 4, 37, 8, 3, 128),     # two overlapped pairs
    ("gru", 2, 70, 4, 2, 32),
    ("gru", 3, 9, 2, 1, 128),
])
def test_overlapped_pairs_match_oracle_and_layers_in_turn(overlap_env, cell, L, T, B, NH, Din):
    """Dh = 128 bf16 stacks run two layers per launch (layer l+1's projection
    and recurrence beside layer l's); RNN355_STACK_OVERLAP=0 runs them in
    turn.  Same kernels, same summation order: equal bits."""
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=128)
    cs = synth.make_stack_case(cell, d, L, "bf16", 9700 + 7 * T + L,
                               bias="forget+1" if cell == "lstm" else "zero",
                               h0_var=0.2, c0_var=0.2)
    got = run(cs)
    os.environ["RNN355_STACK_OVERLAP"] = "0"
    seq = run(cs)
    ref = want(cs)
    for k in got:
        e = nerr(got[k], ref[k])
        print("  %-6s nerr=%.3e" % (k, e), flush=True)
        assert e <= 2e-2, (k, e)
        assert np.array_equal(got[k], seq[k]), k


def test_overlapped_pair_timeout_is_reported_and_cleared(overlap_env):
    """A spin limit of one poll (set from the host) makes the projection's
    wait for layer 0's steps give up: every workgroup stops, the launch ends
    normally and the workspace reports the time-out; the next call clears
    it and is right again."""
    d = synth.Dims(T=64, B=4, Din=64, NH=2, Dh=128)
    cs = synth.make_stack_case("lstm", d, 2, "bf16", 9800, bias="forget+1")
    need = g.workspace_size_stack(g.OP_FWD_LSTM, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), 2,
                                  g.RNN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    os.environ["RNN355_SPIN_LIMIT"] = "1"
    run(cs, ws=ws)
    assert g.workspace_status(ws) == g.RNN_ERR_BARRIER_TIMEOUT
    os.environ.pop("RNN355_SPIN_LIMIT")
    got = run(cs, ws=ws)
    assert g.workspace_status(ws) == g.RNN_OK
    assert nerr(got["h_seq"], want(cs)["h_seq"]) <= 2e-2

"""GPU parity of forward and backward on a seeded set of random shapes.

Cells, head widths (32 .. 384), head counts, batch rows, sequence lengths and
input widths are drawn from a fixed seed, so the set is the same on every
run; among them are ragged lengths and batches, inputs not a multiple of 32
wide (register-staged projection), and (heads x rows) products that do and do
not divide by 8 (the XCD-grouped multi-CU and two-CU paths against the
others).  Each case: the forward (h_seq, hT, cT) and the BPTT gradients
(dx, dW, dR, db, dh0, dc0) against the oracle, normwise 2e-2 (bf16
operands, f32 accumulation), and the workspace status."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402

TOL = 2e-2


def _shapes(n=14, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        cell = ["lstm", "gru"][int(rng.integers(0, 2))]
        Dh = int(rng.choice([32, 64, 128, 256, 384]))
        NH = int(rng.integers(1, 5))
        B = int(rng.integers(1, 9))
        T = int(rng.integers(1, 41))
        Din = int(rng.choice([16, 24, 32, 64, 96]))
        if Dh == 384 and NH * B > 4:  # keep the 384-wide oracle cases small
            continue
        out.append((cell, T, B, NH, Dh, Din))
    return out


# plus shapes the draw may miss: Dh = 256 with (heads x rows) % 8 == 0 (the
# two-CU backward sweep, the XCD-grouped multi-CU forward) and a 384-wide
# head tile group of 8
SHAPES = _shapes() + [("lstm", 23, 4, 2, 256, 48), ("gru", 19, 8, 1, 256, 32),
                      ("lstm", 9, 8, 1, 384, 32)]


@pytest.mark.parametrize("cell,T,B,NH,Dh,Din", SHAPES)
def test_random_shape_forward_and_backward(cell, T, B, NH, Dh, Din):
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    lstm = cell == "lstm"
    seed = 11000 + 7 * T + 13 * B + 17 * NH + Dh + Din
    c = synth.make_case(cell, d, "bf16", seed, bias="forget+1" if lstm else "zero",
                        h0_var=0.2, c0_var=0.2 if lstm else 0.0, backward=True,
                        final_grads=True)
    gd = g.Dims(T, B, Din, NH, Dh)
    fop, bop = (g.OP_FWD_LSTM, g.OP_BWD_LSTM) if lstm else (g.OP_FWD_GRU, g.OP_BWD_GRU)
    print("  plan:", g.plan_describe(fop, gd, g.RNN_BF16), flush=True)
    wf = torch.empty(g.workspace_size(fop, gd, g.RNN_BF16), dtype=torch.uint8, device="cuda")
    wb = torch.empty(g.workspace_size(bop, gd, g.RNN_BF16), dtype=torch.uint8, device="cuda")
    x, W, R, b, h0 = (dev(c, k) for k in ("x", "W", "R", "b", "h0"))
    if lstm:
        c0 = dev(c, "c0")
        h_seq, c_seq, hT, cT = g.lstm_fwd(x, W, R, b, h0, c0, ws=wf)
        fwd = dict(h_seq=h_seq, c_seq=c_seq, hT=hT, cT=cT)
        grads = g.lstm_bwd(x, W, R, b, h0, c0, h_seq, c_seq, dev(c, "dH"), dev(c, "dhT"),
                           dev(c, "dcT"), ws=wb)
    else:
        h_seq, hT = g.gru_fwd(x, W, R, b, h0, ws=wf)
        fwd = dict(h_seq=h_seq, hT=hT)
        grads = g.gru_bwd(x, W, R, b, h0, h_seq, dev(c, "dH"), dev(c, "dhT"), ws=wb)
    torch.cuda.synchronize()
    assert g.workspace_status(wf) == g.RNN_OK
    assert g.workspace_status(wb) == g.RNN_OK
    args = (c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"))
    if lstm:
        ref_f = oracle.lstm_fwd(*args, c.f64("c0"), NH=NH, Dh=Dh)
        ref_b = oracle.lstm_bwd(*args, c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"),
                                NH=NH, Dh=Dh)
    else:
        ref_f = oracle.gru_fwd(*args, NH=NH, Dh=Dh)
        ref_b = oracle.gru_bwd(*args, c.f64("dH"), c.f64("dhT"), NH=NH, Dh=Dh)
    for k, v in fwd.items():
        e = nerr(host(v), ref_f[k])
        print("  fwd %-6s nerr=%.3e" % (k, e), flush=True)
        assert e <= TOL, (k, e)
    for k, v in grads.items():
        e = nerr(host(v), ref_b[k])
        print("  bwd %-4s nerr=%.3e" % (k, e), flush=True)
        assert e <= TOL, (k, e)


def _long_shapes(n=8, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        cell = ["lstm", "gru"][int(rng.integers(0, 2))]
        Dh = int(rng.choice([32, 64, 128, 256]))
        NH = int(rng.integers(1, 5))
        B = int(rng.integers(1, 9))
        T = int(rng.integers(256, 701))
        Din = int(rng.choice([32, 64, 96, 128]))
        out.append((cell, T, B, NH, Dh, Din))
    return out


@pytest.mark.parametrize("cell,T,B,NH,Dh,Din", _long_shapes())
def test_random_long_shape_chunked_against_one_piece(cell, T, B, NH, Dh, Din):
    """Sequences of 256-700 steps, where the backward sweeps in time chunks
    with the gradients on side streams and the forward may run pipelined:
    the backward's dx, dh0 (dc0) are bitwise those of the sweep in one piece
    and dW, dR, db agree to float32 rounding; the forward is bitwise the
    serial one."""
    import os
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    lstm = cell == "lstm"
    c = synth.make_case(cell, d, "bf16", 12000 + 7 * T + 13 * B + 17 * NH + Dh + Din,
                        bias="forget+1" if lstm else "zero", h0_var=0.2,
                        c0_var=0.2 if lstm else 0.0, backward=True, final_grads=True)
    x, W, R, b, h0 = (dev(c, k) for k in ("x", "W", "R", "b", "h0"))
    c0 = dev(c, "c0") if lstm else None

    def fwd():
        return g.lstm_fwd(x, W, R, b, h0, c0) if lstm else g.gru_fwd(x, W, R, b, h0)

    def bwd(f):
        if lstm:
            return g.lstm_bwd(x, W, R, b, h0, c0, f[0], f[1], dev(c, "dH"), dev(c, "dhT"),
                              dev(c, "dcT"))
        return g.gru_bwd(x, W, R, b, h0, f[0], dev(c, "dH"), dev(c, "dhT"))

    keys = ("RNN355_PIPELINE", "RNN355_BWD_OVERLAP")
    old = {k: os.environ.pop(k, None) for k in keys}
    try:
        f = fwd()
        gch = {k: host(v) for k, v in bwd(f).items()}
        os.environ["RNN355_PIPELINE"] = "0"
        os.environ["RNN355_BWD_OVERLAP"] = "0"
        fs = fwd()
        g1 = {k: host(v) for k, v in bwd(fs).items()}
    finally:
        for k in keys:
            os.environ.pop(k, None)
            if old[k] is not None:
                os.environ[k] = old[k]
    torch.cuda.synchronize()
    for a, e in zip(f, fs):
        assert torch.equal(a, e)
    for k in ("dx", "dh0") + (("dc0",) if lstm else ()):
        assert np.array_equal(gch[k], g1[k]), k
    for k in ("dW", "dR", "db"):
        e = nerr(gch[k], g1[k])
        print("  %-3s chunked vs one piece nerr=%.2e" % (k, e), flush=True)
        assert e <= 1e-5, (k, e)

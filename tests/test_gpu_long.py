"""GPU parity of the long-sequence calls: the forward in chunks
(rnn_fwd_*_chunked) gives the same bits as the forward in one piece, and
its checkpoints are the states at the chunk ends; BPTT from checkpoints
(rnn_bwd_*_ckpt) gives the same dx, dh0, dc0 bits as BPTT over the stored
sequences, parameter gradients equal up to float32 summation order, and
every gradient within the backward's bar of the oracle."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402


@pytest.fixture(autouse=True)
def _clean_env():
    keys = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_WIDE", "RNN355_PIPELINE")
    old = {k: os.environ.pop(k, None) for k in keys}
    yield
    for k in keys:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def inputs(c):
    return [dev(c, k) for k in ("x", "W", "R", "b", "h0")] + \
        ([dev(c, "c0")] if c.cell == "lstm" else [])


def whole(c):
    t = inputs(c)
    if c.cell == "lstm":
        h, cs, hT, cT = g.lstm_fwd(*t)
        return dict(h_seq=h, c_seq=cs, hT=hT, cT=cT)
    h, hT = g.gru_fwd(*t)
    return dict(h_seq=h, hT=hT)


def chunked(c, chunk):
    t = inputs(c)
    if c.cell == "lstm":
        h, cs, hT, cT, hk, ck = g.lstm_fwd_chunked(*t, chunk=chunk)
        return dict(h_seq=h, c_seq=cs, hT=hT, cT=cT, h_ckpt=hk, c_ckpt=ck)
    h, hT, hk = g.gru_fwd_chunked(*t, chunk=chunk)
    return dict(h_seq=h, hT=hT, h_ckpt=hk)


@pytest.mark.parametrize("cell,T,B,NH,Dh,Din,dtype,chunk,env", [
    ("lstm", 37, 3, 2, 128, 64, "bf16", 10, None),    # one-CU MFMA kernel, ragged last chunk
    ("lstm", 50, 5, 1, 64, 96, "bf16", 16, None),
    ("lstm", 21, 3, 2, 256, 64, "bf16", 8, None),     # split-R kernel
    ("lstm", 13, 2, 1, 256, 32, "bf16", 5, "0"),      # multi-CU kernel (RNN355_REC_WIDE=0)
    ("lstm", 30, 2, 1, 32, 40, "f32", 7, None),       # f32 LDS kernel, register-staged projection
    ("lstm", 9, 2, 2, 64, 24, "bf16", 100, None),     # one chunk longer than T; Din % 32 != 0
    ("gru", 33, 4, 2, 64, 64, "bf16", 11, None),
    ("gru", 5, 2, 1, 128, 32, "bf16", 1, None),       # one step per chunk
    ("gru", 20, 3, 1, 256, 64, "bf16", 6, None),
    # 64 chains at Dh = 256: the multi-CU plan takes every CU, so each
    # chunk's projection runs on the whole chip in order on the caller's stream
    ("lstm", 21, 16, 4, 256, 64, "bf16", 8, None),
    ("gru", 19, 16, 4, 256, 32, "bf16", 7, None),
])
def test_chunked_forward_is_the_forward_bitwise(cell, T, B, NH, Dh, Din, dtype, chunk, env):
    if env is not None:
        os.environ["RNN355_REC_WIDE"] = env
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    c = synth.make_case(cell, d, dtype, 7100 + T + Dh, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2)
    a = {k: host(v) for k, v in whole(c).items()}
    b = {k: host(v) for k, v in chunked(c, chunk).items()}
    torch.cuda.synchronize()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    ends = [min((k + 1) * chunk, T) - 1 for k in range((T + chunk - 1) // chunk)]
    assert np.array_equal(b["h_ckpt"], a["h_seq"][ends])
    if cell == "lstm":
        assert np.array_equal(b["c_ckpt"], a["c_seq"][ends])
    ref = (oracle.lstm_fwd if cell == "lstm" else oracle.gru_fwd)(
        *[c.f64(k) for k in (["x", "W", "R", "b", "h0"] + (["c0"] if cell == "lstm" else []))],
        NH=NH, Dh=Dh)
    e = nerr(b["h_seq"], ref["h_seq"])
    print("  h_seq nerr vs oracle %.3e" % e, flush=True)
    assert e <= (1e-5 if dtype == "f32" else 2e-2)


def test_chunked_forward_without_sequences_or_checkpoints():
    d = synth.Dims(T=23, B=2, Din=32, NH=2, Dh=128)
    c = synth.make_case("lstm", d, "bf16", 7200, bias="forget+1")
    a = {k: host(v) for k, v in whole(c).items()}
    _, _, hT, cT, hk, ck = g.lstm_fwd_chunked(*inputs(c), chunk=4, with_seq=False, ckpt=False)
    torch.cuda.synchronize()
    assert hk is None and ck is None
    assert np.array_equal(host(hT), a["hT"]) and np.array_equal(host(cT), a["cT"])


def _bwd_both(c, chunk, final):
    t = inputs(c)
    dH = dev(c, "dH")
    lstm = c.cell == "lstm"
    fin = [dev(c, "dhT"), dev(c, "dcT")] if final and lstm else ([dev(c, "dhT")] if final else [])
    if lstm:
        h, cs, _, _ = g.lstm_fwd(*t)
        full = g.lstm_bwd(*t, h, cs, dH, *fin)
        _, _, _, _, hk, ck = g.lstm_fwd_chunked(*t, chunk=chunk, with_seq=False)
        ck_g = g.lstm_bwd_ckpt(*t, hk, ck, dH, *fin, chunk=chunk)
    else:
        h, _ = g.gru_fwd(*t)
        full = g.gru_bwd(*t, h, dH, *fin)
        _, _, hk = g.gru_fwd_chunked(*t, chunk=chunk, with_seq=False)
        ck_g = g.gru_bwd_ckpt(*t, hk, dH, *fin, chunk=chunk)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in full.items()}, {k: host(v) for k, v in ck_g.items()}


@pytest.mark.parametrize("cell,T,B,NH,Dh,chunk,final", [
    ("lstm", 40, 3, 2, 128, 16, True),     # ragged last segment
    ("lstm", 19, 3, 2, 256, 5, False),     # split-R sweep
    ("lstm", 24, 2, 2, 64, 24, True),      # one segment
    ("gru", 31, 4, 2, 64, 8, True),
    ("gru", 17, 3, 1, 256, 6, False),
    ("lstm", 19, 16, 4, 256, 8, True),     # multi-CU forward recompute (every CU)
    ("lstm", 1100, 4, 2, 128, 550, True),  # each segment's sweep in four chunks
    ("gru", 600, 3, 2, 64, 300, True),     # GRU segments swept in two chunks each
])
def test_checkpointed_backward(cell, T, B, NH, Dh, chunk, final):
    d = synth.Dims(T=T, B=B, Din=64, NH=NH, Dh=Dh)
    c = synth.make_case(cell, d, "bf16", 7300 + T + Dh, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2, backward=True, final_grads=final)
    full, ck = _bwd_both(c, chunk, final)
    exact = ("dx", "dh0", "dc0") if cell == "lstm" else ("dx", "dh0")
    for k in exact:
        assert np.array_equal(full[k], ck[k]), k
    for k in ("dW", "dR", "db"):
        e = nerr(ck[k], full[k])
        print("  %-3s nerr vs one-piece BPTT %.2e" % (k, e), flush=True)
        assert e <= 1e-5, (k, e)
    args = [c.f64(k) for k in (["x", "W", "R", "b", "h0"] + (["c0"] if cell == "lstm" else []))]
    args.append(c.f64("dH"))
    if final:
        args += [c.f64("dhT")] + ([c.f64("dcT")] if cell == "lstm" else [])
    ref = (oracle.lstm_bwd if cell == "lstm" else oracle.gru_bwd)(*args, NH=NH, Dh=Dh)
    for k in ("dx", "dW", "dR", "db", "dh0") + (("dc0",) if cell == "lstm" else ()):
        e = nerr(ck[k], ref[k])
        print("  %-3s nerr vs oracle %.3e" % (k, e), flush=True)
        assert e <= 2e-2, (k, e)


def test_long_workload_full_size():
    """The 8192-step workload in chunks of 1024: the same bits as the forward
    in one piece, and two chains against the oracle."""
    w = synth.WORKLOADS["lstm_long_t8k_b16_nh6_dh128"]
    c = synth.workload_case(w)
    a = {k: host(v) for k, v in whole(c).items()}
    b = {k: host(v) for k, v in chunked(c, w.chunk).items()}
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    mask = np.zeros((w.dims.B, w.dims.NH), bool)
    mask[3, 1] = mask[14, 5] = True
    ref = oracle.lstm_fwd(*[c.f64(k) for k in ("x", "W", "R", "b", "h0", "c0")],
                          NH=w.dims.NH, Dh=w.dims.Dh, chain_mask=mask)
    Dh = w.dims.Dh
    for bb, n in ((3, 1), (14, 5)):
        sl = slice(n * Dh, (n + 1) * Dh)
        for k in ("h_seq", "c_seq"):
            e = nerr(b[k][:, bb, sl], ref[k][:, bb, sl])
            print("  chain (%d, %d) %s nerr=%.3e" % (bb, n, k, e), flush=True)
            assert e <= 2e-2

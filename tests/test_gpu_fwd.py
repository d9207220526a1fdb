"""GPU parity of the forward path (input projection + recurrence) against the
CPU oracle, through the C ABI.  Bars: normwise error max|y-y*|/max|y*| of at
most 1e-5 for float32 calls and 2e-2 for bf16 calls (bf16 x, W, R, float32
accumulation and state); 1e-4 for the input projection alone (exact bf16
operands, float32 sums of Din products)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, host, nerr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gru_recurrence_amd as g  # noqa: E402

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(autouse=True)
def _no_plan_override():
    keys = ("RNN355_REC_BT", "RNN355_PIPELINE", "RNN355_HEAD_START", "RNN355_FUSED_TAPER")
    old = {k: os.environ.pop(k, None) for k in keys}
    yield
    for k in keys:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def run_lstm(c, **kw):
    h_seq, c_seq, hT, cT = g.lstm_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"),
                                      dev(c, "h0"), dev(c, "c0"), **kw)
    torch.cuda.synchronize()
    return dict(h_seq=host(h_seq), c_seq=host(c_seq), hT=host(hT), cT=host(cT))


def run_gru(c, **kw):
    h_seq, hT = g.gru_fwd(dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0"), **kw)
    torch.cuda.synchronize()
    return dict(h_seq=host(h_seq), hT=host(hT))


def oracle_of(c, mask=None):
    d = c.dims
    if c.cell == "lstm":
        return oracle.lstm_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                               c.f64("c0"), NH=d.NH, Dh=d.Dh, chain_mask=mask)
    return oracle.gru_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          NH=d.NH, Dh=d.Dh, chain_mask=mask)


def compare(got, want, tol, keys):
    for k in keys:
        check(k, got[k], want[k], tol)


def test_lstm_fp32_tiny_workload_full():
    """The fp32 tiny LSTM workload (T=64, B=2, NH=1, Dh=32, Din=32) in full."""
    c = synth.workload_case(synth.WORKLOADS["lstm_fp32_tiny"])
    compare(run_lstm(c), oracle_of(c), TOL_F32, ("h_seq", "c_seq", "hT", "cT"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N", [(185, 96, 384), (128, 64, 128), (300, 768, 288)])
def test_input_projection(M, K, N, dtype):
    d = synth.Dims(T=M, B=1, Din=K, NH=1, Dh=N // 4)
    c = synth.make_case("lstm", d, dtype, 4242 + M, bias=synth.normal(99, N, 1.0))
    gx = g.input_proj(dev(c, "x"), dev(c, "W"), dev(c, "b"))
    torch.cuda.synchronize()
    want = oracle.input_proj(c.f64("x"), c.f64("W"), c.f64("b"))
    e = nerr(host(gx).reshape(M, N), want)
    print("  gx nerr=%.3e" % e, flush=True)
    assert e <= (1e-4 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("M,K,N", [(185, 96, 384), (300, 768, 288), (2048, 64, 1000),
                                   (1, 32, 8), (4096, 1024, 4096)])
def test_input_projection_transposed_weights(M, K, N):
    """k-major contraction (weights given transposed, tiles loaded straight
    into LDS): matches the oracle, and bitwise the contraction on W as it is
    (same k order).  Covers ragged row and column tiles, a single row, and a
    K of 32 k-tiles in flight through the four-stage ring."""
    d = synth.Dims(T=M, B=1, Din=K, NH=1, Dh=max(N // 4, 1))
    c = synth.make_case("lstm", d, "bf16", 4300 + M, w_var=1.0 / K)
    x = dev(c, "x")
    Wf = torch.from_numpy(synth.normal(4400 + N, K * N, 1.0 / K).reshape(K, N))
    W = Wf.to(torch.bfloat16).to("cuda")
    b = torch.from_numpy(synth.normal(4500 + N, N, 1.0)).float().to("cuda")
    gt = g.input_proj_t(x, W.t().contiguous(), b)
    gr = g.input_proj(x, W, b)
    torch.cuda.synchronize()
    assert torch.equal(gt, gr)
    rows = np.unique(np.r_[0, M - 1, np.arange(0, M, max(1, M // 37))])
    want = oracle.input_proj(c.f64("x"), W.float().cpu().numpy().astype(np.float64),
                             b.cpu().numpy().astype(np.float64), rows=rows)
    e = nerr(host(gt).reshape(M, N)[rows], want)
    print("  gx nerr=%.3e (%d rows)" % (e, len(rows)), flush=True)
    assert e <= 1e-4


@pytest.mark.parametrize("Dh", [32, 64, 128])
@pytest.mark.parametrize("bt", [None, 1, 3, 16])
def test_lstm_bf16_tiles_and_ragged(Dh, bt):
    """T=37, B=5 (ragged against every batch tile), NH=3, Din=96 (M=185 rows
    and N=12*Dh columns end in partial GEMM tiles)."""
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=37, B=5, Din=96, NH=3, Dh=Dh)
    c = synth.make_case("lstm", d, "bf16", 5000 + Dh, bias="forget+1", h0_var=0.2, c0_var=0.2)
    compare(run_lstm(c), oracle_of(c), TOL_BF16, ("h_seq", "c_seq", "hT", "cT"))


@pytest.mark.parametrize("Dh", [32, 64, 128])
@pytest.mark.parametrize("bt", [None, 2, 16])
def test_gru_bf16_tiles_and_ragged(Dh, bt):
    if bt is not None:
        os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=41, B=6, Din=64, NH=2, Dh=Dh)
    c = synth.make_case("gru", d, "bf16", 6000 + Dh, h0_var=0.1)
    compare(run_gru(c), oracle_of(c), TOL_BF16, ("h_seq", "hT"))


@pytest.mark.parametrize("cell", ["lstm", "gru"])
@pytest.mark.parametrize("Dh", [32, 64, 128])
@pytest.mark.parametrize("bt", [2, 4, 5, 8, 9, 16])
def test_rows_per_workgroup_layouts(cell, Dh, bt):
    """Batch tiles of the one-CU kernel in every row layout: 2 to 4 rows (one
    cell update pass over rows in lane groups), 5 to 8 (two passes), 9 to 16
    (four register row slots); B = 13 leaves a ragged last tile."""
    os.environ["RNN355_REC_BT"] = str(bt)
    d = synth.Dims(T=23, B=13, Din=64, NH=2, Dh=Dh)
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    plan = g.plan_describe(op, g.Dims(d.T, d.B, d.Din, d.NH, d.Dh), g.RNN_BF16)
    print("  plan:", plan, flush=True)
    rows = min(bt, d.B)
    assert "mfma_resident_R rows_per_wg=%d " % rows in plan
    passes = 1 if rows <= 4 else 2 if rows <= 8 else 4
    assert "units_per_thread=%d " % passes in plan
    c = synth.make_case(cell, d, "bf16", 5300 + 7 * bt + Dh, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.2, c0_var=0.2 if cell == "lstm" else 0.0)
    got = run_lstm(c) if cell == "lstm" else run_gru(c)
    keys = ("h_seq", "c_seq", "hT", "cT") if cell == "lstm" else ("h_seq", "hT")
    compare(got, oracle_of(c), TOL_BF16, keys)


@pytest.mark.parametrize("cell,dtype,Dh", [("gru", "f32", 32), ("lstm", "f32", 48),
                                           ("lstm", "bf16", 48), ("gru", "bf16", 16)])
def test_lds_kernel_shapes(cell, dtype, Dh):
    """Shapes outside the MFMA kernel run on the LDS kernel (R as float32)."""
    d = synth.Dims(T=19, B=3, Din=40 if dtype == "bf16" else 20, NH=2, Dh=Dh)
    c = synth.make_case(cell, d, dtype, 7000 + Dh, h0_var=0.2, c0_var=0.2)
    got = run_lstm(c) if cell == "lstm" else run_gru(c)
    keys = ("h_seq", "c_seq", "hT", "cT") if cell == "lstm" else ("h_seq", "hT")
    compare(got, oracle_of(c), TOL_F32 if dtype == "f32" else TOL_BF16, keys)


def test_single_step_single_row_single_head():
    d = synth.Dims(T=1, B=1, Din=8, NH=1, Dh=32)
    c = synth.make_case("lstm", d, "bf16", 7100, h0_var=0.5, c0_var=0.5)
    compare(run_lstm(c), oracle_of(c), TOL_BF16, ("h_seq", "c_seq", "hT", "cT"))


def test_run_to_run_bitwise_and_resume():
    d = synth.Dims(T=30, B=4, Din=64, NH=2, Dh=64)
    c = synth.make_case("lstm", d, "bf16", 7200, bias="forget+1", h0_var=0.1, c0_var=0.1)
    a = run_lstm(c)
    b = run_lstm(c)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    # two chunks chained through (hT, cT) equal one call, bitwise
    x, W, R, bb = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b")
    h1, c1, hT1, cT1 = g.lstm_fwd(x[:11].contiguous(), W, R, bb, dev(c, "h0"), dev(c, "c0"))
    h2, c2, hT2, cT2 = g.lstm_fwd(x[11:].contiguous(), W, R, bb, hT1, cT1)
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate([host(h1), host(h2)]), a["h_seq"])
    assert np.array_equal(host(cT2), a["cT"])


def test_head_and_batch_independence_bitwise():
    d = synth.Dims(T=20, B=4, Din=64, NH=3, Dh=32)
    c = synth.make_case("gru", d, "bf16", 7300, h0_var=0.1)
    base = run_gru(c)
    c.vals["h0"][:, 32:64] += 0.5      # head 1 state
    c.vals["h0"][3] -= 0.5             # batch row 3
    c.bits.pop("R")
    c.vals["R"] = c.vals["R"].copy()
    c.vals["R"][1] *= -1.0             # head 1 weights (stays exact in bf16)
    c.bits["R"] = synth.f32_to_bf16_bits(c.vals["R"])
    pert = run_gru(c)
    keep_h = np.r_[0:32, 64:96]
    assert np.array_equal(pert["h_seq"][:, :3][..., keep_h], base["h_seq"][:, :3][..., keep_h])
    assert not np.array_equal(pert["h_seq"][:, 3], base["h_seq"][:, 3])


def test_recurrence_entry_matches_fused_forward():
    d = synth.Dims(T=25, B=3, Din=32, NH=2, Dh=64)
    c = synth.make_case("lstm", d, "bf16", 7400, bias="forget+1")
    full = run_lstm(c)
    gx = g.input_proj(dev(c, "x"), dev(c, "W"), dev(c, "b"))
    h, cs, hT, cT = g.rec_lstm(gx, dev(c, "R"), dev(c, "h0"), dev(c, "c0"))
    torch.cuda.synchronize()
    assert np.array_equal(host(h), full["h_seq"])
    assert np.array_equal(host(cT), full["cT"])


def test_headline_lstm_workload_full_size_every_chain():
    """Multi-head LSTM B=16, NH=6, Dh=128, T=1024, Din=768 at full size in the
    default launch configuration (the projection overlapped with the
    recurrence in one launch); the oracle computes all 96 chains and every
    output is compared."""
    w = synth.WORKLOADS["lstm_mh_b16_nh6_dh128"]
    c = synth.workload_case(w)
    got = run_lstm(c)
    want = oracle_of(c)
    for k in ("h_seq", "c_seq", "hT", "cT"):
        check(k, got[k], want[k], TOL_BF16)


def test_gru_small_batch_workload_full_size_every_chain():
    """Multi-head GRU B=4, NH=12, Dh=64, T=2048, Din=768 at full size; all 48
    chains against the oracle."""
    w = synth.WORKLOADS["gru_mh_b4_nh12_dh64"]
    c = synth.workload_case(w)
    got = run_gru(c)
    want = oracle_of(c)
    for k in ("h_seq", "hT"):
        check(k, got[k], want[k], TOL_BF16)


def _with_env(key, val, fn):
    old = os.environ.get(key)
    os.environ[key] = val
    try:
        return fn()
    finally:
        if old is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = old


@pytest.mark.parametrize("cell,T,B,NH,Dh,Din", [
    ("lstm", 233, 5, 2, 128, 96),    # 1165 rows: 5 row panels, the last one ragged
    ("gru", 300, 16, 3, 128, 64),    # 19 row panels, 16 rows per step
    ("lstm", 96, 11, 4, 128, 32),    # 1056 rows, steps straddle panel edges
])
def test_pipelined_forward_matches_serial_bitwise_and_oracle(cell, T, B, NH, Dh, Din):
    """The forward that overlaps the input projection with the recurrence in
    one launch (row panels published by the projection's workgroups, waited
    on by the recurrence's) gives bitwise the serial result, and that result
    matches the oracle."""
    d = synth.Dims(T=T, B=B, Din=Din, NH=NH, Dh=Dh)
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    gd = g.Dims(T, B, Din, NH, Dh)
    assert "input_proj=serial" in g.plan_describe(op, gd, g.RNN_BF16)   # too small to pay
    assert "input_proj=pipelined" in _with_env("RNN355_PIPELINE", "1",
                                               lambda: g.plan_describe(op, gd, g.RNN_BF16))
    c = synth.make_case(cell, d, "bf16", 7500 + T, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.1, c0_var=0.1 if cell == "lstm" else 0.0)
    run = run_lstm if cell == "lstm" else run_gru
    piped = _with_env("RNN355_PIPELINE", "1", lambda: run(c))
    serial = _with_env("RNN355_PIPELINE", "0", lambda: run(c))
    for k in piped:
        assert np.array_equal(piped[k], serial[k]), k
    keys = ("h_seq", "c_seq", "hT", "cT") if cell == "lstm" else ("h_seq", "hT")
    compare(piped, oracle_of(c), TOL_BF16, keys)


@pytest.mark.parametrize("cell", ["lstm", "gru"])
@pytest.mark.parametrize("bt", [3, 8, 12])
def test_pipelined_forward_row_layouts_match_serial_bitwise(cell, bt):
    """The one-launch forward with several batch rows per recurrence
    workgroup (rows in lane groups, one and two passes; register row slots)
    gives bitwise the serial result, which matches the oracle."""
    d = synth.Dims(T=70, B=24, Din=64, NH=2, Dh=128)
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    gd = g.Dims(d.T, d.B, d.Din, d.NH, d.Dh)
    os.environ["RNN355_REC_BT"] = str(bt)
    plan = _with_env("RNN355_PIPELINE", "1", lambda: g.plan_describe(op, gd, g.RNN_BF16))
    print("  plan:", plan, flush=True)
    assert "rows_per_wg=%d " % bt in plan and "input_proj=pipelined" in plan
    c = synth.make_case(cell, d, "bf16", 7700 + bt, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.1, c0_var=0.1 if cell == "lstm" else 0.0)
    run = run_lstm if cell == "lstm" else run_gru
    piped = _with_env("RNN355_PIPELINE", "1", lambda: run(c))
    serial = _with_env("RNN355_PIPELINE", "0", lambda: run(c))
    for k in piped:
        assert np.array_equal(piped[k], serial[k]), k
    keys = ("h_seq", "c_seq", "hT", "cT") if cell == "lstm" else ("h_seq", "hT")
    compare(piped, oracle_of(c), TOL_BF16, keys)


@pytest.mark.parametrize("cell,T,B,Din,bt,hs,Dh", [
    ("lstm", 200, 16, 256, 1, 4, 128),   # 64 steps x 1 row: two whole row blocks
    ("gru", 150, 8, 128, 1, 1, 128),     # 32 steps x 1 row: one row block
    ("lstm", 120, 48, 128, 1, 3, 128),   # 16 steps x 1 row: a partial row block
    ("gru", 90, 32, 128, 3, 1, 128),     # 8 steps x 3 rows; the last batch tile has 2
    ("lstm", 100, 32, 256, 2, 4, 128),   # 32 steps x 2 rows (rows in lane groups)
    ("lstm", 120, 16, 96, 1, 2, 128),    # three K tiles, fewer than the ring's stages
    ("gru", 300, 4, 256, 1, 1, 64),      # Dh 64 (four waves): 64 steps x 1 row
    ("lstm", 200, 8, 128, 1, 1, 64),     # Dh 64: 32 steps, x resident in LDS
    ("lstm", 150, 16, 96, 2, 2, 64),     # Dh 64: 32 steps x 2 rows, three K tiles
    ("gru", 200, 8, 64, 1, 0, 64),       # Dh 64 one-launch forward without a head start
])
def test_pipelined_forward_head_start_matches_serial_bitwise(cell, T, B, Din, bt, hs, Dh):
    """The one-launch forward whose recurrence workgroups compute the first
    row panels of gx themselves (the projection skipping them) gives bitwise
    the serial result, which matches the oracle: whole and partial 32-row
    blocks, one to three batch rows per workgroup, LSTM and GRU, Dh 128 (eight
    waves) and 64 (four of a workgroup's eight waves)."""
    d = synth.Dims(T=T, B=B, Din=Din, NH=2, Dh=Dh)
    op = g.OP_FWD_LSTM if cell == "lstm" else g.OP_FWD_GRU
    gd = g.Dims(d.T, d.B, d.Din, d.NH, d.Dh)
    os.environ["RNN355_REC_BT"] = str(bt)
    os.environ["RNN355_HEAD_START"] = str(hs)
    plan = _with_env("RNN355_PIPELINE", "1", lambda: g.plan_describe(op, gd, g.RNN_BF16))
    print("  plan:", plan, flush=True)
    assert "rows_per_wg=%d " % bt in plan and "input_proj=pipelined" in plan
    assert "head_start_panels=%d" % hs in plan
    c = synth.make_case(cell, d, "bf16", 7900 + T, bias="forget+1" if cell == "lstm" else "zero",
                        h0_var=0.1, c0_var=0.1 if cell == "lstm" else 0.0)
    run = run_lstm if cell == "lstm" else run_gru
    piped = _with_env("RNN355_PIPELINE", "1", lambda: run(c))
    serial = _with_env("RNN355_PIPELINE", "0", lambda: run(c))
    for k in piped:
        assert np.array_equal(piped[k], serial[k]), k
    keys = ("h_seq", "c_seq", "hT", "cT") if cell == "lstm" else ("h_seq", "hT")
    compare(piped, oracle_of(c), TOL_BF16, keys)


def test_pipelined_headline_forward_repeatable_and_equal_to_serial():
    """Full-size multi-head LSTM (B=16, NH=6, Dh=128, T=1024): three pipelined
    calls on one workspace (panel counters reused), one serial call and one
    pipelined call without the projection's taper agree bitwise."""
    w = synth.WORKLOADS["lstm_mh_b16_nh6_dh128"]
    c = synth.workload_case(w)
    x, W, R, b = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b")
    wd = w.dims
    d = g.Dims(wd.T, wd.B, wd.Din, wd.NH, wd.Dh)
    plan = g.plan_describe(g.OP_FWD_LSTM, d, g.RNN_BF16)
    print("  plan:", plan, flush=True)
    assert "input_proj=pipelined" in plan and "head_start_panels=0" not in plan
    ws = torch.empty(g.workspace_size(g.OP_FWD_LSTM, d, g.RNN_BF16), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for _ in range(3):
        h_seq, _, hT, cT = g.lstm_fwd(x, W, R, b, ws=ws)
        outs.append((h_seq.clone(), hT.clone(), cT.clone()))
    assert g.workspace_status(ws) == g.RNN_OK
    serial = _with_env("RNN355_PIPELINE", "0", lambda: g.lstm_fwd(x, W, R, b, ws=ws))
    torch.cuda.synchronize()
    for o in outs[1:] + [(serial[0], serial[2], serial[3])]:
        for a, e in zip(outs[0], o):
            assert torch.equal(a, e)
    # every projection workgroup to the end (no taper): the same bits
    flat = _with_env("RNN355_FUSED_TAPER", "0", lambda: g.lstm_fwd(x, W, R, b, ws=ws))
    torch.cuda.synchronize()
    for a, e in zip(outs[0], (flat[0], flat[2], flat[3])):
        assert torch.equal(a, e)


def test_pipelined_gru_b4_nh12_dh64_equal_to_serial():
    """Full-size multi-head GRU (B=4, NH=12, Dh=64, T=2048): the one-launch
    forward with its head start (four of eight waves per recurrence
    workgroup), the serial forward and the one-launch forward without the
    projection's taper agree bitwise, twice on one workspace."""
    w = synth.WORKLOADS["gru_mh_b4_nh12_dh64"]
    c = synth.workload_case(w)
    x, W, R, b, h0 = dev(c, "x"), dev(c, "W"), dev(c, "R"), dev(c, "b"), dev(c, "h0")
    wd = w.dims
    d = g.Dims(wd.T, wd.B, wd.Din, wd.NH, wd.Dh)
    plan = g.plan_describe(g.OP_FWD_GRU, d, g.RNN_BF16)
    print("  plan:", plan, flush=True)
    assert "input_proj=pipelined" in plan and "head_start_panels=0" not in plan
    ws = torch.empty(g.workspace_size(g.OP_FWD_GRU, d, g.RNN_BF16), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for _ in range(2):
        h_seq, hT = g.gru_fwd(x, W, R, b, h0, ws=ws)
        outs.append((h_seq.clone(), hT.clone()))
    assert g.workspace_status(ws) == g.RNN_OK
    serial = _with_env("RNN355_PIPELINE", "0", lambda: g.gru_fwd(x, W, R, b, h0, ws=ws))
    flat = _with_env("RNN355_FUSED_TAPER", "0", lambda: g.gru_fwd(x, W, R, b, h0, ws=ws))
    torch.cuda.synchronize()
    for o in outs[1:] + [serial, flat]:
        for a, e in zip(outs[0], o):
            assert torch.equal(a, e)


def test_pipelined_forward_reads_fresh_projection_after_reuse():
    """Two pipelined calls on one workspace with different inputs: the second
    call's projection overwrites gx (4 MiB, about what an XCD's L2 holds) while
    its recurrence reads it; the result must be the serial one for the second
    inputs, never the first call's cached values."""
    d = synth.Dims(T=256, B=4, Din=64, NH=2, Dh=128)
    gd = g.Dims(d.T, d.B, d.Din, d.NH, d.Dh)
    os.environ["RNN355_PIPELINE"] = "1"   # removed by the fixture
    assert "input_proj=pipelined" in g.plan_describe(g.OP_FWD_LSTM, gd, g.RNN_BF16)
    ws = torch.empty(g.workspace_size(g.OP_FWD_LSTM, gd, g.RNN_BF16), dtype=torch.uint8,
                     device="cuda")
    c1 = synth.make_case("lstm", d, "bf16", 7600, bias="forget+1")
    c2 = synth.make_case("lstm", d, "bf16", 7700, bias="forget+1")
    ins = [tuple(dev(c, k) for k in ("x", "W", "R", "b")) for c in (c1, c2)]
    for _ in range(3):
        g.lstm_fwd(*ins[0], ws=ws)
        h2, _, _, cT2 = g.lstm_fwd(*ins[1], ws=ws)
        h2, cT2 = h2.clone(), cT2.clone()
    serial = _with_env("RNN355_PIPELINE", "0", lambda: g.lstm_fwd(*ins[1]))
    torch.cuda.synchronize()
    assert torch.equal(h2, serial[0]) and torch.equal(cT2, serial[3])



@pytest.mark.parametrize("cell,B,NH,Dh,dtype,bt", [
    ("lstm", 3, 2, 64, "bf16", None),    # one row per workgroup
    ("gru", 8, 2, 64, "bf16", "4"),      # rows in lane groups
    ("lstm", 3, 2, 32, "f32", None),     # LDS kernel
])
def test_recurrence_status_is_ok_on_a_workspace_holding_garbage(cell, B, NH, Dh, dtype, bt):
    """The recurrence entry points clear the workspace status word
    themselves: a workspace filled with nonzero bytes reports RNN_OK after a
    call whose kernels never wait (regression: the one-CU and LDS paths left
    the word as it was)."""
    T = 9
    G = synth.gates_of(cell)
    old = os.environ.pop("RNN355_REC_BT", None)
    if bt:
        os.environ["RNN355_REC_BT"] = bt
    try:
        gen = torch.Generator(device="cuda").manual_seed(5)
        gx = torch.randn((T, B, NH * G * Dh), device="cuda", generator=gen)
        R = torch.randn((NH, Dh, G * Dh), device="cuda", generator=gen) / Dh ** 0.5
        if dtype == "bf16":
            R = R.to(torch.bfloat16)
        op = g.OP_REC_LSTM if cell == "lstm" else g.OP_REC_GRU
        dt = g.RNN_BF16 if dtype == "bf16" else g.RNN_F32
        ws = torch.full((g.workspace_size(op, g.Dims(T, B, 64, NH, Dh), dt),), 0xA5,
                        dtype=torch.uint8, device="cuda")
        if cell == "lstm":
            g.rec_lstm(gx, R, ws=ws)
        else:
            g.rec_gru(gx, R, ws=ws)
        assert g.workspace_status(ws) == g.RNN_OK
    finally:
        os.environ.pop("RNN355_REC_BT", None)
        if old is not None:
            os.environ["RNN355_REC_BT"] = old

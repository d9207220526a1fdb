"""The C ABI on the CPU: the library loads, exports every function that
include/rnn355.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import gru_recurrence_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rnn355.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rnn_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = g.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(g.EXPORTS)


def test_status_strings():
    for s in range(6):
        assert g.status_str(s).startswith("RNN_")
    assert "UNKNOWN" in g.status_str(99)


def test_workspace_size_pure_host():
    d = g.Dims(1024, 16, 768, 6, 128)
    fwd = g.workspace_size(g.OP_FWD_LSTM, d, g.RNN_BF16)
    assert fwd >= 1024 * 16 * 6 * 4 * 128 * 4
    assert g.workspace_size(g.OP_FWD_GRU, d, g.RNN_BF16) < fwd
    assert g.workspace_size(g.OP_FWD_LSTM, g.Dims(0, 16, 768, 6, 128), g.RNN_BF16) == 0
    assert g.workspace_size(g.OP_FWD_LSTM, d, 7) == 0


FAKE = 0x7F0000000000  # never dereferenced: validation fails first


def _p(v):
    return ctypes.c_void_p(v)


def test_invalid_arguments_are_rejected_before_launch():
    lib = g.load()
    d = g.Dims(8, 2, 32, 1, 32)
    ok = [_p(FAKE + 256 * i) for i in range(11)]
    # NULL x
    args = list(ok)
    args[0] = None
    s = lib.rnn_fwd_lstm(ctypes.byref(d), g.RNN_BF16, *args[:10], None, 0, None)
    assert s == g.RNN_ERR_INVALID_ARG
    # misaligned W
    args = list(ok)
    args[1] = _p(FAKE + 2)
    s = lib.rnn_fwd_lstm(ctypes.byref(d), g.RNN_BF16, *args[:10], _p(FAKE), 1 << 30, None)
    assert s == g.RNN_ERR_INVALID_ARG
    # bad dims and dtype
    bad = g.Dims(8, 0, 32, 1, 32)
    assert lib.rnn_fwd_lstm(ctypes.byref(bad), g.RNN_BF16, *ok[:10], _p(FAKE), 1 << 30,
                            None) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_fwd_lstm(ctypes.byref(d), 5, *ok[:10], _p(FAKE), 1 << 30,
                            None) == g.RNN_ERR_INVALID_ARG
    # missing / too small workspace
    assert lib.rnn_fwd_lstm(ctypes.byref(d), g.RNN_BF16, *ok[:10], None, 0,
                            None) == g.RNN_ERR_WORKSPACE
    assert lib.rnn_fwd_lstm(ctypes.byref(d), g.RNN_BF16, *ok[:10], _p(FAKE), 64,
                            None) == g.RNN_ERR_WORKSPACE
    # unsupported: bf16 GEMM needs Din % 8 == 0
    d2 = g.Dims(8, 2, 30, 1, 32)
    assert lib.rnn_fwd_lstm(ctypes.byref(d2), g.RNN_BF16, *ok[:10], _p(FAKE), 1 << 30,
                            None) == g.RNN_ERR_UNSUPPORTED
    # unsupported: an f32 head too large for the LDS kernel and not MFMA-shaped
    d3 = g.Dims(8, 2, 32, 1, 256)
    assert lib.rnn_fwd_lstm(ctypes.byref(d3), g.RNN_F32, *ok[:10], _p(FAKE), 1 << 30,
                            None) == g.RNN_ERR_UNSUPPORTED
    # input projection
    assert lib.rnn_input_proj(0, 8, 8, g.RNN_BF16, ok[0], ok[1], None, ok[2],
                              None) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_input_proj(4, 8, 8, g.RNN_BF16, ok[0], None, None, ok[2],
                              None) == g.RNN_ERR_INVALID_ARG
    # transposed-weights projection: bf16 with K % 32 == 0 only
    assert lib.rnn_input_proj_t(4, 32, 8, g.RNN_BF16, ok[0], None, None, ok[2],
                                None) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_input_proj_t(4, 48, 8, g.RNN_BF16, ok[0], ok[1], None, ok[2],
                                None) == g.RNN_ERR_UNSUPPORTED
    assert lib.rnn_input_proj_t(4, 32, 8, g.RNN_F32, ok[0], ok[1], None, ok[2],
                                None) == g.RNN_ERR_UNSUPPORTED
    assert lib.rnn_input_proj_t(4, 32, 8, g.RNN_BF16, _p(FAKE + 8), ok[1], None, ok[2],
                                None) == g.RNN_ERR_INVALID_ARG
    # recurrence alone
    assert lib.rnn_rec_gru(ctypes.byref(d), g.RNN_BF16, None, ok[1], None, None, ok[2],
                           _p(FAKE), 1 << 20, None) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_workspace_status(None, 0, None) == g.RNN_ERR_INVALID_ARG
    # the allocation-free recurrence: same argument checks, and shapes whose
    # scratch would pass the library's fixed array are rejected up front
    dn = g.Dims(8, 2, 1, 1, 32)
    assert lib.rnn_rec_lstm_noalloc(ctypes.byref(dn), g.RNN_BF16, None, ok[1], None, None,
                                    None, None, ok[2], ok[3], None, None) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_rec_lstm_noalloc(ctypes.byref(dn), g.RNN_BF16, ok[0], ok[1], None, None,
                                    None, None, ok[2], ok[3], _p(FAKE + 4),
                                    None) == g.RNN_ERR_INVALID_ARG
    big = g.Dims(8, 2, 1, 64, 256)    # R^T of 64 heads of Dh 256: 32 MiB of scratch
    assert g.workspace_size(g.OP_REC_LSTM, big, g.RNN_BF16) > (8 << 20)
    assert lib.rnn_rec_lstm_noalloc(ctypes.byref(big), g.RNN_BF16, ok[0], ok[1], None, None,
                                    None, None, ok[2], ok[3], None, None) == g.RNN_ERR_WORKSPACE


def test_backward_rejects_unsupported_and_invalid_before_launch():
    lib = g.load()
    d = g.Dims(8, 2, 32, 2, 64)
    ptrs = [_p(FAKE + 256 * i) for i in range(17)]
    # f32 backward: a head whose float32 R block does not fit the sweep's LDS
    # has no kernel; a supported one checks its (float32) workspace
    dbig = g.Dims(8, 2, 32, 2, 256)
    assert lib.rnn_bwd_lstm(ctypes.byref(dbig), g.RNN_F32, *ptrs, _p(FAKE), 1 << 30,
                            None) == g.RNN_ERR_UNSUPPORTED
    assert lib.rnn_bwd_lstm(ctypes.byref(d), g.RNN_F32, *ptrs, _p(FAKE), 64,
                            None) == g.RNN_ERR_WORKSPACE
    assert g.workspace_size(g.OP_BWD_LSTM, d, g.RNN_F32) > 8 * 2 * (2 * 4 * 64) * 4 * 2
    # a required gradient output missing
    bad = list(ptrs)
    bad[11] = None  # dx
    assert lib.rnn_bwd_lstm(ctypes.byref(d), g.RNN_BF16, *bad, _p(FAKE), 1 << 30,
                            None) == g.RNN_ERR_INVALID_ARG
    # workspace too small
    assert lib.rnn_bwd_lstm(ctypes.byref(d), g.RNN_BF16, *ptrs, _p(FAKE), 64,
                            None) == g.RNN_ERR_WORKSPACE
    need = g.workspace_size(g.OP_BWD_LSTM, d, g.RNN_BF16)
    assert need > 8 * 2 * (2 * 4 * 64) * 4  # holds at least the recomputed pre-activations
    # GRU: 13 pointers (no c0, c_seq, dcT, dc0)
    gp = [_p(FAKE + 256 * i) for i in range(13)]
    assert lib.rnn_bwd_gru(ctypes.byref(dbig), g.RNN_F32, *gp, _p(FAKE), 1 << 30,
                           None) == g.RNN_ERR_UNSUPPORTED
    assert lib.rnn_bwd_gru(ctypes.byref(d), g.RNN_F32, *gp, _p(FAKE), 64,
                           None) == g.RNN_ERR_WORKSPACE
    bad = list(gp)
    bad[12] = None  # dh0
    assert lib.rnn_bwd_gru(ctypes.byref(d), g.RNN_BF16, *bad, _p(FAKE), 1 << 30,
                           None) == g.RNN_ERR_INVALID_ARG
    bad = list(gp)
    bad[5] = _p(FAKE + 4)  # misaligned h_seq
    assert lib.rnn_bwd_gru(ctypes.byref(d), g.RNN_BF16, *bad, _p(FAKE), 1 << 30,
                           None) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_bwd_gru(ctypes.byref(d), g.RNN_BF16, *gp, _p(FAKE), 64,
                           None) == g.RNN_ERR_WORKSPACE
    # the GRU workspace keeps Gx and S apart, so it is larger per gate column
    gneed = g.workspace_size(g.OP_BWD_GRU, d, g.RNN_BF16)
    assert gneed > 8 * 2 * (2 * 3 * 64) * 4 * 2


def test_plans_of_the_workloads(monkeypatch):
    """Kernel plans are pure host decisions (256 compute units assumed when
    no device is visible): one-CU resident-R kernel for Dh <= 128, at Dh =
    256 four CUs per chain exchanging through an XCD's L2 (or one CU with R
    split over registers and LDS), multi-CU split above; the forward
    overlaps projection and recurrence (one fused launch, Dh = 128 or 64)
    only when the recurrence leaves half the chip free and the projection is
    large: more than two rounds of tiles on the free CUs, or more than one
    where the recurrence starts on a head start of its own."""
    monkeypatch.delenv("RNN355_PIPELINE", raising=False)
    monkeypatch.delenv("RNN355_REC_BT", raising=False)
    monkeypatch.delenv("RNN355_REC_K", raising=False)
    monkeypatch.delenv("RNN355_REC_WIDE", raising=False)
    monkeypatch.delenv("RNN355_MC_XCD", raising=False)
    if g.plan_describe(g.OP_REC_LSTM, g.Dims(8, 16, 8, 6, 128), g.RNN_BF16).find(" wg=96 ") < 0:
        pytest.skip("a device with other than 256 compute units is visible")
    head = g.Dims(1024, 16, 768, 6, 128)
    p = g.plan_describe(g.OP_FWD_LSTM, head, g.RNN_BF16)
    assert "mfma_resident_R" in p and " wg=96 " in p and "input_proj=pipelined" in p
    assert "head_start_panels=2" in p
    # 288 tiles on 208 free CUs: overlapped with a head start of one panel
    p = g.plan_describe(g.OP_FWD_GRU, g.Dims(2048, 4, 768, 12, 64), g.RNN_BF16)
    assert "mfma_resident_R" in p and " wg=48 " in p and "input_proj=pipelined" in p
    assert "head_start_panels=1" in p
    p = g.plan_describe(g.OP_FWD_LSTM, g.Dims(1024, 16, 768, 1, 768), g.RNN_BF16)
    assert "mfma_multi_cu" in p and "input_proj=serial" in p
    # Dh = 256, 64 (head, row) chains: four CUs per chain, the 64 groups
    # numbered so that each group's four run on one XCD and exchange h
    # through its L2; with that exchange through memory (RNN355_MC_XCD=0),
    # one CU per (head, row) with R split over registers and LDS
    c5 = g.Dims(1024, 16, 1024, 4, 256)
    for op in (g.OP_FWD_LSTM, g.OP_FWD_GRU):
        p = g.plan_describe(op, c5, g.RNN_BF16)
        assert "mfma_multi_cu" in p and " wg=256 " in p and "exchange=xcd_l2" in p
    monkeypatch.setenv("RNN355_MC_XCD", "0")
    p = g.plan_describe(g.OP_FWD_LSTM, c5, g.RNN_BF16)
    assert "split_R" in p and " wg=64 " in p and " threads=256 " in p and "r_lds_bytes=131072" in p
    p = g.plan_describe(g.OP_FWD_GRU, c5, g.RNN_BF16)
    assert "split_R" in p and "r_lds_bytes=0" in p
    monkeypatch.setenv("RNN355_REC_WIDE", "0")
    p = g.plan_describe(g.OP_FWD_LSTM, c5, g.RNN_BF16)
    assert "mfma_multi_cu" in p and "exchange=memory" in p
    monkeypatch.delenv("RNN355_REC_WIDE")
    monkeypatch.delenv("RNN355_MC_XCD")
    # the recurrence-only workspace holds R^T for it (bf16 only)
    rec_f = g.workspace_size(g.OP_REC_LSTM, c5, g.RNN_F32)
    rec_b = g.workspace_size(g.OP_REC_LSTM, c5, g.RNN_BF16)
    assert rec_b - rec_f >= 2 * 4 * 4 * 256 * 256
    p = g.plan_describe(g.OP_FWD_LSTM, g.Dims(64, 2, 32, 1, 32), g.RNN_F32)
    assert "lds_simple" in p and "input_proj=serial" in p
    assert "input_proj" not in g.plan_describe(g.OP_REC_LSTM, head, g.RNN_BF16)
    monkeypatch.setenv("RNN355_PIPELINE", "0")
    assert "input_proj=serial" in g.plan_describe(g.OP_FWD_LSTM, head, g.RNN_BF16)
    monkeypatch.setenv("RNN355_PIPELINE", "1")
    small = g.Dims(233, 5, 96, 2, 128)
    assert "input_proj=pipelined" in g.plan_describe(g.OP_FWD_LSTM, small, g.RNN_BF16)
    # only the one-CU kernel at Dh = 128 or 64 runs fused with the projection,
    # and only with Din % 32 == 0
    assert "input_proj=pipelined" in g.plan_describe(g.OP_FWD_LSTM, g.Dims(233, 5, 96, 2, 64),
                                                     g.RNN_BF16)
    assert "input_proj=serial" in g.plan_describe(g.OP_FWD_LSTM, g.Dims(233, 5, 96, 2, 32),
                                                  g.RNN_BF16)
    assert "input_proj=serial" in g.plan_describe(g.OP_FWD_LSTM, g.Dims(233, 5, 40, 2, 128),
                                                  g.RNN_BF16)
    # never when the recurrence would hold more than half the units
    big = g.Dims(64, 16, 64, 16, 128)
    p = g.plan_describe(g.OP_FWD_LSTM, big, g.RNN_BF16)
    assert " wg=256 " in p and "input_proj=serial" in p


def test_backward_plans(monkeypatch):
    """The backward's sweep and its time chunks are host decisions too:
    two CUs per (head, row) at Dh = 256 where the pairs fit the XCD
    grouping, four chunks at T = 1024 and two at T = 256 (chunks of at
    least 128 steps) where the sweep leaves at least 64 CUs free, one piece
    with RNN355_BWD_OVERLAP=0, for short sequences and in float32."""
    for k in ("RNN355_BWD_OVERLAP", "RNN355_BWD_CHUNKS", "RNN355_BWD_WIDE2", "RNN355_REC_WIDE",
              "RNN355_MC_XCD", "RNN355_REC_BT", "RNN355_REC_K"):
        monkeypatch.delenv(k, raising=False)
    if g.plan_describe(g.OP_REC_LSTM, g.Dims(8, 16, 8, 6, 128), g.RNN_BF16).find(" wg=96 ") < 0:
        pytest.skip("a device with other than 256 compute units is visible")
    c5 = g.Dims(1024, 16, 1024, 4, 256)
    p = g.plan_describe(g.OP_BWD_LSTM, c5, g.RNN_BF16)
    assert "bwd_sweep=split_R_two_cu" in p and " wg=128 " in p and " chunks=4 " in p, p
    assert "free_cus=128" in p
    assert " chunks=2 " in g.plan_describe(g.OP_BWD_LSTM, g.Dims(256, 16, 1024, 4, 256),
                                           g.RNN_BF16)
    assert " chunks=1 " in g.plan_describe(g.OP_BWD_LSTM, g.Dims(255, 16, 1024, 4, 256),
                                           g.RNN_BF16)
    p = g.plan_describe(g.OP_BWD_GRU, g.Dims(600, 5, 96, 2, 64), g.RNN_BF16)
    assert "bwd_sweep=exchange" in p and " chunks=4 " in p, p
    monkeypatch.setenv("RNN355_BWD_CHUNKS", "3")
    assert " chunks=3 " in g.plan_describe(g.OP_BWD_LSTM, c5, g.RNN_BF16)
    monkeypatch.setenv("RNN355_BWD_OVERLAP", "0")
    assert " chunks=1 " in g.plan_describe(g.OP_BWD_LSTM, c5, g.RNN_BF16)
    monkeypatch.delenv("RNN355_BWD_OVERLAP")
    monkeypatch.delenv("RNN355_BWD_CHUNKS")
    monkeypatch.setenv("RNN355_BWD_WIDE2", "0")
    p = g.plan_describe(g.OP_BWD_LSTM, c5, g.RNN_BF16)
    assert "bwd_sweep=split_R " in p and " wg=64 " in p and " chunks=4 " in p, p
    p = g.plan_describe(g.OP_BWD_LSTM, g.Dims(64, 2, 32, 1, 32), g.RNN_F32)
    assert "bwd_sweep=f32_lds" in p and "chunks=1" in p, p


def test_stack_entry_points_reject_before_launch():
    lib = g.load()
    d = g.Dims(8, 2, 32, 1, 32)
    P3 = ctypes.c_void_p * 3
    W, R = P3(*[FAKE + 256 * i for i in range(3)]), P3(*[FAKE + 4096 + 256 * i for i in range(3)])
    ok = [_p(FAKE + 65536 + 256 * i) for i in range(8)]
    big = 1 << 30
    ws1 = g.workspace_size_stack(g.OP_FWD_LSTM, d, 1, g.RNN_BF16)
    ws3 = g.workspace_size_stack(g.OP_FWD_LSTM, d, 3, g.RNN_BF16)
    assert ws1 > 0 and ws3 == ws1  # the buffers are reused layer after layer
    assert g.workspace_size_stack(g.OP_FWD_LSTM, d, 0, g.RNN_BF16) == 0
    assert g.workspace_size_stack(g.OP_FWD_LSTM, d, 65, g.RNN_BF16) == 0
    assert g.workspace_size_stack(g.OP_BWD_LSTM, d, 2, g.RNN_BF16) == 0

    def lstm(dd, L, W_, R_, hT=ok[4], ws=_p(FAKE), nb=big, x=ok[0]):
        return lib.rnn_fwd_lstm_stack(ctypes.byref(dd), L, g.RNN_BF16, x, W_, R_, None, None,
                                      None, ok[2], ok[3], hT, ok[5], ws, nb, None)

    assert lstm(d, 0, W, R) == g.RNN_ERR_INVALID_ARG
    assert lstm(d, 65, W, R) == g.RNN_ERR_INVALID_ARG
    assert lstm(d, 3, W, R, x=None) == g.RNN_ERR_INVALID_ARG
    assert lstm(d, 3, None, R) == g.RNN_ERR_INVALID_ARG
    assert lstm(d, 3, W, R, hT=None) == g.RNN_ERR_INVALID_ARG
    holed = P3(FAKE, 0, FAKE + 512)
    assert lstm(d, 3, holed, R) == g.RNN_ERR_INVALID_ARG
    assert lstm(d, 2, holed, R) == g.RNN_ERR_INVALID_ARG
    misal = P3(FAKE, FAKE + 6, FAKE + 512)
    assert lstm(d, 3, misal, R) == g.RNN_ERR_INVALID_ARG
    assert lstm(d, 3, W, R, ws=None, nb=0) == g.RNN_ERR_WORKSPACE
    assert lstm(d, 3, W, R, nb=ws3 - 1) == g.RNN_ERR_WORKSPACE
    # Din % 8 != 0 rejects layer 0's projection
    assert lstm(g.Dims(8, 2, 30, 1, 32), 2, W, R) == g.RNN_ERR_UNSUPPORTED
    assert lib.rnn_fwd_gru_stack(ctypes.byref(d), 2, g.RNN_BF16, ok[0], W, R, None, None, None,
                                 None, _p(FAKE), big, None) == g.RNN_ERR_INVALID_ARG


def test_chunked_and_checkpointed_entry_points_reject_before_launch():
    lib = g.load()
    d = g.Dims(64, 2, 32, 1, 64)
    ok = [_p(FAKE + 256 * i) for i in range(24)]
    big = 1 << 30
    f = g.workspace_size_chunked(g.OP_FWD_LSTM, d, 16, g.RNN_BF16)
    d2 = g.Dims(6400, 2, 32, 1, 64)
    assert f > 0 and g.workspace_size_chunked(g.OP_FWD_LSTM, d2, 16, g.RNN_BF16) == f
    bk = g.workspace_size_chunked(g.OP_BWD_LSTM, d, 16, g.RNN_BF16)
    assert bk > 0 and g.workspace_size_chunked(g.OP_BWD_LSTM, d2, 16, g.RNN_BF16) == bk
    assert bk < g.workspace_size(g.OP_BWD_LSTM, d2, g.RNN_BF16)
    assert g.workspace_size_chunked(g.OP_FWD_LSTM, d, 0, g.RNN_BF16) == 0
    assert g.workspace_size_chunked(g.OP_REC_LSTM, d, 16, g.RNN_BF16) == 0

    def fwd(chunk, hck=ok[11], cck=ok[12], ws=_p(FAKE), nb=big):
        return lib.rnn_fwd_lstm_chunked(ctypes.byref(d), g.RNN_BF16, chunk, *ok[:10], hck, cck, ws,
                                        nb, None)
    assert fwd(0) == g.RNN_ERR_INVALID_ARG
    assert fwd(16, cck=None) == g.RNN_ERR_INVALID_ARG       # h and c checkpoints go together
    assert fwd(16, ws=None, nb=0) == g.RNN_ERR_WORKSPACE
    assert fwd(16, nb=f - 1) == g.RNN_ERR_WORKSPACE
    assert fwd(16, hck=_p(FAKE + 8), cck=_p(FAKE + 8)) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_fwd_gru_chunked(ctypes.byref(d), g.RNN_BF16, -1, *ok[:8], _p(FAKE), big,
                                   None) == g.RNN_ERR_INVALID_ARG

    def bwd(chunk, dt=g.RNN_BF16, hck=ok[6], cck=ok[7], nb=big):
        a = list(ok[:17])
        a[6], a[7] = hck, cck
        return lib.rnn_bwd_lstm_ckpt(ctypes.byref(d), dt, chunk, *a, _p(FAKE), nb, None)
    assert bwd(0) == g.RNN_ERR_INVALID_ARG
    assert bwd(16, hck=None) == g.RNN_ERR_INVALID_ARG       # checkpoints needed when chunk < T
    assert bwd(16, cck=None) == g.RNN_ERR_INVALID_ARG
    assert bwd(16, dt=g.RNN_F32) == g.RNN_ERR_UNSUPPORTED
    assert bwd(16, nb=bk - 1) == g.RNN_ERR_WORKSPACE
    assert lib.rnn_bwd_gru_ckpt(ctypes.byref(d), g.RNN_BF16, 16, *ok[:5], None, *ok[6:13],
                                _p(FAKE), big, None) == g.RNN_ERR_INVALID_ARG

"""Pins of the oracle's input projection (``oracle.input_proj``) and of the
stacked-layer composition with bf16 rounding between layers.

Input projection: the dense input part of every gate (FlashRNN card,
paperdance.org/p/2412.07752, abstract: the input contribution does not
depend on the recurrence, so it is one dense product over all steps).  Pinned
to ``torch.nn.functional.linear`` in float64, a library routine: the whole
matrix, a row subset (unsorted, repeated, ragged), no bias, and the [T,B,K]
input form.  Operands are non-square and the bias is non-zero, so a dropped
bias, a transposed W or a wrong row index changes the result.

Stacked layers with bf16 between them (blog.hotdry.top, 2025-09-21, the
list of framework-level optimisations, first item: layers of a multi-layer
RNN): layer l+1 reads layer l's h_1..h_T rounded to bfloat16 as any bf16
input would be.  Pinned to torch float64 single-layer modules, one per
layer, chained through an explicit float32 -> bfloat16 rounding done by
torch itself (not by the oracle's ``round_bf16``), at L = 2 and 3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.torch_pins import embed


def nrm(seed, shape, var=1.0):
    return synth.normal(seed, int(np.prod(shape)), var).reshape(shape)


def torch_linear(x, W, b):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    wt = torch.from_numpy(np.asarray(W, np.float64)).t().contiguous()   # [N, K]
    bt = None if b is None else torch.from_numpy(np.asarray(b, np.float64))
    return torch.nn.functional.linear(xt, wt, bt).numpy()


@pytest.mark.parametrize("M,K,N", [(37, 13, 20), (5, 64, 3), (1, 7, 11)])
def test_input_proj_full_matches_torch_linear(M, K, N):
    x, W, b = nrm(1100 + M, (M, K)), nrm(1200 + K, (K, N), 1.0 / K), nrm(1300 + N, (N,))
    got = oracle.input_proj(x, W, b)
    assert got.shape == (M, N)
    assert np.max(np.abs(got - torch_linear(x, W, b))) < 1e-12


def test_input_proj_rows_subset_matches_torch_linear():
    M, K, N = 41, 17, 24
    x, W, b = nrm(1401, (M, K)), nrm(1402, (K, N), 1.0 / K), nrm(1403, (N,))
    rows = np.array([40, 0, 7, 7, 33, 1, 39])   # unsorted, repeated, both ends
    got = oracle.input_proj(x, W, b, rows=rows)
    assert got.shape == (rows.size, N)
    want = torch_linear(x, W, b)[rows]
    assert np.max(np.abs(got - want)) < 1e-12


def test_input_proj_without_bias_and_3d_input():
    T, B, K, N = 6, 3, 9, 15
    x, W = nrm(1501, (T, B, K)), nrm(1502, (K, N), 1.0 / K)
    got = oracle.input_proj(x, W, None)
    want = torch_linear(x.reshape(T * B, K), W, None)
    assert np.max(np.abs(got - want)) < 1e-12
    # the bias is added exactly once per entry
    b = nrm(1503, (N,))
    assert np.max(np.abs(oracle.input_proj(x, W, b) - (got + b))) < 1e-12


def test_input_proj_rejects_out_of_range_rows():
    x, W = nrm(1601, (4, 3)), nrm(1602, (3, 5))
    with pytest.raises(ValueError):
        oracle.input_proj(x, W, None, rows=np.array([0, 4]))
    with pytest.raises(ValueError):
        oracle.input_proj(x, W, None, rows=np.array([-1]))


def _bf16_torch(a):
    """Round float64 values to bfloat16 the way a bf16 input is stored: to
    float32 (nearest even), then to bfloat16 (nearest even), by torch."""
    return torch.from_numpy(np.asarray(a, np.float64)).float().to(torch.bfloat16).double().numpy()


def _torch_layer(cell, x, W, R, b, h0, c0, NH, Dh):
    G = 4 if cell == "lstm" else 3
    T, B, Din = x.shape
    H = NH * Dh
    mod = (torch.nn.LSTM if cell == "lstm" else torch.nn.GRU)(Din, H).double()
    w_ih, w_hh, bb = embed(W, R, b, NH, Dh, G)
    with torch.no_grad():
        mod.weight_ih_l0.copy_(torch.from_numpy(w_ih))
        mod.weight_hh_l0.copy_(torch.from_numpy(w_hh))
        mod.bias_ih_l0.copy_(torch.from_numpy(bb))
        mod.bias_hh_l0.zero_()
        xt = torch.from_numpy(np.asarray(x, np.float64))
        if cell == "lstm":
            y, (hn, cn) = mod(xt, (torch.from_numpy(h0[None]), torch.from_numpy(c0[None])))
            return y.numpy(), hn[0].numpy(), cn[0].numpy()
        y, hn = mod(xt, torch.from_numpy(h0[None]))
        return y.numpy(), hn[0].numpy(), None


@pytest.mark.parametrize("cell,L", [("lstm", 2), ("lstm", 3), ("gru", 2), ("gru", 3)])
def test_stack_bf16_between_matches_torch_chain(cell, L):
    T, B, Din, NH, Dh = 9, 3, 6, 2, 4
    G = 4 if cell == "lstm" else 3
    H, N = NH * Dh, NH * G * Dh
    # bf16-exact weights and x, as a bf16 run stores them
    Ws = [_bf16_torch(nrm(1700 + 10 * l, (Din if l == 0 else H, N), 1.0 / (Din if l == 0 else H)))
          for l in range(L)]
    Rs = [_bf16_torch(nrm(1701 + 10 * l, (NH, Dh, G * Dh), 1.0 / Dh)) for l in range(L)]
    bs = [nrm(1702 + 10 * l, (N,), 0.1) for l in range(L)]
    h0 = nrm(1790, (L, B, H), 0.2)
    c0 = nrm(1791, (L, B, H), 0.2)
    x = _bf16_torch(nrm(1792, (T, B, Din)))
    if cell == "lstm":
        o = oracle.lstm_stack_fwd(x, Ws, Rs, bs, h0, c0, NH=NH, Dh=Dh, bf16_between=True)
    else:
        o = oracle.gru_stack_fwd(x, Ws, Rs, bs, h0, NH=NH, Dh=Dh, bf16_between=True)
    inp = x
    for l in range(L):
        y, hn, cn = _torch_layer(cell, inp, Ws[l], Rs[l], bs[l], h0[l], c0[l], NH, Dh)
        assert np.max(np.abs(o["hT"][l] - hn)) < 1e-12, l
        if cell == "lstm":
            assert np.max(np.abs(o["cT"][l] - cn)) < 1e-12, l
        inp = _bf16_torch(y)
    assert np.max(np.abs(o["h_seq"] - y)) < 1e-12
    # the rounding is really in effect: without it the upper layers differ
    plain = (oracle.lstm_stack_fwd(x, Ws, Rs, bs, h0, c0, NH=NH, Dh=Dh) if cell == "lstm"
             else oracle.gru_stack_fwd(x, Ws, Rs, bs, h0, NH=NH, Dh=Dh))
    assert np.max(np.abs(plain["h_seq"] - o["h_seq"])) > 1e-6
    # rounding c (LSTM) or nothing between the layers would not match torch
    assert np.max(np.abs(plain["hT"][1] - o["hT"][1])) > 1e-6

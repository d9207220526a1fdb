"""Pins of the stacked-layer oracle (lstm_stack_fwd / gru_stack_fwd):

* ``torch.nn.LSTM`` / ``torch.nn.GRU`` with ``num_layers`` = L in float64 (a
  library routine), fed every layer's multi-head parameters embedded
  block-diagonally into dense ones -- fixes the layer wiring (layer l's
  input is layer l-1's h_1..h_T), the per-layer states and the outputs;
* the bf16 rounding between layers against exact small cases (ties to
  even, carries into the exponent) and against an independent evaluation of
  the rule on random values.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.torch_pins import embed


def nrm(seed, shape, var):
    return synth.normal(seed, int(np.prod(shape)), var).reshape(shape)


def layers(cell, L, Din, NH, Dh, seed):
    G = 4 if cell == "lstm" else 3
    H, N = NH * Dh, NH * G * Dh
    Ws, Rs, bs = [], [], []
    for layer in range(L):
        k = Din if layer == 0 else H
        Ws.append(nrm(seed + 10 * layer + 1, (k, N), 0.5 / k))
        Rs.append(nrm(seed + 10 * layer + 2, (NH, Dh, G * Dh), 0.5 / Dh))
        bs.append(nrm(seed + 10 * layer + 3, (N,), 0.1))
    return Ws, Rs, bs


def torch_stack(cell, x, Ws, Rs, bs, h0, c0, NH, Dh):
    G = 4 if cell == "lstm" else 3
    T, B, Din = x.shape
    L, H = len(Ws), NH * Dh
    mod = (torch.nn.LSTM if cell == "lstm" else torch.nn.GRU)(Din, H, num_layers=L).double()
    with torch.no_grad():
        for layer in range(L):
            w_ih, w_hh, bb = embed(Ws[layer], Rs[layer], bs[layer], NH, Dh, G)
            getattr(mod, "weight_ih_l%d" % layer).copy_(torch.from_numpy(w_ih))
            getattr(mod, "weight_hh_l%d" % layer).copy_(torch.from_numpy(w_hh))
            getattr(mod, "bias_ih_l%d" % layer).copy_(torch.from_numpy(bb))
            getattr(mod, "bias_hh_l%d" % layer).zero_()
        xt = torch.from_numpy(np.asarray(x, np.float64))
        if cell == "lstm":
            y, (hn, cn) = mod(xt, (torch.from_numpy(h0), torch.from_numpy(c0)))
            return y.numpy(), hn.numpy(), cn.numpy()
        y, hn = mod(xt, torch.from_numpy(h0))
        return y.numpy(), hn.numpy(), None


@pytest.mark.parametrize("cell,L,NH,Dh", [("lstm", 2, 1, 5), ("lstm", 3, 2, 3),
                                          ("gru", 2, 1, 4), ("gru", 3, 3, 2)])
def test_stack_matches_torch_multilayer(cell, L, NH, Dh):
    T, B, Din = 7, 3, 4
    H = NH * Dh
    Ws, Rs, bs = layers(cell, L, Din, NH, Dh, 600 + L + NH)
    x = nrm(690, (T, B, Din), 1.0)
    h0 = nrm(691, (L, B, H), 0.2)
    c0 = nrm(692, (L, B, H), 0.2)
    if cell == "lstm":
        o = oracle.lstm_stack_fwd(x, Ws, Rs, bs, h0, c0, NH=NH, Dh=Dh)
    else:
        o = oracle.gru_stack_fwd(x, Ws, Rs, bs, h0, NH=NH, Dh=Dh)
    y, hn, cn = torch_stack(cell, x, Ws, Rs, bs, h0, c0, NH, Dh)
    assert np.max(np.abs(o["h_seq"] - y)) < 1e-12
    assert np.max(np.abs(o["hT"] - hn)) < 1e-12
    if cell == "lstm":
        assert np.max(np.abs(o["cT"] - cn)) < 1e-12


def test_single_layer_stack_is_the_layer():
    NH, Dh = 2, 3
    Ws, Rs, bs = layers("lstm", 1, 4, NH, Dh, 700)
    x = nrm(701, (5, 2, 4), 1.0)
    a = oracle.lstm_stack_fwd(x, Ws, Rs, bs, NH=NH, Dh=Dh, bf16_between=True)
    b = oracle.lstm_fwd(x, Ws[0], Rs[0], bs[0], NH=NH, Dh=Dh)
    assert np.array_equal(a["h_seq"], b["h_seq"]) and np.array_equal(a["cT"][0], b["cT"])


def test_round_bf16_exact_cases():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 (odd) and 1 + 2^-6: rounds up
    cases = {1.0: 1.0, 1.0 + 2.0 ** -8: 1.0, 1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,
             1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7, -2.5: -2.5,
             (2.0 - 2.0 ** -9): 2.0,            # carry into the exponent
             3.0e38: 226.0 * 2.0 ** 120}        # 3e38 = 225.69 * 2^120: 8 bits, up
    for v, want in cases.items():
        got = oracle.round_bf16(np.array([v]))[0]
        assert abs(got - want) <= abs(want) * 1e-7, (v, got, want)


def test_round_bf16_is_nearest_on_random_values():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))
    r = oracle.round_bf16(v)
    # r has 8 significant bits, and no bf16 neighbour is closer to float32(v)
    f = v.astype(np.float32).astype(np.float64)
    m, e = np.frexp(r)
    assert np.all(np.abs(m * 256 - np.round(m * 256)) == 0)
    ulp = np.ldexp(1.0, e - 8)
    assert np.all(np.abs(f - r) <= ulp / 2 * (1 + 1e-12))

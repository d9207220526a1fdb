"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of ``oracle/oracle.c`` (or in the stacked-layer
composition), builds it on the CPU, and checks that a named pin fails with
it while the same pin passes on the real oracle.

A pin that passed on a mutant would be a pin that cannot see that kind of
mistake; the list covers every oracle function: the input projection (bias,
operand orientation, row selection), the LSTM and GRU forward cells, both
BPTT sweeps (carries, gate derivatives, the R^T product), the parameter
gradients, and the bf16 rounding between stacked layers.
"""
import contextlib
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_gru as pin_gru
from tests import test_oracle_lstm as pin_lstm
from tests import test_oracle_proj as pin_proj

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted text, pins that must fail: (callable, args))
MUTANTS = [
    ("input_proj drops the bias",
     "for (int c = 0; c < N; ++c) o[c] = bias ? bias[c] : 0.0;",
     "for (int c = 0; c < N; ++c) o[c] = 0.0;",
     [(pin_proj.test_input_proj_full_matches_torch_linear, (37, 13, 20))]),
    ("input_proj reads W transposed",
     "const double *w = W + (size_t)k * N;\n            for (int c = 0; c < N; ++c) o[c] += xv * w[c];",
     "for (int c = 0; c < N; ++c) o[c] += xv * W[(size_t)c * K + k];",
     [(pin_proj.test_input_proj_full_matches_torch_linear, (37, 13, 20))]),
    ("input_proj ignores the row list",
     "const long m = rows ? rows[e] : e;",
     "const long m = e;",
     [(pin_proj.test_input_proj_rows_subset_matches_torch_linear, ())]),
    ("per-step projection drops the bias",
     "for (int c = 0; c < GD; ++c) gx[c] = bias ? bias[c0 + c] : 0.0;",
     "for (int c = 0; c < GD; ++c) gx[c] = 0.0;",
     [(pin_lstm.test_forward_matches_torch_lstmcell, (3, 4)),
      (pin_gru.test_forward_matches_torch_grucell, (3, 4))]),
    ("LSTM cell input uses o instead of z",
     "const double c = fg * cp[j] + ig * zg;",
     "const double c = fg * cp[j] + ig * og;",
     [(pin_lstm.test_forward_matches_torch_lstmcell, (1, 6)),
      (pin_lstm.test_single_step_by_hand, ())]),
    ("LSTM BPTT cell carry misses the forget gate",
     "dcn[j] = dc * fg;",
     "dcn[j] = dc;",
     [(pin_lstm.test_backward_matches_torch_autograd, ()),
      (pin_lstm.test_backward_matches_finite_differences, ())]),
    ("LSTM BPTT dA_f uses c_t instead of c_{t-1}",
     "d[Dh + j] = dc * cprev * fg * (1.0 - fg);",
     "d[Dh + j] = dc * ct * fg * (1.0 - fg);",
     [(pin_lstm.test_backward_matches_torch_autograd, ())]),
    ("LSTM BPTT R^T product skips the o gate",
     "for (int c = 0; c < GD; ++c) acc += d[c] * rr[c];",
     "for (int c = 0; c < 3 * Dh; ++c) acc += d[c] * rr[c];",
     [(pin_lstm.test_backward_matches_torch_autograd, ())]),
    ("GRU reset and update gates swapped",
     "const double rg = sigm(a[j] + s[j]);\n            const double ug = sigm(a[Dh + j] + s[Dh + j]);",
     "const double ug = sigm(a[j] + s[j]);\n            const double rg = sigm(a[Dh + j] + s[Dh + j]);",
     [(pin_gru.test_forward_matches_torch_grucell, (1, 6))]),
    ("GRU candidate without the reset gate",
     "const double ng = tanh(a[2 * Dh + j] + rg * s[2 * Dh + j]);",
     "const double ng = tanh(a[2 * Dh + j] + s[2 * Dh + j]);",
     [(pin_gru.test_forward_matches_torch_grucell, (1, 6)),
      (pin_gru.test_closed_reset_gate_cuts_the_candidate_recurrence, ())]),
    ("GRU BPTT drops the direct carry dh*u",
     "dd[j] = dh * ug;",
     "dd[j] = 0.0;",
     [(pin_gru.test_backward_matches_torch_autograd, ()),
      (pin_gru.test_backward_matches_finite_differences, ())]),
    ("dR pairs dS_t with h_t instead of h_{t-1}",
     "const double hv = t > 0 ? h_seq[((size_t)(t - 1) * B + b) * H + n * Dh + mm]",
     "const double hv = t + 1 < T ? h_seq[((size_t)t * B + b) * H + n * Dh + mm]",
     [(pin_lstm.test_backward_matches_torch_autograd, ())]),
]


def _build(tmp_path, name, text):
    src = tmp_path / (name + ".c")
    lib = tmp_path / ("lib" + name + ".so")
    src.write_text(text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                           str(src), "-lm"])
    return str(src), str(lib)


@contextlib.contextmanager
def _oracle_from(src, lib):
    saved = (oracle._SRC, oracle._LIB, oracle._lib)
    oracle._SRC, oracle._LIB, oracle._lib = src, lib, None
    try:
        yield
    finally:
        oracle._SRC, oracle._LIB, oracle._lib = saved


def _fails(fn, args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,orig,planted,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_oracle_mistake(tmp_path, name, orig, planted, pins):
    text = open(SRC).read()
    assert text.count(orig) == 1, "mutation site not found once: %r" % orig
    src, lib = _build(tmp_path, "mutant", text.replace(orig, planted))
    with _oracle_from(src, lib):
        for fn, args in pins:
            assert _fails(fn, args), "%s: pin %s passed on the mutant" % (name, fn.__name__)
    for fn, args in pins:          # and the real oracle passes the same pins
        fn(*args)


def _stack_pin():
    pin_proj.test_stack_bf16_between_matches_torch_chain("lstm", 3)


@pytest.mark.parametrize("name,rounding", [
    ("no rounding between layers", lambda a: np.asarray(a, np.float64)),
    ("float32 rounding only", lambda a: np.asarray(a, np.float64).astype(np.float32).astype(np.float64)),
    ("bf16 by truncation", lambda a: (np.asarray(a, np.float64).astype(np.float32).view(np.uint32)
                                      & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)),
])
def test_stack_pin_catches_wrong_rounding_between_layers(monkeypatch, name, rounding):
    monkeypatch.setattr(oracle, "round_bf16", rounding)
    assert _fails(_stack_pin, ()), name


def test_stack_pin_catches_cell_state_fed_forward(monkeypatch):
    real = oracle.lstm_fwd

    def feeds_c(*a, **k):
        r = dict(real(*a, **k))
        r["h_seq"], r["c_seq"] = r["c_seq"], r["h_seq"]
        return r

    monkeypatch.setattr(oracle, "lstm_fwd", feeds_c)
    assert _fails(_stack_pin, ())

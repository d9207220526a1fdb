"""Pins of the LSTM oracle against things other than itself:

* ``torch.nn.LSTMCell`` in float64 (a library routine), both for one head and
  for several heads embedded block-diagonally into one dense cell -- this
  fixes the gate order, the W column order and the block-diagonal layout;
* torch autograd on that dense cell for every gradient, and central finite
  differences of the oracle's own forward on a tiny case (brute force);
* closed forms: saturated gates, constant gates, one step;
* exact invariants: head and batch independence, head-permutation
  equivariance, causality and chunked resume (all bitwise).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.torch_pins import run_cell

G = 4


def case(T=5, B=3, Din=7, NH=2, Dh=4, seed=100, bias=None, h0_var=0.3, c0_var=0.3,
         backward=True, final=True):
    d = synth.Dims(T, B, Din, NH, Dh)
    if bias is None:
        bias_arr = synth.normal(seed + 50, NH * G * Dh, 0.5)
    else:
        bias_arr = bias
    return synth.make_case("lstm", d, "f32", seed, w_var=0.5, r_var=0.5, bias=bias_arr,
                           h0_var=h0_var, c0_var=c0_var, backward=backward,
                           final_grads=final)


def fwd(c, **kw):
    d = c.dims
    return oracle.lstm_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"),
                           c.f64("h0"), c.f64("c0"), NH=d.NH, Dh=d.Dh, **kw)


@pytest.mark.parametrize("NH,Dh", [(1, 6), (3, 4)])
def test_forward_matches_torch_lstmcell(NH, Dh):
    c = case(T=9, B=3, Din=5, NH=NH, Dh=Dh, seed=200 + NH)
    o = fwd(c)
    t = run_cell("lstm", c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"),
                 c.f64("h0"), c.f64("c0"), NH, Dh)
    assert np.max(np.abs(o["h_seq"] - t["h_seq"])) < 1e-12
    assert np.max(np.abs(o["c_seq"] - t["c_seq"])) < 1e-12
    assert np.array_equal(o["hT"], o["h_seq"][-1])
    assert np.array_equal(o["cT"], o["c_seq"][-1])


def test_backward_matches_torch_autograd():
    NH, Dh = 3, 4
    c = case(T=6, B=2, Din=5, NH=NH, Dh=Dh, seed=300)
    o = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                        c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"), NH=NH, Dh=Dh)
    t = run_cell("lstm", c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                 c.f64("c0"), NH, Dh, dH=c.f64("dH"), dhT=c.f64("dhT"), dcT=c.f64("dcT"))
    for k in ("dx", "dW", "dR", "db", "dh0", "dc0"):
        err = np.max(np.abs(o[k] - t[k])) / max(1.0, np.max(np.abs(t[k])))
        assert err < 1e-12, (k, err)


def _loss(c, x=None, W=None, R=None, b=None, h0=None, c0=None):
    d = c.dims
    o = oracle.lstm_fwd(c.f64("x") if x is None else x, c.f64("W") if W is None else W,
                        c.f64("R") if R is None else R, c.f64("b") if b is None else b,
                        c.f64("h0") if h0 is None else h0, c.f64("c0") if c0 is None else c0,
                        NH=d.NH, Dh=d.Dh)
    return (np.sum(o["h_seq"] * c.f64("dH")) + np.sum(o["hT"] * c.f64("dhT"))
            + np.sum(o["cT"] * c.f64("dcT")))


def test_backward_matches_finite_differences():
    c = case(T=4, B=2, Din=5, NH=2, Dh=3, seed=400)
    o = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                        c.f64("c0"), c.f64("dH"), c.f64("dhT"), c.f64("dcT"),
                        NH=2, Dh=3)
    names = {"x": "dx", "W": "dW", "R": "dR", "b": "db", "h0": "dh0", "c0": "dc0"}
    for p, g in names.items():
        base = c.f64(p)
        num = np.zeros_like(base)
        flat = base.reshape(-1)
        for i in range(flat.size):
            eps = 1e-6 * max(1.0, abs(flat[i]))
            up, dn = flat.copy(), flat.copy()
            up[i] += eps
            dn[i] -= eps
            num.reshape(-1)[i] = (_loss(c, **{p: up.reshape(base.shape)})
                                  - _loss(c, **{p: dn.reshape(base.shape)})) / (2 * eps)
        err = np.max(np.abs(num - o[g]))
        assert err < 2e-7, (p, err)


def test_saturated_gates_keep_cell_constant():
    """Forget bias +40, input bias -40: sigma(40) is 1.0 in double and
    sigma(-40) ~ 4e-18, so c_t = c0 for every t and h_t = sigma(A_o) tanh(c0)."""
    NH, Dh = 2, 5
    b = np.zeros((NH, G, Dh))
    b[:, 0] = -40.0
    b[:, 1] = 40.0
    c = case(T=12, B=3, Din=4, NH=NH, Dh=Dh, seed=500, bias=b.reshape(-1), backward=False)
    # shrink W and R so |A_i|, |A_f| stay far from the bias
    c.vals["W"] *= 0.1
    c.vals["R"] *= 0.1
    o = fwd(c)
    c0 = c.f64("c0")
    assert np.max(np.abs(o["c_seq"] - c0[None])) < 1e-15
    assert np.all(np.abs(o["h_seq"]) <= np.abs(np.tanh(c0))[None] + 1e-15)


def test_constant_gates_closed_form():
    """W = 0, R = 0: every gate is its constant bias, so
    c_t = f^t c0 + i z (1 - f^t)/(1 - f) and h_t = o tanh(c_t)."""
    NH, Dh, T = 2, 3, 17
    bias = synth.normal(600, NH * G * Dh, 1.0)
    c = case(T=T, B=2, Din=3, NH=NH, Dh=Dh, seed=600, bias=bias, backward=False)
    c.vals["W"][:] = 0
    c.vals["R"][:] = 0
    o = fwd(c)
    bb = c.f64("b").reshape(NH, G, Dh)
    sig = lambda a: 1 / (1 + np.exp(-a))
    i, f, z, og = sig(bb[:, 0]), sig(bb[:, 1]), np.tanh(bb[:, 2]), sig(bb[:, 3])
    i, f, z, og = (v.reshape(-1) for v in (i, f, z, og))
    c0 = c.f64("c0")
    for t in range(1, T + 1):
        ct = f ** t * c0 + i * z * (1 - f ** t) / (1 - f)
        assert np.max(np.abs(o["c_seq"][t - 1] - ct)) < 1e-13
        assert np.max(np.abs(o["h_seq"][t - 1] - og * np.tanh(ct))) < 1e-13


def test_single_step_by_hand():
    """T = 1 with x = 0 and h0 = 0: A = b exactly, so h_1 = o tanh(i z + f c0)."""
    NH, Dh = 2, 3
    bias = synth.normal(700, NH * G * Dh, 2.0)
    c = case(T=1, B=2, Din=3, NH=NH, Dh=Dh, seed=700, bias=bias, h0_var=0.0,
             backward=False)
    c.vals["x"][:] = 0
    o = fwd(c)
    bb = c.f64("b").reshape(NH, G, Dh)
    sig = lambda a: 1 / (1 + np.exp(-a))
    i, f, z, og = (v.reshape(-1) for v in (sig(bb[:, 0]), sig(bb[:, 1]),
                                            np.tanh(bb[:, 2]), sig(bb[:, 3])))
    c1 = f * c.f64("c0") + i * z
    assert np.max(np.abs(o["h_seq"][0] - og * np.tanh(c1))) < 1e-15


def test_head_and_batch_independence_bitwise():
    NH, Dh = 3, 4
    c = case(T=7, B=3, Din=5, NH=NH, Dh=Dh, seed=800, backward=False)
    base = fwd(c)
    # perturb head 1's R block, bias block and initial state
    c2 = case(T=7, B=3, Din=5, NH=NH, Dh=Dh, seed=800, backward=False)
    c2.vals["R"][1] += 0.5
    c2.vals["b"].reshape(NH, G, Dh)[1] += 0.5
    c2.vals["h0"][:, Dh:2 * Dh] += 1.0
    c2.vals["c0"][:, Dh:2 * Dh] -= 1.0
    pert = fwd(c2)
    keep = np.r_[0:Dh, 2 * Dh:3 * Dh]
    assert np.array_equal(base["h_seq"][..., keep], pert["h_seq"][..., keep])
    assert np.array_equal(base["c_seq"][..., keep], pert["c_seq"][..., keep])
    assert not np.array_equal(base["h_seq"][..., Dh:2 * Dh], pert["h_seq"][..., Dh:2 * Dh])
    # perturb batch row 2
    c3 = case(T=7, B=3, Din=5, NH=NH, Dh=Dh, seed=800, backward=False)
    c3.vals["x"][:, 2] += 1.0
    c3.vals["h0"][2] += 1.0
    p3 = fwd(c3)
    assert np.array_equal(base["h_seq"][:, :2], p3["h_seq"][:, :2])
    assert not np.array_equal(base["h_seq"][:, 2], p3["h_seq"][:, 2])


def test_head_permutation_equivariance_bitwise():
    NH, Dh = 3, 4
    c = case(T=6, B=2, Din=5, NH=NH, Dh=Dh, seed=900, backward=False)
    base = fwd(c)
    perm = [2, 0, 1]
    c2 = case(T=6, B=2, Din=5, NH=NH, Dh=Dh, seed=900, backward=False)
    Din = c.dims.Din
    c2.vals["R"] = c.vals["R"][perm].copy()
    c2.vals["W"] = c.vals["W"].reshape(Din, NH, G * Dh)[:, perm].reshape(Din, -1).copy()
    c2.vals["b"] = c.vals["b"].reshape(NH, G * Dh)[perm].reshape(-1).copy()
    hidx = np.concatenate([np.arange(p * Dh, (p + 1) * Dh) for p in perm])
    c2.vals["h0"] = c.vals["h0"][:, hidx].copy()
    c2.vals["c0"] = c.vals["c0"][:, hidx].copy()
    p = fwd(c2)
    assert np.array_equal(p["h_seq"], base["h_seq"][..., hidx])
    assert np.array_equal(p["c_seq"], base["c_seq"][..., hidx])


def test_causality_and_chunked_resume_bitwise():
    c = case(T=10, B=2, Din=5, NH=2, Dh=3, seed=1000, backward=False)
    full = fwd(c)
    d = c.dims
    x = c.f64("x")
    a = oracle.lstm_fwd(x[:4], c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                        c.f64("c0"), NH=d.NH, Dh=d.Dh)
    assert np.array_equal(a["h_seq"], full["h_seq"][:4])
    bpart = oracle.lstm_fwd(x[4:], c.f64("W"), c.f64("R"), c.f64("b"), a["hT"], a["cT"],
                            NH=d.NH, Dh=d.Dh)
    assert np.array_equal(bpart["h_seq"], full["h_seq"][4:])
    assert np.array_equal(bpart["cT"], full["cT"])


def test_chain_mask_and_thread_count_do_not_change_bits():
    c = case(T=8, B=3, Din=6, NH=3, Dh=4, seed=1100, backward=False)
    full = fwd(c)
    mask = np.zeros((3, 3), bool)
    mask[1, 2] = mask[0, 0] = True
    part = fwd(c, chain_mask=mask)
    H = c.dims.H
    for b, n in [(1, 2), (0, 0)]:
        sl = slice(n * 4, (n + 1) * 4)
        assert np.array_equal(part["h_seq"][:, b, sl], full["h_seq"][:, b, sl])
    assert np.isnan(part["h_seq"][:, 2]).all()
    assert H == 12


def test_db_is_sum_of_gate_grads_and_dR_of_zero_block():
    """db = sum_{t,b} dA; a head whose R block is zero still has
    dR = H_prev^T dA (not zero)."""
    NH, Dh = 2, 3
    c = case(T=5, B=2, Din=4, NH=NH, Dh=Dh, seed=1200)
    c.vals["R"][1] = 0
    o = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                        c.f64("c0"), c.f64("dH"), NH=NH, Dh=Dh)
    assert np.allclose(o["db"], o["dA"].sum(axis=(0, 1)), rtol=0, atol=1e-13)
    assert np.max(np.abs(o["dR"][1])) > 1e-3
    t = run_cell("lstm", c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                 c.f64("c0"), NH, Dh, dH=c.f64("dH"))
    assert np.max(np.abs(o["dR"] - t["dR"])) < 1e-12


def test_grad_entries_match_full_grads():
    NH, Dh = 2, 3
    c = case(T=5, B=2, Din=4, NH=NH, Dh=Dh, seed=1300)
    o = oracle.lstm_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                        c.f64("c0"), c.f64("dH"), NH=NH, Dh=Dh)
    args = (c.f64("x"), c.f64("W"), c.f64("h0"), o["h_seq"], o["dA"], o["dA"])
    kw = dict(NH=NH, Dh=Dh, G=4)
    assert np.array_equal(oracle.param_grad_entries("db", [[3], [20]], *args, **kw),
                          o["db"][[3, 20]])
    assert np.array_equal(oracle.param_grad_entries("dW", [[1, 3], [3, 20]], *args, **kw),
                          o["dW"][[1, 3], [3, 20]])
    dx = o["dx"].reshape(10, 4)
    assert np.array_equal(oracle.param_grad_entries("dx", [[7, 2], [0, 3]], *args, **kw),
                          dx[[7, 0], [2, 3]])
    assert np.array_equal(oracle.param_grad_entries("dR", [[1, 2, 11], [0, 0, 5]], *args, **kw),
                          o["dR"][[1, 0], [2, 0], [11, 5]])

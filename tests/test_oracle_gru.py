"""Pins of the GRU oracle: ``torch.nn.GRUCell`` float64 (reset-after form,
the library routine) for one and several heads, torch autograd and finite
differences for the backward, closed forms and exact invariants."""
import numpy as np
import pytest

import oracle
import synth
from tests.torch_pins import run_cell

G = 3


def case(T=5, B=3, Din=7, NH=2, Dh=4, seed=100, bias=None, h0_var=0.3, backward=True):
    d = synth.Dims(T, B, Din, NH, Dh)
    bias_arr = synth.normal(seed + 50, NH * G * Dh, 0.5) if bias is None else bias
    return synth.make_case("gru", d, "f32", seed, w_var=0.5, r_var=0.5, bias=bias_arr,
                           h0_var=h0_var, backward=backward, final_grads=True)


def fwd(c, **kw):
    d = c.dims
    return oracle.gru_fwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                          NH=d.NH, Dh=d.Dh, **kw)


@pytest.mark.parametrize("NH,Dh", [(1, 6), (3, 4)])
def test_forward_matches_torch_grucell(NH, Dh):
    c = case(T=9, B=3, Din=5, NH=NH, Dh=Dh, seed=2200 + NH)
    o = fwd(c)
    t = run_cell("gru", c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                 None, NH, Dh)
    assert np.max(np.abs(o["h_seq"] - t["h_seq"])) < 1e-12
    assert np.array_equal(o["hT"], o["h_seq"][-1])


def test_backward_matches_torch_autograd():
    NH, Dh = 3, 4
    c = case(T=6, B=2, Din=5, NH=NH, Dh=Dh, seed=2300)
    o = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                       c.f64("dH"), c.f64("dhT"), NH=NH, Dh=Dh)
    t = run_cell("gru", c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                 None, NH, Dh, dH=c.f64("dH"), dhT=c.f64("dhT"))
    for k in ("dx", "dW", "dR", "db", "dh0"):
        err = np.max(np.abs(o[k] - t[k])) / max(1.0, np.max(np.abs(t[k])))
        assert err < 1e-12, (k, err)


def test_backward_matches_finite_differences():
    c = case(T=4, B=2, Din=5, NH=2, Dh=3, seed=2400)
    d = c.dims
    o = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                       c.f64("dH"), c.f64("dhT"), NH=d.NH, Dh=d.Dh)

    def loss(**over):
        a = {k: over.get(k, c.f64(k)) for k in ("x", "W", "R", "b", "h0")}
        r = oracle.gru_fwd(a["x"], a["W"], a["R"], a["b"], a["h0"], NH=d.NH, Dh=d.Dh)
        return np.sum(r["h_seq"] * c.f64("dH")) + np.sum(r["hT"] * c.f64("dhT"))

    for p, g in {"x": "dx", "W": "dW", "R": "dR", "b": "db", "h0": "dh0"}.items():
        base = c.f64(p)
        flat = base.reshape(-1)
        num = np.zeros(flat.size)
        for i in range(flat.size):
            eps = 1e-6 * max(1.0, abs(flat[i]))
            up, dn = flat.copy(), flat.copy()
            up[i] += eps
            dn[i] -= eps
            num[i] = (loss(**{p: up.reshape(base.shape)})
                      - loss(**{p: dn.reshape(base.shape)})) / (2 * eps)
        err = np.max(np.abs(num - o[g].reshape(-1)))
        assert err < 2e-7, (p, err)


def test_constant_gates_closed_form():
    """W = 0, R = 0: r, u, nn are constants (nn = tanh(b_n) since the
    recurrent term is zero), so h_t = nn + u^t (h0 - nn)."""
    NH, Dh, T = 2, 3, 15
    c = case(T=T, B=2, Din=3, NH=NH, Dh=Dh, seed=2600, bias=synth.normal(2601, 18, 1.0),
             backward=False)
    c.vals["W"][:] = 0
    c.vals["R"][:] = 0
    o = fwd(c)
    bb = c.f64("b").reshape(NH, G, Dh)
    u = (1 / (1 + np.exp(-bb[:, 1]))).reshape(-1)
    nn = np.tanh(bb[:, 2]).reshape(-1)
    h0 = c.f64("h0")
    for t in range(1, T + 1):
        assert np.max(np.abs(o["h_seq"][t - 1] - (nn + u ** t * (h0 - nn)))) < 1e-14


def test_saturated_update_gate_holds_state_exactly():
    """Update bias +40: u = sigma(40) rounds to 1.0 in double, so h_t = h0 bitwise."""
    NH, Dh = 2, 4
    b = np.zeros((NH, G, Dh))
    b[:, 1] = 40.0
    c = case(T=9, B=3, Din=4, NH=NH, Dh=Dh, seed=2700, bias=b.reshape(-1), backward=False)
    c.vals["W"] *= 0.1
    c.vals["R"] *= 0.1
    o = fwd(c)
    assert np.array_equal(o["h_seq"], np.broadcast_to(c.f64("h0"), o["h_seq"].shape))


def test_closed_reset_gate_cuts_the_candidate_recurrence():
    """Reset bias -40 (r ~ 4e-18): the n-gate block of R only enters through
    r * S_n, so changing it moves h by less than 1e-15."""
    NH, Dh = 2, 4
    b = np.zeros((NH, G, Dh))
    b[:, 0] = -40.0
    c = case(T=8, B=2, Din=4, NH=NH, Dh=Dh, seed=2800, bias=b.reshape(-1), backward=False)
    c.vals["W"] *= 0.1
    base = fwd(c)
    c.vals["R"].reshape(NH, Dh, G, Dh)[:, :, 2] += 3.0
    pert = fwd(c)
    assert np.max(np.abs(base["h_seq"] - pert["h_seq"])) < 1e-15


def test_head_independence_and_resume_bitwise():
    NH, Dh = 3, 4
    c = case(T=8, B=2, Din=5, NH=NH, Dh=Dh, seed=2900, backward=False)
    base = fwd(c)
    c2 = case(T=8, B=2, Din=5, NH=NH, Dh=Dh, seed=2900, backward=False)
    c2.vals["R"][2] *= -1
    c2.vals["h0"][:, 2 * Dh:] += 1
    pert = fwd(c2)
    assert np.array_equal(base["h_seq"][..., :2 * Dh], pert["h_seq"][..., :2 * Dh])
    d = c.dims
    x = c.f64("x")
    a = oracle.gru_fwd(x[:3], c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"), NH=d.NH, Dh=d.Dh)
    r = oracle.gru_fwd(x[3:], c.f64("W"), c.f64("R"), c.f64("b"), a["hT"], NH=d.NH, Dh=d.Dh)
    assert np.array_equal(np.concatenate([a["h_seq"], r["h_seq"]]), base["h_seq"])


def test_gate_grad_split_only_differs_in_candidate_gate():
    NH, Dh = 2, 3
    c = case(T=5, B=2, Din=4, NH=NH, Dh=Dh, seed=3000)
    o = oracle.gru_bwd(c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"),
                       c.f64("dH"), NH=NH, Dh=Dh, grads=())
    gx = o["dGx"].reshape(5, 2, NH, G, Dh)
    s = o["dS"].reshape(5, 2, NH, G, Dh)
    assert np.array_equal(gx[:, :, :, :2], s[:, :, :, :2])
    assert not np.array_equal(gx[:, :, :, 2], s[:, :, :, 2])

"""The recurrence's plan search (rnn_plan_search) on the CPU: every
candidate it calls feasible meets the constraints it reports, the choice is
the fastest feasible candidate, the split-R fragment split follows from the
register and LDS budgets, overrides fix variables, and the latency model
tracks and ranks the measured recurrence times of this library's kernels
(tests/golden/plan_measurements.json, measured on one MI355X)."""
import json
import os

import pytest
from hypothesis import given, settings, strategies as st

import gru_recurrence_amd as g

HERE = os.path.dirname(os.path.abspath(__file__))
POINTS = json.load(open(os.path.join(HERE, "golden", "plan_measurements.json")))["points"]
CUS = 256
ENV = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_KCW", "RNN355_REC_WIDE", "RNN355_MC_XCD")


@pytest.fixture(autouse=True)
def _clean_env():
    old = {k: os.environ.pop(k, None) for k in ENV}
    yield
    for k, v in old.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


def search(cell, T, B, NH, Dh, dtype="bf16", cus=CUS):
    op = g.OP_REC_LSTM if cell == "lstm" else g.OP_REC_GRU
    dt = g.RNN_BF16 if dtype == "bf16" else g.RNN_F32
    return g.plan_search(op, g.Dims(T, B, 64, NH, Dh), dt, cus)


def plan_vars(plan, Dh):
    """Family and integers of a rnn_plan_describe string."""
    kv = dict(t.split("=") for t in plan.split() if "=" in t)
    fam = {"mfma_resident_R": 1, "mfma_split_R": 2, "mfma_multi_cu": 3, "lds_simple": 4}[kv["rec_kernel"]]
    v = dict(family=fam, rows_per_wg=int(kv["rows_per_wg"]))
    if fam == 3:
        v["wg_per_head"] = int(kv["wg_per_head_row_tile"])
        v["blocks_per_wg"] = int(kv["units_per_wg"]) // 16
        v["k_splits"] = int(kv["k_splits"])
        v["kchunks_per_wave"] = Dh // 32 // v["k_splits"]
        v["xcd_local"] = int(kv.get("exchange", "memory") == "xcd_l2")
    return v


def match(cands, v):
    hits = [c for c in cands if all(c[k] == x for k, x in v.items())]
    if v["family"] == 2:
        hits = [c for c in hits if c["feasible"]]
    assert len(hits) >= 1, v
    return hits[0]


def test_feasible_candidates_meet_their_constraints_on_the_workload_shapes():
    for shape in [("lstm", 1024, 16, 6, 128), ("gru", 2048, 4, 12, 64), ("lstm", 1024, 16, 1, 768),
                  ("lstm", 1024, 16, 4, 256), ("gru", 1024, 16, 4, 256)]:
        cands, best = search(*shape)
        _check_all(shape[0], shape[2], shape[4], "bf16", cands, best)


@settings(max_examples=60, deadline=None)
@given(cell=st.sampled_from(["lstm", "gru"]), B=st.integers(1, 80), NH=st.integers(1, 16),
       Dh=st.sampled_from([16, 32, 48, 64, 96, 128, 256, 384, 512, 768, 1024]),
       dtype=st.sampled_from(["bf16", "f32"]), cus=st.sampled_from([64, 128, 256, 304]))
def test_feasible_candidates_meet_their_constraints(cell, B, NH, Dh, dtype, cus):
    cands, best = search(cell, 64, B, NH, Dh, dtype, cus)
    _check_all(cell, B, Dh, dtype, cands, best, cus)


def _check_all(cell, B, Dh, dtype, cands, best, cus=CUS):
    G = 4 if cell == "lstm" else 3
    feas = [c for c in cands if c["feasible"]]
    for c in cands:
        assert (c["violated"] == 0) == bool(c["feasible"])
    for c in feas:
        assert 1 <= c["rows_per_wg"] <= min(B, 16)
        assert c["r_vgpr"] <= 128 and c["wg_per_cu"] >= 1
        if c["family"] == 1:
            assert dtype == "bf16" and Dh in (32, 64, 128)
            assert c["waves"] == Dh // 16 and c["lds_bytes"] <= 160 * 1024
        elif c["family"] == 2:
            assert dtype == "bf16" and Dh == 256 and c["wg_per_cu"] == 1
            assert 4 * c["frags_agpr"] <= 256 and 4 * c["frags_vgpr"] + 128 <= 256
            assert c["frags_agpr"] + c["frags_vgpr"] + c["frags_lds"] == 2 * G * 16
            assert c["lds_bytes"] <= 160 * 1024
        elif c["family"] == 3:
            assert dtype == "bf16" and Dh >= 256 and Dh % 128 == 0
            assert Dh == 16 * c["blocks_per_wg"] * c["wg_per_head"] and c["wg_per_head"] >= 2
            assert Dh // 32 == c["kchunks_per_wave"] * c["k_splits"]
            assert c["waves"] == c["blocks_per_wg"] * c["k_splits"] <= 8
            assert c["grid"] <= cus and c["lds_bytes"] <= 160 * 1024
        else:
            assert c["lds_bytes"] <= 64 * 1024
    if not feas:
        assert best == -1
        return
    assert best >= 0 and cands[best]["feasible"]
    assert cands[best]["ns_total"] <= min(c["ns_total"] for c in feas) * (1 + 1e-9)


@pytest.mark.parametrize("cell,fl", [("lstm", 32), ("gru", 0)])
def test_split_r_fragment_split_follows_from_the_budgets(cell, fl):
    """Among the split-R splits that the register and LDS budgets allow
    (feasible, or only not compiled), the cheapest is the compiled one:
    every AGPR used, then VGPRs, the rest in LDS; it is the choice where the
    multi-CU exchange goes through memory."""
    os.environ["RNN355_MC_XCD"] = "0"
    cands, best = search(cell, 1024, 16, 4, 256)
    ok = [c for c in cands if c["family"] == 2 and c["violated"] in (0, 1)]
    top = min(ok, key=lambda c: c["ns_total"])
    assert (top["frags_agpr"], top["frags_vgpr"], top["frags_lds"]) == (64, 32, fl)
    assert top["feasible"] and cands[best] == top


def test_overrides_fix_variables():
    os.environ["RNN355_REC_BT"] = "4"
    cands, best = search("lstm", 1024, 16, 6, 128)
    assert cands[best]["rows_per_wg"] == 4
    os.environ.pop("RNN355_REC_BT")
    os.environ["RNN355_REC_WIDE"] = "0"
    cands, best = search("lstm", 1024, 16, 4, 256)
    assert cands[best]["family"] == 3
    os.environ["RNN355_REC_K"] = "2"
    cands, best = search("lstm", 1024, 16, 4, 256)
    assert cands[best]["family"] == 3 and cands[best]["wg_per_head"] == 2
    assert cands[best]["xcd_local"] == 1
    os.environ["RNN355_MC_XCD"] = "0"
    cands, best = search("lstm", 1024, 16, 4, 256)
    assert cands[best]["family"] == 3 and cands[best]["xcd_local"] == 0


@pytest.mark.parametrize("shape,want", [
    (("lstm", 1024, 16, 6, 128, "bf16"), dict(family=1, rows_per_wg=1, grid=96)),
    (("gru", 2048, 4, 12, 64, "bf16"), dict(family=1, rows_per_wg=1, grid=48)),
    (("lstm", 1024, 16, 1, 768, "bf16"), dict(family=3, rows_per_wg=2, wg_per_head=24,
                                             kchunks_per_wave=8)),
    (("lstm", 1024, 16, 4, 256, "bf16"), dict(family=3, wg_per_head=4, rows_per_wg=1,
                                             xcd_local=1)),
    (("lstm", 64, 2, 1, 384, "bf16"), dict(family=3, xcd_local=0)),   # 2 groups: memory
    (("lstm", 64, 2, 1, 32, "f32"), dict(family=4, rows_per_wg=2)),
])
def test_workload_plans(shape, want):
    cands, best = search(*shape)
    for k, v in want.items():
        assert cands[best][k] == v, (k, cands[best])


def _predicted(p):
    """The model's time for the measured plan (under the point's exchange and
    row layout settings: RNN355_MC_XCD=0 prices the multi-CU exchange through
    memory, RNN355_MC_ROWLANES=0 the cell update over register slots)."""
    keys = ("RNN355_MC_XCD", "RNN355_MC_ROWLANES")
    for k in keys:
        if k in p["env"]:
            os.environ[k] = p["env"][k]
    try:
        cands, _ = search(p["cell"], p["T"], p["B"], p["NH"], p["Dh"], p["dtype"])
    finally:
        for k in keys:
            os.environ.pop(k, None)
    c = match(cands, plan_vars(p["plan"], p["Dh"]))
    return c["ns_total"] / p["T"], c


def test_predictions_track_the_measured_times():
    worst = 0.0
    for p in POINTS:
        pred, c = _predicted(p)
        assert c["feasible"], p
        r = pred / p["ns_step"]
        print("  %-4s B=%-3d NH=%-2d Dh=%-4d %-4s %-45s meas %7.1f pred %7.1f" % (
            p["cell"], p["B"], p["NH"], p["Dh"], p["dtype"], json.dumps(p["env"]), p["ns_step"],
            pred))
        worst = max(worst, abs(r - 1))
        assert 0.6 <= r <= 1.5, (p, pred)
    print("  worst relative error %.2f" % worst)


def _groups():
    out = {}
    for p in POINTS:
        out.setdefault((p["cell"], p["T"], p["B"], p["NH"], p["Dh"], p["dtype"]), []).append(p)
    return out


def test_model_ranks_measured_alternatives_like_the_measurements():
    pairs = 0
    for key, ps in _groups().items():
        pl = [(p["ns_step"], _predicted(p)[0], p["plan"]) for p in ps]
        for i in range(len(pl)):
            for j in range(i + 1, len(pl)):
                (ma, pa, qa), (mb, pb, qb) = pl[i], pl[j]
                if qa == qb or abs(ma - mb) < 0.05 * min(ma, mb):
                    continue
                pairs += 1
                assert (ma < mb) == (pa < pb), (key, qa, ma, pa, qb, mb, pb)
    assert pairs >= 10


def test_default_choice_is_the_best_measured_plan():
    for key, ps in _groups().items():
        if len(ps) < 2:
            continue
        cands, best = search(*key)
        chosen = {k: cands[best][k] for k in ("family", "rows_per_wg", "wg_per_head")}
        meas = {}
        for p in ps:
            if "RNN355_MC_XCD" in p["env"] or "RNN355_MC_ROWLANES" in p["env"]:
                continue  # the defaults keep the XCD grouping and row lanes on
            v = plan_vars(p["plan"], key[4])
            meas[(v["family"], v["rows_per_wg"], v.get("wg_per_head", 1))] = p["ns_step"]
        k = (chosen["family"], chosen["rows_per_wg"], chosen["wg_per_head"])
        if k in meas:
            assert meas[k] <= min(meas.values()) * 1.03, (key, k, meas)


def test_plan_search_rejects_bad_arguments():
    import ctypes
    lib = g.load()
    n, b = ctypes.c_int(0), ctypes.c_int(0)
    d = g.Dims(8, 2, 32, 1, 64)
    assert lib.rnn_plan_search(g.OP_REC_LSTM, ctypes.byref(d), g.RNN_BF16, 256, None, 4,
                               ctypes.byref(n), ctypes.byref(b)) == g.RNN_ERR_INVALID_ARG
    assert lib.rnn_plan_search(9, ctypes.byref(d), g.RNN_BF16, 256, None, 0, ctypes.byref(n),
                               ctypes.byref(b)) == g.RNN_ERR_INVALID_ARG
    bad = g.Dims(8, 0, 32, 1, 64)
    assert lib.rnn_plan_search(g.OP_REC_LSTM, ctypes.byref(bad), g.RNN_BF16, 256, None, 0,
                               ctypes.byref(n), ctypes.byref(b)) == g.RNN_ERR_INVALID_ARG
    # no kernel for a 16-unit f32 head too large for LDS: unsupported, -1
    big = g.Dims(8, 2, 32, 1, 512)
    assert lib.rnn_plan_search(g.OP_REC_LSTM, ctypes.byref(big), g.RNN_F32, 256, None, 0,
                               ctypes.byref(n), ctypes.byref(b)) == g.RNN_ERR_UNSUPPORTED
    assert b.value == -1 and n.value > 0


def test_rows_override_is_clamped_to_the_batch():
    os.environ["RNN355_REC_BT"] = "4"
    cands, best = search("lstm", 19, 3, 2, 128)
    assert best >= 0 and cands[best]["rows_per_wg"] == 3

"""Writes plan_measurements.json: the recurrence's time per step on one
MI355X for a fixed list of shapes and plan overrides, the calibration and
validation data of the plan search's latency model (tests/test_plan_search.py
checks the model against it).  These are measurements of this library's
kernels, not values from the pages and not expected outputs of any parity
test.

    python tests/golden/make_plan_measurements.py [--out PATH]

Each point: random Gx and R (bf16 R for bf16 points), one warm-up launch of
the recurrence entry point (rnn_rec_lstm / rnn_rec_gru) with the point's
RNN355_* overrides set, then three launches each bracketed by HIP events on
the stream they run on; ns_step = mean launch time / T.  `plan` is
rnn_plan_describe of the plan that ran (without its predicted time).
"""
import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

OVERRIDES = ("RNN355_REC_BT", "RNN355_REC_K", "RNN355_REC_WIDE", "RNN355_MC_XCD",
             "RNN355_MC_ROWLANES", "RNN355_REC_KCW")

# (cell, T, B, NH, Dh, dtype, overrides)
POINTS = [
    ("lstm", 1024, 16, 6, 128, "bf16", {}),
    ("lstm", 1024, 16, 6, 128, "bf16", {"RNN355_REC_BT": "2"}),
    ("lstm", 1024, 16, 6, 128, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 1024, 16, 6, 128, "bf16", {"RNN355_REC_BT": "16"}),
    ("gru", 2048, 4, 12, 64, "bf16", {}),
    ("lstm", 512, 64, 12, 64, "bf16", {}),
    ("lstm", 512, 64, 12, 64, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 64, 12, 128, "bf16", {}),
    ("lstm", 512, 64, 12, 128, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 16, 4, 256, "bf16", {}),
    ("gru", 512, 16, 4, 256, "bf16", {}),
    ("lstm", 512, 4, 4, 32, "f32", {}),
    ("lstm", 512, 4, 4, 32, "f32", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 64, 6, 64, "bf16", {}),
    ("lstm", 512, 64, 6, 64, "bf16", {"RNN355_REC_BT": "2"}),
    ("lstm", 512, 64, 12, 32, "bf16", {}),
    ("lstm", 512, 64, 12, 32, "bf16", {"RNN355_REC_BT": "4"}),
    ("gru", 512, 64, 12, 64, "bf16", {}),
    ("gru", 512, 64, 12, 64, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 2, 1, 32, "f32", {}),
    ("gru", 512, 8, 2, 48, "f32", {}),
    ("lstm", 512, 16, 1, 768, "bf16", {}),
    ("lstm", 512, 16, 1, 768, "bf16", {"RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 2, 768, "bf16", {}),
    ("lstm", 512, 16, 2, 768, "bf16", {"RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 2, 768, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 16, 2, 768, "bf16", {"RNN355_REC_BT": "4", "RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_REC_K": "2"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_REC_K": "2",
                                       "RNN355_MC_XCD": "0"}),
    ("lstm", 512, 2, 1, 384, "bf16", {}),
    ("lstm", 512, 2, 1, 384, "bf16", {"RNN355_REC_K": "12"}),
    ("lstm", 512, 1, 1, 768, "bf16", {}),
    ("lstm", 512, 1, 1, 768, "bf16", {"RNN355_REC_K": "24"}),
    ("lstm", 512, 16, 6, 384, "bf16", {}),
    ("lstm", 512, 16, 6, 384, "bf16", {"RNN355_REC_BT": "8"}),
    ("gru", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0"}),
    ("gru", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_MC_XCD": "0"}),
    ("lstm", 512, 8, 1, 512, "bf16", {}),
    ("lstm", 512, 8, 1, 512, "bf16", {"RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 2, 512, "bf16", {}),
    ("lstm", 512, 16, 2, 512, "bf16", {"RNN355_MC_XCD": "0"}),
    ("gru", 512, 16, 1, 768, "bf16", {}),
    ("gru", 512, 16, 1, 768, "bf16", {"RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 1, 384, "bf16", {}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_REC_BT": "1"}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_REC_BT": "1", "RNN355_MC_XCD": "0"}),
    ("lstm", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "4"}),
    ("gru", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_REC_BT": "2"}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_REC_BT": "4"}),
    ("lstm", 512, 16, 6, 384, "bf16", {"RNN355_MC_ROWLANES": "0"}),
    ("lstm", 512, 16, 6, 384, "bf16", {"RNN355_REC_BT": "8", "RNN355_MC_ROWLANES": "0"}),
    ("lstm", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "8"}),
    ("lstm", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "8", "RNN355_MC_ROWLANES": "0"}),
    ("lstm", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "16"}),
    ("lstm", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "16", "RNN355_MC_ROWLANES": "0"}),
    ("gru", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "8"}),
    ("gru", 512, 16, 1, 768, "bf16", {"RNN355_REC_BT": "8", "RNN355_MC_ROWLANES": "0"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_REC_BT": "8"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_REC_BT": "8",
                                       "RNN355_MC_ROWLANES": "0"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_REC_BT": "16"}),
    ("lstm", 512, 16, 4, 256, "bf16", {"RNN355_REC_WIDE": "0", "RNN355_REC_BT": "16",
                                       "RNN355_MC_ROWLANES": "0"}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_REC_BT": "8"}),
    ("lstm", 512, 16, 1, 384, "bf16", {"RNN355_REC_BT": "8", "RNN355_MC_ROWLANES": "0"}),
    # one CU per (head, rows), rows in lane groups (2 to 8 rows per workgroup)
    ("lstm", 1024, 16, 6, 128, "bf16", {"RNN355_REC_BT": "8"}),
    ("lstm", 512, 64, 12, 64, "bf16", {"RNN355_REC_BT": "8"}),
    ("lstm", 512, 64, 12, 128, "bf16", {"RNN355_REC_BT": "8"}),
    ("lstm", 512, 64, 12, 32, "bf16", {"RNN355_REC_BT": "2"}),
    ("gru", 512, 64, 12, 64, "bf16", {"RNN355_REC_BT": "8"}),
    ("gru", 512, 64, 12, 64, "bf16", {"RNN355_REC_BT": "1"}),
    ("lstm", 512, 64, 12, 64, "bf16", {"RNN355_REC_BT": "1"}),
]

ABOUT = (
    "Recurrence time per step (ns) of this library's kernels on one MI355X, measured with HIP "
    "events over 3 launches after one warm-up (T steps, random Gx, Din=64 irrelevant to the "
    "recurrence), for given plan overrides; the plan column is rnn_plan_describe of the plan "
    "that ran.  Calibration and validation data of the plan search's latency model "
    "(measurements of this library, not values from the pages).  Multi-CU points: the plan "
    "string names the exchange (exchange=xcd_l2: the head tile's workgroups on one XCD, h "
    "through its L2; exchange=memory: through memory, RNN355_MC_XCD=0 or groups that do not "
    "divide over the 8 XCDs).  Points with RNN355_MC_ROWLANES=0 ran the multi-CU cell update "
    "over register row slots (one pass per slot) instead of the default rows in lane groups "
    "(one pass per four rows).  Written by tests/golden/make_plan_measurements.py.")


def measure(cell, T, B, NH, Dh, dtype, env, reps=3):
    import torch
    import gru_recurrence_amd as g
    for k in OVERRIDES:
        os.environ.pop(k, None)
    os.environ.update(env)
    G = 4 if cell == "lstm" else 3
    gen = torch.Generator(device="cuda").manual_seed(T * 7 + B * 13 + NH * 17 + Dh)
    gx = torch.randn((T, B, NH * G * Dh), device="cuda", generator=gen)
    R = torch.randn((NH, Dh, G * Dh), device="cuda", generator=gen) / Dh ** 0.5
    if dtype == "bf16":
        R = R.to(torch.bfloat16)
    op = g.OP_REC_LSTM if cell == "lstm" else g.OP_REC_GRU
    d = g.Dims(T, B, 64, NH, Dh)
    dt = g.RNN_BF16 if dtype == "bf16" else g.RNN_F32
    plan = g.plan_describe(op, d, dt).split(" predicted_ns_per_step")[0]
    ws = torch.empty(g.workspace_size(op, d, dt), dtype=torch.uint8, device="cuda")
    run = (lambda: g.rec_lstm(gx, R, ws=ws)) if cell == "lstm" else (lambda: g.rec_gru(gx, R, ws=ws))
    run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        run()
        e[1].record()
        torch.cuda.synchronize()
        ms.append(e[0].elapsed_time(e[1]))
    assert g.workspace_status(ws) == g.RNN_OK
    for k in env:
        os.environ.pop(k, None)
    return round(sum(ms) / len(ms) * 1e6 / T, 1), plan


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "plan_measurements.json"))
    args = ap.parse_args()
    pts = []
    for cell, T, B, NH, Dh, dtype, env in POINTS:
        ns, plan = measure(cell, T, B, NH, Dh, dtype, env)
        print("%-4s T%-5d B%-3d NH%-3d Dh%-4d %-4s %-70s %8.1f ns  %s"
              % (cell, T, B, NH, Dh, dtype, json.dumps(env), ns, plan), flush=True)
        pts.append(dict(cell=cell, T=T, B=B, NH=NH, Dh=Dh, dtype=dtype, env=env, ns_step=ns,
                        plan=plan))
    with open(args.out, "w") as f:
        json.dump({"about": ABOUT, "points": pts}, f, indent=1)


if __name__ == "__main__":
    main()

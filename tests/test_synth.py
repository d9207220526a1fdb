"""The shared input generator: SplitMix64 stream, Box-Muller normals and
bf16 round-to-nearest-even (checked against torch's own conversion)."""
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.txt")


def test_splitmix64_published_values():
    want = [int(l, 16) for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    got = synth.splitmix64(0, len(want))
    assert [int(v) for v in got] == want


def test_normal_moments_and_determinism():
    z = synth.normal(1234, 200001, 0.1)
    assert abs(z.mean()) < 3e-3
    assert abs(z.var() - 0.1) < 2e-3
    assert np.array_equal(z, synth.normal(1234, 200001, 0.1))
    assert not np.array_equal(z[:10], synth.normal(1235, 10, 0.1))


def test_bf16_rne_matches_torch():
    a = synth.normal(7, 100000, 4.0).astype(np.float32)
    # include exact halfway cases of both parities
    halves = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000],
                      dtype=np.uint32).view(np.float32)
    a = np.concatenate([a, halves])
    ours = synth.f32_to_bf16_bits(a)
    theirs = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_workload_recipes():
    w = synth.WORKLOADS["lstm_mh_b16_nh6_dh128"]
    d = synth.Dims(T=3, B=16, Din=768, NH=6, Dh=128)
    c = synth.workload_case(w, d)
    assert c.vals["x"].shape == (3, 16, 768)
    assert c.vals["W"].shape == (768, 6 * 4 * 128)
    assert c.vals["R"].shape == (6, 128, 512)
    b = c.vals["b"].reshape(6, 4, 128)
    assert np.all(b[:, 1] == 1.0) and np.all(b[:, [0, 2, 3]] == 0.0)
    assert np.all(c.vals["h0"] == 0) and np.all(c.vals["c0"] == 0)
    # stored values are exactly representable in bf16
    assert np.array_equal(synth.bf16_bits_to_f32(c.bits["R"]), c.vals["R"])
    g = synth.workload_case(synth.WORKLOADS["gru_mh_b4_nh12_dh64"],
                            synth.Dims(T=2, B=4, Din=768, NH=12, Dh=64))
    assert abs(g.vals["h0"].std() - np.sqrt(0.1)) < 0.02

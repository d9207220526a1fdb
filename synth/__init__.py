"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests
and the benchmark.

This module holds no arithmetic of the recurrence itself: it only draws
random numbers and rounds them to the storage precision.  Both sides of
every parity check receive the very same buffers from here.

Recipe (one stream per tensor):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014) seeded with ``seed`` gives 64-bit words;
  * the top 53 bits of each word give a uniform in (0, 1);
  * Box-Muller (Box & Muller 1958) turns consecutive uniform pairs into
    standard normals, in float64;
  * the normals are scaled by sqrt(variance), rounded once to float32, and
    then to bfloat16 with round-to-nearest-even where the workload stores
    that tensor in bf16.

Seeds follow ``1000 * workload_id + tensor_id`` with tensor ids
x=1, W=2, R=3, b=4, h0=5, c0=6, dH=7.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {"x": 1, "W": 2, "R": 3, "b": 4, "h0": 5, "c0": 6, "dH": 7,
              "dhT": 8, "dcT": 9}


def splitmix64(seed: int, n: int) -> np.ndarray:
    """First ``n`` outputs of SplitMix64 started from state ``seed``."""
    with np.errstate(over="ignore"):
        k = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform_open01(seed: int, n: int) -> np.ndarray:
    """Uniforms in the open interval (0, 1): (top53 + 0.5) * 2^-53."""
    top = (splitmix64(seed, n) >> np.uint64(11)).astype(np.float64)
    return (top + 0.5) * (2.0 ** -53)


def normal(seed: int, n: int, variance: float = 1.0) -> np.ndarray:
    """``n`` draws of N(0, variance) as float64 (second parameter = variance)."""
    m = (n + 1) // 2
    u = uniform_open01(seed, 2 * m)
    u1, u2 = u[0::2], u[1::2]
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = rad * np.cos(ang)
    z[1::2] = rad * np.sin(ang)
    return z[:n] * np.sqrt(variance)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returning the 16-bit pattern."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def quantize(a64: np.ndarray, dtype: str):
    """float64 -> storage dtype.  Returns (values as float32, bf16 bits or None)."""
    a32 = np.asarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32, None
    if dtype == "bf16":
        bits = f32_to_bf16_bits(a32)
        return bf16_bits_to_f32(bits), bits
    raise ValueError(dtype)


@dataclass(frozen=True)
class Dims:
    T: int
    B: int
    Din: int
    NH: int
    Dh: int

    @property
    def H(self) -> int:
        return self.NH * self.Dh


def gates_of(cell: str) -> int:
    return {"lstm": 4, "gru": 3}[cell]


@dataclass
class Workload:
    """A named synthetic workload: shapes, storage precision and the
    distributions of every input (variances, bias pattern, initial state)."""
    wid: int
    name: str
    cell: str                    # "lstm" | "gru"
    dims: Dims
    dtype: str                   # storage of x, W, R: "f32" | "bf16"
    x_var: float = 1.0
    w_var: Optional[float] = None   # default 1/Din
    r_var: Optional[float] = None   # default 1/Dh
    bias: str = "zero"           # "zero" | "forget+1"
    h0_var: float = 0.0          # 0 -> zero initial state
    c0_var: float = 0.0
    backward: bool = False
    dH_var: float = 1.0
    layers: int = 1              # stacked layers (layer l > 0 reads layer l-1's h)
    chunk: int = 0               # > 0: forward in chunks of this many steps, BPTT from
                                 # checkpoints at the chunk ends
    note: str = ""


WORKLOADS: Dict[str, Workload] = {
    "lstm_fp32_tiny": Workload(
        1, "lstm_fp32_tiny", "lstm", Dims(T=64, B=2, Din=32, NH=1, Dh=32), "f32",
        note="LSTM forward, fp32 throughout, tiny case the oracle finishes at once"),
    "lstm_mh_b16_nh6_dh128": Workload(
        2, "lstm_mh_b16_nh6_dh128", "lstm", Dims(T=1024, B=16, Din=768, NH=6, Dh=128), "bf16",
        bias="forget+1",
        note="multi-head LSTM forward, bf16 x/W/R, fp32 state; the headline workload"),
    "gru_mh_b4_nh12_dh64": Workload(
        3, "gru_mh_b4_nh12_dh64", "gru", Dims(T=2048, B=4, Din=768, NH=12, Dh=64), "bf16",
        h0_var=0.1,
        note="multi-head GRU forward, small-batch latency case"),
    "lstm_1h_b16_dh768": Workload(
        4, "lstm_1h_b16_dh768", "lstm", Dims(T=1024, B=16, Din=768, NH=1, Dh=768), "bf16",
        bias="forget+1",
        note="single large head: R spans several CUs with a step barrier"),
    "lstm_fwdbwd_b16_nh4_dh256": Workload(
        5, "lstm_fwdbwd_b16_nh4_dh256", "lstm", Dims(T=1024, B=16, Din=1024, NH=4, Dh=256), "bf16",
        bias="forget+1", backward=True,
        note="multi-head LSTM forward plus BPTT backward"),
    "lstm_stack2_b16_nh6_dh128": Workload(
        6, "lstm_stack2_b16_nh6_dh128", "lstm", Dims(T=1024, B=16, Din=768, NH=6, Dh=128), "bf16",
        bias="forget+1", layers=2,
        note="two stacked layers of the multi-head LSTM (second layer's W is [H][N])"),
    "lstm_long_t8k_b16_nh6_dh128": Workload(
        7, "lstm_long_t8k_b16_nh6_dh128", "lstm", Dims(T=8192, B=16, Din=768, NH=6, Dh=128),
        "bf16", bias="forget+1", chunk=1024,
        note="the headline LSTM over a sequence 8x longer, forward in chunks of 1024 steps"),
    "lstm_fwdbwd_ckpt_b16_nh4_dh256": Workload(
        8, "lstm_fwdbwd_ckpt_b16_nh4_dh256", "lstm", Dims(T=1024, B=16, Din=1024, NH=4, Dh=256),
        "bf16", bias="forget+1", backward=True, chunk=256,
        note="forward plus BPTT of the Dh=256 workload with checkpoints every 256 steps"),
}

BY_ID = {w.wid: w for w in WORKLOADS.values()}


def bias_vector(cell: str, dims: Dims, pattern: str) -> np.ndarray:
    """Bias laid out [NH][G][Dh] (float64).  'forget+1' sets the LSTM forget
    gate (gate index 1 in the order i, f, z, o) to +1 and the rest to 0."""
    G = gates_of(cell)
    b = np.zeros((dims.NH, G, dims.Dh), dtype=np.float64)
    if pattern == "forget+1":
        if cell != "lstm":
            raise ValueError("forget bias only exists for the LSTM")
        b[:, 1, :] = 1.0
    elif pattern != "zero":
        raise ValueError(pattern)
    return b.reshape(-1)


@dataclass
class Case:
    """Quantised inputs of one case.  ``vals`` holds every tensor as float32
    carrying exactly the stored value; ``bits`` holds the bf16 patterns of
    the tensors stored in bf16."""
    cell: str
    dims: Dims
    dtype: str
    vals: Dict[str, np.ndarray] = field(default_factory=dict)
    bits: Dict[str, np.ndarray] = field(default_factory=dict)

    @property
    def G(self) -> int:
        return gates_of(self.cell)

    def f64(self, name: str) -> np.ndarray:
        return self.vals[name].astype(np.float64)


def make_case(cell: str, dims: Dims, dtype: str, seed_base: int, *,
              x_var: float = 1.0, w_var: Optional[float] = None,
              r_var: Optional[float] = None, bias="zero",
              h0_var: float = 0.0, c0_var: float = 0.0,
              backward: bool = False, dH_var: float = 1.0,
              final_grads: bool = False) -> Case:
    """Draw every input of a case.  ``bias`` is a pattern name or an explicit
    array of NH*G*Dh values; seeds are ``seed_base + tensor_id``."""
    G = gates_of(cell)
    T, B, Din, NH, Dh = dims.T, dims.B, dims.Din, dims.NH, dims.Dh
    H = NH * Dh
    w_var = 1.0 / Din if w_var is None else w_var
    r_var = 1.0 / Dh if r_var is None else r_var
    c = Case(cell, dims, dtype)

    def draw(name, shape, var, storage):
        n = int(np.prod(shape))
        if var == 0.0:
            z = np.zeros(n)
        else:
            z = normal(seed_base + TENSOR_IDS[name], n, var)
        v, bits = quantize(z.reshape(shape), storage)
        c.vals[name] = v.reshape(shape)
        if bits is not None:
            c.bits[name] = bits.reshape(shape)

    draw("x", (T, B, Din), x_var, dtype)
    draw("W", (Din, NH * G * Dh), w_var, dtype)
    draw("R", (NH, Dh, G * Dh), r_var, dtype)
    if isinstance(bias, str):
        c.vals["b"] = bias_vector(cell, dims, bias).astype(np.float32)
    else:
        c.vals["b"] = np.asarray(bias, dtype=np.float32).reshape(NH * G * Dh)
    draw("h0", (B, H), h0_var, "f32")
    if cell == "lstm":
        draw("c0", (B, H), c0_var, "f32")
    if backward:
        draw("dH", (T, B, H), dH_var, "f32")
        if final_grads:
            draw("dhT", (B, H), dH_var, "f32")
            if cell == "lstm":
                draw("dcT", (B, H), dH_var, "f32")
    return c


def make_stack_case(cell: str, dims: Dims, layers: int, dtype: str, seed_base: int,
                    **kw) -> list:
    """Inputs of a stack of ``layers`` layers: one Case per layer.  Layer 0 is
    make_case(dims); layer l > 0 has input width H (its x is never used) and
    seeds seed_base + 100*l; its W variance defaults to 1/H."""
    out = [make_case(cell, dims, dtype, seed_base, **kw)]
    for layer in range(1, layers):
        d = Dims(dims.T, dims.B, dims.H, dims.NH, dims.Dh)
        kl = dict(kw)
        kl.pop("w_var", None)
        out.append(make_case(cell, d, dtype, seed_base + 100 * layer, **kl))
    return out


def workload_case(w: Workload, dims: Optional[Dims] = None) -> Case:
    """Inputs of a named workload, optionally at other dims (same recipe)."""
    d = dims or w.dims
    return make_case(w.cell, d, w.dtype, 1000 * w.wid, x_var=w.x_var,
                     w_var=w.w_var, r_var=w.r_var, bias=w.bias,
                     h0_var=w.h0_var, c0_var=w.c0_var, backward=w.backward,
                     dH_var=w.dH_var)


def workload_stack_case(w: Workload) -> list:
    """Per-layer inputs of a stacked workload (same recipe per layer)."""
    return make_stack_case(w.cell, w.dims, w.layers, w.dtype, 1000 * w.wid, x_var=w.x_var,
                           w_var=w.w_var, r_var=w.r_var, bias=w.bias, h0_var=w.h0_var,
                           c0_var=w.c0_var)

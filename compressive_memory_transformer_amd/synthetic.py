"""Seeded synthetic inputs for the Infini-attention segment forward.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic.  It is the one module that both the
checks against the float64 reference and the GPU path take their inputs from.

Every (tensor, batch, head, segment) tile is drawn from its own counter-keyed
stream, ``PCG64(SeedSequence([workload_seed, tensor_id, b, h, s]))`` with
tensor_id Q = 0, K = 1, V = 2, so any tile can be regenerated on its own without
materialising a whole stream.  Tiles are drawn as float32 standard normals,
multiplied by the workload's input scale and, for bf16 workloads, rounded to
bfloat16 with round-to-nearest-even.  The per-head gate logits come from
``SeedSequence([workload_seed, 3])``.

The workloads stand in for the long-context tasks of the source pages (a
32K-token language-model stream cut into 2048-token segments, a 1M-token
passkey stream, a 500K-token book stream); those datasets are not used.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

Q_ID, K_ID, V_ID, BETA_ID, PLANT_ID = 0, 1, 2, 3, 4
# output gradient tiles (d_value wide, like V), the final-state gradients and a
# starting state for streams that resume from a non-empty memory
DOUT_ID, STATE_GRAD_ID, STATE0_ID = 5, 6, 7
# the layer around the stream: input rows and the two projection weights
X_ID, WQKV_ID, WO_ID = 8, 9, 10


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    heads: int
    d_key: int
    d_value: int
    segment_len: int
    segments: int
    dtype: str                 # "f32" or "bf16": storage dtype of Q, K, V and the output
    rules: tuple               # update rules run on this workload
    beta_kind: str             # "normal" (sd 1) or "uniform" (symmetric, half-width beta_width)
    beta_width: float
    input_scale: float         # Q/K/V = scale * N(0, 1) before rounding
    planted: bool = False      # one key/value pair written in segment 0, queried in the last
    notes: str = field(default="", compare=False)

    @property
    def seq_len(self) -> int:
        return self.segment_len * self.segments

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_f32", 1, 1, 2, 32, 32, 64, 4, "f32", ("linear", "delta"),
                 "normal", 1.0, 1.0,
                 notes="fp32 correctness case: B=1, H=2, d=32, N=64, 4 segments"),
        Workload("layer_32k_linear", 2, 1, 8, 128, 128, 2048, 16, "bf16", ("linear",),
                 "uniform", 2.0, 1.0 / math.sqrt(128.0),
                 notes="one layer of a 32K-token LM stream, 2048-token segments"),
        Workload("batched_64k_delta", 3, 8, 16, 128, 128, 2048, 32, "bf16", ("delta",),
                 "uniform", 2.0, 1.0 / math.sqrt(128.0),
                 notes="batched delta-rule stream, 8 x 16 heads, 64K tokens"),
        Workload("stream_1m_delta", 4, 1, 8, 128, 128, 2048, 512, "bf16", ("delta",),
                 "uniform", 2.0, 1.0 / math.sqrt(128.0), planted=True,
                 notes="1M-token stream with one planted key/value pair (passkey stand-in)"),
        Workload("wide_500k", 5, 1, 32, 128, 128, 2048, 256, "bf16", ("linear", "delta"),
                 "uniform", 3.0, 1.0 / math.sqrt(128.0),
                 notes="500K-token stream over 32 heads (book-length stand-in)"),
    )
}


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7F800000) == 0x7F800000
    nan &= (u & 0x007FFFFF) != 0
    rounded = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | np.uint32(0x40)).astype(np.uint16), rounded)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def planted_pair(w: Workload):
    """Positions (p0 in segment 0, p1 in the last segment) and per-head key/value
    vectors of the planted pair; unscaled N(0, 1), rounded to the storage dtype."""
    g = rng(w.seed, PLANT_ID)
    p0, p1 = (int(x) for x in g.integers(0, w.segment_len, size=2))
    kstar = g.standard_normal((w.heads, w.d_key), dtype=np.float32)
    vstar = g.standard_normal((w.heads, w.d_value), dtype=np.float32)
    if w.dtype == "bf16":
        kstar, vstar = round_bf16(kstar), round_bf16(vstar)
    return p0, p1, kstar, vstar


def tile(w: Workload, tensor_id: int, b: int, h: int, s: int) -> np.ndarray:
    """One [segment_len, d] tile of Q (0), K (1) or V (2) as float32 values that are
    exact in the workload's storage dtype."""
    d = w.d_value if tensor_id in (V_ID, DOUT_ID) else w.d_key
    x = rng(w.seed, tensor_id, b, h, s).standard_normal((w.segment_len, d), dtype=np.float32)
    if w.input_scale != 1.0:
        x *= np.float32(w.input_scale)
    if w.dtype == "bf16":
        x = round_bf16(x)
    if w.planted:
        p0, p1, kstar, vstar = planted_pair(w)
        if s == 0 and tensor_id == K_ID:
            x[p0] = kstar[h]
        elif s == 0 and tensor_id == V_ID:
            x[p0] = vstar[h]
        elif s == w.segments - 1 and tensor_id == Q_ID:
            x[p1] = kstar[h]
    return x


def state_grads(w: Workload):
    """Gradients of the final state: dM [B, H, d_key, d_value] and dz [B, H, d_key],
    float32 standard normals scaled by the input scale."""
    g = rng(w.seed, STATE_GRAD_ID)
    dM = g.standard_normal((w.batch, w.heads, w.d_key, w.d_value), dtype=np.float32) * np.float32(w.input_scale)
    dz = g.standard_normal((w.batch, w.heads, w.d_key), dtype=np.float32) * np.float32(w.input_scale)
    return dM, dz


def initial_state(w: Workload, segments: int = 2):
    """A starting state (M0, z0) shaped like the memory after `segments` segments
    of the workload's inputs: z0 about segments * N per entry (positive), M0 entries
    of standard deviation sqrt(segments * N) times the input scale.  float32."""
    g = rng(w.seed, STATE0_ID)
    n0 = float(segments * w.segment_len)
    M0 = (g.standard_normal((w.batch, w.heads, w.d_key, w.d_value)) * math.sqrt(n0) * w.input_scale)
    z0 = n0 * (1.0 + 0.05 * np.abs(g.standard_normal((w.batch, w.heads, w.d_key))))
    return M0.astype(np.float32), z0.astype(np.float32)


def layer_tensors(w: Workload, d_model: int):
    """Input x [B, L, d_model] ~ N(0, 1), fused projection weights w_qkv
    [d_model, H (2 d_key + d_value)] ~ N(0, 1 / d_model) times the input scale (so
    the projected q, k, v have the spread of the workload's own inputs) and w_o
    [H d_value, d_model] ~ N(0, 1 / (H d_value)); float32 values, rounded to bf16
    for bf16 workloads."""
    H = w.heads
    x = rng(w.seed, X_ID).standard_normal((w.batch, w.seq_len, d_model), dtype=np.float32)
    wq = rng(w.seed, WQKV_ID).standard_normal((d_model, H * (2 * w.d_key + w.d_value)), dtype=np.float32)
    wq *= np.float32(w.input_scale / math.sqrt(d_model))
    wo = rng(w.seed, WO_ID).standard_normal((H * w.d_value, d_model), dtype=np.float32)
    wo *= np.float32(1.0 / math.sqrt(H * w.d_value))
    if w.dtype == "bf16":
        x, wq, wo = round_bf16(x), round_bf16(wq), round_bf16(wo)
    return x, wq, wo


def betas(w: Workload) -> np.ndarray:
    g = rng(w.seed, BETA_ID)
    if w.beta_kind == "normal":
        return g.standard_normal(w.heads).astype(np.float32)
    return g.uniform(-w.beta_width, w.beta_width, size=w.heads).astype(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def full_tensor(w: Workload, tensor_id: int, as_bits: bool = False,
                heads: list | None = None, segments: int | None = None) -> np.ndarray:
    """The whole [B, H, L, d] tensor (or a subset of heads / a prefix of segments).

    With ``as_bits`` and a bf16 workload the result is the uint16 bit pattern,
    ready to be viewed as bfloat16 on the device."""
    d = w.d_value if tensor_id in (V_ID, DOUT_ID) else w.d_key
    hs = list(range(w.heads)) if heads is None else list(heads)
    S = w.segments if segments is None else segments
    bits = as_bits and w.dtype == "bf16"
    out = np.empty((w.batch, len(hs), S * w.segment_len, d), dtype=np.uint16 if bits else np.float32)

    def fill(job):
        b, hi, s = job
        t = tile(w, tensor_id, b, hs[hi], s)
        out[b, hi, s * w.segment_len:(s + 1) * w.segment_len] = f32_to_bf16_bits(t) if bits else t

    jobs = [(b, hi, s) for b in range(w.batch) for hi in range(len(hs)) for s in range(S)]
    if len(jobs) < 64:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, jobs, chunksize=16))
    return out


def stress_variant(w: Workload, name_suffix: str = "_stress") -> Workload:
    """Same shapes with unscaled N(0, 1) inputs: at d = 128 with the 1/sqrt(d)
    softmax scale the scores have a spread of about one unit, ten times that of
    the scaled workloads, so the softmax weights are far from uniform."""
    return Workload(w.name + name_suffix, w.seed + 100, w.batch, w.heads, w.d_key, w.d_value,
                    w.segment_len, w.segments, w.dtype, w.rules, w.beta_kind, w.beta_width, 1.0,
                    False, notes="stress variant of " + w.name)


def custom(name: str, seed: int, batch: int, heads: int, d: int, segment_len: int, segments: int,
           dtype: str = "bf16", rules=("linear", "delta"), input_scale: float | None = None,
           beta_width: float = 2.0, d_value: int | None = None) -> Workload:
    """A workload of arbitrary shape for tests (several tiles and a ragged tail);
    d is the key width and, unless d_value is given, the value width too."""
    if input_scale is None:
        input_scale = 1.0 / math.sqrt(d) if dtype == "bf16" else 1.0
    return Workload(name, seed, batch, heads, d, d if d_value is None else d_value, segment_len, segments, dtype,
                    tuple(rules), "uniform", beta_width, input_scale)

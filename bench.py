#!/usr/bin/env python3
"""Throughput of the Infini-attention segment forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rule RULE]

One step = one pass of the whole path over one batch of the workload's synthetic
stream for each update rule the workload names (the default, the 500K-token
stream over 32 heads, names both): reset the rule's state, then forward_sequence
over all segments of every head (memory-state stage + fused
attention/retrieval/gate stage), inputs resident in HBM.  The timed region is K
steps bracketed by device synchronisation.  Prints one JSON line with the
whole-job tokens/s (tokens of every rule's pass), the roofline position of the
dominant kernel (the fused attention kernel, timed live with HIP events around
its stage on the stream it runs on), a per-rule breakdown and the float64 oracle
timed on the host cores over a bounded prefix of the same stream.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
VALU_F32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector (256 CUs x 2.4 GHz x 256 FLOP/clk)
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_traffic.json")
DOMINANT_SOURCES = ["compressive_memory_transformer_amd/csrc/fa_fwd.hip",
                    "compressive_memory_transformer_amd/csrc/common.h"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None,
                   help="synthetic workload (default: the 500K-token stream over 32 heads; the 32K-token "
                        "stream for --decode, --backward, --layer and --kla)")
    p.add_argument("--rule", default=None,
                   help="update rule to time (default: every rule the workload names, one pass each per step)")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="budget of the oracle leg (0 disables it)")
    p.add_argument("--decode", type=int, default=0, metavar="FILLED",
                   help="time single-token decode steps (infini_attn_append of one token per (b, h)) with "
                        "the open segment holding FILLED tokens when the timed steps start and the memory "
                        "holding all but the last segment of the workload; prints its own JSON line")
    p.add_argument("--backward", action="store_true",
                   help="time infini_attn_backward_sequence over the workload (gradients of a forward from an "
                        "empty memory); prints its own JSON line")
    p.add_argument("--saved", action="store_true",
                   help="with --backward: time infini_attn_backward_sequence_saved, given the output and the "
                        "softmax log-normalisers of an (untimed) infini_attn_forward_sequence_train call")
    p.add_argument("--layer", type=int, default=0, metavar="D_MODEL",
                   help="time infini_attn_layer_forward (QKV projection, stream, output projection) with model "
                        "width D_MODEL (0: off); prints its own JSON line")
    p.add_argument("--kla", type=int, default=0, metavar="CHUNK",
                   help="time causal kernel linear attention over the workload's q, k, v with chunks of CHUNK "
                        "tokens (0: off); prints its own JSON line")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 launches), to calibrate "
                        "the HBM byte counters of a profiler against a known size")
    return p.parse_args()


def hip_runtime():
    """The HIP runtime already mapped into this process (the one torch uses)."""
    maps = open("/proc/self/maps").read()
    paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", maps)))
    return ctypes.CDLL(paths[0] if paths else "libamdhip64.so")


PROFILE_EVERY = 4   # timed steps per step that carries the stage events


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev.append(e.value)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def attention_flops(w, first_segment_global: int = 0) -> int:
    """Algorithmic FLOPs of one launch of the fused kernel: causal pairs only,
    2 * d * N (N + 1) per (b, h, segment) for QK^T and PV, plus the retrieval GEMM
    and its denominator 2 * N * d_k * (d_v + 1) for every segment that reads a
    non-empty memory."""
    N, dk, dv = w.segment_len, w.d_key, w.d_value
    att = 2 * dk * N * (N + 1) // 2 + 2 * dv * N * (N + 1) // 2
    ret = 2 * N * dk * dv + 2 * N * dk
    seg_with_memory = sum(1 for s in range(w.segments) if first_segment_global + s > 0)
    return w.batch * w.heads * (w.segments * att + seg_with_memory * ret)


def state_bytes(w) -> int:
    """Algorithmic HBM bytes of the memory-state stage (either rule): K and V read
    once, one snapshot per (b, h, segment) written (M^T in bf16 or fp32, z and the
    column sums of M in fp32), and the state (M, z) read and written once per head."""
    el = 2 if w.dtype == "bf16" else 4
    N, dk, dv = w.segment_len, w.d_key, w.d_value
    per_seg = N * (dk + dv) * el + dk * dv * el + (dk + dv) * 4
    per_head = 2 * (dk * dv + dk) * 4
    return w.batch * w.heads * (w.segments * per_seg + per_head)


def state_flops(w, rule: str) -> int:
    N, dk, dv = w.segment_len, w.d_key, w.d_value
    upd = 2 * N * dk * dv + N * dk
    if rule == "delta":
        upd += 2 * N * dk * dv + 2 * N * dk
    return w.batch * w.heads * w.segments * upd


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, rule: str):
    """HBM bytes per launch of the fused kernel from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    entry = rec.get("workloads", {}).get(f"{workload}/{rule}")
    return None if entry is None else entry.get("bytes_per_launch")


def blas_info() -> str:
    """The BLAS library numpy runs on and its thread count."""
    from threadpoolctl import threadpool_info
    libs = [f"{i.get('internal_api', '?')} {i.get('version', '')} ({i.get('num_threads', 1)} threads)"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return ", ".join(libs) or "unknown"


def cpu_baseline(w, rules, budget_s: float):
    """The float64 oracle on the host over a prefix of the same stream, for each
    rule with an equal share of the budget: segments in order, all heads of a
    segment before the next, until the rule's share is spent.  The value is the
    tokens of all rules over the time of all rules (the rate of the GPU step's
    mix)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from compressive_memory_transformer_amd import synthetic as syn
    from oracle import infini_ref as ref

    if isinstance(rules, str):
        rules = [rules]
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    sc = ref.default_scale(w.d_key)
    betas = syn.betas(w)
    total_tok, total_s, samples = 0.0, 0.0, []
    for rule in rules:
        share = budget_s / len(rules)
        M = {(b, h): np.zeros((w.d_key, w.d_value)) for b in range(w.batch) for h in range(w.heads)}
        z = {key: np.zeros(w.d_key) for key in M}
        done = 0
        spent = 0.0
        for s in range(w.segments):
            for (b, h) in M:
                q, k, v = (syn.tile(w, i, b, h, s).astype(np.float64) for i in (0, 1, 2))
                t0 = time.perf_counter()
                _, M[(b, h)], z[(b, h)], _, _ = ref.segment_forward(q, k, v, M[(b, h)], z[(b, h)],
                                                                    float(betas[h]), rule, s == 0, sc)
                spent += time.perf_counter() - t0
                done += 1
                if spent >= share:
                    break
            if spent >= share:
                break
        total_tok += done * w.segment_len / w.heads
        total_s += spent
        samples.append(f"{done} of {w.batch * w.heads * w.segments} (batch, head, segment) tiles of "
                       f"{w.name}/{rule} in stream order ({spent:.1f}s)")
    return {"value": total_tok / total_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(samples) + f"; float64 numpy on {blas_info()}"}


def decode_bytes(w, filled: int, steps: int) -> int:
    """Algorithmic HBM bytes of `steps` decode steps starting at an open segment of
    `filled` tokens: per (b, h) and step, the open segment's keys and values up to
    the new token, M and z, and the token's q, k, v in and A out."""
    esz = 2 if w.dtype == "bf16" else 4
    bh = w.batch * w.heads
    kv = sum(filled + i + 1 for i in range(steps)) * (w.d_key + w.d_value) * esz
    per_step = (w.d_key * w.d_value + w.d_key) * 4 + (2 * w.d_key + 2 * w.d_value) * esz
    return bh * (kv + steps * per_step)


def decode_cpu_baseline(w, rule: str, filled: int, budget_s: float):
    """The float64 oracle's decode: tokens appended one at a time to an open
    segment of `filled` tokens, all heads, until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from compressive_memory_transformer_amd import synthetic as syn
    from oracle import infini_ref as ref

    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    s = w.segments - 1
    q, k, v = (np.stack([np.stack([syn.tile(w, i, b, h, s) for h in range(w.heads)]) for b in range(w.batch)])
               .astype(np.float64) for i in (0, 1, 2))
    rng = np.random.default_rng(0)
    M = rng.standard_normal((w.batch, w.heads, w.d_key, w.d_value))
    z = np.abs(rng.standard_normal((w.batch, w.heads, w.d_key))) + 1.0
    ok, ov = k[:, :, :filled], v[:, :, :filled]
    spent, n = 0.0, 0
    while spent < budget_s and filled + n < w.segment_len - 1:
        t = filled + n
        t0 = time.perf_counter()
        res = ref.forward_stream(q[:, :, t:t + 1], k[:, :, t:t + 1], v[:, :, t:t + 1], syn.betas(w), rule,
                                 w.segment_len, M0=M, z0=z, segments_done=s, open_k=ok, open_v=ov)
        spent += time.perf_counter() - t0
        ok, ov = res["open_k"], res["open_v"]
        n += 1
    return {"value": n * w.batch / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode steps of {w.name}/{rule} from an open segment of {filled} tokens, all "
                      f"{w.batch * w.heads} heads, float64 numpy, {spent:.1f}s"}


def backward_flops(w, rule: str) -> float:
    """Algorithmic FLOP of one backward over the whole workload.  Per seg-head: the
    local attention's five products over the causal pairs (scores recomputed, dP,
    dV, dQ, dK: (3 d_key + 2 d_value) N (N + 1)), the retrieval's three (numerator
    recomputed, d sigma(q), dM: 6 N d_key d_value), the update's (linear: dV and
    d sigma(K), 4 N d_k d_v; delta: R recomputed, dV, two d sigma(K) terms and dM,
    10 N d_k d_v) and its replay (linear 2, delta 4 N d_k d_v)."""
    N, dk, dv = w.segment_len, w.d_key, w.d_value
    att = (3 * dk + 2 * dv) * N * (N + 1)
    mem = 6 * N * dk * dv + (6 if rule == "linear" else 14) * N * dk * dv
    return float(att + mem) * w.batch * w.heads * w.segments


def backward_cpu_baseline(w, rule: str, budget_s: float):
    """The float64 gradient oracle on the first segments of one (batch, head),
    doubling the number of segments until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from compressive_memory_transformer_amd import synthetic as syn
    from oracle import infini_grad as og

    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    beta = syn.betas(w)[:1]
    dM, dz = syn.state_grads(w)
    spent, segs, n = 0.0, 0, 1
    while spent < budget_s / 3 and n <= w.segments:
        q, k, v, do = (np.concatenate([syn.tile(w, i, 0, 0, s) for s in range(n)])[None, None].astype(np.float64)
                       for i in (syn.Q_ID, syn.K_ID, syn.V_ID, syn.DOUT_ID))
        t0 = time.perf_counter()
        og.backward_sequence(q, k, v, beta, rule, w.segment_len, do, dM=dM[:1, :1], dz=dz[:1, :1])
        spent, segs = time.perf_counter() - t0, n
        n *= 2
    tokens = segs * w.segment_len / w.heads   # a token is all heads of one position
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"backward of the first {segs} segments of one (batch, head) of {w.name}/{rule}, "
                      f"float64 numpy, {spent:.1f}s"}


def bench_backward(args):
    import numpy as np
    import torch

    from compressive_memory_transformer_amd import infini as ia
    from compressive_memory_transformer_amd import synthetic as syn

    w = syn.WORKLOADS[args.workload]
    rule = args.rule or w.rules[0]
    ia.load_library()

    def upload(tid):
        arr = syn.full_tensor(w, tid, as_bits=True)
        if w.dtype == "bf16":
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(arr).to("cuda")

    q, k, v, dout = (upload(i) for i in (syn.Q_ID, syn.K_ID, syn.V_ID, syn.DOUT_ID))
    beta = torch.from_numpy(syn.betas(w)).to("cuda")
    dM, dz = (torch.from_numpy(x).to("cuda") for x in syn.state_grads(w))
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, w.dtype, rule)
    M0, z0 = torch.zeros_like(eng.M), torch.zeros_like(eng.z)
    st = ia.State.from_buffer_copy(eng.state)
    st.M, st.z, st.segments_done = M0.data_ptr(), z0.data_ptr(), 0
    L = w.seq_len
    need = ia.backward_workspace_bytes(st, L)
    raw = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    ws = raw[(-raw.data_ptr()) % 256:][:need]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbeta = torch.empty(w.heads, dtype=torch.float32, device="cuda")
    dM0, dz0 = torch.empty_like(M0), torch.empty_like(z0)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    saved = None
    if args.saved:
        # the training forward from the same (empty) starting state keeps what the
        # backward then reads instead of recomputing the softmax statistics
        eng.reset()
        saved = eng.forward_sequence_train(q, k, v, beta)
        torch.cuda.synchronize()

    def step():
        if saved is None:
            ia.backward_sequence(st, q, k, v, L, beta, dout, dM, dz, dq, dk, dv, dbeta, dM0, dz0, ws, need, sh)
        else:
            ia.backward_sequence_saved(st, q, k, v, L, beta, saved[0], saved[1], dout, dM, dz, dq, dk, dv, dbeta,
                                       dM0, dz0, ws, need, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    fl = backward_flops(w, rule)
    tf = fl / gpu_s / 1e12
    cpu = backward_cpu_baseline(w, rule, args.cpu_seconds) if args.cpu_seconds > 0 else None
    line = {
        "metric": ("Infini-attention backward tokens/sec on 1 MI355X (gradients of forward_sequence"
                   + (", given the training forward's output and softmax log-normalisers)" if saved else ")")),
        "value": w.tokens * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"backward{'_saved' if saved else ''}/{w.name}", "batch": w.batch,
                   "heads": w.heads, "segment_len": w.segment_len, "segments": w.segments, "d_key": w.d_key,
                   "d_value": w.d_value, "rule": rule, "parallelism": "single GPU"},
        "roofline": ({"bound": "mfma", "kernel": "whole backward (all launches of one call)", "achieved": tf,
                      "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                      "traffic": None, "flops_per_step": fl, "avg_step_ms_on_stream": gpu_s * 1e3}
                     if w.dtype == "bf16" else
                     {"bound": "alu", "kernel": "whole backward (fp32 VALU kernels)", "achieved": tf,
                      "peak": VALU_F32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / VALU_F32_PEAK_TFLOPS,
                      "traffic": None, "flops_per_step": fl, "avg_step_ms_on_stream": gpu_s * 1e3}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def layer_flops(w, rule: str, d_model: int) -> int:
    """Algorithmic FLOP of one layer call: the two projections (2 B L d_model
    H (2 d_k + d_v) and 2 B L H d_v d_model), the fused kernel's and the state
    stage's."""
    H, dk, dv, BL = w.heads, w.d_key, w.d_value, w.batch * w.seq_len
    proj = 2 * BL * d_model * H * (2 * dk + dv) + 2 * BL * H * dv * d_model
    return proj + attention_flops(w) + state_flops(w, rule)


def layer_cpu_baseline(w, rule: str, d_model: int, budget_s: float):
    """The float64 layer oracle on the first segments of batch 0 (all heads),
    doubling the number of segments until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from compressive_memory_transformer_amd import synthetic as syn
    from oracle import infini_layer as ol

    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    x, wq, wo = syn.layer_tensors(w, d_model)
    beta = syn.betas(w)
    spent, segs, n = 0.0, 0, 1
    while spent < budget_s / 3 and n <= w.segments:
        t0 = time.perf_counter()
        ol.layer_forward(x[:1, :n * w.segment_len], wq, wo, beta, rule, w.segment_len, w.heads, w.d_key, w.d_value)
        spent, segs = time.perf_counter() - t0, n
        n *= 2
    return {"value": segs * w.segment_len / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"layer over the first {segs} segments of batch 0 of {w.name}/{rule}, d_model {d_model}, "
                      f"float64 numpy, {spent:.1f}s"}


def bench_layer(args):
    import numpy as np
    import torch

    from compressive_memory_transformer_amd import infini as ia
    from compressive_memory_transformer_amd import synthetic as syn

    w = syn.WORKLOADS[args.workload]
    rule = args.rule or w.rules[0]
    dm = args.layer
    ia.load_library()
    dev = [torch.from_numpy(t).to("cuda").to(torch.bfloat16) for t in syn.layer_tensors(w, dm)]
    x, wq, wo = dev
    beta = torch.from_numpy(syn.betas(w)).to("cuda")
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, w.dtype, rule)
    y = torch.empty_like(x)
    L = w.seq_len
    need = ia.layer_workspace_bytes(eng.state, dm, L)
    raw = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    ws = raw[(-raw.data_ptr()) % 256:][:need]
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        ia.reset(eng.state, sh)
        ia.layer_forward(eng.state, x, dm, wq, wo, L, beta, y, ws, need, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    fl = layer_flops(w, rule, dm)
    tf = fl / gpu_s / 1e12
    cpu = layer_cpu_baseline(w, rule, dm, args.cpu_seconds) if args.cpu_seconds > 0 else None
    line = {
        "metric": "Infini-attention layer tokens/sec on 1 MI355X (projections + segment stream)",
        "value": w.tokens * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"layer/{w.name}", "batch": w.batch, "heads": w.heads, "d_model": dm,
                   "segment_len": w.segment_len, "segments": w.segments, "d_key": w.d_key, "d_value": w.d_value,
                   "rule": rule, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "whole layer call (reset + 2 GEMMs + state stage + fused kernel)",
                     "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None, "flops_per_step": fl,
                     "avg_step_ms_on_stream": gpu_s * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def kla_work(w, chunk: int):
    """Algorithmic FLOP and HBM bytes of one causal kernel linear attention pass in
    chunks of `chunk` tokens: per chunk and head, the weights and their product
    with V over the causal pairs (2 (d_k + d_v) C (C + 1) / 2), the retrieval from
    the chunk's starting state (2 C d_k d_v) and the chunk's contribution to the
    state (2 C d_k d_v); bytes: q, k, v read and the output written once, plus one
    starting state (bf16 M^T and two fp32 vectors) per chunk."""
    C, dk, dv = chunk, w.d_key, w.d_value
    chunks = w.batch * w.heads * (w.seq_len // C)
    fl = chunks * ((dk + dv) * C * (C + 1) + 4 * C * dk * dv)
    by = w.batch * w.heads * w.seq_len * (2 * dk + 2 * dv) * 2 + chunks * (dk * dv * 2 + 8 * dk)
    return fl, by


def kla_cpu_baseline(w, chunk: int, budget_s: float):
    """The float64 oracle on the first tokens of one (batch, head), doubling the
    length until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from compressive_memory_transformer_amd import synthetic as syn
    from oracle import kernel_linear as kl

    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    spent, segs, n = 0.0, 0, 1
    while spent < budget_s / 3 and n <= w.segments:
        q, k, v = (np.concatenate([syn.tile(w, i, 0, 0, s) for s in range(n)])[None, None].astype(np.float64)
                   for i in (syn.Q_ID, syn.K_ID, syn.V_ID))
        t0 = time.perf_counter()
        kl.causal_kernel_linear_attention(q, k, v)
        spent, segs = time.perf_counter() - t0, n
        n *= 2
    tokens = segs * w.segment_len / w.heads   # a token is all heads of one position
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {segs * w.segment_len} tokens of one (batch, head) of {w.name}, float64 numpy, "
                      f"{spent:.1f}s"}


def bench_kla(args):
    import numpy as np
    import torch

    from compressive_memory_transformer_amd import infini as ia
    from compressive_memory_transformer_amd import synthetic as syn

    w = syn.WORKLOADS[args.workload]
    C = args.kla
    if w.seq_len % C != 0:
        print(f"--kla {C} does not divide the workload's {w.seq_len} tokens", file=sys.stderr)
        sys.exit(2)
    ia.load_library()

    def upload(tid):
        return torch.from_numpy(syn.full_tensor(w, tid, as_bits=True).view(np.int16)).view(torch.bfloat16).to("cuda")

    q, k, v = (upload(i) for i in (syn.Q_ID, syn.K_ID, syn.V_ID))
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, C, "bf16", "linear")
    out = torch.empty_like(v)
    L = w.seq_len
    ws, nbytes = eng.workspace(L)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        ia.reset(eng.state, sh)
        ia.kernel_linear_attention(eng.state, q, k, v, L, out, ws, nbytes, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    fl, by = kla_work(w, C)
    tf, gbs = fl / gpu_s / 1e12, by / gpu_s / 1e9
    mfma_bound = fl / by > MFMA_BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS
    roof = ({"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": tf / MFMA_BF16_PEAK_TFLOPS} if mfma_bound else
            {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS})
    roof.update({"kernel": "whole call (reset + contributions + prefix scan + chunk kernel)", "traffic": None,
                 "flops_per_step": fl, "bytes_per_step": by, "tflops": tf, "gbs": gbs,
                 "avg_step_ms_on_stream": gpu_s * 1e3})
    cpu = kla_cpu_baseline(w, C, args.cpu_seconds) if args.cpu_seconds > 0 else None
    line = {
        "metric": "Causal kernel linear attention tokens/sec on 1 MI355X",
        "value": w.tokens * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"kla/{w.name}", "batch": w.batch, "heads": w.heads, "chunk": C,
                   "seq_len": w.seq_len, "d_key": w.d_key, "d_value": w.d_value, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_decode(args):
    import torch

    from compressive_memory_transformer_amd import infini as ia
    from compressive_memory_transformer_amd import synthetic as syn

    w = syn.WORKLOADS[args.workload]
    rule = args.rule or w.rules[0]
    filled, N = args.decode, w.segment_len
    if filled + args.warmup + args.steps > N - 1:
        print(f"--decode {filled} plus {args.warmup + args.steps} steps does not fit one open segment of {N}",
              file=sys.stderr)
        sys.exit(2)
    ia.load_library()

    def upload(tid):
        arr = syn.full_tensor(w, tid, as_bits=True)
        if w.dtype == "bf16":
            import numpy as np
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(arr).to("cuda")

    q, k, v = (upload(i) for i in (0, 1, 2))
    beta = torch.from_numpy(syn.betas(w)).to("cuda")
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, N, w.dtype, rule)
    L0 = (w.segments - 1) * N
    eng.forward_sequence(q[:, :, :L0].contiguous(), k[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), beta)
    eng.open_stream()
    if filled:
        sl = slice(L0, L0 + filled)
        eng.append(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), beta)
    toks = [tuple(x[:, :, L0 + filled + i:L0 + filled + i + 1].contiguous() for x in (q, k, v))
            for i in range(args.warmup + args.steps)]
    out = torch.empty((w.batch, w.heads, 1, w.d_value), dtype=q.dtype, device="cuda")
    ws, nbytes = eng.append_workspace(1)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(args.warmup):
        ia.append(eng.state, eng.open, *toks[i], 1, beta, out, ws, nbytes, sh)
    torch.cuda.synchronize()
    start = filled + args.warmup
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()   # torch's current stream: the stream the steps are enqueued on
    for i in range(args.warmup, args.warmup + args.steps):
        ia.append(eng.state, eng.open, *toks[i], 1, beta, out, ws, nbytes, sh)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) * 1e-3
    byts = decode_bytes(w, start, args.steps)
    gbs = byts / gpu_s / 1e9
    cpu = decode_cpu_baseline(w, rule, start, args.cpu_seconds) if args.cpu_seconds > 0 else None
    line = {
        "metric": "Infini-attention decode tokens/sec on 1 MI355X (one new token per (b, h) per step)",
        "value": w.batch * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"decode/{w.name}", "batch": w.batch, "heads": w.heads, "segment_len": N,
                   "d_key": w.d_key, "d_value": w.d_value, "rule": rule, "open_segment_filled": start,
                   "segments_in_memory": w.segments - 1, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "open_attn_partial + open_attn_combine",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "bytes_per_step": byts / args.steps,
                     "avg_step_ms_on_stream": gpu_s / args.steps * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); "
              "this library has no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": {"read": n * 4, "write": n * 4}, "launches": 3}))
        return

    from compressive_memory_transformer_amd import infini as ia
    from compressive_memory_transformer_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload is None:
        side = args.backward or args.layer or args.kla or args.decode
        args.workload = "layer_32k_linear" if side else "wide_500k"
    if args.backward:
        bench_backward(args)
        return
    if args.layer:
        bench_layer(args)
        return
    if args.kla:
        bench_kla(args)
        return
    if args.decode:
        bench_decode(args)
        return
    w = syn.WORKLOADS[args.workload]
    rules = [args.rule] if args.rule else list(w.rules)
    ia.load_library()

    def upload(tid):
        arr = syn.full_tensor(w, tid, as_bits=True)
        if w.dtype == "bf16":
            import numpy as np
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(arr).to("cuda")

    t_in = time.perf_counter()
    q, k, v = (upload(i) for i in (0, 1, 2))
    beta = torch.from_numpy(syn.betas(w)).to("cuda")
    print(f"inputs of {w.name} on the device in {time.perf_counter() - t_in:.1f}s", file=sys.stderr, flush=True)
    # one engine (state + workspace) per rule; the output buffer is shared
    engs = {r: ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, w.dtype, r) for r in rules}
    out = torch.empty((w.batch, w.heads, w.seq_len, w.d_value), dtype=q.dtype, device="cuda")
    wss = {r: engs[r].workspace(w.seq_len) for r in rules}
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    hip = hip_runtime()
    # Stage events go into every PROFILE_EVERY-th timed step (at least one): each
    # event record costs a few microseconds of GPU time, so stamping every step
    # would slow down the very steps being timed.
    prof_steps = [i for i in range(args.steps) if i % PROFILE_EVERY == 0]
    ev = Events(hip, 3 * len(prof_steps) * len(rules))

    def step(j=None):
        """One pass of the path: for each rule, reset its state and stream the whole
        workload through forward_sequence."""
        for ri, r in enumerate(rules):
            eng = engs[r]
            ws, ws_bytes = wss[r]
            ia.reset(eng.state, sh)
            if j is None:
                ia.forward_sequence(eng.state, q, k, v, w.seq_len, beta, out, ws, ws_bytes, sh)
            else:
                b = 3 * (j * len(rules) + ri)
                ia.forward_sequence_profiled(eng.state, q, k, v, w.seq_len, beta, out, ws, ws_bytes, sh,
                                             ev.ev[b:b + 3])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i // PROFILE_EVERY if i % PROFILE_EVERY == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    wall = t1 - t0
    tokens = w.batch * w.seq_len * len(rules)
    per_rule = {}
    fa_all = []
    for ri, r in enumerate(rules):
        idx = [3 * (j * len(rules) + ri) for j in range(len(prof_steps))]
        fa_ms = [ev.elapsed_ms(b + 1, b + 2) for b in idx]
        st_ms = [ev.elapsed_ms(b, b + 1) for b in idx]
        fw_ms = [ev.elapsed_ms(b, b + 2) for b in idx]
        fa_all += fa_ms
        st_avg = sum(st_ms) / len(st_ms)
        fw_avg = sum(fw_ms) / len(fw_ms)
        per_rule[r] = {
            "forward_ms": fw_avg,
            "tokens_per_s": w.batch * w.seq_len / (fw_avg * 1e-3),
            "stages_ms": {"state": st_avg, "attention": sum(fa_ms) / len(fa_ms),
                          "attention_min": min(fa_ms), "attention_max": max(fa_ms)},
            # the memory-state stage against its own bounds: HBM for the linear rule
            # (contributions + prefix scan), the dependent chain for the delta rule
            "state_roofline": {"bound": "hbm" if r == "linear" else "latency",
                               "achieved_GBps": state_bytes(w) / (st_avg * 1e-3) / 1e9,
                               "peak_GBps": HBM_PEAK_GBS,
                               "frac_hbm": state_bytes(w) / (st_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "tflops": state_flops(w, r) / (st_avg * 1e-3) / 1e12,
                               "frac_mfma": state_flops(w, r) / (st_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                               "bytes": state_bytes(w), "flops": state_flops(w, r)},
        }
    ev.destroy()
    fa_avg = sum(fa_all) / len(fa_all)
    fl = attention_flops(w)
    achieved = fl / (fa_avg * 1e-3) / 1e12
    step_fl = len(rules) * fl + sum(state_flops(w, r) for r in rules)
    traffic = traffic_for(w.name, "+".join(rules))

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, rules, args.cpu_seconds)

    line = {
        "metric": "Infini-attention fwd tokens/sec on 1 MI355X + % of bf16 MFMA/HBM roofline",
        "value": tokens * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "segment_len": w.segment_len, "d_key": w.d_key, "d_value": w.d_value, "rules": rules,
                   "step": "reset + forward_sequence over the whole stream, once per rule",
                   "tokens_per_step": tokens, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "fa_fwd_kernel", "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic, "flops_per_launch": fl, "avg_launch_ms": fa_avg,
                     "launches_sampled": len(fa_all)},
        "per_rule": per_rule,
        "step_tflops": step_fl / (wall / args.steps) / 1e12,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

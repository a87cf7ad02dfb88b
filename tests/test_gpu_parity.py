"""GPU parity of the HIP library against the float64 oracle, through the C ABI.

Small shapes (several query/key tiles, a ragged last query tile, both rules,
both head widths), the tiny fp32 workload and the full 32K-token single-layer
workload, plus the diagnostics: pure-memory and pure-local gates, a stress input
with widely spread scores, segment-by-segment streaming == one sequence call
(bitwise, also on the pipelined delta path), the persistent fused-kernel grid
with an odd number of query tiles and a ragged last tile, reset, determinism
and a NaN-poisoned workspace.
"""

import math

import numpy as np
import pytest

from compressive_memory_transformer_amd import synthetic as syn
from oracle import infini_ref as ref
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = gh.torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressive_memory_transformer_amd import infini as ia
    ia.load_library()
    yield


SMALL = [
    # name, seed, B, H, d_key, N, S, dtype[, d_value]
    ("f32_tiny_shape", 11, 1, 2, 32, 64, 4, "f32"),
    ("f32_ragged", 12, 2, 3, 20, 37, 3, "f32"),
    ("bf16_d128_n192", 13, 2, 3, 128, 192, 3, "bf16"),
    ("bf16_d64_n256", 14, 1, 4, 64, 256, 4, "bf16"),
    ("bf16_d128_n64", 15, 1, 2, 128, 64, 5, "bf16"),
    ("bf16_d64_n320", 16, 2, 1, 64, 320, 2, "bf16"),
    # bf16 shapes the MFMA kernels do not take (the VALU path): the tiny
    # workload's shape, different key and value widths, a ragged segment length
    ("bf16_d32_n64", 17, 1, 2, 32, 64, 4, "bf16"),
    ("bf16_dk64_dv32_n100", 18, 2, 2, 64, 100, 3, "bf16", 32),
    ("bf16_dk32_dv128_n96", 19, 1, 3, 32, 96, 3, "bf16", 128),
]


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case, rule):
    name, seed, B, H, d, N, S, dtype = case[:8]
    dv = case[8] if len(case) > 8 else None
    gh.log(f"case {name} rule={rule}")
    w = syn.custom(name, seed, B, H, d, N, S, dtype=dtype, d_value=dv)
    q, k, v, beta = gh.device_inputs(w)
    out, eng = gh.run(w, rule, q, k, v, beta)
    gh.torch_mod().cuda.synchronize()
    res = gh.oracle_full(w, rule)
    gh.compare_full(w, rule, out, eng, res, label=f"{name}/{rule}")
    assert eng.segments_done == S


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_tiny_f32_workload(rule):
    w = syn.WORKLOADS["tiny_f32"]
    gh.log(f"workload {w.name} rule={rule}")
    q, k, v, beta = gh.device_inputs(w)
    out, eng = gh.run(w, rule, q, k, v, beta)
    res = gh.oracle_full(w, rule)
    gh.compare_full(w, rule, out, eng, res, label=f"{w.name}/{rule}")


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_gate_limits(rule, sign):
    """beta = +inf: A is exactly A_mem (0 in the first segment); beta = -inf: A_dot."""
    w = syn.custom("gate_case", 21, 1, 3, 128, 256, 4)
    gh.log(f"gate limit sign={sign} rule={rule}")
    q, k, v, _ = gh.device_inputs(w)
    out, eng = gh.run(w, rule, q, k, v, gh.inf_beta(w.heads, sign))
    res = gh.oracle_full(w, rule, beta_np=np.full(w.heads, math.inf * sign), keep_parts=True)
    part = res["A_mem"] if sign > 0 else res["A_dot"]
    got = gh.to_host(out)
    N = w.segment_len
    for h in range(w.heads):
        for s in range(w.segments):
            sl = slice(s * N, (s + 1) * N)
            if sign > 0 and s == 0:
                assert np.all(got[0, h, sl] == 0.0)
                continue
            e = gh.metric(got[0, h, sl], part[0, h, sl], "bf16")
            assert e <= gh.BF16_TOL, (h, s, e)
    gh.log(f"  gate sign={sign} ok")


def test_stress_scores():
    """Unscaled N(0, 1) queries and keys: scores with a spread of about one unit
    (ten times the workloads'), so the softmax weights are far from uniform and the
    exponentials span several binades."""
    base = syn.custom("stress_case", 31, 1, 2, 128, 512, 3)
    w = syn.stress_variant(base)
    gh.log("stress input")
    q, k, v, beta = gh.device_inputs(w)
    for rule in ("linear", "delta"):
        out, eng = gh.run(w, rule, q, k, v, beta)
        res = gh.oracle_full(w, rule)
        gh.compare_full(w, rule, out, eng, res, label=f"stress/{rule}")


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segments_equal_sequence_bitwise(rule, dtype):
    torch = gh.torch_mod()
    d, N = (128, 256) if dtype == "bf16" else (32, 64)
    w = syn.custom("stream_case", 41, 2, 2, d, N, 4, dtype=dtype)
    gh.log(f"segment-vs-sequence {dtype}/{rule}")
    q, k, v, beta = gh.device_inputs(w)
    out1, e1 = gh.run(w, rule, q, k, v, beta, mode="sequence")
    out2, e2 = gh.run(w, rule, q, k, v, beta, mode="segments")
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(e1.M, e2.M) and torch.equal(e1.z, e2.z)
    assert e1.segments_done == e2.segments_done == w.segments


@pytest.mark.parametrize("d", [64, 128])
def test_delta_pipeline_bitwise(d):
    """A delta stream whose chain leaves most compute units free (8 heads, 8 x
    CUs / 8 segments of 128 tokens) takes the pipelined path: the chain in ranges
    of segments on a side stream, the fused kernel of each range on the caller's
    stream as soon as the range is chained.  Its output and final state equal,
    bitwise, those of the same stream fed in calls of CUs / 8 segments, which are
    not pipelined but tile the contributions the same way (as many (b, h,
    segment) tiles per call as compute units); and the oracle's at the bf16
    tolerance."""
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    H = 8
    per_call = torch.cuda.get_device_properties(0).multi_processor_count // H
    S, N = 8 * per_call, 128
    w = syn.custom("pipeline_case", 43, 1, H, d, N, S, rules=("delta",))
    gh.log(f"delta pipeline d={d}, {S} segments, reference calls of {per_call}")
    q, k, v, beta = gh.device_inputs(w)
    out1, e1 = gh.run(w, "delta", q, k, v, beta, mode="sequence")
    e2 = ia.InfiniAttention(1, H, d, d, N, "bf16", "delta")
    out2 = torch.empty_like(out1)
    for c in range(0, S, per_call):
        rows = slice(c * N, (c + per_call) * N)
        out2[:, :, rows] = e2.forward_sequence(q[:, :, rows].contiguous(), k[:, :, rows].contiguous(),
                                               v[:, :, rows].contiguous(), beta)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(e1.M, e2.M) and torch.equal(e1.z, e2.z)
    res = gh.oracle_full(w, "delta")
    gh.compare_full(w, "delta", out1, e1, res, label=f"pipeline d={d}")


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("d", [64, 128])
def test_persistent_grid_odd_tiles(rule, d):
    """A call with more (b, h, segment) x query-tile-pair items than compute units
    runs the fused kernel persistent (one workgroup per CU walking its XCD's items,
    passes chained across items).  Segments of 1216 tokens give five query tiles:
    pairs (4, 0) and (3, 1) and a middle pair with a single tile (2), the last
    tile ragged (192 rows: two waves idle), and 4 x 80 x 3 = 960 items, which the
    8 XCD ranges do not split evenly.  At d = 64 the output and final state equal,
    bitwise, those of the same stream fed one segment per call (12 items: one
    workgroup each); at both widths every tile of two heads matches the oracle."""
    torch = gh.torch_mod()
    H, N, S = 4, 1216, 80
    w = syn.custom(f"persistent_odd_d{d}", 47, 1, H, d, N, S)
    gh.log(f"persistent grid d={d} rule={rule}: {H * S * 3} items")
    q, k, v, beta = gh.device_inputs(w)
    out1, e1 = gh.run(w, rule, q, k, v, beta, mode="sequence")
    if d == 64:
        out2, e2 = gh.run(w, rule, q, k, v, beta, mode="segments")
        torch.cuda.synchronize()
        assert torch.equal(out1, out2)
        assert torch.equal(e1.M, e2.M) and torch.equal(e1.z, e2.z)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    res = gh.oracle_full(w, rule, heads=heads)
    got = gh.to_host(out1)[:, heads]
    worst = 0.0
    for j, h in enumerate(heads):
        for s in range(S):
            sl = slice(s * N, (s + 1) * N)
            e = gh.metric(got[0, j, sl], res["A"][0, j, sl], "bf16")
            worst = max(worst, e)
            assert e <= gh.tol("bf16"), f"head {h} segment {s}: error {e:.3e}"
    eM = gh.metric(gh.to_host(e1.M)[:, heads], res["M"], "bf16")
    gh.log(f"  persistent d={d}/{rule}: worst tile {worst:.3e}, final M {eM:.3e}")
    assert eM <= gh.tol("bf16")


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_reset_determinism_and_poisoned_workspace(rule):
    torch = gh.torch_mod()
    w = syn.custom("repeat_case", 51, 1, 4, 128, 384, 3)
    gh.log(f"repeat/reset/poison rule={rule}")
    q, k, v, beta = gh.device_inputs(w)
    out1, eng = gh.run(w, rule, q, k, v, beta)
    M1, z1 = eng.M.clone(), eng.z.clone()
    eng.reset()
    assert eng.segments_done == 0
    ws, _ = eng.workspace(q.shape[2])
    ws.fill_(0xFF)  # NaN bit patterns everywhere
    out2, _ = gh.run(w, rule, q, k, v, beta, engine=eng)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(M1, eng.M) and torch.equal(z1, eng.z)


def test_resume_from_saved_state():
    """The compressive state is the checkpoint: copying (M, z, counter) out and back
    in continues the stream bitwise."""
    torch = gh.torch_mod()
    from compressive_memory_transformer_amd import infini as ia
    w = syn.custom("resume_case", 61, 1, 2, 128, 256, 4)
    q, k, v, beta = gh.device_inputs(w)
    for rule in ("linear", "delta"):
        whole, _ = gh.run(w, rule, q, k, v, beta)
        half = 2 * w.segment_len
        e1 = ia.InfiniAttention(1, 2, 128, 128, w.segment_len, "bf16", rule)
        a1 = e1.forward_sequence(q[:, :, :half].contiguous(), k[:, :, :half].contiguous(),
                                 v[:, :, :half].contiguous(), beta)
        saved = (e1.M.clone(), e1.z.clone(), e1.segments_done)
        e2 = ia.InfiniAttention(1, 2, 128, 128, w.segment_len, "bf16", rule)
        e2.M.copy_(saved[0])
        e2.z.copy_(saved[1])
        e2.state.segments_done = saved[2]
        a2 = e2.forward_sequence(q[:, :, half:].contiguous(), k[:, :, half:].contiguous(),
                                 v[:, :, half:].contiguous(), beta)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([a1, a2], dim=2), whole)


def test_single_layer_32k_linear_full():
    """The 32K-token single-layer workload (B=1, H=8, N=2048, 16 segments, linear),
    every tile against the oracle."""
    w = syn.WORKLOADS["layer_32k_linear"]
    gh.log(f"workload {w.name}")
    q, k, v, beta = gh.device_inputs(w)
    out, eng = gh.run(w, "linear", q, k, v, beta)
    gh.torch_mod().cuda.synchronize()
    res = gh.oracle_full(w, "linear")
    gh.compare_full(w, "linear", out, eng, res, label=w.name)


OVERFLOW_CASES = [
    # name, seed, N, segments, (query row, key row) pairs: query row i is made a
    # large multiple of key row j (j <= i), so its score against key j exceeds the
    # maximum over the first 32-key block by far more than 64 ln 2
    ("n2048", 71, 2048, 2, [(200, 100), (1000, 1000), (1800, 1000), (2047, 40)]),
    ("n192", 72, 192, 3, [(150, 64), (191, 33), (40, 40)]),
]


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", OVERFLOW_CASES, ids=[c[0] for c in OVERFLOW_CASES])
def test_softmax_overflow_recompute(case, rule):
    """Scores far above the reference maximum the fused kernel takes from the
    first 32-key block: the block's probability sums leave the safe range and the
    query block is recomputed exactly.  Queries in the first and in later query
    tiles, on the diagonal tile and left of it, in a segment without memory and in
    one with memory; every tile against the oracle."""
    name, seed, N, S, pairs = case
    w = syn.custom(f"overflow_{name}", seed, 1, 2, 128, N, S)
    q, k, v = (syn.full_tensor(w, i) for i in (syn.Q_ID, syn.K_ID, syn.V_ID))
    sc = 1.0 / math.sqrt(128.0)
    for h in range(w.heads):
        for seg in (0, S - 1):
            for (i, j) in pairs:
                kj = k[0, h, seg * N + j].astype(np.float64)
                c = 150.0 / (sc * float(kj @ kj))      # score about 150 (natural units)
                q[0, h, seg * N + i] = syn.round_bf16((c * kj).astype(np.float32))
    # on the host: every planted row's best score beats its first block's maximum
    # by far more than 64 ln 2 (where the kernel's sums would pass 2^64)
    for seg in (0, S - 1):
        for (i, j) in pairs:
            qi = q[0, 0, seg * N + i].astype(np.float64)
            s_row = sc * (k[0, 0, seg * N:seg * N + i + 1].astype(np.float64) @ qi)
            assert s_row.max() - s_row[:min(32, i + 1)].max() > 64 * math.log(2) + 20 or j < 32
    gh.log(f"overflow case {name} rule={rule}")
    dq, dk, dv = (gh.upload_values(x, "bf16") for x in (q, k, v))
    beta = gh.torch_mod().from_numpy(syn.betas(w)).to("cuda")
    out, eng = gh.run(w, rule, dq, dk, dv, beta)
    gh.torch_mod().cuda.synchronize()
    res = ref.forward_sequence(q, k, v, syn.betas(w), rule, N)
    gh.compare_full(w, rule, out, eng, res, label=f"overflow_{name}/{rule}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_nonfinite_inputs_propagate(rule, dtype):
    """A NaN in one query element and an infinity in one key element are carried
    to the outputs and the state the way the float64 oracle carries them: the rows
    and state entries that are not finite there are not finite on the GPU, and
    every other row and entry matches."""
    d, N = (128, 256) if dtype == "bf16" else (32, 64)
    w = syn.custom(f"nonfinite_{dtype}", 81, 1, 2, d, N, 3, dtype=dtype)
    q, k, v = (syn.full_tensor(w, i) for i in (syn.Q_ID, syn.K_ID, syn.V_ID))
    q[0, 0, 1 * N + 77, 5] = np.nan          # head 0, segment 1
    k[0, 1, 2 * N + 30, 9] = np.inf          # head 1, last segment
    gh.log(f"non-finite inputs {dtype}/{rule}")
    dq, dk, dv = (gh.upload_values(x, dtype) for x in (q, k, v))
    beta = gh.torch_mod().from_numpy(syn.betas(w)).to("cuda")
    out, eng = gh.run(w, rule, dq, dk, dv, beta)
    gh.torch_mod().cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        res = ref.forward_sequence(q, k, v, syn.betas(w), rule, N)
    got = gh.to_host(out)
    fin_ref = np.isfinite(res["A"]).all(axis=-1)
    fin_gpu = np.isfinite(got).all(axis=-1)
    assert (~fin_ref).any(), "the planted values must make some output rows non-finite"
    assert np.array_equal(fin_ref, fin_gpu), (np.argwhere(fin_ref != fin_gpu)[:5])
    for h in range(w.heads):
        for s in range(w.segments):
            rows = slice(s * N, (s + 1) * N)
            ok = fin_ref[0, h, rows]
            e = gh.metric(got[0, h, rows][ok], res["A"][0, h, rows][ok], dtype)
            assert e <= gh.tol(dtype), (h, s, e)
    for name, g, o in (("M", gh.to_host(eng.M), res["M"]), ("z", gh.to_host(eng.z), res["z"])):
        assert np.array_equal(np.isfinite(g), np.isfinite(o)), name
        for h in range(w.heads):
            ok = np.isfinite(o[0, h])
            if ok.any():
                assert gh.metric(g[0, h][ok], o[0, h][ok], dtype) <= gh.tol(dtype), (name, h)
    gh.log(f"  non-finite {dtype}/{rule}: {int((~fin_ref).sum())} non-finite rows, all matched")

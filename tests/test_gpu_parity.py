"""GPU parity of the HIP library against the float64 oracle, through the C ABI.

Small shapes (several query/key tiles, a ragged last query tile, both rules,
both head widths), the tiny fp32 workload and the full 32K-token single-layer
workload, plus the diagnostics: pure-memory and pure-local gates, a stress input
with widely spread scores, segment-by-segment streaming == one sequence call
(bitwise), reset, determinism and a NaN-poisoned workspace.
"""

import math

import numpy as np
import pytest

from compressive_memory_transformer_amd import synthetic as syn
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
    # name, seed, B, H, d, N, S, dtype
    ("f32_tiny_shape", 11, 1, 2, 32, 64, 4, "f32"),
    ("f32_ragged", 12, 2, 3, 20, 37, 3, "f32"),
    ("bf16_d128_n192", 13, 2, 3, 128, 192, 3, "bf16"),
    ("bf16_d64_n256", 14, 1, 4, 64, 256, 4, "bf16"),
    ("bf16_d128_n64", 15, 1, 2, 128, 64, 5, "bf16"),
    ("bf16_d64_n320", 16, 2, 1, 64, 320, 2, "bf16"),
]


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case, rule):
    name, seed, B, H, d, N, S, dtype = case
    gh.log(f"case {name} rule={rule}")
    w = syn.custom(name, seed, B, H, d, N, S, dtype=dtype)
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
    """Unscaled N(0, 1) queries and keys: scores spread over tens of units, so the
    running maximum of the online softmax moves and rescales."""
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

"""GPU parity on the full-size workloads, sampled: for chosen heads the oracle
walks the whole stream (memory updates only) and produces complete segment
outputs at chosen segments; those tiles and the final state of the head are
compared with the GPU run of the whole workload.

  batched 64K-token stream, delta rule       (B=8, H=16, 32 segments of 2048)
  1M-token stream, delta rule, planted pair  (B=1, H=8, 512 segments)
  500K-token wide stream, both rules         (B=1, H=32, 256 segments)

Each also runs with beta = +inf, where the output is the memory retrieval alone,
so that a wrong A_mem cannot hide behind the local attention term.
"""

import dataclasses
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
    yield
    torch.cuda.empty_cache()


def _memory_only_check(w, rule, q, k, v, heads_bh, segments):
    """beta = +inf on the GPU against the oracle's A_mem at the sampled tiles."""
    out, _ = gh.run(w, rule, q, k, v, gh.inf_beta(w.heads, 1))
    N = w.segment_len
    worst = 0.0
    for (b, h) in heads_bh:
        parts = {}
        gh.oracle_walk(w, rule, b, h, segments, parts=parts)
        for s, (_, a_mem) in parts.items():
            got = gh.to_host(out[b, h, s * N:(s + 1) * N])
            if s == 0:
                assert np.all(got == 0.0)
                continue
            e = gh.metric(got, a_mem, w.dtype)
            worst = max(worst, e)
            assert e <= gh.BF16_TOL, (b, h, s, e)
    gh.log(f"  {w.name}/{rule} beta=+inf: worst sampled A_mem tile {worst:.3e}")
    del out


def test_batched_64k_delta():
    w = syn.WORKLOADS["batched_64k_delta"]
    gh.log(f"workload {w.name}")
    q, k, v, beta = gh.device_inputs(w)
    out, eng = gh.run(w, "delta", q, k, v, beta)
    heads = [(0, 0), (3, 7), (7, 15)]
    segs = [0, 1, 16, 31]
    gh.compare_sampled(w, "delta", out, eng, heads, segs, label=w.name)
    del out
    _memory_only_check(w, "delta", q, k, v, heads[:2], [0, 1, 31])


def test_stream_1m_delta_with_planted_pair():
    torch = gh.torch_mod()
    w = syn.WORKLOADS["stream_1m_delta"]
    gh.log(f"workload {w.name}")
    q, k, v, beta = gh.device_inputs(w)
    out, eng = gh.run(w, "delta", q, k, v, beta)
    heads = [(0, 0), (0, 5)]
    segs = [0, 1, 255, 511]
    gh.compare_sampled(w, "delta", out, eng, heads, segs, label=w.name)
    del out
    _memory_only_check(w, "delta", q, k, v, heads[:1], [0, 511])

    # planted-pair retrieval: the change of A_mem at the query row of the last
    # segment caused by the plant, GPU against oracle, head 5
    p0, p1, _, _ = syn.planted_pair(w)
    h = 5
    N, S = w.segment_len, w.segments
    last = slice((S - 1) * N, S * N)
    got_planted = gh.run(w, "delta", q, k, v, gh.inf_beta(w.heads, 1))[0][0, h, last][p1]
    bare = dataclasses.replace(w, planted=False)
    for tid, t, seg, row in ((syn.K_ID, k, 0, p0), (syn.V_ID, v, 0, p0), (syn.Q_ID, q, S - 1, p1)):
        for hh in range(w.heads):
            t[0, hh, seg * N + row] = torch.from_numpy(syn.tile(bare, tid, 0, hh, seg)[row]).to(t.dtype).to("cuda")
    got_bare = gh.run(w, "delta", q, k, v, gh.inf_beta(w.heads, 1))[0][0, h, last][p1]
    d_gpu = gh.to_host(got_planted) - gh.to_host(got_bare)
    parts_p, parts_b = {}, {}
    gh.oracle_walk(w, "delta", 0, h, [S - 1], parts=parts_p)
    gh.oracle_walk(bare, "delta", 0, h, [S - 1], parts=parts_b)
    # the GPU rows are bf16 outputs: take the oracle rows through the same rounding
    # before differencing, so both sides compare the change of the stored values
    rnd = lambda x: syn.round_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)
    d_ref = rnd(parts_p[S - 1][1][p1]) - rnd(parts_b[S - 1][1][p1])
    rel = np.linalg.norm(d_gpu - d_ref) / np.linalg.norm(d_ref)
    share = np.linalg.norm(d_ref) / np.linalg.norm(parts_p[S - 1][1][p1])
    gh.log(f"  planted pair: |delta| / |A_mem row| = {share:.3e}; GPU delta vs oracle delta: {rel:.3e}")
    assert rel <= 0.10


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_wide_500k(rule):
    w = syn.WORKLOADS["wide_500k"]
    gh.log(f"workload {w.name} rule={rule}")
    q, k, v, beta = gh.device_inputs(w)
    out, eng = gh.run(w, rule, q, k, v, beta)
    heads = [(0, 0), (0, 17), (0, 31)]
    segs = [0, 1, 128, 255]
    gh.compare_sampled(w, rule, out, eng, heads, segs, label=f"{w.name}/{rule}")
    del out
    _memory_only_check(w, rule, q, k, v, heads[:1], [0, 1, 255])

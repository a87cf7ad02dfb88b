"""GPU parity on the full-size workloads:

  batched 64K-token stream, delta rule       (B=8, H=16, 32 segments of 2048)
  1M-token stream, delta rule, planted pair  (B=1, H=8, 512 segments)
  500K-token wide stream, both rules         (B=1, H=32, 256 segments)

For every head the oracle walks the whole stream (memory updates only) and the
final (M, z) of every head is compared with the GPU's.  For one head per
workload every segment's output is compared with the oracle's segment output,
built from that head's walk.  Each workload also runs with beta = +inf, where
the output is the memory retrieval alone, so that a wrong A_mem cannot hide
behind the local attention term: every segment of the chosen head is checked
there too (exactly 0 in the first segment).  On the 1M-token stream the change
of the retrieval at the planted query caused by the planted pair is compared
with the oracle's for every head.
"""

import dataclasses

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
    yield
    torch.cuda.empty_cache()


def _full_check(w, rule, q, k, v, beta, full_head):
    """The GPU stream against the oracle: every head's final state, every
    segment of `full_head` (gated output and, in a beta = +inf run, the
    retrieval alone).  Returns the oracle walks."""
    gh.log(f"workload {w.name} rule={rule}")
    out, eng = gh.run(w, rule, q, k, v, beta)
    gh.torch_mod().cuda.synchronize()
    walks = gh.walk_all_heads(w, rule, keep_heads=[full_head])
    gh.check_final_states(w, eng, walks, f"{w.name}/{rule}")
    snaps = walks[full_head][2]
    gh.check_every_segment(w, rule, out, *full_head, snaps, f"{w.name}/{rule}")
    del out, eng
    mem, _ = gh.run(w, rule, q, k, v, gh.inf_beta(w.heads, 1))
    gh.check_every_segment(w, rule, mem, *full_head, snaps, f"{w.name}/{rule} beta=+inf", part="A_mem")
    del mem
    return walks


def test_batched_64k_delta():
    w = syn.WORKLOADS["batched_64k_delta"]
    q, k, v, beta = gh.device_inputs(w)
    _full_check(w, "delta", q, k, v, beta, (3, 7))


def test_stream_1m_delta_with_planted_pair():
    torch = gh.torch_mod()
    w = syn.WORKLOADS["stream_1m_delta"]
    q, k, v, beta = gh.device_inputs(w)
    walks = _full_check(w, "delta", q, k, v, beta, (0, 5))

    # planted-pair retrieval, every head: the change of A_mem at the query row of
    # the last segment caused by the plant, GPU against oracle
    p0, p1, _, _ = syn.planted_pair(w)
    N, S = w.segment_len, w.segments
    last = slice((S - 1) * N, S * N)
    got_planted = gh.to_host(gh.run(w, "delta", q, k, v, gh.inf_beta(w.heads, 1))[0][0, :, last][:, p1])
    bare = dataclasses.replace(w, planted=False)
    for tid, t, seg, row in ((syn.K_ID, k, 0, p0), (syn.V_ID, v, 0, p0), (syn.Q_ID, q, S - 1, p1)):
        for hh in range(w.heads):
            t[0, hh, seg * N + row] = torch.from_numpy(syn.tile(bare, tid, 0, hh, seg)[row]).to(t.dtype).to("cuda")
    got_bare = gh.to_host(gh.run(w, "delta", q, k, v, gh.inf_beta(w.heads, 1))[0][0, :, last][:, p1])
    torch.cuda.synchronize()
    # the memory the last segment reads, with the plant (from the walks above)
    # and without it (walks of the bare stream)
    pre_b = gh.walk_all_heads(bare, "delta")
    # the GPU rows are bf16 outputs: the oracle rows go through the same rounding
    # before differencing, so both sides compare the change of the stored values
    rnd = lambda x: syn.round_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)
    worst = 0.0
    all_gpu, all_ref = [], []
    for h in range(w.heads):
        qp = syn.tile(w, syn.Q_ID, 0, h, S - 1)[p1:p1 + 1].astype(np.float64)
        qb = syn.tile(bare, syn.Q_ID, 0, h, S - 1)[p1:p1 + 1].astype(np.float64)
        Mp, zp = walks[(0, h)][3]
        Mb, zb = pre_b[(0, h)][3]
        a_p = ref.memory_retrieval(qp, Mp, zp, False)[0]
        a_b = ref.memory_retrieval(qb, Mb, zb, False)[0]
        d_ref = rnd(a_p) - rnd(a_b)
        d_gpu = got_planted[h] - got_bare[h]
        rel = np.linalg.norm(d_gpu - d_ref) / np.linalg.norm(d_ref)
        share = np.linalg.norm(d_ref) / np.linalg.norm(a_p)
        worst = max(worst, rel)
        all_gpu.append(d_gpu)
        all_ref.append(d_ref)
        gh.log(f"  planted pair head {h}: |delta| / |A_mem row| = {share:.3e}; GPU delta vs oracle delta {rel:.3e}")
        assert rel <= 0.10, (h, rel)
    tot = np.linalg.norm(np.concatenate(all_gpu) - np.concatenate(all_ref)) / np.linalg.norm(np.concatenate(all_ref))
    gh.log(f"  planted pair: worst head {worst:.3e}; all {w.heads} heads together {tot:.3e}")
    assert tot <= 0.10


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_wide_500k(rule):
    w = syn.WORKLOADS["wide_500k"]
    q, k, v, beta = gh.device_inputs(w)
    _full_check(w, rule, q, k, v, beta, (0, 17))

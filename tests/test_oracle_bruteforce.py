"""The oracle against a scalar-loop transcription on the tiny fp32 workload's
inputs (transcription guard only; the readings are pinned elsewhere)."""

import math

import numpy as np
import pytest

from compressive_memory_transformer_amd import synthetic as syn
from oracle import infini_ref
from tests import brute_force


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_oracle_matches_scalar_loops(rule):
    w = syn.custom("bf_case", 21, 1, 2, 8, 16, 3, dtype="f32")
    q, k, v = (syn.full_tensor(w, t) for t in (0, 1, 2))
    beta = syn.betas(w)
    res = infini_ref.forward_sequence(q, k, v, beta, rule, w.segment_len)
    A, M, z = brute_force.run(q[0].tolist(), k[0].tolist(), v[0].tolist(), beta.tolist(), rule,
                              w.segment_len, 1.0 / math.sqrt(w.d_key))
    assert np.allclose(res["A"][0], np.array(A), rtol=1e-12, atol=1e-12)
    assert np.allclose(res["M"][0], np.array(M), rtol=1e-12, atol=1e-12)
    assert np.allclose(res["z"][0], np.array(z), rtol=1e-13, atol=0)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_oracle_matches_scalar_loops_tiny_workload(rule):
    w = syn.WORKLOADS["tiny_f32"]
    q, k, v = (syn.full_tensor(w, t) for t in (0, 1, 2))
    beta = syn.betas(w)
    res = infini_ref.forward_sequence(q, k, v, beta, rule, w.segment_len)
    A, M, z = brute_force.run(q[0].tolist(), k[0].tolist(), v[0].tolist(), beta.tolist(), rule,
                              w.segment_len, 1.0 / math.sqrt(w.d_key))
    assert np.allclose(res["A"][0], np.array(A), rtol=1e-11, atol=1e-12)
    assert np.allclose(res["M"][0], np.array(M), rtol=1e-11, atol=1e-11)
    assert np.allclose(res["z"][0], np.array(z), rtol=1e-13, atol=0)

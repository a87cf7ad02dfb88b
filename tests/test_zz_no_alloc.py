"""The allocation-free forward (infini_attn_forward_sequence_noalloc, which runs on
the library's own device scratch array) against infini_attn_forward_sequence with
a caller workspace, through the C ABI: two calls in a row on one GPU, the second
with a smaller input, both update rules.  The outputs and final states must be
bitwise equal (the same kernels on the same inputs), and the smaller stream is
also checked against the float64 oracle at the bf16 tile bar."""

import ctypes

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


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_noalloc_matches_workspace_entry_point(rule):
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = syn.WORKLOADS["layer_32k_linear"]          # 32K tokens x 8 heads
    small = syn.custom("noalloc_small", 91, 1, 2, 128, 256, 3)
    for w in (big, small):
        gh.log(f"no-alloc forward {w.name} rule={rule}")
        q, k, v, beta = gh.device_inputs(w)
        ref_eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, "bf16", rule)
        want = ref_eng.forward_sequence(q, k, v, beta)
        eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, "bf16", rule)
        assert 0 < ia.workspace_bytes(eng.state, w.seq_len) <= ia.noalloc_scratch_bytes()
        out = torch.empty_like(want)
        ia.forward_sequence_noalloc(eng.state, q, k, v, w.seq_len, beta, out, sh)
        torch.cuda.synchronize()
        assert eng.segments_done == w.segments
        assert torch.equal(out, want)
        assert torch.equal(eng.M, ref_eng.M) and torch.equal(eng.z, ref_eng.z)
        if w is small:
            res = gh.oracle_full(w, rule)
            gh.compare_full(w, rule, out, eng, res, label=f"no-alloc {w.name}/{rule}")
        gh.log(f"  bitwise equal to forward_sequence ({ia.workspace_bytes(eng.state, w.seq_len)} bytes of scratch)")

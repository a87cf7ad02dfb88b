"""GPU parity of infini_attn_layer_forward (projections + segment stream + output
projection) against the float64 layer oracle, through the C ABI."""

import numpy as np
import pytest

from compressive_memory_transformer_amd import synthetic as syn
from oracle import infini_layer as ol
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


CASES = [
    # name, seed, B, H, d, N, S, d_model
    ("d64_dm128", 41, 1, 2, 64, 128, 2, 128),
    ("d128_dm512", 42, 2, 4, 128, 256, 2, 512),
    # d_model = 192: the output projection's last 128-column tile is partial
    ("d128_dm192", 43, 1, 2, 128, 128, 3, 192),
    # enough output tiles for the 256 x 256 GEMM tiling in both projections
    ("d64_dm1024_big", 44, 2, 8, 64, 128, 64, 1024),
    # 256 x 256 tiling of the QKV projection with a partial last row tile (8320
    # rows) and a partial last column tile (1920 columns)
    ("d64_h10_dm512_ragged", 45, 1, 10, 64, 128, 65, 512),
]


def _bf16(torch, arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda").to(torch.bfloat16)


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_matches_oracle(case, rule):
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    name, seed, B, H, d, N, S, dm = case
    gh.log(f"layer {name} rule={rule}")
    w = syn.custom(name, seed, B, H, d, N, S, dtype="bf16")
    x, wq, wo = syn.layer_tensors(w, dm)
    beta = syn.betas(w)
    eng = ia.InfiniAttention(B, H, d, d, N, "bf16", rule)
    y = eng.layer_forward(_bf16(torch, x), _bf16(torch, wq), _bf16(torch, wo), torch.from_numpy(beta).cuda())
    torch.cuda.synchronize()
    want = ol.layer_forward(x, wq, wo, beta, rule, N, H, d, d)
    got = gh.to_host(y)
    worst = 0.0
    for b in range(B):
        for s in range(S):
            rows = slice(s * N, (s + 1) * N)
            e = gh.metric(got[b, rows], want["y"][b, rows], "bf16")
            worst = max(worst, e)
            assert e <= gh.tol("bf16"), f"{name}/{rule} y b={b} s={s}: error {e:.3e}"
    eM = gh.metric(gh.to_host(eng.M), want["M"], "bf16")
    ez = gh.metric(gh.to_host(eng.z), want["z"], "bf16")
    gh.log(f"  worst y tile {worst:.3e}; M {eM:.3e}; z {ez:.3e}")
    assert eM <= gh.tol("bf16") and ez <= gh.tol("bf16")
    assert eng.segments_done == S


def test_full_size_layer():
    """The 32K-token stream with d_model 1024 (the shape bench.py --layer 1024 times):
    every output tile against the oracle."""
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    w = syn.WORKLOADS["layer_32k_linear"]
    dm = 1024
    gh.log(f"layer full size {w.name}, d_model {dm}")
    x, wq, wo = syn.layer_tensors(w, dm)
    beta = syn.betas(w)
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, "bf16", "linear")
    y = eng.layer_forward(_bf16(torch, x), _bf16(torch, wq), _bf16(torch, wo), torch.from_numpy(beta).cuda())
    torch.cuda.synchronize()
    want = ol.layer_forward(x, wq, wo, beta, "linear", w.segment_len, w.heads, w.d_key, w.d_value)
    got = gh.to_host(y)
    N, worst = w.segment_len, 0.0
    for s in range(w.segments):
        rows = slice(s * N, (s + 1) * N)
        e = gh.metric(got[0, rows], want["y"][0, rows], "bf16")
        worst = max(worst, e)
        assert e <= gh.tol("bf16"), f"y segment {s}: error {e:.3e}"
    gh.log(f"  worst y tile {worst:.3e}")

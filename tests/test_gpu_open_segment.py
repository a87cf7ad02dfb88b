"""GPU parity of the open-segment entry point (tokens appended in any number per
call, single-token decode steps, ragged tails) against the oracle's
forward_stream, through the C ABI."""

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


CASES = [
    # name, seed, B, H, d, N, segments generated, dtype, chunk sizes (tokens per append call)
    ("f32_tiny_chunks", 21, 1, 2, 32, 64, 5, "f32", [1, 5, 58, 1, 64, 70, 3, 1, 17]),
    ("f32_ragged_dims", 22, 2, 1, 20, 37, 4, "f32", [36, 1, 1, 40, 50, 2]),
    ("bf16_d128_chunks", 23, 1, 2, 128, 128, 5, "bf16", [1, 127, 3, 260, 1, 60, 7]),
    ("bf16_d64_chunks", 24, 2, 2, 64, 192, 4, "bf16", [100, 92, 384, 1, 1, 50]),
    # a bf16 shape without MFMA kernels (d = 32, N = 80): the VALU path throughout
    ("bf16_d32_n80", 27, 1, 2, 32, 80, 4, "bf16", [1, 70, 9, 90, 1, 1, 40]),
]


def _per_row(got, want, dtype, label):
    """Every output row graded on its own (the tile measure applied to one row):
    a decode step answers one row, so one wrong token cannot hide in a tile."""
    worst = 0.0
    B, H, T, _ = got.shape
    for b in range(B):
        for h in range(H):
            for t in range(T):
                e = gh.metric(got[b, h, t], want[b, h, t], dtype)
                worst = max(worst, e)
                assert e <= gh.tol(dtype), f"{label} b={b} h={h} token {t}: row error {e:.3e}"
    return worst


def _stream_case(w, rule, chunks):
    """Appends the first sum(chunks) tokens of workload w in the given chunks and
    compares every output row (grouped by segment, the last one partial), the
    final state and the open segment with the oracle."""
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    T, N = sum(chunks), w.segment_len
    q, k, v, beta = gh.device_inputs(w)
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, N, w.dtype, rule)
    eng.open_stream()
    outs, pos = [], 0
    for c in chunks:
        sl = slice(pos, pos + c)
        outs.append(eng.append(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), beta))
        pos += c
    torch.cuda.synchronize()
    got = gh.to_host(torch.cat(outs, dim=2))
    qn, kn, vn = (syn.full_tensor(w, i)[:, :, :T] for i in (0, 1, 2))
    res = ref.forward_stream(qn, kn, vn, syn.betas(w), rule, N)
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            for s in range((T + N - 1) // N):
                rows = slice(s * N, min(T, (s + 1) * N))
                e = gh.metric(got[b, h, rows], res["A"][b, h, rows], w.dtype)
                worst = max(worst, e)
                assert e <= gh.tol(w.dtype), f"{w.name}/{rule} b={b} h={h} s={s}: error {e:.3e}"
    worst_row = _per_row(got, res["A"], w.dtype, f"{w.name}/{rule}")
    gh.log(f"  {w.name}/{rule}: worst single row {worst_row:.3e}")
    eM = gh.metric(gh.to_host(eng.M), res["M"], w.dtype)
    ez = gh.metric(gh.to_host(eng.z), res["z"], w.dtype)
    gh.log(f"  {w.name}/{rule}: {len(chunks)} appends, {T} tokens; worst tile {worst:.3e}; M {eM:.3e}; z {ez:.3e}")
    assert eM <= gh.tol(w.dtype) and ez <= gh.tol(w.dtype)
    assert eng.segments_done == T // N and eng.filled == T % N
    f = T % N
    if f:   # the open segment holds exactly the last f keys and values (copied bit for bit)
        assert torch.equal(eng.k_open[:, :, :f], k[:, :, T - f:T])
        assert torch.equal(eng.v_open[:, :, :f], v[:, :, T - f:T])


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_appends_in_chunks(case, rule):
    name, seed, B, H, d, N, S, dtype, chunks = case
    gh.log(f"case {name} rule={rule}")
    w = syn.custom(name, seed, B, H, d, N, S, dtype=dtype)
    _stream_case(w, rule, chunks)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_decode_token_by_token(rule, dtype):
    """Two whole segments and a ragged tail, one token per call."""
    N = 64
    gh.log(f"decode {dtype}/{rule}")
    w = syn.custom(f"decode_{dtype}", 25, 1, 2, 128 if dtype == "bf16" else 32, N, 3, dtype=dtype)
    _stream_case(w, rule, [1] * (2 * N + 9))


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_whole_segments_take_the_segment_path(rule):
    """Appending whole segments at a segment boundary equals forward_sequence bit
    for bit (it runs the same kernels), then a ragged tail continues the stream."""
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    w = syn.custom("whole_segments", 26, 1, 2, 128, 128, 3, dtype="bf16")
    q, k, v, beta = gh.device_inputs(w)
    N = w.segment_len
    a = ia.InfiniAttention(1, 2, 128, 128, N, "bf16", rule)
    a.open_stream()
    b = ia.InfiniAttention(1, 2, 128, 128, N, "bf16", rule)
    sl = slice(0, 2 * N)
    out_a = a.append(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), beta)
    out_b = b.forward_sequence(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), beta)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(a.M, b.M) and torch.equal(a.z, b.z)
    assert a.segments_done == b.segments_done == 2 and a.filled == 0


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_full_size_decode_shape(rule):
    """The shape bench.py --decode 1024 times: the 32K-token stream's first 15
    segments through forward_sequence, then 1024 tokens of the last segment in one
    append (the many-query path) and 10 single-token appends; one head's outputs
    of the open segment, the state and the open buffers against the oracle."""
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    w = syn.WORKLOADS["layer_32k_linear"]
    N, h, F, T = w.segment_len, 5, 1024, 10
    L0 = (w.segments - 1) * N
    gh.log(f"open segment full size {w.name} rule={rule}, head {h}")
    q, k, v, beta = gh.device_inputs(w)
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, N, "bf16", rule)
    eng.forward_sequence(q[:, :, :L0].contiguous(), k[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(), beta)
    eng.open_stream()
    outs = [eng.append(*(x[:, :, L0:L0 + F].contiguous() for x in (q, k, v)), beta)]
    for i in range(T):
        sl = slice(L0 + F + i, L0 + F + i + 1)
        outs.append(eng.append(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), beta))
    torch.cuda.synchronize()
    got = gh.to_host(torch.cat(outs, dim=2)[:, h:h + 1])
    qn, kn, vn = (syn.full_tensor(w, i, heads=[h]) for i in (0, 1, 2))
    bn = syn.betas(w)[[h]]
    pre = ref.forward_sequence(qn[:, :, :L0], kn[:, :, :L0], vn[:, :, :L0], bn, rule, N)
    sl = slice(L0, L0 + F + T)
    res = ref.forward_stream(qn[:, :, sl], kn[:, :, sl], vn[:, :, sl], bn, rule, N, M0=pre["M"], z0=pre["z"],
                             segments_done=w.segments - 1)
    e_big = gh.metric(got[0, 0, :F], res["A"][0, 0, :F], "bf16")
    e_dec = _per_row(got[:, :, F:], res["A"][:, :, F:], "bf16", f"decode steps {rule}")
    eM = gh.metric(gh.to_host(eng.M)[:, h:h + 1], res["M"], "bf16")
    gh.log(f"  1024-token append {e_big:.3e}; decode steps {e_dec:.3e}; M {eM:.3e}")
    assert e_big <= gh.tol("bf16") and e_dec <= gh.tol("bf16") and eM <= gh.tol("bf16")
    assert eng.filled == F + T and eng.segments_done == w.segments - 1
    assert torch.equal(eng.k_open[:, :, :F + T], k[:, :, L0:L0 + F + T])

"""GPU parity of infini_attn_backward_sequence (the gradients of forward_sequence)
against the float64 gradient oracle, through the C ABI."""

import numpy as np
import pytest

from compressive_memory_transformer_amd import synthetic as syn
from oracle import infini_grad as og
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


def _workload(name, seed, B, H, dk, dv, N, S, dtype):
    scale = 1.0 / np.sqrt(dk) if dtype == "bf16" else 1.0
    return syn.Workload(name, seed, B, H, dk, dv, N, S, dtype, ("linear", "delta"), "uniform", 2.0, scale)


CASES = [
    # name, seed, B, H, d_key, d_value, N, S, dtype, segments already in the memory
    ("f32_tiny", 31, 1, 2, 32, 32, 64, 4, "f32", 0),
    ("f32_ragged_resume", 32, 2, 1, 20, 24, 37, 3, "f32", 2),
    ("bf16_d64", 33, 1, 2, 64, 64, 128, 3, "bf16", 0),
    ("bf16_d128_resume", 34, 1, 2, 128, 128, 256, 3, "bf16", 2),
    # N = 192: the 256-row tile of the attention kernels has two idle waves
    ("bf16_d128_n192", 35, 2, 1, 128, 128, 192, 2, "bf16", 1),
    # 256-row tiles of the attention kernels: three tiles (a pair and a lone
    # middle one), and a pair whose second tile holds 64 rows
    ("bf16_d128_n768", 37, 1, 2, 128, 128, 768, 2, "bf16", 1),
    ("bf16_d64_n320", 38, 1, 2, 64, 64, 320, 3, "bf16", 0),
    # a bf16 shape without MFMA kernels (different widths, ragged N): the VALU kernels
    ("bf16_dk32_dv48_n80", 36, 1, 2, 32, 48, 80, 3, "bf16", 1),
]


def _device(torch, arr, dtype):
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case, rule):
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    name, seed, B, H, dk, dv, N, S, dtype, done = case
    gh.log(f"backward {name} rule={rule}")
    w = _workload(name, seed, B, H, dk, dv, N, S, dtype)
    qn, kn, vn, don = (syn.full_tensor(w, i) for i in (syn.Q_ID, syn.K_ID, syn.V_ID, syn.DOUT_ID))
    beta = syn.betas(w)
    dM, dz = syn.state_grads(w)
    if done:
        M0, z0 = syn.initial_state(w, done)
    else:
        M0, z0 = np.zeros((B, H, dk, dv), np.float32), np.zeros((B, H, dk), np.float32)
    # bf16 values are exact in float32, so the device gets exactly what the oracle sees
    q, k, v, dout = (_device(torch, x, dtype) for x in (qn, kn, vn, don))
    eng = ia.InfiniAttention(B, H, dk, dv, N, dtype, rule)
    g = eng.backward_sequence(q, k, v, torch.from_numpy(beta).cuda(), dout, torch.from_numpy(M0).cuda(),
                              torch.from_numpy(z0).cuda(), done, dM=torch.from_numpy(dM).cuda(),
                              dz=torch.from_numpy(dz).cuda())
    torch.cuda.synchronize()
    want = og.backward_sequence(qn, kn, vn, beta, rule, N, don, dM=dM, dz=dz, M0=M0, z0=z0, segments_done=done)
    _check_grads(g, want, name, rule, dtype, B, H, S, N)


def _check_grads(g, want, name, rule, dtype, B, H, S, N):
    tol = gh.tol(dtype)
    worst = {}
    for key in ("dq", "dk", "dv"):
        got = gh.to_host(g[key])
        for b in range(B):
            for h in range(H):
                for s in range(S):
                    rows = slice(s * N, (s + 1) * N)
                    e = gh.metric(got[b, h, rows], want[key][b, h, rows], dtype)
                    worst[key] = max(worst.get(key, 0.0), e)
                    assert e <= tol, f"{name}/{rule} {key} b={b} h={h} s={s}: error {e:.3e}"
    for key in ("dM0", "dz0"):
        got = gh.to_host(g[key])
        for b in range(B):
            for h in range(H):
                e = gh.metric(got[b, h], want[key][b, h], "f32" if dtype == "f32" else "bf16")
                worst[key] = max(worst.get(key, 0.0), e)
                assert e <= tol, f"{name}/{rule} {key} b={b} h={h}: error {e:.3e}"
    gb = gh.to_host(g["dbeta"])
    e = float(np.abs(gb - want["dbeta"]).max() / max(np.abs(want["dbeta"]).max(), 1e-30))
    worst["dbeta"] = e
    gh.log("  " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert e <= tol, f"{name}/{rule} dbeta: error {e:.3e} ({gb} vs {want['dbeta']})"


# the saved-statistics pair runs on the MFMA shapes only
SAVED_CASES = [c for c in CASES if c[8] == "bf16" and c[4] == c[5] and c[4] in (64, 128) and c[6] % 64 == 0]


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("case", SAVED_CASES, ids=[c[0] for c in SAVED_CASES])
def test_backward_saved_matches_oracle(case, rule):
    """forward_sequence_train writes the output of forward_sequence bitwise and the
    rows' base-2 log-normalisers (against the oracle's); backward_sequence_saved
    on them gives the oracle's gradients."""
    from compressive_memory_transformer_amd import infini as ia
    from oracle import infini_ref as ref
    torch = gh.torch_mod()
    name, seed, B, H, dk, dv, N, S, dtype, done = case
    gh.log(f"backward saved {name} rule={rule}")
    w = _workload(name, seed, B, H, dk, dv, N, S, dtype)
    qn, kn, vn, don = (syn.full_tensor(w, i) for i in (syn.Q_ID, syn.K_ID, syn.V_ID, syn.DOUT_ID))
    beta = syn.betas(w)
    dM, dz = syn.state_grads(w)
    if done:
        M0, z0 = syn.initial_state(w, done)
    else:
        M0, z0 = np.zeros((B, H, dk, dv), np.float32), np.zeros((B, H, dk), np.float32)
    q, k, v, dout = (_device(torch, x, dtype) for x in (qn, kn, vn, don))
    beta_t, M0t, z0t = (torch.from_numpy(x).cuda() for x in (beta, M0, z0))
    eng = ia.InfiniAttention(B, H, dk, dv, N, dtype, rule)

    def start():
        eng.M.copy_(M0t)
        eng.z.copy_(z0t)
        eng.state.segments_done = done

    start()
    out_plain = eng.forward_sequence(q, k, v, beta_t)
    start()
    out, lse = eng.forward_sequence_train(q, k, v, beta_t)
    torch.cuda.synchronize()
    assert eng.segments_done == done + S
    assert torch.equal(out, out_plain), f"{name}/{rule}: the training forward's output differs"
    e = float(np.abs(gh.to_host(lse) - ref.log_normalisers(qn, kn, N)).max())
    gh.log(f"  lse max abs error {e:.2e} (log2 units)")
    assert e <= gh.tol(dtype), f"{name}/{rule} lse: error {e:.3e}"
    g = eng.backward_sequence(q, k, v, beta_t, dout, M0t, z0t, done, dM=torch.from_numpy(dM).cuda(),
                              dz=torch.from_numpy(dz).cuda(), saved=(out, lse))
    torch.cuda.synchronize()
    want = og.backward_sequence(qn, kn, vn, beta, rule, N, don, dM=dM, dz=dz, M0=M0, z0=z0, segments_done=done)
    _check_grads(g, want, name + "/saved", rule, dtype, B, H, S, N)


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_full_size_sampled_head(rule, saved):
    """The 32K-token single-layer stream at its full size (the shape bench.py times):
    one head's gradients over all 16 segments against the oracle (heads are
    independent; with one batch row dbeta of that head is that head's alone), from
    the backward that recomputes the softmax statistics and from the one given the
    training forward's output and log-normalisers."""
    from compressive_memory_transformer_amd import infini as ia
    torch = gh.torch_mod()
    w = syn.WORKLOADS["layer_32k_linear"]
    h = 3
    gh.log(f"backward full size {w.name} rule={rule}, head {h}, saved={saved}")
    q, k, v, beta = gh.device_inputs(w)
    dout = gh.upload(w, syn.DOUT_ID)
    dM, dz = syn.state_grads(w)
    eng = ia.InfiniAttention(w.batch, w.heads, w.d_key, w.d_value, w.segment_len, "bf16", rule)
    zM, zz = torch.zeros_like(eng.M), torch.zeros_like(eng.z)
    keep = None
    if saved:
        eng.reset()
        keep = eng.forward_sequence_train(q, k, v, beta)
    g = eng.backward_sequence(q, k, v, beta, dout, zM, zz, 0, dM=torch.from_numpy(dM).cuda(),
                              dz=torch.from_numpy(dz).cuda(), saved=keep)
    torch.cuda.synchronize()
    qn, kn, vn, don = (syn.full_tensor(w, i, heads=[h]) for i in (syn.Q_ID, syn.K_ID, syn.V_ID, syn.DOUT_ID))
    want = og.backward_sequence(qn, kn, vn, syn.betas(w)[[h]], rule, w.segment_len, don, dM=dM[:, [h]],
                                dz=dz[:, [h]])
    N, worst = w.segment_len, {}
    for key in ("dq", "dk", "dv"):
        got = gh.to_host(g[key][:, h:h + 1])
        for s in range(w.segments):
            rows = slice(s * N, (s + 1) * N)
            e = gh.metric(got[0, 0, rows], want[key][0, 0, rows], "bf16")
            worst[key] = max(worst.get(key, 0.0), e)
            assert e <= gh.tol("bf16"), f"{rule} {key} segment {s}: error {e:.3e}"
    for key in ("dM0", "dz0"):
        e = gh.metric(gh.to_host(g[key][:, h:h + 1]), want[key], "bf16")
        worst[key] = e
        assert e <= gh.tol("bf16"), f"{rule} {key}: error {e:.3e}"
    gb, wb = float(gh.to_host(g["dbeta"])[h]), float(want["dbeta"][0])
    worst["dbeta"] = abs(gb - wb) / max(abs(wb), 1e-30)
    gh.log("  " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert worst["dbeta"] <= gh.tol("bf16")

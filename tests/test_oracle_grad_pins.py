"""Pins of the gradient oracle (oracle/infini_grad.py), CPU, float64.

The gradient is pinned to the mathematics of the derivative, not to itself:
central finite differences of the (separately pinned) forward oracle for every
input of tiny streams, both rules, a first and a later segment position; the
beta = -inf single segment against torch autograd of causal SDPA.  Planted
mistakes in the gradient oracle must each fail a pin."""


import numpy as np
import pytest

from oracle import infini_grad as og
from oracle import infini_ref as ref


def _stream(seed, B=1, H=2, N=3, S=3, dk=3, dv=2, done=0):
    rng = np.random.default_rng(seed)
    L = N * S
    x = {
        "q": 0.8 * rng.standard_normal((B, H, L, dk)),
        "k": 0.8 * rng.standard_normal((B, H, L, dk)),
        "v": rng.standard_normal((B, H, L, dv)),
        "beta": rng.standard_normal(H),
        "M0": rng.standard_normal((B, H, dk, dv)) if done else np.zeros((B, H, dk, dv)),
        "z0": (np.abs(rng.standard_normal((B, H, dk))) + 0.5) if done else np.zeros((B, H, dk)),
    }
    w = {"dA": rng.standard_normal((B, H, L, dv)), "dM": rng.standard_normal((B, H, dk, dv)),
         "dz": rng.standard_normal((B, H, dk))}
    return x, w, N, done


def _loss(x, w, rule, N, done):
    r = ref.forward_sequence(x["q"], x["k"], x["v"], x["beta"], rule, N, M0=x["M0"], z0=x["z0"],
                             segments_done=done)
    return float((w["dA"] * r["A"]).sum() + (w["dM"] * r["M"]).sum() + (w["dz"] * r["z"]).sum())


def _analytic(x, w, rule, N, done):
    return og.backward_sequence(x["q"], x["k"], x["v"], x["beta"], rule, N, w["dA"], dM=w["dM"], dz=w["dz"],
                                M0=x["M0"], z0=x["z0"], segments_done=done)


KEYS = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "M0": "dM0", "z0": "dz0"}


def _check_fd(seed, rule, done, h=1e-6, rtol=1e-6):
    x, w, N, done = _stream(seed, done=done)
    g = _analytic(x, w, rule, N, done)
    for name, gname in KEYS.items():
        arr = x[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            up = _loss(x, w, rule, N, done)
            arr[idx] = keep - h
            dn = _loss(x, w, rule, N, done)
            arr[idx] = keep
            fd[idx] = (up - dn) / (2 * h)
        scale = max(1.0, float(np.abs(fd).max()))
        err = float(np.abs(g[gname] - fd).max()) / scale
        assert err < rtol, f"{rule} done={done}: d/d{name} differs from finite differences by {err:.2e}"


def pin_fd_linear_from_empty():
    _check_fd(1, ref.RULE_LINEAR, 0)


def pin_fd_linear_with_history():
    _check_fd(2, ref.RULE_LINEAR, 3)


def pin_fd_delta_from_empty():
    _check_fd(3, ref.RULE_DELTA, 0)


def pin_fd_delta_with_history():
    _check_fd(4, ref.RULE_DELTA, 3)


def pin_single_segment_attention_is_sdpa_autograd():
    """beta = -inf, one segment, empty memory: A = causal SDPA, so dq, dk, dv are
    torch autograd's (float64, CPU) for the same output gradient."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 16, 8
    q, k, v, dA = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    beta = np.full(H, -np.inf)
    g = og.backward_sequence(q, k, v, beta, ref.RULE_LINEAR, N, dA)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    out.backward(torch.tensor(dA, dtype=torch.float64))
    assert np.allclose(g["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    # the update's share of dk, dv vanishes when the state gradient is zero
    assert np.allclose(g["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dv"], tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(g["dbeta"] == 0.0)


def pin_state_only_loss_is_linear_in_the_keys_and_values():
    """Linear rule, dA = 0: L = <dM, M_S> + <dz, z_S> with M_S = M_0 + sigma(K)^T V
    and z_S = z_0 + sum sigma(K) (both pinned forward identities), so dv = sigma(K) dM,
    dq = 0, dbeta = 0, dM0 = dM, dz0 = dz; checked on a longer stream than the
    finite differences can afford."""
    rng = np.random.default_rng(6)
    B, H, N, S, d = 1, 2, 8, 5, 4
    q, k, v = (rng.standard_normal((B, H, N * S, d)) for _ in range(3))
    dM, dz = rng.standard_normal((B, H, d, d)), rng.standard_normal((B, H, d))
    g = og.backward_sequence(q, k, v, rng.standard_normal(H), ref.RULE_LINEAR, N, np.zeros_like(v), dM=dM, dz=dz)
    assert np.allclose(g["dv"], ref.sigma(k) @ dM, rtol=1e-12, atol=1e-12)
    assert np.all(g["dq"] == 0.0) and np.all(g["dbeta"] == 0.0)
    assert np.allclose(g["dM0"], dM) and np.allclose(g["dz0"], dz)


ALL_GRAD_PINS = [pin_fd_linear_from_empty, pin_fd_linear_with_history, pin_fd_delta_from_empty,
                 pin_fd_delta_with_history, pin_single_segment_attention_is_sdpa_autograd,
                 pin_state_only_loss_is_linear_in_the_keys_and_values]


@pytest.mark.parametrize("pin", ALL_GRAD_PINS, ids=[p.__name__ for p in ALL_GRAD_PINS])
def test_grad_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes

def _softmax_jacobian_without_rowsum(q, k, v, scale, d_out):
    n = q.shape[0]
    s = np.where(ref.causal_mask(n), scale * (q @ k.T), -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    ds = p * (d_out @ v.T)
    return scale * ds @ k, scale * ds.T @ q, p.T @ d_out


def _retrieval_without_denominator_term(q, M, z, first, d_mem):
    n, d_key = q.shape
    if first:
        return np.zeros((n, d_key)), np.zeros_like(M), np.zeros(d_key)
    fq = ref.sigma(q)
    den = fq @ z
    dnum = d_mem / den[:, None]
    return (dnum @ M.T) * og.sigma_prime(q), fq.T @ dnum, np.zeros(d_key)


def _update_without_z_gradient(k, v, M, z, rule, first, gM, gz):
    dk, dv, gMp, gzp = ORIGINAL_UPDATE(k, v, M, z, rule, first, gM, gz)
    return dk - gz[None, :] * og.sigma_prime(k), dv, gMp, gzp


def _update_delta_without_state_term(k, v, M, z, rule, first, gM, gz):
    dk, dv, gMp, gzp = ORIGINAL_UPDATE(k, v, M, z, rule, first, gM, gz)
    if rule == ref.RULE_DELTA and not first:
        gMp = gM.copy()
    return dk, dv, gMp, gzp


def _sigma_prime_is_one(x):
    return np.ones_like(np.asarray(x, dtype=np.float64))


ORIGINAL_UPDATE = og.update_backward


def _segment_backward_without_gate_slope(q, k, v, M, z, beta, rule, first, scale, dA, gM, gz):
    dq, dk, dv, db, gMp, gzp = ORIGINAL_SEGMENT(q, k, v, M, z, beta, rule, first, scale, dA, gM, gz)
    g = og.gate_value(beta)
    return dq, dk, dv, (db / (g * (1 - g)) if 0 < g < 1 else db), gMp, gzp


def _segment_backward_reads_updated_state(q, k, v, M, z, beta, rule, first, scale, dA, gM, gz):
    Mn, zn = ref.memory_update(k, v, M, z, rule, first)
    return ORIGINAL_SEGMENT(q, k, v, Mn, zn, beta, rule, first, scale, dA, gM, gz)


ORIGINAL_SEGMENT = og.segment_backward

GRAD_MUTANTS = {
    "softmax_jacobian_without_rowsum": ("local_attention_backward", _softmax_jacobian_without_rowsum),
    "retrieval_without_denominator_term": ("retrieval_backward", _retrieval_without_denominator_term),
    "update_without_z_gradient": ("update_backward", _update_without_z_gradient),
    "delta_without_state_term": ("update_backward", _update_delta_without_state_term),
    "sigma_prime_is_one": ("sigma_prime", _sigma_prime_is_one),
    "gate_slope_dropped": ("segment_backward", _segment_backward_without_gate_slope),
    "backward_reads_updated_state": ("segment_backward", _segment_backward_reads_updated_state),
}


@pytest.mark.parametrize("name", sorted(GRAD_MUTANTS))
def test_grad_mutant_is_caught(name, monkeypatch):
    attr, fn = GRAD_MUTANTS[name]
    monkeypatch.setattr(og, attr, fn)
    failed = []
    for pin in ALL_GRAD_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every gradient pin"

"""Pins of the causal kernel linear attention oracle (oracle/kernel_linear.py),
CPU, float64; planted mistakes must each fail a pin."""

import numpy as np
import pytest

from oracle import infini_ref as ref
from oracle import kernel_linear as kl


def _x(seed, B=1, H=2, L=12, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, L, dk)), rng.standard_normal((B, H, L, dk)),
            rng.standard_normal((B, H, L, dv)))


def pin_equals_lower_triangular_form():
    """O = (W masked to j <= i) V / row sums, W = phi(Q) phi(K)^T (chapter-24
    page section 24.4: the prefix states reproduce the explicit masked kernel
    attention)."""
    q, k, v = _x(1)
    got = kl.causal_kernel_linear_attention(q, k, v)["O"]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            W = ref.sigma(q[b, h]) @ ref.sigma(k[b, h]).T
            W = np.where(ref.causal_mask(q.shape[2]), W, 0.0)
            want = (W @ v[b, h]) / W.sum(axis=1, keepdims=True)
            assert np.allclose(got[b, h], want, rtol=1e-12, atol=1e-12)


def pin_single_token_returns_its_value():
    """One token and an empty state: phi(q).phi(k) v / phi(q).phi(k) = v for any q."""
    q, k, v = _x(2, L=1)
    got = kl.causal_kernel_linear_attention(q, k, v)["O"]
    assert np.allclose(got, v, rtol=1e-13, atol=1e-13)


def pin_split_stream_equals_one_call():
    q, k, v = _x(3, L=20)
    whole = kl.causal_kernel_linear_attention(q, k, v)
    a = kl.causal_kernel_linear_attention(q[:, :, :7], k[:, :, :7], v[:, :, :7])
    b = kl.causal_kernel_linear_attention(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:], S0=a["S"], Z0=a["Z"])
    assert np.allclose(np.concatenate([a["O"], b["O"]], axis=2), whole["O"], rtol=1e-12, atol=1e-12)
    assert np.allclose(b["S"], whole["S"]) and np.allclose(b["Z"], whole["Z"])


def pin_final_state_is_the_linear_memory():
    """The final (S, Z) is the Infini-attention linear-rule memory after the same
    keys and values (the forward oracle's update, any segment length)."""
    q, k, v = _x(4, L=12)
    got = kl.causal_kernel_linear_attention(q, k, v)
    mem = ref.forward_sequence(q, k, v, np.zeros(q.shape[1]), ref.RULE_LINEAR, 4)
    assert np.allclose(got["S"], mem["M"]) and np.allclose(got["Z"], mem["z"])


ALL_KLA_PINS = [pin_equals_lower_triangular_form, pin_single_token_returns_its_value,
                pin_split_stream_equals_one_call, pin_final_state_is_the_linear_memory]


@pytest.mark.parametrize("pin", ALL_KLA_PINS, ids=[p.__name__ for p in ALL_KLA_PINS])
def test_kla_pin(pin):
    pin()


def _exclusive_prefix(q, k, v, S0=None, Z0=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    S_in = np.zeros((B, H, dk, dv)) if S0 is None else S0
    Z_in = np.ones((B, H, dk)) if Z0 is None else Z0
    O = np.zeros((B, H, L, dv))
    for b in range(B):
        for h in range(H):
            S, Z = S_in[b, h].copy(), Z_in[b, h].copy()
            for i in range(L):
                fq, fk = ref.sigma(q[b, h, i]), ref.sigma(k[b, h, i])
                O[b, h, i] = (fq @ S) / (fq @ Z)
                S = S + np.outer(fk, v[b, h, i])
                Z = Z + fk
    return {"O": O, "S": S_in + 0, "Z": Z_in + 0}


ORIGINAL_KLA = kl.causal_kernel_linear_attention


def _raw_key_normalizer(q, k, v, S0=None, Z0=None):
    """The normaliser accumulating the raw keys instead of phi(k)."""
    out = ORIGINAL_KLA(q, k, v, S0, Z0)
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    fq = ref.sigma(q)
    Zraw = (0.0 if Z0 is None else np.asarray(Z0)[:, :, None, :]) + np.cumsum(k, axis=2)
    Zphi = (0.0 if Z0 is None else np.asarray(Z0)[:, :, None, :]) + np.cumsum(ref.sigma(k), axis=2)
    scale = (fq * Zphi).sum(-1, keepdims=True) / (fq * Zraw).sum(-1, keepdims=True)
    return {"O": out["O"] * scale, "S": out["S"], "Z": Zraw[:, :, -1]}


# (phi itself is pinned with the forward oracle against torch's ELU + 1)
KLA_MUTANTS = {"exclusive_prefix": _exclusive_prefix, "raw_key_normaliser": _raw_key_normalizer}


@pytest.mark.parametrize("name", sorted(KLA_MUTANTS))
def test_kla_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(kl, "causal_kernel_linear_attention", KLA_MUTANTS[name])
    failed = []
    for pin in ALL_KLA_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"

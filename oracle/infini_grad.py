"""Float64 CPU oracle for the gradients of the Infini-attention segment forward.

TEST INFRASTRUCTURE ONLY, like ``infini_ref`` (imported by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg, never by the
product path, sharing no code with it).

What is differentiated is the forward of ``infini_ref.forward_sequence``: for each
(batch, head) and segment, in stream order, retrieval from (M_{s-1}, z_{s-1})
(close-reading page "精读笔记：Infini-attention", section 3.3), causal local
attention (section 3.1 with the mask of section 3.8 step 2), the gate (section
3.5), then the memory update, linear or delta (section 3.4; CSDN page section
2.1 for the delta fraction).  The pages train the layer end to end (close-reading
page, section 4; the chapter-24 page mentions gradient agreement in section
24.4) but print no backward formulas: everything here is the chain rule applied
to those forward equations, step by step in reverse order, with the readings of
the forward oracle (scale, first segment, zero denominators, segment-batched
delta correction, gate in every segment).

Given the loss L = <dA, A> + <dM, M_S> + <dz, z_S> (dA the output gradient,
dM, dz the gradients of the final state, zero when omitted), ``backward_sequence``
returns dL/dq, dL/dk, dL/dv, dL/dbeta and dL/dM_0, dL/dz_0 (the initial state).

Pins (``tests/test_oracle_grad_pins.py``): central finite differences of the
forward oracle on tiny shapes for every input, both rules, first and later
segments; the beta = -inf single-segment case against torch autograd of causal
SDPA; closed forms for the state-only loss of the linear rule; planted mistakes
in this module are each caught.  The delta rule's gradient is pinned by finite
differences of the forward oracle, whose own delta parity is pinned only through
special cases: that residual carries over.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import infini_ref as ref


def sigma_prime(x: np.ndarray) -> np.ndarray:
    """Derivative of ELU(alpha=1) + 1: 1 for x > 0, e^x otherwise (both sides give
    1 at x = 0)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


def gate_value(beta: float) -> float:
    beta = float(beta)
    if beta == math.inf:
        return 1.0
    if beta == -math.inf:
        return 0.0
    return 1.0 / (1.0 + math.exp(-beta))


def local_attention_backward(q, k, v, scale, d_out):
    """Gradients of A_dot = softmax(scale q k^T, causal) v with respect to q, k, v
    for the output gradient d_out (one head, one segment).

    P is the masked softmax; dP = d_out v^T; the softmax Jacobian gives
    dS = P * (dP - rowsum(P * dP)); then dq = scale dS k, dk = scale dS^T q,
    dv = P^T d_out.  Masked entries have P = 0 and so no gradient."""
    n = q.shape[0]
    scores = scale * (q @ k.T)
    scores = np.where(ref.causal_mask(n), scores, -np.inf)
    p = np.exp(scores - scores.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    dp = d_out @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * ds @ k, scale * ds.T @ q, p.T @ d_out


def retrieval_backward(q, M, z, first, d_mem):
    """Gradients of A_mem = sigma(q) M / (sigma(q) z) for the output gradient d_mem:
    returns (dq, dM, dz).  Rows with a zero denominator (and the whole first
    segment) are constant zero and pass no gradient.

    With num = sigma(q) M and den = sigma(q) z: dnum = d_mem / den,
    dden = -<d_mem, num> / den^2; d sigma(q) = dnum M^T + dden z^T; dM = sigma(q)^T dnum;
    dz = sigma(q)^T dden."""
    n, d_key = q.shape
    d_value = M.shape[1]
    if first:
        return np.zeros((n, d_key)), np.zeros((d_key, d_value)), np.zeros(d_key)
    fq = ref.sigma(q)
    num = fq @ M
    den = fq @ z
    ok = den > 0.0
    dnum = np.zeros((n, d_value))
    dden = np.zeros(n)
    dnum[ok] = d_mem[ok] / den[ok, None]
    dden[ok] = -(d_mem[ok] * num[ok]).sum(axis=1) / den[ok] ** 2
    dfq = dnum @ M.T + dden[:, None] * z[None, :]
    return dfq * sigma_prime(q), fq.T @ dnum, fq.T @ dden


def update_backward(k, v, M, z, rule, first, gM, gz):
    """Gradients through one memory update (M_s, z_s) = update(k, v, M_{s-1}, z_{s-1})
    given gM = dL/dM_s and gz = dL/dz_s: returns (dk, dv, dL/dM_{s-1}, dL/dz_{s-1}).

    Linear rule: M_s = M + sigma(K)^T V, z_s = z + sum_t sigma(K_t).
    Delta rule: R = sigma(K) M / (sigma(K) z) (0 in the first segment), U = V - R,
    M_s = M + sigma(K)^T U, z_s as in the linear rule."""
    fk = ref.sigma(k)
    gM_prev = gM.copy()
    gz_prev = gz.copy()
    if rule == ref.RULE_LINEAR:
        dfk = v @ gM.T + gz[None, :]
        dv = fk @ gM
    elif rule == ref.RULE_DELTA:
        R = ref.delta_correction(k, M, z, first)
        U = v - R
        dU = fk @ gM
        dv = dU.copy()
        dfk = U @ gM.T + gz[None, :]
        if not first:
            r = fk @ M
            e = fk @ z
            ok = e > 0.0
            dR = -dU
            dr = np.zeros_like(dR)
            de = np.zeros(k.shape[0])
            dr[ok] = dR[ok] / e[ok, None]
            de[ok] = -(dR[ok] * r[ok]).sum(axis=1) / e[ok] ** 2
            dfk = dfk + dr @ M.T + de[:, None] * z[None, :]
            gM_prev = gM_prev + fk.T @ dr
            gz_prev = gz_prev + fk.T @ de
    else:
        raise ValueError(f"unknown rule {rule!r}")
    return dfk * sigma_prime(k), dv, gM_prev, gz_prev


def segment_backward(q, k, v, M, z, beta, rule, first, scale, dA, gM, gz):
    """Reverse of ``infini_ref.segment_forward`` for one head and segment: the
    update's gradient first (it was applied last), then the gate, the local
    attention and the retrieval.  Returns (dq, dk, dv, dbeta, dL/dM_{s-1},
    dL/dz_{s-1})."""
    dk_u, dv_u, gM_prev, gz_prev = update_backward(k, v, M, z, rule, first, gM, gz)
    g = gate_value(beta)
    a_mem = ref.memory_retrieval(q, M, z, first)
    a_dot = ref.local_causal_attention(q, k, v, scale)
    dbeta = float((dA * (a_mem - a_dot)).sum()) * g * (1.0 - g)
    dq_a, dk_a, dv_a = local_attention_backward(q, k, v, scale, (1.0 - g) * dA)
    dq_m, dM_r, dz_r = retrieval_backward(q, M, z, first, g * dA)
    return (dq_a + dq_m, dk_a + dk_u, dv_a + dv_u, dbeta, gM_prev + dM_r, gz_prev + dz_r)


def backward_sequence(q, k, v, beta, rule, segment_len, dA, dM=None, dz=None, M0=None, z0=None,
                      segments_done=0, scale=None):
    """Gradients of ``infini_ref.forward_sequence`` (same arguments) for the loss
    <dA, A> + <dM, M_S> + <dz, z_S>.

    The forward is replayed to recover every M_{s-1}, z_{s-1}; then the segments
    are walked in reverse, carrying dL/dM_s and dL/dz_s backwards.  Returns a dict
    with dq, dk [B, H, L, d_key], dv [B, H, L, d_value], dbeta [H] (summed over the
    batch: beta is shared) and dM0 [B, H, d_key, d_value], dz0 [B, H, d_key]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dA = np.asarray(dA, dtype=np.float64)
    B, H, L, d_key = q.shape
    d_value = v.shape[-1]
    N = segment_len
    if L % N != 0:
        raise ValueError("sequence length must be a multiple of the segment length")
    S = L // N
    sc = ref.default_scale(d_key, scale)
    M_init = np.zeros((B, H, d_key, d_value)) if M0 is None else np.asarray(M0, dtype=np.float64)
    z_init = np.zeros((B, H, d_key)) if z0 is None else np.asarray(z0, dtype=np.float64)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dbeta": np.zeros(H), "dM0": np.zeros((B, H, d_key, d_value)), "dz0": np.zeros((B, H, d_key))}
    for b in range(B):
        for h in range(H):
            Ms, zs = [M_init[b, h].copy()], [z_init[b, h].copy()]
            for s in range(S):
                rows = slice(s * N, (s + 1) * N)
                first = (segments_done + s) == 0
                Mn, zn = ref.memory_update(k[b, h, rows], v[b, h, rows], Ms[-1], zs[-1], rule, first)
                Ms.append(Mn)
                zs.append(zn)
            gM = np.zeros((d_key, d_value)) if dM is None else np.array(dM[b, h], dtype=np.float64)
            gz = np.zeros(d_key) if dz is None else np.array(dz[b, h], dtype=np.float64)
            for s in reversed(range(S)):
                rows = slice(s * N, (s + 1) * N)
                first = (segments_done + s) == 0
                dq_s, dk_s, dv_s, db, gM, gz = segment_backward(
                    q[b, h, rows], k[b, h, rows], v[b, h, rows], Ms[s], zs[s], beta[h], rule, first, sc,
                    dA[b, h, rows], gM, gz)
                out["dq"][b, h, rows] = dq_s
                out["dk"][b, h, rows] = dk_s
                out["dv"][b, h, rows] = dv_s
                out["dbeta"][h] += db
            out["dM0"][b, h] = gM
            out["dz0"][b, h] = gz
    return out

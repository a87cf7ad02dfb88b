"""Float64 CPU oracle for causal kernel linear attention.

TEST INFRASTRUCTURE ONLY, like ``infini_ref`` (imported by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg, never by the
product path, sharing no code with it).

Definition (page "第24章 Sparse与Infinite Attention", section 24.4, kernelised
linear attention): with the non-negative feature map phi = ELU + 1 (the same
sigma as the Infini-attention memory), each query i of one head reads the
prefix states over the keys j <= i (the query's own key included)
    S_i = S_0 + sum_{j <= i} phi(k_j) v_j^T,   Z_i = Z_0 + sum_{j <= i} phi(k_j),
    O_i = phi(q_i)^T S_i / (phi(q_i)^T Z_i),
where (S_0, Z_0) is the state carried in from earlier tokens of the stream (zero
at its start).  Here the prefix states are cumulative sums over the tokens in
their order; the test pins this against the explicit lower-triangular form
(phi(Q) phi(K)^T masked to j <= i, times V, over its row sums), single-token and
split-stream cases, and the Infini-attention linear memory update.
"""

from __future__ import annotations

import numpy as np

from oracle import infini_ref as ref


def causal_kernel_linear_attention(q, k, v, S0=None, Z0=None):
    """q, k: [B, H, L, d_key]; v: [B, H, L, d_value]; S0 [B, H, d_key, d_value] and
    Z0 [B, H, d_key] (zeros when omitted).  Returns a dict with O [B, H, L, d_value]
    and the final S, Z."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    S_in = np.zeros((B, H, dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Z_in = np.zeros((B, H, dk)) if Z0 is None else np.asarray(Z0, dtype=np.float64)
    O = np.zeros((B, H, L, dv))
    S_out = np.zeros((B, H, dk, dv))
    Z_out = np.zeros((B, H, dk))
    for b in range(B):
        for h in range(H):
            fq, fk = ref.sigma(q[b, h]), ref.sigma(k[b, h])
            S = S_in[b, h] + np.cumsum(fk[:, :, None] * v[b, h][:, None, :], axis=0)   # S_i for every i
            Z = Z_in[b, h] + np.cumsum(fk, axis=0)
            num = np.einsum("ic,icd->id", fq, S)
            den = np.einsum("ic,ic->i", fq, Z)
            O[b, h] = num / den[:, None]
            S_out[b, h], Z_out[b, h] = S[-1], Z[-1]
    return {"O": O, "S": S_out, "Z": Z_out}

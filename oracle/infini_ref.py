"""Float64 CPU oracle for the Infini-attention segment forward pass.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py`` and by
nothing else.  The product path (the HIP library and its Python binding) never
imports, calls or links it, and it shares no code with that path: every step
below is written out from the equations of the source pages in plain numpy
float64, in the pages' order, without blocking, fusion or reordering.

Source: "Leave No Context Behind: Efficient Infinite Context Transformers with
Infini-attention" (Munkhdalai, Faruqui, Golovnev, arXiv 2404.07143), as quoted
and restated on the five pages of the reference text:

* page "精读笔记：Infini-attention" (llm-papers-study close-reading notes),
  sections 3.1 (scaled dot-product attention), 3.3 (memory retrieval),
  3.4 (memory update, linear and Linear+Delta), 3.5 (long-term context
  injection / gate), 3.6 (multi-head memories), 3.7 (Table 1), 3.8 (forward
  pseudo-code);
* page "忘记遗忘：解锁无限上下文的 Infini-attention" (CSDN), section 2.1, whose
  LaTeX gives the delta-rule fraction without ambiguity;
* page "第24章 Sparse与Infinite Attention" (waylandz.com), sections 24.4
  (kernel linear attention, sigma = ELU + 1) and 24.5 (one head, one segment:
  read M_{s-1}, z_{s-1} first, write M_s, z_s after the output).

Readings taken where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):

* scale: 1/sqrt(d_key) by default (the per-head key width; the pages write
  sqrt(d_model) in section 3.1 and sqrt(d) in section 3.8, and the chapter-24
  code uses the SDPA default 1/sqrt(d_key));
* mask: causal with the diagonal, inside the current segment only;
* sigma(x) = ELU(x; alpha=1) + 1, evaluated as x + 1 for x > 0 and exp(x)
  otherwise (same function, no (e^x - 1) + 1 cancellation);
* first segment after init or reset: A_mem = 0 and the delta correction is 0,
  so the first delta update equals the linear one; "first" is decided by the
  segment counter, not by testing z;
* a zero retrieval denominator (only possible with no stored key) yields a zero
  row; there is no clamp otherwise;
* the delta correction is segment-batched: every token of segment s reads the
  same M_{s-1} and z_{s-1}; z is updated exactly as in the linear rule;
* the gate is g * A_mem + (1 - g) * A_dot with g = sigmoid(beta_h), one beta per
  head shared over the batch, applied in every segment including the first;
* the local softmax's log-normaliser (``local_log_normaliser``, what a training
  forward keeps for the backward) is reported in base 2: log2 of the causal
  denominator of section 3.1, so the probabilities are 2^(scale q.k log2 e - lse);
* streaming (the pages' "streaming inference", abstract of the close-reading
  page and point 4 of the key-idea list of the CSDN page): a token that arrives
  before its segment is complete attends causally to the tokens of its segment
  that have arrived (itself included) and reads the memory as of the segment's
  start; the segment is folded into (M, z) once its N-th token has arrived.
  Because the local attention is causal, this gives every token the output it
  has when the segment is processed whole.

Parity status per function (see the pins in ``tests/test_oracle_pins.py``):
every function here is pinned by at least one closed form, invariant, special
case or library routine, except the delta rule for s >= 2 with general V,
which is pinned only through its special cases (delta = linear in the first
segment, zero update when V equals the retrieved value, zero update for a
re-written single pair, equality with the linear rule when all earlier V are
zero, and affinity in V) and by its matrix form (I - A) M + sigma(K)^T V, a
second computation of the same equation: beyond those its parity is unpinned.
"""

from __future__ import annotations

import math

import numpy as np

RULE_LINEAR = "linear"
RULE_DELTA = "delta"


def default_scale(d_key: int, scale: float | None = None) -> float:
    """Softmax scale: 1/sqrt(d_key) unless a positive scale is given.

    Page "精读笔记" section 3.1 (A_dot equation) divides the scores by a square
    root of the model width; the chapter-24 page's code (section 24.5) uses the
    SDPA default, which is 1/sqrt of the per-head key width."""
    if scale is not None and scale > 0:
        return float(scale)
    return 1.0 / math.sqrt(d_key)


def sigma(x: np.ndarray) -> np.ndarray:
    """ELU(alpha=1) + 1, the element-wise feature map of section 3.3 ("ELU + 1")
    of the close-reading page and section 24.4 of the chapter-24 page."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def causal_mask(n: int) -> np.ndarray:
    """Boolean [n, n] mask, True where key j may be seen by query i (j <= i).

    The local attention is causal inside the segment (close-reading page,
    section 3.8 step 2; chapter-24 page section 24.5 uses is_causal=True)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return j <= i


def local_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """A_dot = softmax(scale * q k^T, causal) v for one head and one segment.

    Close-reading page, section 3.1 (A_dot equation) with the causal mask of
    section 3.8 step 2.  q, k: [n, d_key]; v: [n, d_value]; float64."""
    n = q.shape[0]
    scores = scale * (q @ k.T)
    scores = np.where(causal_mask(n), scores, -np.inf)
    row_max = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - row_max)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def local_log_normaliser(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Per query row i of one segment, the base-2 logarithm of the causal softmax
    denominator of A_dot: log2 of the sum over keys j <= i of exp(scale q_i.k_j)
    (close-reading page, section 3.1, with the causal mask of section 3.8 step 2).
    In base 2 the row's probabilities are 2^(scale q_i.k_j log2(e) - lse_i).
    q, k: [n, d_key]; returns [n], float64."""
    n = q.shape[0]
    scores = scale * (q @ k.T)
    scores = np.where(causal_mask(n), scores, -np.inf)
    row_max = scores.max(axis=1)
    natural = row_max + np.log(np.exp(scores - row_max[:, None]).sum(axis=1))
    return natural / math.log(2.0)


def log_normalisers(q, k, segment_len: int, scale=None) -> np.ndarray:
    """local_log_normaliser of every query row of a stream, segment by segment
    (each segment attends only to itself): q, k [B, H, L, d_key] -> [B, H, L]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, L, dk = q.shape
    sc = default_scale(dk, scale)
    out = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            for s0 in range(0, L, segment_len):
                rows = slice(s0, s0 + segment_len)
                out[b, h, rows] = local_log_normaliser(q[b, h, rows], k[b, h, rows], sc)
    return out


def prefix_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, offset: int,
                            scale: float) -> np.ndarray:
    """A_dot for queries that sit at positions offset, offset + 1, ... of a segment
    whose first offset + len(q) keys and values are k, v: query i sees keys
    j <= offset + i (close-reading page section 3.1 with the causal mask of
    section 3.8 step 2, for a segment that has not received all its tokens)."""
    n = q.shape[0]
    scores = scale * (q @ k.T)
    visible = np.arange(k.shape[0])[None, :] <= offset + np.arange(n)[:, None]
    scores = np.where(visible, scores, -np.inf)
    row_max = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - row_max)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def memory_retrieval(q: np.ndarray, M: np.ndarray, z: np.ndarray, first: bool) -> np.ndarray:
    """A_mem = sigma(q) M_{s-1} / (sigma(q) z_{s-1}), row-normalised.

    Close-reading page, section 3.3 (memory retrieval equation).  In the first
    segment the memory is empty (M_0 = 0, z_0 = 0) and A_mem is defined as 0."""
    n, d_value = q.shape[0], M.shape[1]
    if first:
        return np.zeros((n, d_value))
    fq = sigma(q)
    numerator = fq @ M
    denominator = fq @ z
    out = np.zeros((n, d_value))
    ok = denominator > 0.0
    out[ok] = numerator[ok] / denominator[ok, None]
    return out


def gate(beta: float, a_mem: np.ndarray, a_dot: np.ndarray) -> np.ndarray:
    """A = sigmoid(beta) * A_mem + (1 - sigmoid(beta)) * A_dot.

    Close-reading page, section 3.5 (long-term context injection)."""
    beta = float(beta)
    if beta == math.inf:
        g = 1.0
    elif beta == -math.inf:
        g = 0.0
    else:
        g = 1.0 / (1.0 + math.exp(-beta))
    return g * a_mem + (1.0 - g) * a_dot


def update_linear(k: np.ndarray, v: np.ndarray, M: np.ndarray, z: np.ndarray):
    """Linear rule: M_s = M_{s-1} + sigma(K)^T V and z_s = z_{s-1} + sum_t sigma(K_t).

    Close-reading page, section 3.4 (memory update equations)."""
    fk = sigma(k)
    return M + fk.T @ v, z + fk.sum(axis=0)


def delta_correction(k: np.ndarray, M: np.ndarray, z: np.ndarray, first: bool) -> np.ndarray:
    """The value the memory already holds for each key:
    sigma(K) M_{s-1} / (sigma(K) z_{s-1}), row-wise; 0 in the first segment.

    CSDN page section 2.1 (the delta fraction); close-reading page section 3.4."""
    if first:
        return np.zeros((k.shape[0], M.shape[1]))
    fk = sigma(k)
    numerator = fk @ M
    denominator = fk @ z
    out = np.zeros_like(numerator)
    ok = denominator > 0.0
    out[ok] = numerator[ok] / denominator[ok, None]
    return out


def update_delta(k: np.ndarray, v: np.ndarray, M: np.ndarray, z: np.ndarray, first: bool):
    """Linear+Delta rule: M_s = M_{s-1} + sigma(K)^T (V - sigma(K) M_{s-1} / (sigma(K) z_{s-1})),
    with z updated as in the linear rule.

    Close-reading page section 3.4 (second equation and the sentence after it);
    CSDN page section 2.1."""
    fk = sigma(k)
    residual = v - delta_correction(k, M, z, first)
    return M + fk.T @ residual, z + fk.sum(axis=0)


def segment_forward(q, k, v, M, z, beta, rule, first, scale):
    """One head, one segment, in the order of the chapter-24 page section 24.5
    and the close-reading page section 3.8: retrieve from (M_{s-1}, z_{s-1}),
    local causal attention, gate, then update to (M_s, z_s).

    Returns (A, M_s, z_s, A_dot, A_mem)."""
    a_mem = memory_retrieval(q, M, z, first)
    a_dot = local_causal_attention(q, k, v, scale)
    a = gate(beta, a_mem, a_dot)
    if rule == RULE_LINEAR:
        M_new, z_new = update_linear(k, v, M, z)
    elif rule == RULE_DELTA:
        M_new, z_new = update_delta(k, v, M, z, first)
    else:
        raise ValueError(f"unknown rule {rule!r}")
    return a, M_new, z_new, a_dot, a_mem


def memory_update(k, v, M, z, rule, first):
    """The state step alone (no attention), for memory-only walks over long streams."""
    if rule == RULE_LINEAR:
        return update_linear(k, v, M, z)
    if rule == RULE_DELTA:
        return update_delta(k, v, M, z, first)
    raise ValueError(f"unknown rule {rule!r}")


def forward_sequence(q, k, v, beta, rule, segment_len, M0=None, z0=None,
                     segments_done=0, scale=None, keep_parts=False):
    """Stream all segments of every (batch, head) in order.

    q, k: [B, H, L, d_key]; v: [B, H, L, d_value]; beta: [H]; L a multiple of
    segment_len.  M0: [B, H, d_key, d_value], z0: [B, H, d_key] (zeros when
    omitted).  ``segments_done`` counts segments already folded into (M0, z0):
    when it is 0 the first segment reads an empty memory.

    Multi-head layout follows the close-reading page section 3.6: one memory per
    head, heads independent.  Returns a dict with A [B, H, L, d_value], the final
    M and z, the new segment count and, if ``keep_parts``, A_dot and A_mem."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d_key = q.shape
    d_value = v.shape[-1]
    if L % segment_len != 0:
        raise ValueError("sequence length must be a multiple of the segment length")
    S = L // segment_len
    sc = default_scale(d_key, scale)
    M = np.zeros((B, H, d_key, d_value)) if M0 is None else np.array(M0, dtype=np.float64)
    z = np.zeros((B, H, d_key)) if z0 is None else np.array(z0, dtype=np.float64)
    A = np.zeros((B, H, L, d_value))
    A_dot = np.zeros_like(A) if keep_parts else None
    A_mem = np.zeros_like(A) if keep_parts else None
    for b in range(B):
        for h in range(H):
            for s in range(S):
                rows = slice(s * segment_len, (s + 1) * segment_len)
                first = (segments_done + s) == 0
                a, M[b, h], z[b, h], ad, am = segment_forward(
                    q[b, h, rows], k[b, h, rows], v[b, h, rows], M[b, h], z[b, h],
                    beta[h], rule, first, sc)
                A[b, h, rows] = a
                if keep_parts:
                    A_dot[b, h, rows] = ad
                    A_mem[b, h, rows] = am
    out = {"A": A, "M": M, "z": z, "segments_done": segments_done + S}
    if keep_parts:
        out["A_dot"] = A_dot
        out["A_mem"] = A_mem
    return out


def forward_stream(q, k, v, beta, rule, segment_len, M0=None, z0=None, segments_done=0,
                   open_k=None, open_v=None, scale=None):
    """Append T tokens per (batch, head) to a stream whose current segment already
    holds the keys and values open_k, open_v ([B, H, f, d], f < segment_len; none
    when omitted).  Each token is answered with the segment it falls in as it
    stands when the token arrives (streaming reading in the module notes): local
    causal attention over the segment's tokens up to itself, retrieval from the
    memory as of the segment's start, gate; a segment is folded into (M, z) when
    its last token arrives.

    q, k: [B, H, T, d_key]; v: [B, H, T, d_value]; T >= 1 and any length.  Returns
    a dict with A [B, H, T, d_value], the final M, z, segment count and the keys
    and values of the segment left open (possibly empty)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, d_key = q.shape
    d_value = v.shape[-1]
    N = segment_len
    sc = default_scale(d_key, scale)
    M = np.zeros((B, H, d_key, d_value)) if M0 is None else np.array(M0, dtype=np.float64)
    z = np.zeros((B, H, d_key)) if z0 is None else np.array(z0, dtype=np.float64)
    f0 = 0 if open_k is None else np.asarray(open_k).shape[2]
    if f0 >= N:
        raise ValueError("the open segment must hold fewer than segment_len tokens")
    A = np.zeros((B, H, T, d_value))
    f_end = (f0 + T) % N                      # tokens left in the open segment
    open_k_out = np.zeros((B, H, f_end, d_key))
    open_v_out = np.zeros((B, H, f_end, d_value))
    done = segments_done
    for b in range(B):
        for h in range(H):
            seg_k = np.zeros((0, d_key)) if f0 == 0 else np.asarray(open_k[b, h], dtype=np.float64)
            seg_v = np.zeros((0, d_value)) if f0 == 0 else np.asarray(open_v[b, h], dtype=np.float64)
            done = segments_done
            pos = 0
            while pos < T:
                f = seg_k.shape[0]
                m = min(N - f, T - pos)
                new = slice(pos, pos + m)
                seg_k = np.concatenate([seg_k, k[b, h, new]])
                seg_v = np.concatenate([seg_v, v[b, h, new]])
                first = done == 0
                a_mem = memory_retrieval(q[b, h, new], M[b, h], z[b, h], first)
                a_dot = prefix_causal_attention(q[b, h, new], seg_k, seg_v, f, sc)
                A[b, h, new] = gate(beta[h], a_mem, a_dot)
                if f + m == N:
                    M[b, h], z[b, h] = memory_update(seg_k, seg_v, M[b, h], z[b, h], rule, first)
                    seg_k, seg_v = np.zeros((0, d_key)), np.zeros((0, d_value))
                    done += 1
                pos += m
            open_k_out[b, h] = seg_k
            open_v_out[b, h] = seg_v
    return {"A": A, "M": M, "z": z, "segments_done": done, "open_k": open_k_out, "open_v": open_v_out}


def state_floats_per_head(d_key: int, d_value: int) -> int:
    """Size of the compressive state of one head: d_key * d_value for M plus d_key
    for z (close-reading page section 3.7, Table 1: d_key x (d_value + 1))."""
    return d_key * d_value + d_key

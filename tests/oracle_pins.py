"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError (or
any exception) when the oracle disagrees with a closed form, an invariant, a
special case that reduces to a library routine, or a value printed on the
source pages.  ``test_oracle_pins.py`` runs them against the real oracle and
``test_oracle_mutants.py`` checks that plausible mistakes planted into the
oracle make at least one of them fail.

Independent ground truth used here: torch's ``scaled_dot_product_attention``
and ``elu`` on CPU in float64, scipy's ``expit``, the pair-count table of
section 24.1.1 of the chapter-24 page (tests/golden/causal_pairs.txt), and
closed forms derived from the equations (running means, single stored pairs,
fixed points of the delta rule).
"""

from __future__ import annotations

import math
import os

import numpy as np
import torch
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _randn(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _phi(x):
    """sigma = ELU + 1 computed by torch, independent of the oracle's own sigma."""
    return torch.nn.functional.elu(torch.from_numpy(np.asarray(x, dtype=np.float64)), alpha=1.0).numpy() + 1.0


def _sdpa(q, k, v):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)[0, 0].numpy()


def _stream(seed, B, H, S, N, dk, dv, scale=1.0):
    q = _randn(seed, B, H, S * N, dk, scale=scale)
    k = _randn(seed + 1, B, H, S * N, dk, scale=scale)
    v = _randn(seed + 2, B, H, S * N, dv, scale=scale)
    return q, k, v


# ---------------------------------------------------------------- feature map

def pin_sigma_is_elu_plus_one(o):
    """sigma = ELU(alpha=1) + 1 (close-reading page section 3.3; chapter-24 page
    section 24.4), against torch's elu; positive everywhere; sigma(0) = 1."""
    x = np.concatenate([np.linspace(-30, 30, 6001), [0.0, -0.0, 1e-300, -1e-300]])
    got = o.sigma(x)
    # torch evaluates (e^x - 1) + 1 for x < 0, which loses up to one ulp of 1.0
    assert np.allclose(got, _phi(x), rtol=1e-15, atol=4.5e-16)
    neg = x < 0
    assert np.allclose(got[neg], np.exp(x[neg]), rtol=1e-15, atol=0.0)
    assert np.all(got > 0.0)
    assert o.sigma(np.array([0.0]))[0] == 1.0


# ---------------------------------------------------------- local attention

def pin_local_attention_is_causal_sdpa(o):
    """A_dot of one segment equals torch's causal SDPA with the default scale
    1/sqrt(d_key) (chapter-24 page section 24.5 uses exactly that call)."""
    for seed, n, dk, dv in [(1, 1, 4, 3), (2, 7, 8, 5), (3, 16, 16, 16), (4, 33, 8, 12)]:
        q, k, v = _randn(seed, n, dk), _randn(seed + 10, n, dk), _randn(seed + 20, n, dv)
        got = o.local_causal_attention(q, k, v, o.default_scale(dk))
        assert np.allclose(got, _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


def pin_zero_query_gives_running_mean(o):
    """With q = 0 every allowed score is equal, so row i of A_dot is the mean of
    v_0..v_i: pins the mask (diagonal included, no future key) and the
    normalisation without any library call."""
    n, dk, dv = 12, 6, 5
    q = np.zeros((n, dk))
    k, v = _randn(5, n, dk), _randn(6, n, dv)
    got = o.local_causal_attention(q, k, v, o.default_scale(dk))
    want = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(got, want, rtol=1e-13, atol=1e-14)


def pin_causal_pair_counts(o):
    """The mask admits N(N+1)/2 of N^2 pairs: the values printed in the table of
    section 24.1.1 of the chapter-24 page (tests/golden/causal_pairs.txt)."""
    rows = []
    with open(os.path.join(GOLDEN, "causal_pairs.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(tuple(int(x) for x in line.split()))
    assert len(rows) == 4
    for n, dense, causal in rows:
        if n <= 4096:
            m = o.causal_mask(n)
            assert m.size == dense
            assert int(m.sum()) == causal


def pin_each_segment_attends_only_to_itself(o):
    """With beta = -inf the streamed output of every segment equals causal SDPA
    over that segment alone (local attention discards earlier segments; page 3,
    method section; chapter-24 page section 24.5)."""
    B, H, S, N, dk, dv = 1, 2, 3, 5, 4, 6
    q, k, v = _stream(30, B, H, S, N, dk, dv)
    res = o.forward_sequence(q, k, v, np.array([-np.inf, -np.inf]), o.RULE_LINEAR, N)
    for h in range(H):
        for s in range(S):
            r = slice(s * N, (s + 1) * N)
            assert np.allclose(res["A"][0, h, r], _sdpa(q[0, h, r], k[0, h, r], v[0, h, r]),
                               rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ memory

def pin_linear_memory_is_order_free_sum(o):
    """Linear rule: the final M equals sigma(K_all)^T V_all, whatever the order of
    the segments, and z equals the column sums of sigma(K_all) (close-reading
    page section 3.4: M_s = M_{s-1} + sigma(K)^T V, z_s = z_{s-1} + sum sigma(K_t))."""
    B, H, S, N, dk, dv = 2, 2, 5, 4, 3, 7
    q, k, v = _stream(40, B, H, S, N, dk, dv)
    beta = np.array([0.3, -0.7])
    res = o.forward_sequence(q, k, v, beta, o.RULE_LINEAR, N)
    fk = _phi(k)
    want_M = np.einsum("bhtk,bhtv->bhkv", fk, v)
    assert np.allclose(res["M"], want_M, rtol=1e-12, atol=1e-12)
    assert np.allclose(res["z"], fk.sum(axis=2), rtol=1e-13, atol=0)
    perm = [3, 0, 4, 2, 1]
    idx = np.concatenate([np.arange(p * N, (p + 1) * N) for p in perm])
    res_p = o.forward_sequence(q[:, :, idx], k[:, :, idx], v[:, :, idx], beta, o.RULE_LINEAR, N)
    assert np.allclose(res_p["M"], res["M"], rtol=1e-12, atol=1e-12)


def pin_z_is_column_sum_for_both_rules(o):
    """z tracks the same sum of sigma(K) under both rules (close-reading page
    section 3.4, the sentence after the delta equation)."""
    B, H, S, N, dk, dv = 1, 3, 4, 6, 5, 4
    q, k, v = _stream(50, B, H, S, N, dk, dv)
    for rule in (o.RULE_LINEAR, o.RULE_DELTA):
        res = o.forward_sequence(q, k, v, np.zeros(H), rule, N)
        assert np.allclose(res["z"], _phi(k).sum(axis=2), rtol=1e-13, atol=0)


def pin_single_stored_pair_retrieves_its_value(o):
    """After storing one pair (k1, v1) the retrieval returns v1 for every query:
    (sigma(q).sigma(k1)) v1 / (sigma(q).sigma(k1)) (close-reading page section 3.3).
    With beta = +inf the output is exactly A_mem (section 3.5)."""
    dk, dv = 6, 4
    k1, v1 = _randn(60, 1, dk), _randn(61, 1, dv)
    q = _randn(62, 2, dk) * 3.0
    qq = np.concatenate([_randn(63, 1, dk), q[1:]])[None, None]
    kk = np.concatenate([k1, _randn(64, 1, dk)])[None, None]
    vv = np.concatenate([v1, _randn(65, 1, dv)])[None, None]
    res = o.forward_sequence(qq, kk, vv, np.array([np.inf]), o.RULE_LINEAR, 1, keep_parts=True)
    assert np.allclose(res["A"][0, 0, 1], v1[0], rtol=1e-13, atol=1e-14)
    assert np.array_equal(res["A"][0, 0, 0], np.zeros(dv))  # first segment reads an empty memory


def pin_retrieval_is_block_causal_kernel_attention(o):
    """Linear rule: A_mem of a token in segment s equals kernel linear attention
    (chapter-24 page section 24.4, sim = sigma(q).sigma(k)) over all tokens of
    segments 0..s-1, built quadratically; the first segment retrieves 0."""
    B, H, S, N, dk, dv = 1, 2, 4, 3, 5, 6
    q, k, v = _stream(70, B, H, S, N, dk, dv)
    res = o.forward_sequence(q, k, v, np.array([np.inf, np.inf]), o.RULE_LINEAR, N)
    for h in range(H):
        fq, fk = _phi(q[0, h]), _phi(k[0, h])
        for t in range(S * N):
            s = t // N
            if s == 0:
                assert np.array_equal(res["A"][0, h, t], np.zeros(dv))
                continue
            w = np.array([fq[t] @ fk[j] for j in range(s * N)])
            want = (w[:, None] * v[0, h, :s * N]).sum(axis=0) / w.sum()
            assert np.allclose(res["A"][0, h, t], want, rtol=1e-12, atol=1e-13)


def pin_delta_keeps_memory_when_binding_exists(o):
    """Delta rule: if V equals what the memory already returns for K, M is left
    unchanged (close-reading page section 3.4, sentence after the delta
    equation).  The target values come from the retrieval function, which is
    pinned on its own."""
    dk, dv, N = 5, 4, 7
    k0, v0 = _randn(80, N, dk), _randn(81, N, dv)
    M1, z1 = o.update_delta(k0, v0, np.zeros((dk, dv)), np.zeros(dk), True)
    k1 = _randn(82, N, dk)
    v1 = o.memory_retrieval(k1, M1, z1, False)
    M2, z2 = o.update_delta(k1, v1, M1, z1, False)
    assert np.allclose(M2, M1, rtol=1e-13, atol=1e-13 * np.abs(M1).max())
    assert np.allclose(z2, z1 + _phi(k1).sum(axis=0), rtol=1e-14, atol=0)


def pin_delta_rewrite_of_single_pair(o):
    """Delta rule: storing (k1, v1) and then the same pair again leaves M as it
    was and doubles z."""
    dk, dv = 6, 3
    k1, v1 = _randn(90, 1, dk), _randn(91, 1, dv)
    kk = np.concatenate([k1, k1])[None, None]
    vv = np.concatenate([v1, v1])[None, None]
    qq = _randn(92, 1, 1, 2, dk)
    one = o.forward_sequence(qq[:, :, :1], kk[:, :, :1], vv[:, :, :1], np.zeros(1), o.RULE_DELTA, 1)
    two = o.forward_sequence(qq, kk, vv, np.zeros(1), o.RULE_DELTA, 1)
    assert np.allclose(two["M"], one["M"], rtol=1e-13, atol=1e-14)
    assert np.allclose(two["z"], 2.0 * one["z"], rtol=1e-15, atol=0)
    assert np.allclose(one["M"][0, 0], np.outer(_phi(k1[0]), v1[0]), rtol=1e-14, atol=0)


def pin_delta_equals_linear_in_first_segment(o):
    """With an empty memory there is nothing to subtract: the first delta update
    equals the linear one."""
    B, H, S, N, dk, dv = 2, 2, 1, 6, 4, 5
    q, k, v = _stream(100, B, H, S, N, dk, dv)
    lin = o.forward_sequence(q, k, v, np.zeros(H), o.RULE_LINEAR, N)
    dlt = o.forward_sequence(q, k, v, np.zeros(H), o.RULE_DELTA, N)
    assert np.array_equal(lin["M"], dlt["M"]) and np.array_equal(lin["z"], dlt["z"])
    assert np.allclose(dlt["M"], np.einsum("bhtk,bhtv->bhkv", _phi(k), v), rtol=1e-13, atol=1e-14)


def pin_delta_equals_linear_after_zero_values(o):
    """If every earlier value was 0 then M = 0 and z > 0, so the retrieved value is
    0 and the delta update of the next segment equals the linear one."""
    B, H, S, N, dk, dv = 1, 2, 3, 4, 5, 3
    q, k, v = _stream(110, B, H, S, N, dk, dv)
    v[:, :, : (S - 1) * N] = 0.0
    lin = o.forward_sequence(q, k, v, np.zeros(H), o.RULE_LINEAR, N)
    dlt = o.forward_sequence(q, k, v, np.zeros(H), o.RULE_DELTA, N)
    assert np.allclose(dlt["M"], lin["M"], rtol=1e-14, atol=1e-15)
    last = slice((S - 1) * N, S * N)
    assert np.allclose(lin["M"], np.einsum("bhtk,bhtv->bhkv", _phi(k[:, :, last]), v[:, :, last]),
                       rtol=1e-13, atol=1e-14)


def pin_delta_update_is_affine_in_values(o):
    """For fixed (M_{s-1}, z_{s-1}, K) the delta update is affine in V with slope
    sigma(K)^T: M_s(V) - M_s(V') = sigma(K)^T (V - V')."""
    dk, dv, N = 4, 6, 5
    M0 = _randn(120, dk, dv)
    z0 = np.abs(_randn(121, dk)) + 0.5
    k = _randn(122, N, dk)
    v, v2 = _randn(123, N, dv), _randn(124, N, dv)
    Ma, _ = o.update_delta(k, v, M0, z0, False)
    Mb, _ = o.update_delta(k, v2, M0, z0, False)
    assert np.allclose(Ma - Mb, _phi(k).T @ (v - v2), rtol=1e-12, atol=1e-12)
    # and with V' = 0 the remaining part is the memory's own read-back, which is
    # independent of V: M_s(0) - M_{s-1} does not depend on the values.
    M0b, _ = o.update_delta(k, np.zeros((N, dv)), M0, z0, False)
    M0c, _ = o.update_delta(k, np.zeros((N, dv)), M0, z0, False)
    assert np.array_equal(M0b, M0c)


# -------------------------------------------------------------------- gate

def pin_gate_limits_and_mix(o):
    """beta -> -inf gives pure local attention and beta -> +inf pure retrieval,
    exactly; a finite beta mixes with weight expit(beta) on the memory
    (close-reading page section 3.5 and the remark on the learned gates in its
    section 4.4)."""
    B, H, S, N, dk, dv = 1, 3, 3, 4, 5, 6
    q, k, v = _stream(130, B, H, S, N, dk, dv)
    for rule in (o.RULE_LINEAR, o.RULE_DELTA):
        res = o.forward_sequence(q, k, v, np.array([-np.inf, np.inf, 1.3]), rule, N, keep_parts=True)
        assert np.array_equal(res["A"][0, 0], res["A_dot"][0, 0])
        assert np.array_equal(res["A"][0, 1], res["A_mem"][0, 1])
        g = expit(1.3)
        assert np.allclose(res["A"][0, 2], g * res["A_mem"][0, 2] + (1 - g) * res["A_dot"][0, 2],
                           rtol=1e-14, atol=1e-15)
    x, y = _randn(131, 3, 2), _randn(132, 3, 2)
    for beta in (-4.0, -0.5, 0.0, 2.0, 30.0):
        assert np.allclose(o.gate(beta, x, y), expit(beta) * x + (1 - expit(beta)) * y, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------- streaming

def pin_stream_equals_chained_segments(o):
    """Processing L tokens at once equals feeding the segments one at a time with
    the state carried over (the recurrence of close-reading page section 3.4);
    a stream that resumes from a saved state equals an uninterrupted one."""
    B, H, S, N, dk, dv = 2, 2, 4, 3, 4, 4
    q, k, v = _stream(140, B, H, S, N, dk, dv)
    beta = np.array([0.2, -1.1])
    for rule in (o.RULE_LINEAR, o.RULE_DELTA):
        whole = o.forward_sequence(q, k, v, beta, rule, N)
        M = z = None
        done = 0
        for s in range(S):
            r = slice(s * N, (s + 1) * N)
            part = o.forward_sequence(q[:, :, r], k[:, :, r], v[:, :, r], beta, rule, N,
                                      M0=M, z0=z, segments_done=done)
            assert np.allclose(part["A"], whole["A"][:, :, r], rtol=1e-13, atol=1e-14)
            M, z, done = part["M"], part["z"], part["segments_done"]
        assert done == S
        assert np.allclose(M, whole["M"], rtol=1e-13, atol=1e-13)
        assert np.allclose(z, whole["z"], rtol=1e-14, atol=0)


def pin_prefix_attention_is_masked_sdpa(o):
    """Queries at positions f, f + 1, ... of a segment prefix attend to keys j <= f + i:
    torch's scaled_dot_product_attention with that boolean mask."""
    f, m, dk, dv = 5, 4, 3, 2
    q, k, v = _randn(160, m, dk), _randn(161, f + m, dk), _randn(162, f + m, dv)
    mask = np.arange(f + m)[None, :] <= f + np.arange(m)[:, None]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask))
    assert np.allclose(o.prefix_causal_attention(q, k, v, f, 1.0 / math.sqrt(dk)), ref[0, 0].numpy(),
                       rtol=1e-13, atol=1e-14)


def pin_stream_of_whole_segments_equals_forward_sequence(o):
    """Appending whole segments to an empty open segment is forward_sequence (every
    segment completes, so each is processed whole)."""
    B, H, S, N, dk, dv = 1, 2, 3, 4, 3, 3
    q, k, v = _stream(170, B, H, S, N, dk, dv)
    beta = np.array([0.4, -0.7])
    for rule in (o.RULE_LINEAR, o.RULE_DELTA):
        a = o.forward_stream(q, k, v, beta, rule, N)
        b = o.forward_sequence(q, k, v, beta, rule, N)
        assert np.allclose(a["A"], b["A"], rtol=1e-13, atol=1e-14)
        assert np.allclose(a["M"], b["M"], rtol=1e-13, atol=1e-13)
        assert np.allclose(a["z"], b["z"], rtol=1e-14, atol=0)
        assert a["segments_done"] == S and a["open_k"].shape[2] == 0


def pin_stream_outputs_do_not_depend_on_chunking(o):
    """Feeding a ragged stream in chunks of 1, 2, N - 1, N + 2, ... tokens (carrying the
    state and the open segment) gives the outputs, state and open segment of one
    call: the streaming reading makes a token's output a function of the stream
    up to it."""
    B, H, N, dk, dv, T = 1, 2, 4, 3, 2, 23
    q, k, v = (_randn(180 + i, B, H, T, d) for i, d in enumerate((dk, dk, dv)))
    beta = np.array([1.1, -0.3])
    for rule in (o.RULE_LINEAR, o.RULE_DELTA):
        whole = o.forward_stream(q, k, v, beta, rule, N)
        M = z = ok = ov = None
        done, pos, A = 0, 0, []
        for c in (1, 2, 3, 1, 6, 2, 5, 3):
            r = slice(pos, pos + c)
            part = o.forward_stream(q[:, :, r], k[:, :, r], v[:, :, r], beta, rule, N, M0=M, z0=z,
                                    segments_done=done, open_k=ok, open_v=ov)
            A.append(part["A"])
            M, z, done, ok, ov = part["M"], part["z"], part["segments_done"], part["open_k"], part["open_v"]
            pos += c
        assert pos == T and done == whole["segments_done"] == T // N
        assert np.allclose(np.concatenate(A, axis=2), whole["A"], rtol=1e-12, atol=1e-13)
        assert np.allclose(M, whole["M"], rtol=1e-12, atol=1e-12)
        assert np.allclose(ok, whole["open_k"]) and np.allclose(ov, whole["open_v"])
        assert ok.shape[2] == T % N


def pin_open_segment_rows_match_whole_segment(o):
    """The first p tokens of a segment, answered before the rest arrive, get the rows
    they get when the segment is processed whole (the local attention is causal),
    and (M, z) do not change until the segment's last token has arrived."""
    B, H, S, N, dk, dv = 1, 1, 2, 5, 3, 3
    q, k, v = _stream(190, B, H, S, N, dk, dv)
    beta = np.array([0.25])
    for rule in (o.RULE_LINEAR, o.RULE_DELTA):
        whole = o.forward_sequence(q, k, v, beta, rule, N)
        first_seg = o.forward_sequence(q[:, :, :N], k[:, :, :N], v[:, :, :N], beta, rule, N)
        for p in range(1, N):
            r = slice(0, N + p)
            part = o.forward_stream(q[:, :, r], k[:, :, r], v[:, :, r], beta, rule, N)
            assert np.allclose(part["A"], whole["A"][:, :, r], rtol=1e-13, atol=1e-14)
            assert part["segments_done"] == 1
            assert np.array_equal(part["M"], first_seg["M"]) and np.array_equal(part["z"], first_seg["z"])


def pin_state_size_matches_table_1(o):
    """The carried state of one head is d_key x d_value + d_key numbers, for any
    segment count (close-reading page section 3.7, Table 1)."""
    B, H, S, N, dk, dv = 1, 2, 3, 2, 3, 5
    q, k, v = _stream(150, B, H, S, N, dk, dv)
    res = o.forward_sequence(q, k, v, np.zeros(H), o.RULE_DELTA, N)
    per_head = (res["M"].size + res["z"].size) // (B * H)
    assert per_head == dk * (dv + 1) == o.state_floats_per_head(dk, dv)



def pin_delta_matrix_form(o):
    """For any segment with a non-empty memory and general V, the delta update
    equals M_s = (I - A) M_{s-1} + sigma(K)^T V with A = sigma(K)^T diag(1/e) sigma(K),
    e_t = sigma(K_t) . z_{s-1}: the row-wise correction sigma(K)^T (sigma(K) M / e)
    rewritten as one d_key x d_key operator (and A symmetric)."""
    rng = np.random.default_rng(77)
    for n, dk, dv in ((5, 3, 4), (16, 8, 8), (9, 6, 2)):
        k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
        M = rng.standard_normal((dk, dv))
        z = np.abs(rng.standard_normal(dk)) + 0.3
        got, gz = o.update_delta(k, v, M, z, first=False)
        fk = o.sigma(k)
        A = fk.T @ np.diag(1.0 / (fk @ z)) @ fk
        assert np.allclose(A, A.T, rtol=0, atol=1e-13)
        assert np.allclose(got, (np.eye(dk) - A) @ M + fk.T @ v, rtol=1e-12, atol=1e-12)
        assert np.allclose(gz, z + fk.sum(axis=0))

def pin_log_normaliser_of_equal_keys(o):
    """Every key equal: row i sees i + 1 equal scores s, so the base-2
    log-normaliser is s log2(e) + log2(i + 1)."""
    n, d = 9, 4
    q = _randn(61, n, d)
    k = np.tile(_randn(62, 1, d), (n, 1))
    scale = 0.37
    s = scale * (q @ k[0])
    want = s / math.log(2.0) + np.log2(np.arange(1, n + 1))
    got = o.local_log_normaliser(q, k, scale)
    assert np.allclose(got, want, rtol=0, atol=1e-12), (got, want)


def pin_log_normaliser_is_scipy_logsumexp(o):
    """Against scipy's logsumexp over each row's visible keys, in base 2."""
    from scipy.special import logsumexp
    n, d = 12, 5
    q, k = _randn(63, n, d, scale=2.0), _randn(64, n, d, scale=2.0)
    scale = 0.6
    got = o.local_log_normaliser(q, k, scale)
    for i in range(n):
        want = logsumexp(scale * (q[i] @ k[: i + 1].T)) / math.log(2.0)
        assert abs(got[i] - want) < 1e-12, (i, got[i], want)


def pin_log_normaliser_normalises_the_attention(o):
    """The probabilities 2^(scale q.k log2 e - lse) over the visible keys give
    torch's causal SDPA output when applied to V (the default scale of the
    attention), across the segments of a stream."""
    B, H, N, S, d = 1, 2, 6, 2, 4
    q, k, v = (_randn(65 + i, B, H, N * S, d) for i in range(3))
    lse = o.log_normalisers(q, k, N)
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        for s0 in range(0, N * S, N):
            rows = slice(s0, s0 + N)
            qs, ks, vs = q[0, h, rows], k[0, h, rows], v[0, h, rows]
            p = np.exp2(scale * (qs @ ks.T) / math.log(2.0) - lse[0, h, rows][:, None])
            p = np.where(np.tril(np.ones((N, N), bool)), p, 0.0)
            assert np.allclose(p @ vs, _sdpa(qs * math.sqrt(d) * scale, ks, vs), atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]

"""Plausible mistakes planted into the oracle (on the CPU) must each make at least
one pin fail: evidence that the pins constrain every step of the oracle."""

import math

import numpy as np
import pytest

from oracle import infini_ref as o
from tests.oracle_pins import ALL_PINS


def _strict_mask(n):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return j < i


def _scale_model_width(d_key, scale=None):
    return 1.0 / math.sqrt(2 * d_key)


def _elu_without_plus_one(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x, np.exp(np.minimum(x, 0.0)) - 1.0)


def _retrieval_with_raw_query(q, M, z, first):
    if first:
        return np.zeros((q.shape[0], M.shape[1]))
    return (q @ M) / (q @ z)[:, None]


def _retrieval_sum_denominator(q, M, z, first):
    if first:
        return np.zeros((q.shape[0], M.shape[1]))
    return (o.sigma(q) @ M) / z.sum()


def _linear_without_sigma_in_z(k, v, M, z):
    return M + o.sigma(k).T @ v, z + k.sum(axis=0)


def _linear_transposed(k, v, M, z):
    return M + (v.T @ o.sigma(k)).T[::-1], z + o.sigma(k).sum(axis=0)


def _delta_sign_flipped(k, v, M, z, first):
    fk = o.sigma(k)
    return M + fk.T @ (v + o.delta_correction(k, M, z, first)), z + fk.sum(axis=0)


def _delta_unnormalised(k, M, z, first):
    if first:
        return np.zeros((k.shape[0], M.shape[1]))
    return o.sigma(k) @ M


def _delta_with_new_z(k, v, M, z, first):
    fk = o.sigma(k)
    z_new = z + fk.sum(axis=0)
    return M + fk.T @ (v - o.delta_correction(k, M, z_new, False if not first else True)), z_new


def _delta_per_token(k, v, M, z, first):
    fk = o.sigma(k)
    M = M.copy()
    z = z.copy()
    for t in range(k.shape[0]):
        den = fk[t] @ z
        r = (fk[t] @ M) / den if den > 0 else np.zeros(M.shape[1])
        M += np.outer(fk[t], v[t] - r)
        z += fk[t]
    return M, z


def _gate_swapped(beta, a_mem, a_dot):
    g = 1.0 / (1.0 + math.exp(-beta)) if math.isfinite(beta) else (1.0 if beta > 0 else 0.0)
    return g * a_dot + (1.0 - g) * a_mem


def _softmax_over_all_keys(q, k, v, scale):
    n = q.shape[0]
    scores = scale * (q @ k.T)
    p = np.exp(scores - scores.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    p = np.where(o.causal_mask(n), p, 0.0)
    return p @ v


_real_segment_forward = o.segment_forward


def _write_before_read(q, k, v, M, z, beta, rule, first, scale):
    M2, z2 = o.memory_update(k, v, M, z, rule, first)
    a_mem = o.memory_retrieval(q, M2, z2, False)
    a_dot = o.local_causal_attention(q, k, v, scale)
    return o.gate(beta, a_mem, a_dot), M2, z2, a_dot, a_mem


def _prefix_mask_excludes_diagonal(q, k, v, offset, scale):
    scores = scale * (q @ k.T)
    visible = np.arange(k.shape[0])[None, :] < offset + np.arange(q.shape[0])[:, None]
    scores = np.where(visible, scores, -np.inf)
    p = np.exp(scores - scores.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


def _prefix_offset_ignored(q, k, v, offset, scale):
    return _real_prefix(q, k, v, 0, scale)


_real_prefix = o.prefix_causal_attention
_real_stream = o.forward_stream


def _stream_commits_every_call(q, k, v, beta, rule, segment_len, M0=None, z0=None, segments_done=0,
                               open_k=None, open_v=None, scale=None):
    # folds whatever the call brought into the memory, complete segment or not
    res = _real_stream(q, k, v, beta, rule, segment_len, M0, z0, segments_done, open_k, open_v, scale)
    if res["open_k"].shape[2]:
        M, z = res["M"].copy(), res["z"].copy()
        for b in range(M.shape[0]):
            for h in range(M.shape[1]):
                M[b, h], z[b, h] = o.memory_update(res["open_k"][b, h], res["open_v"][b, h], M[b, h], z[b, h],
                                                   rule, res["segments_done"] == 0)
        res = dict(res, M=M, z=z, open_k=res["open_k"][:, :, :0], open_v=res["open_v"][:, :, :0])
    return res


def _log_normaliser_natural(q, k, scale):
    return _real_lse(q, k, scale) * math.log(2.0)


def _log_normaliser_unscaled(q, k, scale):
    return _real_lse(q, k, 1.0)


def _log_normaliser_shifted_row(q, k, scale):
    x = _real_lse(q, k, scale)
    return np.concatenate([x[:1], x[:-1]])


_real_lse = o.local_log_normaliser


MUTANTS = {
    "prefix_mask_excludes_diagonal": ("prefix_causal_attention", _prefix_mask_excludes_diagonal),
    "prefix_offset_ignored": ("prefix_causal_attention", _prefix_offset_ignored),
    "stream_commits_every_call": ("forward_stream", _stream_commits_every_call),
    "mask_excludes_diagonal": ("causal_mask", _strict_mask),
    "scale_uses_model_width": ("default_scale", _scale_model_width),
    "sigma_is_plain_elu": ("sigma", _elu_without_plus_one),
    "retrieval_without_sigma": ("memory_retrieval", _retrieval_with_raw_query),
    "retrieval_wrong_denominator": ("memory_retrieval", _retrieval_sum_denominator),
    "z_sums_raw_keys": ("update_linear", _linear_without_sigma_in_z),
    "linear_binding_rows_permuted": ("update_linear", _linear_transposed),
    "delta_adds_retrieved_value": ("update_delta", _delta_sign_flipped),
    "delta_without_normaliser": ("delta_correction", _delta_unnormalised),
    "delta_reads_updated_z": ("update_delta", _delta_with_new_z),
    "delta_token_by_token": ("update_delta", _delta_per_token),
    "gate_weights_swapped": ("gate", _gate_swapped),
    "softmax_normalised_before_mask": ("local_causal_attention", _softmax_over_all_keys),
    "memory_written_before_read": ("segment_forward", _write_before_read),
    "log_normaliser_in_natural_log": ("local_log_normaliser", _log_normaliser_natural),
    "log_normaliser_without_scale": ("local_log_normaliser", _log_normaliser_unscaled),
    "log_normaliser_of_previous_row": ("local_log_normaliser", _log_normaliser_shifted_row),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(o, attr, bad)
    caught = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(o)
            except Exception:  # noqa: BLE001 - any failure of a pin counts
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"

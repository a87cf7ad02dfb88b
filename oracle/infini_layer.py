"""Float64 CPU oracle for the Infini-attention layer with its projections.

TEST INFRASTRUCTURE ONLY, like ``infini_ref`` (imported by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg, never by the
product path, sharing no code with it).

The steps on either side of the segment forward: the per-head projections
Q = X W_Q, K = X W_K, V = X W_V of the input (close-reading page
"精读笔记：Infini-attention", section 3.1, where the per-head weight matrices map
the model width to d_key and d_value), the segment stream of every head
(``infini_ref.forward_sequence``), then the heads' outputs concatenated and
projected back to the model width with W_O (section 3.6: O = [A^1; ...; A^H] W_O).

Weight layout (the plainest reading of those equations for a fused projection):
``w_qkv`` is [d_model, H (2 d_key + d_value)], its columns the H query heads (d_key
each, head-major), then the H key heads, then the H value heads; ``w_o`` is
[H d_value, d_model], its rows the heads' outputs in head order.  ``x`` is
[B, L, d_model]; the output is [B, L, d_model].

Pins (``tests/test_oracle_layer_pins.py``): a pure-Python loop version of the two
projections on tiny shapes; head-selector weights that reduce the layer to the
per-head stream (checks the head split and the concatenation order); linearity in
W_O; planted mistakes (swapped K/V blocks, heads interleaved instead of head-major,
the concatenation in reverse head order) are each caught.
"""

from __future__ import annotations

import numpy as np

from oracle import infini_ref as ref


def split_heads(qkv: np.ndarray, heads: int, d_key: int, d_value: int):
    """[B, L, H (2 d_key + d_value)] -> q, k [B, H, L, d_key], v [B, H, L, d_value]."""
    B, L, _ = qkv.shape
    hq, hk = heads * d_key, 2 * heads * d_key
    q = qkv[:, :, :hq].reshape(B, L, heads, d_key).transpose(0, 2, 1, 3)
    k = qkv[:, :, hq:hk].reshape(B, L, heads, d_key).transpose(0, 2, 1, 3)
    v = qkv[:, :, hk:].reshape(B, L, heads, d_value).transpose(0, 2, 1, 3)
    return q, k, v


def concat_heads(a: np.ndarray) -> np.ndarray:
    """[B, H, L, d_value] -> [B, L, H d_value] (head h in columns h d_value ...)."""
    B, H, L, dv = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B, L, H * dv)


def layer_forward(x, w_qkv, w_o, beta, rule, segment_len, heads, d_key, d_value, M0=None, z0=None,
                  segments_done=0, scale=None):
    """y = concat_h(segment stream of head h) W_O with q, k, v = x W_QKV split into
    heads, all in float64.  Returns a dict with y, the stream's A, the final M, z
    and the projected q, k, v."""
    x = np.asarray(x, dtype=np.float64)
    qkv = x @ np.asarray(w_qkv, dtype=np.float64)
    q, k, v = split_heads(qkv, heads, d_key, d_value)
    res = ref.forward_sequence(q, k, v, beta, rule, segment_len, M0=M0, z0=z0, segments_done=segments_done,
                               scale=scale)
    y = concat_heads(res["A"]) @ np.asarray(w_o, dtype=np.float64)
    return {"y": y, "A": res["A"], "M": res["M"], "z": res["z"], "q": q, "k": k, "v": v}

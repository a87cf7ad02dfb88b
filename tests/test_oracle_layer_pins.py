"""Pins of the layer oracle (oracle/infini_layer.py), CPU, float64: the projections
against pure-Python loops, head-selector weights that reduce the layer to the
per-head stream, linearity in W_O; planted mistakes must each fail a pin."""

import numpy as np
import pytest

from oracle import infini_layer as ol
from oracle import infini_ref as ref


def _tiny(seed, B=1, L=8, dm=5, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, dm))
    w_qkv = rng.standard_normal((dm, H * (2 * dk + dv))) / np.sqrt(dm)
    w_o = rng.standard_normal((H * dv, dm)) / np.sqrt(H * dv)
    beta = rng.standard_normal(H)
    return x, w_qkv, w_o, beta


def pin_projections_match_loops():
    """q, k, v and y against scalar loops over the projection definitions: q[b,h,t,c]
    = sum_i x[b,t,i] W[i, h dk + c] (K and V from the next column blocks), and
    y[b,t,j] = sum_h sum_c A[b,h,t,c] W_O[h dv + c, j]."""
    B, L, dm, H, dk, dv, N = 1, 8, 5, 2, 3, 2, 4
    x, w_qkv, w_o, beta = _tiny(1, B, L, dm, H, dk, dv)
    r = ol.layer_forward(x, w_qkv, w_o, beta, ref.RULE_LINEAR, N, H, dk, dv)
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for c in range(dk):
                    q = sum(x[b, t, i] * w_qkv[i, h * dk + c] for i in range(dm))
                    k = sum(x[b, t, i] * w_qkv[i, H * dk + h * dk + c] for i in range(dm))
                    assert abs(q - r["q"][b, h, t, c]) < 1e-12 and abs(k - r["k"][b, h, t, c]) < 1e-12
                for c in range(dv):
                    v = sum(x[b, t, i] * w_qkv[i, 2 * H * dk + h * dv + c] for i in range(dm))
                    assert abs(v - r["v"][b, h, t, c]) < 1e-12
    for b in range(B):
        for t in range(L):
            for j in range(dm):
                y = sum(r["A"][b, h, t, c] * w_o[h * dv + c, j] for h in range(H) for c in range(dv))
                assert abs(y - r["y"][b, t, j]) < 1e-12


def pin_head_selectors_reduce_to_the_stream():
    """d_model = H d: W_QKV made of identity blocks makes q = k = v = the head's slice
    of x, and W_O = identity makes y the concatenated heads; the layer then equals
    the per-head stream of those slices."""
    B, L, H, d, N = 2, 12, 3, 4, 4
    rng = np.random.default_rng(2)
    x = rng.standard_normal((B, L, H * d))
    eye = np.eye(H * d)
    w_qkv = np.concatenate([eye, eye, eye], axis=1)
    beta = rng.standard_normal(H)
    r = ol.layer_forward(x, w_qkv, eye, beta, ref.RULE_DELTA, N, H, d, d)
    heads = x.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    want = ref.forward_sequence(heads, heads, heads, beta, ref.RULE_DELTA, N)
    assert np.allclose(r["A"], want["A"], atol=1e-13)
    assert np.allclose(r["y"], want["A"].transpose(0, 2, 1, 3).reshape(B, L, H * d), atol=1e-13)


def pin_output_projection_is_linear():
    B, L, dm, H, dk, dv, N = 1, 8, 6, 2, 3, 2, 4
    x, w_qkv, w_o, beta = _tiny(3, B, L, dm, H, dk, dv)
    w2 = np.random.default_rng(4).standard_normal(w_o.shape)
    y1 = ol.layer_forward(x, w_qkv, w_o, beta, ref.RULE_LINEAR, N, H, dk, dv)["y"]
    y2 = ol.layer_forward(x, w_qkv, w2, beta, ref.RULE_LINEAR, N, H, dk, dv)["y"]
    y3 = ol.layer_forward(x, w_qkv, 2 * w_o - w2, beta, ref.RULE_LINEAR, N, H, dk, dv)["y"]
    assert np.allclose(y3, 2 * y1 - y2, atol=1e-12)


ALL_LAYER_PINS = [pin_projections_match_loops, pin_head_selectors_reduce_to_the_stream,
                  pin_output_projection_is_linear]


@pytest.mark.parametrize("pin", ALL_LAYER_PINS, ids=[p.__name__ for p in ALL_LAYER_PINS])
def test_layer_pin(pin):
    pin()


ORIGINAL_SPLIT = ol.split_heads
ORIGINAL_CONCAT = ol.concat_heads


def _split_kv_swapped(qkv, heads, d_key, d_value):
    q, k, v = ORIGINAL_SPLIT(qkv, heads, d_key, d_value)
    return (q, v, k) if d_key == d_value else (q, k, v[..., ::-1])


def _split_heads_interleaved(qkv, heads, d_key, d_value):
    B, L, _ = qkv.shape
    hq, hk = heads * d_key, 2 * heads * d_key
    q = qkv[:, :, :hq].reshape(B, L, d_key, heads).transpose(0, 3, 1, 2)
    k = qkv[:, :, hq:hk].reshape(B, L, d_key, heads).transpose(0, 3, 1, 2)
    v = qkv[:, :, hk:].reshape(B, L, d_value, heads).transpose(0, 3, 1, 2)
    return q, k, v


def _concat_heads_reversed(a):
    return ORIGINAL_CONCAT(a[:, ::-1])


LAYER_MUTANTS = {
    "kv_blocks_swapped": ("split_heads", _split_kv_swapped),
    "heads_interleaved": ("split_heads", _split_heads_interleaved),
    "concat_reversed": ("concat_heads", _concat_heads_reversed),
}


@pytest.mark.parametrize("name", sorted(LAYER_MUTANTS))
def test_layer_mutant_is_caught(name, monkeypatch):
    attr, fn = LAYER_MUTANTS[name]
    monkeypatch.setattr(ol, attr, fn)
    failed = []
    for pin in ALL_LAYER_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every layer pin"

"""The seeded input generator: determinism, per-tile independence, bf16 rounding
and the planted pair; CPU only."""

import numpy as np
import torch

from compressive_memory_transformer_amd import synthetic as syn


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 3.0e38, 1e-40],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = syn.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_tiles_are_deterministic_and_independent():
    w = syn.WORKLOADS["layer_32k_linear"]
    a = syn.tile(w, syn.K_ID, 0, 3, 5)
    b = syn.tile(w, syn.K_ID, 0, 3, 5)
    c = syn.tile(w, syn.K_ID, 0, 3, 6)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert a.shape == (2048, 128) and a.dtype == np.float32
    assert np.array_equal(syn.round_bf16(a), a)  # already exact in bf16
    assert abs(float(a.std()) - 1 / np.sqrt(128)) < 2e-3


def test_full_tensor_matches_tiles():
    w = syn.custom("t", 7, 2, 3, 16, 32, 3)
    full = syn.full_tensor(w, syn.V_ID)
    bits = syn.full_tensor(w, syn.V_ID, as_bits=True)
    assert full.shape == (2, 3, 96, 16)
    assert np.array_equal(full[1, 2, 32:64], syn.tile(w, syn.V_ID, 1, 2, 1))
    assert np.array_equal(syn.bf16_bits_to_f32(bits), full)


def test_planted_pair_positions():
    w = syn.WORKLOADS["stream_1m_delta"]
    p0, p1, kstar, vstar = syn.planted_pair(w)
    assert 0 <= p0 < w.segment_len and 0 <= p1 < w.segment_len
    k0 = syn.tile(w, syn.K_ID, 0, 5, 0)
    v0 = syn.tile(w, syn.V_ID, 0, 5, 0)
    ql = syn.tile(w, syn.Q_ID, 0, 5, w.segments - 1)
    assert np.array_equal(k0[p0], kstar[5]) and np.array_equal(v0[p0], vstar[5])
    assert np.array_equal(ql[p1], kstar[5])
    assert np.abs(kstar).mean() > 5 * np.abs(k0).mean()  # unscaled against the 1/sqrt(128) background


def test_betas():
    assert syn.betas(syn.WORKLOADS["tiny_f32"]).shape == (2,)
    b = syn.betas(syn.WORKLOADS["wide_500k"])
    assert b.shape == (32,) and b.dtype == np.float32 and np.all(np.abs(b) <= 3.0)

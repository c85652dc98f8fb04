"""Pins for the decode-step oracle (oracle/decode_oracle.py): each part of the
decoder block against a closed form, a special case or brute force."""

import math

import numpy as np
import pytest

from oracle import decode_oracle as D
from oracle import prox_oracle as O
from prox_workloads import bf16_round, bf16_to_f32


def test_rmsnorm_closed_form():
    x = np.array([3.0, -3.0, 3.0, -3.0])
    g = np.array([1.0, 2.0, 0.5, 1.0])
    y = D.rmsnorm(x, g)
    s = 3.0 / math.sqrt(9.0 + D.EPS)
    assert np.allclose(y, np.array([s, -2 * s, 0.5 * s, -s]), rtol=1e-15, atol=0)


def test_rope_identity_norms_and_hand_angle():
    r = np.random.default_rng(0)
    v = r.standard_normal((3, 8))
    assert np.array_equal(D.rope(v, 0), v)                       # position 0: no rotation
    w = D.rope(v, 17)
    assert np.allclose(w[:, 0::2] ** 2 + w[:, 1::2] ** 2, v[:, 0::2] ** 2 + v[:, 1::2] ** 2, rtol=1e-13)
    e = np.zeros(4)
    e[0] = 1.0                                                   # pair 0 rotates by pos * theta^0 = pos
    assert np.allclose(D.rope(e, 2)[:2], [math.cos(2.0), math.sin(2.0)], rtol=1e-15)
    e = np.zeros(4)
    e[2] = 1.0                                                   # pair 1: angle pos * theta^(-2/4)
    a = 3 * D.THETA ** -0.5
    assert np.allclose(D.rope(e, 3)[2:], [math.cos(a), math.sin(a)], rtol=1e-14)


def test_attention_special_cases():
    r = np.random.default_rng(1)
    q = r.standard_normal((4, 8))
    V = r.standard_normal((1, 2, 8))
    K = r.standard_normal((1, 2, 8))
    out = D.attention(q, K, V, 4, 2)
    # one cached position: every head returns its value row (heads 0, 1 -> kv 0)
    assert np.allclose(out, V[0][[0, 0, 1, 1]], rtol=1e-15)
    # equal keys: the mean of the value rows
    K2 = np.repeat(K, 3, axis=0)
    V2 = r.standard_normal((3, 2, 8))
    out2 = D.attention(q, K2, V2, 4, 2)
    assert np.allclose(out2[0], V2[:, 0].mean(axis=0), rtol=1e-13)
    # brute force against scalar loops
    K3, V3 = r.standard_normal((5, 2, 8)), r.standard_normal((5, 2, 8))
    out3 = D.attention(q, K3, V3, 4, 2)
    for h in range(4):
        kv = h // 2
        s = [math.fsum(q[h, i] * K3[t, kv, i] for i in range(8)) / math.sqrt(8) for t in range(5)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = math.fsum(e)
        ref = [math.fsum(e[t] / z * V3[t, kv, i] for t in range(5)) for i in range(8)]
        assert np.allclose(out3[h], ref, rtol=1e-12)


def _layers(n, d, F, n_kv, hd, seed):
    r = np.random.default_rng(seed)
    f = lambda *s: bf16_to_f32(bf16_round((r.standard_normal(s) * 0.05).astype(np.float32))).astype(np.float64)  # noqa: E731
    out = []
    for _ in range(n):
        out.append(D.LayerWeights(f(d, d), f(n_kv * hd, d), f(n_kv * hd, d), f(d, d), np.ones(d), np.ones(d),
                                  f(F, d), f(F, d), f(F, d)))
    return out


def test_full_k_prox_block_is_dense_block():
    # every channel kept: the block with the Prox FFN is the dense block
    d, F, H, KV = 64, 96, 4, 2
    layers = _layers(2, d, F, KV, d // H, 3)
    a = D.DecoderOracle(layers, H, KV, ffn="dense")
    b = D.DecoderOracle(layers, H, KV, ffn="int8", keep_k=40, k_ff=F)
    x = np.random.default_rng(4).standard_normal(d)
    for pos in range(4):
        ya, yb = a.step(x, pos), b.step(x, pos)
        assert np.max(np.abs(ya - yb)) <= 1e-12 * np.max(np.abs(ya))
        x = ya


def test_ffn_taps_are_the_prox_forward():
    d, F, H, KV = 64, 96, 4, 4
    layers = _layers(1, d, F, KV, d // H, 5)
    o = D.DecoderOracle(layers, H, KV, ffn="int8", keep_k=40, k_ff=30)
    taps = {}
    o.step(np.random.default_rng(6).standard_normal(d), 0, taps=taps)
    L = layers[0]
    ref = O.oracle_forward(taps["ffn_in"][0][None], L.wg_t, L.wu_t, L.wd, "int8", 40, 30).y[0]
    assert np.array_equal(taps["ffn_out"][0], ref)


def test_mutant_rope_reversed(monkeypatch):
    orig = D.rope
    monkeypatch.setattr(D, "rope", lambda v, pos: orig(v, -pos))
    with pytest.raises(AssertionError):
        test_rope_identity_norms_and_hand_angle()

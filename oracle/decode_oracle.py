"""CPU oracle for one decode step of a Llama-shaped decoder layer around the
Prox FFN -- TEST INFRASTRUCTURE ONLY (the tests and the bench's baseline leg
use it; the product path never does).

Plain numpy, float64.  The layer is the usual pre-norm decoder block: the
FFN is the SwiGLU FFN of "PrunePath: Towards Highly Structured Sparse
Language Models", §2.1, Eq. (1), run as the Prox two-stage sparse FFN ("Prox:
Training-Free FFN Activation Sparsity via Approximate Intermediate-Channel
Salience in LLMs", Abstract) by ``prox_oracle``; the pages leave the rest of
the block as the standard one, so the readings below are the plainest ones:

* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, eps = 1e-5.
* Rotary position embedding on q and k, pairs (2i, 2i + 1) of each head
  rotated by angle pos * theta^(-2i / head_dim), theta = 10000.
* Attention over the cached positions 0..pos, softmax of q.k / sqrt(head_dim),
  grouped heads: query head h reads key/value head h // (n_heads / n_kv).
* Residuals around the attention and the FFN.

The GPU harness rounds activations to bf16 where its matrix products take
them (the inputs of each projection and of the FFN); ``step`` takes a
``rnd`` hook for those points so a test can mirror them.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional

import numpy as np

from . import prox_oracle as O

EPS = 1e-5
THETA = 10000.0


def rmsnorm(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS) * g


def rope(v: np.ndarray, pos: int) -> np.ndarray:
    """v [..., head_dim]: pairs (2i, 2i + 1) rotated by pos * theta^(-2i / head_dim)."""
    hd = v.shape[-1]
    i = np.arange(hd // 2, dtype=np.float64)
    ang = pos * THETA ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(v, dtype=np.float64)
    a, b = v[..., 0::2], v[..., 1::2]
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def softmax(z: np.ndarray) -> np.ndarray:
    z = z - np.max(z, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_heads: int, n_kv: int) -> np.ndarray:
    """q [n_heads][hd], K, V [T][n_kv][hd] -> [n_heads][hd]."""
    hd = q.shape[-1]
    rep = n_heads // n_kv
    out = np.empty_like(q, dtype=np.float64)
    for h in range(n_heads):
        kv = h // rep
        p = softmax(K[:, kv, :] @ q[h] / np.sqrt(hd))
        out[h] = p @ V[:, kv, :]
    return out


@dataclass
class LayerWeights:
    """float64 values of the bf16 weights of one layer (nn.Linear layout
    [out][in]); FFN weights [F][d] as in prox_oracle."""

    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    g_attn: np.ndarray
    g_ffn: np.ndarray
    wg_t: np.ndarray
    wu_t: np.ndarray
    wd: np.ndarray


class DecoderOracle:
    """Decode steps of a stack of layers for one token sequence (batch 1)."""

    def __init__(self, layers: List[LayerWeights], n_heads: int, n_kv: int, ffn: str = "int8",
                 keep_k: Optional[int] = None, k_ff: Optional[int] = None):
        self.layers = layers
        self.n_heads, self.n_kv = n_heads, n_kv
        self.ffn = ffn            # "dense" or a proxy kind of prox_oracle
        self.keep_k, self.k_ff = keep_k, k_ff
        self.K: List[list] = [[] for _ in layers]
        self.V: List[list] = [[] for _ in layers]
        self.proxies = [None] * len(layers)

    def step(self, x: np.ndarray, pos: int, rnd: Callable[[np.ndarray], np.ndarray] = lambda a: a,
             taps: Optional[dict] = None) -> np.ndarray:
        """x [d] -> [d] after every layer; rnd rounds the inputs of the
        projections and of the FFN (identity: pure fp64)."""
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[0]
        hd = d // self.n_heads
        for li, L in enumerate(self.layers):
            a = rnd(rmsnorm(x, L.g_attn))
            q = rope((L.wq @ a).reshape(self.n_heads, hd), pos)
            k = rope((L.wk @ a).reshape(self.n_kv, hd), pos)
            v = (L.wv @ a).reshape(self.n_kv, hd)
            self.K[li].append(k)
            self.V[li].append(v)
            att = attention(q, np.stack(self.K[li]), np.stack(self.V[li]), self.n_heads, self.n_kv)
            x = x + L.wo @ rnd(att.reshape(d))
            f_in = rnd(rmsnorm(x, L.g_ffn))
            if self.ffn == "dense":
                f_out = O.dense_ffn(f_in[None], L.wg_t, L.wu_t, L.wd)[0]
            else:
                if self.proxies[li] is None:
                    self.proxies[li] = (O.build_proxy(L.wg_t.T, self.ffn), O.build_proxy(L.wu_t.T, self.ffn))
                f_out = O.oracle_forward(f_in[None], L.wg_t, L.wu_t, L.wd, self.ffn, self.keep_k, self.k_ff,
                                         proxies=self.proxies[li]).y[0]
            if taps is not None:
                taps.setdefault("ffn_in", []).append(f_in)
                taps.setdefault("ffn_out", []).append(f_out)
            x = x + f_out
        return x

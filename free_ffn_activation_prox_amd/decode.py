"""Decode-step harness: a random-weight, Llama-shaped decoder whose FFNs run
either dense or through the Prox library, to put the FFN speed-up next to the
end-to-end decode step ("Prox: ...", Abstract, reports 1.99x end-to-end at
70 % FFN sparsity; "PrunePath: ...", §4.5: the parts other than the FFN cap
the end-to-end gain).

Everything but the FFN is the unchanged decoder block, in torch on the GPU:
pre-norm RMSNorm (eps 1e-5), q/k/v/o projections (bf16, nn.Linear layout),
rotary embedding (theta 10000, pairs (2i, 2i + 1)), attention over a bf16 KV
cache, residuals.  The FFN is one of:
  "dense"  the SwiGLU FFN as three bf16 matrix products (torch / hipBLASLt);
  "prox"   prox_ffn_forward (a proxy kind, k_in, k_ff);
  "q8"     prox_ffn_forward_q8 (int8 Stage-2 rows);
  "exact"  the exact-mask mode.
One step = one token through every layer, at the next cache position.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import Weights, alloc_workspace, build_proxy, build_qweights, ffn_forward

EPS = 1e-5
THETA = 10000.0


@dataclass
class DecoderShape:
    n_layers: int
    d: int
    F: int
    n_heads: int
    n_kv: int

    @property
    def hd(self) -> int:
        return self.d // self.n_heads


def _rope_tables(hd: int, max_ctx: int, device):
    i = torch.arange(hd // 2, dtype=torch.float64)
    inv = THETA ** (-2.0 * i / hd)
    ang = torch.arange(max_ctx, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).float().to(device), torch.sin(ang).float().to(device)


class DecodeHarness:
    """Decode steps (batch 1) of a stack of decoder layers with bf16 weights.

    ``layers``: per layer a dict of bf16 device tensors wq [d][d],
    wk, wv [n_kv * hd][d], wo [d][d], g_attn, g_ffn [d], wg_t, wu_t, wd [F][d]
    (wd row j = W_down[j, :]).  ``ffn``: "dense" | "prox" | "q8" | "exact"."""

    def __init__(self, shape: DecoderShape, layers: List[dict], max_ctx: int, ffn: str = "prox",
                 proxy: str = "int8", k_in: Optional[int] = None, k_ff: Optional[int] = None, device="cuda"):
        self.shape, self.layers, self.ffn = shape, layers, ffn
        self.max_ctx = max_ctx
        d, F, hd = shape.d, shape.F, shape.hd
        self.k_in = d if ffn == "exact" else (k_in if k_in is not None else d)
        self.k_ff = k_ff if k_ff is not None else F
        self.cos, self.sin = _rope_tables(hd, max_ctx, device)
        # K cache stored transposed ([kv][hd][ctx]) so q.K is a product with a
        # row-major right operand; V cache [kv][ctx][hd]
        self.Kt = [torch.zeros(shape.n_kv, hd, max_ctx, dtype=torch.bfloat16, device=device) for _ in layers]
        self.V = [torch.zeros(shape.n_kv, max_ctx, hd, dtype=torch.bfloat16, device=device) for _ in layers]
        self.pos = 0
        if ffn != "dense":
            kind = "exact" if ffn == "exact" else proxy
            self.w = [Weights(L["wg_t"], L["wu_t"], L["wd"]) for L in layers]
            self.px = [build_proxy(w, kind) for w in self.w]
            self.s2 = [build_qweights(w) for w in self.w] if ffn == "q8" else self.w
            self.ws = alloc_workspace(d, F, 1, kind, device)
            self.y = torch.empty(1, d, dtype=torch.float32, device=device)
            self.mask = torch.empty(1, F, dtype=torch.uint8, device=device)
            self.idx = torch.empty(1, max(self.k_ff, 1), dtype=torch.int32, device=device)
        self.taps: Optional[dict] = None

    def fill_cache(self, n: int, seed: int = 0):
        """Random keys and values at positions 0..n-1 (a context of n tokens)."""
        g = torch.Generator(device="cpu").manual_seed(seed)
        for Kt, V in zip(self.Kt, self.V):
            Kt[:, :, :n] = torch.randn(Kt[:, :, :n].shape, generator=g).to(Kt.dtype).to(Kt.device)
            V[:, :n, :] = torch.randn(V[:, :n, :].shape, generator=g).to(V.dtype).to(V.device)
        self.pos = n

    def _rmsnorm(self, x, g):
        return (x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + EPS) * g.float()).to(torch.bfloat16)

    def _rope(self, v, pos):
        c, s = self.cos[pos], self.sin[pos]
        a, b = v[..., 0::2].float(), v[..., 1::2].float()
        out = torch.empty(v.shape, dtype=torch.float32, device=v.device)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
        return out.to(torch.bfloat16)

    def _ffn(self, li: int, f_in: torch.Tensor) -> torch.Tensor:
        L = self.layers[li]
        if self.ffn == "dense":
            g = torch.nn.functional.linear(f_in, L["wg_t"])
            u = torch.nn.functional.linear(f_in, L["wu_t"])
            h = (torch.nn.functional.silu(g.float()) * u.float()).to(torch.bfloat16)
            return torch.matmul(h, L["wd"]).float()
        ffn_forward(f_in, self.s2[li], self.px[li], self.k_in, self.k_ff, y=self.y, mask=self.mask, idx=self.idx,
                    workspace=self.ws)
        return self.y

    def step(self, x: torch.Tensor) -> torch.Tensor:
        """x fp32 [1][d] -> fp32 [1][d] after every layer; the cache advances."""
        sh, pos = self.shape, self.pos
        H, KV, hd = sh.n_heads, sh.n_kv, sh.hd
        rep = H // KV
        for li, L in enumerate(self.layers):
            a = self._rmsnorm(x, L["g_attn"])
            q = self._rope(torch.nn.functional.linear(a, L["wq"]).view(H, hd), pos)
            k = self._rope(torch.nn.functional.linear(a, L["wk"]).view(KV, hd), pos)
            v = torch.nn.functional.linear(a, L["wv"]).view(KV, hd)
            self.Kt[li][:, :, pos] = k
            self.V[li][:, pos, :] = v
            T = pos + 1
            qg = q.view(KV, rep, hd)                                   # heads grouped by their kv head
            sc = torch.matmul(qg, self.Kt[li][:, :, :T]).float() / math.sqrt(hd)
            p = torch.softmax(sc, dim=-1).to(torch.bfloat16)
            att = torch.matmul(p, self.V[li][:, :T, :]).reshape(1, sh.d)
            x = x + torch.nn.functional.linear(att, L["wo"]).float()
            f_in = self._rmsnorm(x, L["g_ffn"])
            f_out = self._ffn(li, f_in)
            if self.taps is not None:
                self.taps.setdefault("ffn_in", []).append(f_in.clone())
                self.taps.setdefault("ffn_out", []).append(f_out.clone())
                self.taps.setdefault("attn_in", []).append(a.clone())
                self.taps.setdefault("x_mid", []).append(x.clone())
                if self.ffn != "dense":
                    self.taps.setdefault("mask", []).append(self.mask.clone())
            x = x + f_out
        self.pos += 1
        return x


def random_layers(shape: DecoderShape, ffn_weights, seed: int = 0, device="cuda", std: float = 0.02):
    """Random bf16 decoder weights: attention N(0, std); FFN weights from
    ``ffn_weights(layer)`` (bf16 bit arrays wg_t, wu_t, wd [F][d]); RMSNorm
    gains 1."""
    d, kvd = shape.d, shape.n_kv * shape.hd
    g = torch.Generator(device="cpu").manual_seed(seed)

    def rnd(*s):
        return (torch.randn(s, generator=g) * std).to(torch.bfloat16).to(device)

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    out = []
    for li in range(shape.n_layers):
        w = ffn_weights(li)
        out.append({"wq": rnd(d, d), "wk": rnd(kvd, d), "wv": rnd(kvd, d), "wo": rnd(d, d),
                    "g_attn": torch.ones(d, dtype=torch.bfloat16, device=device),
                    "g_ffn": torch.ones(d, dtype=torch.bfloat16, device=device),
                    "wg_t": bits(w["wg_t"]), "wu_t": bits(w["wu_t"]), "wd": bits(w["wd"])})
    return out

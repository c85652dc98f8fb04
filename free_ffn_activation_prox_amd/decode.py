"""Decode-step harness: a random-weight, Llama-shaped decoder whose FFNs run
either dense or through the Prox library, to put the FFN speed-up next to the
end-to-end decode step ("Prox: ...", Abstract, reports 1.99x end-to-end at
70 % FFN sparsity; "PrunePath: ...", §4.5: the parts other than the FFN cap
the end-to-end gain).

Everything but the FFN is the unchanged decoder block, in torch on the GPU:
pre-norm RMSNorm (eps 1e-5), q/k/v/o projections (bf16, nn.Linear layout; q,
k and v as one product), rotary embedding (theta 10000, pairs (2i, 2i + 1),
one complex product for q and one for k, the attention scale 1/sqrt(head_dim)
folded into q's), attention over a bf16 KV cache, residuals, written with few
kernels so that the step is not dominated by launches of tiny ones.  The FFN
is one of:
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
        # q, k and v projections as one product (rows of wq, wk, wv stacked)
        self.wqkv = [torch.cat([L["wq"], L["wk"], L["wv"]], 0).contiguous() for L in layers]
        # rotary factors e^{i pos theta^(-2i/hd)} per position; the query's
        # carry the attention scale 1/sqrt(hd)
        i = torch.arange(hd // 2, dtype=torch.float64)
        ang = torch.arange(max_ctx, dtype=torch.float64)[:, None] * (THETA ** (-2.0 * i / hd))[None, :]
        rot = torch.polar(torch.ones_like(ang), ang)
        self.rot_k = rot.to(torch.complex64).to(device)
        self.rot_q = (rot / math.sqrt(hd)).to(torch.complex64).to(device)
        self.g_attn = [L["g_attn"].float() for L in layers]
        self.g_ffn = [L["g_ffn"].float() for L in layers]
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
        return torch.nn.functional.rms_norm(x, (x.shape[-1],), g, EPS).to(torch.bfloat16)

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
        d, kvd = sh.d, sh.n_kv * sh.hd
        rep = H // KV
        T = pos + 1
        for li, L in enumerate(self.layers):
            a = self._rmsnorm(x, self.g_attn[li])
            qkv = torch.nn.functional.linear(a, self.wqkv[li])                     # [1][d + 2 kvd] bf16
            qk = torch.view_as_complex(qkv[0, :d + kvd].float().view(H + KV, hd // 2, 2))
            q = torch.view_as_real(qk[:H] * self.rot_q[pos]).to(torch.bfloat16).view(KV, rep, hd)
            self.Kt[li][:, :, pos].copy_(torch.view_as_real(qk[H:] * self.rot_k[pos]).view(KV, hd))
            self.V[li][:, pos, :].copy_(qkv[0, d + kvd:].view(KV, hd))
            sc = torch.matmul(q, self.Kt[li][:, :, :T])                          # heads grouped by kv head
            p = torch.softmax(sc, dim=-1, dtype=torch.float32).to(torch.bfloat16)
            att = torch.matmul(p, self.V[li][:, :T, :]).reshape(1, d)
            x = x + torch.nn.functional.linear(att, L["wo"])
            f_in = self._rmsnorm(x, self.g_ffn[li])
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

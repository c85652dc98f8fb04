"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, run the oracle on the same inputs, and compare.

Acceptance per token (the bar the path is held to):
  * proxy codes and scales bit-exact with the oracle's quantiser;
  * kept-input lists identical;
  * channel masks identical except channels whose oracle score lies within
    1e-6 (relative) of the k-th score t ("excused");
  * max |y_gpu - y_ref| <= 2e-2 * max |y_ref| (the contract), where y_ref is
    the oracle's Stage 2 on the GPU's own mask (identical to the oracle's y
    when the masks agree); and a second bar of 1e-4 * max |y_ref|, the fp32
    accumulation bound below, which a lost or doubled channel exceeds;
  * below 4 tokens per call: the channels the Stage-2 blocks stream are a
    permutation of idx (no channel lost, none streamed twice).

The second y bar: y is a sum of at most F fp32 products h_j W_down[j, c],
accumulated in fp32 (per block, then a fixed-order sum of the block
partials); h_j itself carries the fp32 error of a d-term dot product (the
matrix-core path adds the rounding of h to 16 significant bits, as two bf16
halves).  Measured errors are below 5e-6 of max |y|; 1e-4 leaves a factor
of 20 while one channel near the threshold moves y by about 1e-2 of max |y|.
"""

from __future__ import annotations

import numpy as np
import torch

import free_ffn_activation_prox_amd as P
from oracle import prox_oracle as O

Y_TOL = 2e-2
Y_TIGHT = 1e-4
BAND = 1e-6


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def decode_proxy(proxy: P.Proxy, d: int, F: int):
    """GPU proxy buffer -> (q_gate [d][F], q_up [d][F], s_gate, s_up) as numpy.

    Tile-major layout: [tile][row i][8 blocks of 16 B]; int8 block = 8 gate then
    8 up codes; int4 block = 16 gate then 16 up nibbles (low nibble first)."""
    codes, scales = proxy.codes_and_scales()
    c = codes.cpu().numpy()                       # [tiles][d][128]
    tiles = c.shape[0]
    if proxy.kind == "int8":
        blk = c.reshape(tiles, d, 8, 2, 8).view(np.int8)          # tile, i, block, g/u, ch
        q = blk.transpose(3, 1, 0, 2, 4).reshape(2, d, tiles * 64)
    else:
        blk = c.reshape(tiles, d, 8, 2, 8)                          # bytes
        lo = (blk & 0xF).astype(np.int8)
        hi = (blk >> 4).astype(np.int8)
        nib = np.stack([lo, hi], axis=-1).reshape(tiles, d, 8, 2, 16)
        nib = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
        q = nib.transpose(3, 1, 0, 2, 4).reshape(2, d, tiles * 128)
    qg, qu = q[0][:, :F], q[1][:, :F]
    s = scales.cpu().numpy()
    sg, su = s[0][:, :F], s[1][:, :F]
    if proxy.kind == "int8":
        sg, su = sg[0], su[0]
    return qg, qu, sg, su


class Case:
    """One layer's tensors on host (bf16 bits + float64) and device."""

    def __init__(self, x_bits, wg_bits, wu_bits, wd_bits, kind):
        self.kind = kind
        self.xb = x_bits
        self.x = O.bf16_bits_to_f64(x_bits)
        self.wg = O.bf16_bits_to_f64(wg_bits)
        self.wu = O.bf16_bits_to_f64(wu_bits)
        self.wd = O.bf16_bits_to_f64(wd_bits)
        self.B, self.d = self.x.shape
        self.F = self.wg.shape[0]
        self.dx = to_dev(x_bits)
        self.weights = P.Weights(to_dev(wg_bits), to_dev(wu_bits), to_dev(wd_bits))
        self.proxy = P.build_proxy(self.weights, kind)
        self._oproxies = None
        self.gq = None        # quantized Stage-2 weights (GPU), when in use
        self.oq = None        # the oracle's

    def use_q8(self):
        """Run Stage 2 on the quantized rows (prox_ffn_forward_q8) from now on."""
        self.gq = P.build_qweights(self.weights)
        self.oq = O.build_qweights(self.wg, self.wu, self.wd)
        return self

    def check_qweights(self):
        codes, scales = self.gq.codes_and_scales()
        codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
        for m, (q, s) in enumerate(((self.oq.qg, self.oq.sg), (self.oq.qu, self.oq.su), (self.oq.qd, self.oq.sd))):
            assert np.array_equal(codes[m], q), f"matrix {m}: codes differ"
            assert np.array_equal(scales[m].view(np.uint32), s.astype(np.float32).view(np.uint32)), \
                f"matrix {m}: scales differ"

    def oracle_proxies(self):
        if self._oproxies is None:
            self._oproxies = (O.build_proxy(self.wg.T, self.kind), O.build_proxy(self.wu.T, self.kind))
        return self._oproxies

    def check_proxy(self):
        qg, qu, sg, su = decode_proxy(self.proxy, self.d, self.F)
        pg, pu = self.oracle_proxies()
        assert np.array_equal(qg, pg.q), "gate codes differ"
        assert np.array_equal(qu, pu.q), "up codes differ"
        assert np.array_equal(sg.view(np.uint32), pg.s.astype(np.float32).view(np.uint32)), "gate scales differ"
        assert np.array_equal(su.view(np.uint32), pu.s.astype(np.float32).view(np.uint32)), "up scales differ"

    def run_gpu(self, k_in, k_ff, taps=True):
        out = P.ffn_forward(self.dx, self.gq if self.gq is not None else self.weights, self.proxy, k_in, k_ff,
                            taps=taps)
        torch.cuda.synchronize()
        return out

    def check(self, k_in, k_ff, tokens=None, label=""):
        """Full comparison for the listed tokens (default: all).  Returns stats."""
        y, mask, idx, taps = self.run_gpu(k_in, k_ff, taps=True)
        y, mask, idx = y.cpu().numpy(), mask.cpu().numpy(), idx.cpu().numpy()
        in_idx = taps["in_idx"].cpu().numpy()
        key = taps["key"].cpu().numpy()
        hh = taps["h_hat"].cpu().numpy()
        sidx = taps["stream_idx"].cpu().numpy()
        toks = list(range(self.B)) if tokens is None else list(tokens)
        pg, pu = self.oracle_proxies()
        stats = {"excused": 0, "unexcused": 0, "key_bits_differ": 0, "max_rel_y": 0.0,
                 "max_rel_h": 0.0}
        s1 = O.stage1_batch(self.x[toks], pg, pu, k_in, k_ff)
        gms = [np.flatnonzero(mask[b]) for b in toks]
        sw = (self.oq.wg_t, self.oq.wu_t, self.oq.wd) if self.gq is not None else (self.wg, self.wu, self.wd)
        _, yrefs = O.stage2_batch(self.x[toks], *sw, gms)
        for n, b in enumerate(toks):
            s_in, g_hat, u_hat, h_hat, okey, omask, t = s1[n]
            assert np.array_equal(in_idx[b], s_in), f"{label} token {b}: kept inputs differ"
            sc = max(np.max(np.abs(h_hat)), 1e-300)
            stats["max_rel_h"] = max(stats["max_rel_h"], float(np.max(np.abs(hh[b] - h_hat)) / sc))
            stats["key_bits_differ"] += int(np.sum(key[b].view(np.uint32) != okey.view(np.uint32)))
            gm = gms[n]
            assert gm.size == k_ff, f"{label} token {b}: mask has {gm.size} channels, want {k_ff}"
            assert np.array_equal(idx[b], gm), f"{label} token {b}: idx is not the ascending mask"
            if self.B < 4:
                assert np.array_equal(np.sort(sidx[b]), gm), \
                    f"{label} token {b}: the streamed channels are not the kept ones"
            tok = O.TokenResult(s_in, g_hat, u_hat, h_hat, okey, omask, t, None, None)
            exc, unexc, diff = O.mask_diff(tok, gm, BAND)
            stats["excused"] += exc
            stats["unexcused"] += unexc
            assert unexc == 0, f"{label} token {b}: {unexc} unexcused mask differences {diff[:8]}"
            yref = yrefs[n]
            scale = np.max(np.abs(yref))
            err = np.max(np.abs(y[b] - yref))
            rel = float(err / scale) if scale > 0 else float(err)
            stats["max_rel_y"] = max(stats["max_rel_y"], rel)
            assert rel <= Y_TOL, f"{label} token {b}: y error {rel:.3e} > {Y_TOL}"
            assert rel <= Y_TIGHT, f"{label} token {b}: y error {rel:.3e} > {Y_TIGHT} (accumulation bound)"
        return stats

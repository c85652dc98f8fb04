"""CPU oracle for the Prox two-stage sparse SwiGLU FFN (decode path).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module; only the tests, the package's smoke check and the bench's
CPU-baseline leg do.  It shares no code with the HIP library: both take their
inputs from ``prox_workloads`` (random draws only) and compute independently.

Plain numpy, float64 for all floating-point arithmetic, written to be checked
by eye against the sources:

* "Prox: Training-Free FFN Activation Sparsity via Approximate
  Intermediate-Channel Salience in LLMs", Abstract — two stages: Stage 1 uses
  input sparsity and quantized proxy weights to build one shared channel mask
  from the magnitude ranking of the SwiGLU intermediate state; Stage 2
  computes the selected channels exactly, so all three projections run sparse.
* "PrunePath: Towards Highly Structured Sparse Language Models", §2.1, Eq. (1)
  — FFN(x) = (phi(x W_gate) ⊙ x W_up) W_down with phi = SiLU, W_gate, W_up in
  R^{d x d_ff}, W_down in R^{d_ff x d}; the intermediate h is element-wise
  along d_ff, so channels are separable.
* "COUNTDOWN: Contextually Sparse Activation Filtering Out Unnecessary Weights
  in Down Projection", Abstract — the FFN output is a linear combination of
  the rows of W_down, weighted by the intermediate coefficients.

Readings where the pages are silent (each is also listed in the design notes):

* proxy "int8": symmetric, per output channel j: s_j = fl32(max_i |W[i,j]| / 127),
  q = clamp(rne(fl32(W / s_j)), -127, 127); "int4": symmetric per (group of 128
  inputs, channel), s = fl32(max / 7), q in [-7, 7].  A zero column/group gives
  s = 0 and q = 0.  "exact": the proxy is the weight itself (W~ = W).
* input sparsity: keep the k_in largest |x_i|; among equal |x_i| the lower
  index wins.  Stage 2 uses the full, dense x.
* channel ranking: by |h~_j| with h~ = silu(g~) * u~ computed in float64 and
  the ranking key rounded once to fp32; among equal keys the lower index wins.
  The pages fix no precision for the magnitude ranking.  A top-k is a discrete
  decision, so two implementations can only be compared when both rank one
  stated quantity; rounding to fp32 moves a key by at most 2^-24 of its value,
  about 17 times inside the 1e-6 relative band in which masks may differ, so
  ranking the float64 |h~| instead changes the mask only among channels that
  band already excuses (pinned by brute force against the float64 ranking).
* silu(z) = z / (1 + exp(-z)).
* the output y is returned in float64; h is never rounded.

Array layout: ``x`` is [B][d]; ``wg_t`` and ``wu_t`` are [F][d] (row j = the
weights of channel j, i.e. W_gate[:, j]); ``wd`` is [F][d] (row j =
W_down[j, :]).  All inputs are float64 arrays holding bf16 values exactly.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

INT8_QMAX = 127
INT4_QMAX = 7
INT4_GROUP = 128


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU, the activation phi of the SwiGLU FFN (PrunePath, §2.1, Eq. (1))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# Proxy weights (Prox, Abstract: "quantized proxy weights", built training-free
# from the weights alone).  W is taken in the page's orientation [d][F].
# --------------------------------------------------------------------------

def _quantize_block(w32: np.ndarray, amax32: np.ndarray, qmax: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric quantisation of ``w32`` with one scale per entry of ``amax32``
    (broadcast along the reduced axis).  All divisions are fp32 IEEE."""
    s = (amax32 / np.float32(qmax)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (w32 / s).astype(np.float32)
    q = np.where(s > 0, np.clip(np.rint(ratio), -qmax, qmax), 0.0)
    return q.astype(np.int8), s


def quantize_int8_pc(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """int8 per-output-channel proxy of W [d][F].  Returns (q [d][F] int8, s [F] fp32)."""
    w32 = np.asarray(w, dtype=np.float32)           # bf16 values: exact in fp32
    amax = np.max(np.abs(w32), axis=0, keepdims=True)
    q, s = _quantize_block(w32, amax, INT8_QMAX)
    return q, s.reshape(-1)


def quantize_int4_g128(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """int4 proxy of W [d][F], one scale per (group of 128 inputs, channel).

    Returns (q [d][F] int8 holding values in [-7, 7], s [d/128][F] fp32)."""
    w32 = np.asarray(w, dtype=np.float32)
    d, F = w32.shape
    if d % INT4_GROUP:
        raise ValueError("int4 group-128 proxy needs d % 128 == 0")
    g = w32.reshape(d // INT4_GROUP, INT4_GROUP, F)
    amax = np.max(np.abs(g), axis=1, keepdims=True)
    q, s = _quantize_block(g, amax, INT4_QMAX)
    return q.reshape(d, F), s.reshape(d // INT4_GROUP, F)


@dataclass
class Proxy:
    """One proxy matrix: codes, scales and the real-valued W~ = s * q."""

    kind: str
    q: Optional[np.ndarray]
    s: Optional[np.ndarray]
    w_tilde: np.ndarray          # [d][F] float64


def build_proxy(w: np.ndarray, kind: str) -> Proxy:
    """Proxy of W [d][F] (float64 bf16 values) for ``kind`` in int8/int4/exact."""
    if kind == "int8":
        q, s = quantize_int8_pc(w)
        wt = q.astype(np.float64) * s.astype(np.float64)[None, :]
    elif kind == "int4":
        q, s = quantize_int4_g128(w)
        d, F = q.shape
        # W~[i, j] = s[i // 128, j] * q[i, j]: rows of group g take scale row g
        wt = (q.astype(np.float64).reshape(d // INT4_GROUP, INT4_GROUP, F)
              * s.astype(np.float64)[:, None, :]).reshape(d, F)
    elif kind == "exact":
        q, s, wt = None, None, np.asarray(w, dtype=np.float64)
    else:
        raise ValueError(f"unknown proxy kind {kind!r}")
    return Proxy(kind, q, s, wt)


# --------------------------------------------------------------------------
# Selection: "keep the k largest magnitudes, lower index wins ties".
# --------------------------------------------------------------------------

def select_topk(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the first k entries of the order (key descending, index
    ascending), returned in ascending index order.  ``keys`` are magnitudes."""
    keys = np.asarray(keys)
    n = keys.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(n), -keys))   # primary: -key ascending, then index
    return np.sort(order[:k])


# --------------------------------------------------------------------------
# The forward pass, one token at a time (tokens are independent problems).
# --------------------------------------------------------------------------

@dataclass
class TokenResult:
    s_in: np.ndarray        # selected inputs, ascending
    g_hat: np.ndarray       # [F] proxy gate pre-activation
    u_hat: np.ndarray       # [F] proxy up pre-activation
    h_hat: np.ndarray       # [F] approximate intermediate
    key: np.ndarray         # [F] fp32 ranking key |h~|
    mask: np.ndarray        # selected channels, ascending
    t: float                # |h~| (float64) of the k-th ranked channel (nan if k == 0)
    h: np.ndarray           # [k] exact intermediate on the mask
    y: np.ndarray           # [d] output


@dataclass
class ForwardResult:
    tokens: List[TokenResult] = field(default_factory=list)

    @property
    def y(self) -> np.ndarray:
        return np.stack([t.y for t in self.tokens])

    @property
    def masks(self) -> List[np.ndarray]:
        return [t.mask for t in self.tokens]


def keep_mask(x: np.ndarray, k_in: int) -> Tuple[np.ndarray, np.ndarray]:
    """Input sparsity for one token: S_in (ascending) and x with every input
    outside S_in set to zero."""
    s_in = select_topk(np.abs(x), k_in)
    xk = np.zeros_like(x)
    xk[s_in] = x[s_in]
    return s_in, xk


def stage1_batch(x: np.ndarray, pg: Proxy, pu: Proxy, k_in: int, k_ff: int):
    """Stage 1 for tokens x [B][d] (Prox, Abstract): input sparsity, proxy
    pre-activations, approximate intermediate, magnitude ranking, mask.

    g~_j = sum over i in S_in of x_i W~_gate[i, j] is evaluated as one matrix
    product of x with its dropped inputs set to zero (each dropped term is an
    exact zero), one row per token.  Returns one tuple per token:
    (s_in, g~, u~, h~, key, mask, t)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    kept = [keep_mask(x[b], k_in) for b in range(x.shape[0])]
    xk = np.stack([k[1] for k in kept])
    g_hat = xk @ pg.w_tilde
    u_hat = xk @ pu.w_tilde
    h_hat = silu(g_hat) * u_hat
    out = []
    for b in range(x.shape[0]):
        key = np.abs(h_hat[b]).astype(np.float32)
        mask = select_topk(key, k_ff)
        if k_ff > 0:
            kth = np.lexsort((np.arange(key.shape[0]), -key))[k_ff - 1]
            t = float(abs(h_hat[b, kth]))
        else:
            t = float("nan")
        out.append((kept[b][0], g_hat[b], u_hat[b], h_hat[b], key, mask, t))
    return out


def stage1_token(x: np.ndarray, pg: Proxy, pu: Proxy, k_in: int, k_ff: int):
    """Stage 1 for one token x [d]; see stage1_batch."""
    return stage1_batch(np.asarray(x, dtype=np.float64)[None, :], pg, pu, k_in, k_ff)[0]


def stage2_batch(x: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray,
                 masks) -> Tuple[List[np.ndarray], np.ndarray]:
    """Stage 2 for tokens x [B][d] with per-token masks (Prox, Abstract: the
    selected channels computed exactly; COUNTDOWN, Abstract: y is a
    combination of W_down rows).

    g_j = sum_i x_i W_gate[i, j] over the dense x, h_j = silu(g_j) u_j for j in
    the token's mask, y = sum over the mask of h_j W_down[j, :], evaluated as
    matrix products with h set to zero outside the mask (exact zeros).
    Returns (h on each mask, in mask order; y [B][d])."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B = x.shape[0]
    g = x @ wg_t.T
    u = x @ wu_t.T
    h_all = silu(g) * u
    hm = np.zeros_like(h_all)
    hs = []
    for b in range(B):
        m = np.asarray(masks[b], dtype=np.int64)
        hm[b, m] = h_all[b, m]
        hs.append(h_all[b, m])
    return hs, hm @ wd


def stage2_token(x: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray,
                 mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Stage 2 for one token x [d]; see stage2_batch.  Returns (h [k], y [d])."""
    hs, y = stage2_batch(np.asarray(x, dtype=np.float64)[None, :], wg_t, wu_t, wd, [mask])
    return hs[0], y[0]


def oracle_stage2(x: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray,
                  masks) -> np.ndarray:
    """Stage 2 for a batch with caller-given per-token masks -> y [B][d]."""
    return stage2_batch(x, wg_t, wu_t, wd, masks)[1]


def oracle_forward(x: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray,
                   kind: str, k_in: int, k_ff: int,
                   proxies: Optional[Tuple[Proxy, Proxy]] = None) -> ForwardResult:
    """Full Prox forward for x [B][d]; per-token masks, nothing shared across tokens."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    wg_t = np.asarray(wg_t, dtype=np.float64)
    wu_t = np.asarray(wu_t, dtype=np.float64)
    wd = np.asarray(wd, dtype=np.float64)
    F, d = wg_t.shape
    if x.shape[1] != d or wu_t.shape != (F, d) or wd.shape != (F, d):
        raise ValueError("shape mismatch")
    if not (0 <= k_in <= d and 0 <= k_ff <= F):
        raise ValueError("k out of range")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite x")
    if proxies is None:
        proxies = (build_proxy(wg_t.T, kind), build_proxy(wu_t.T, kind))
    pg, pu = proxies
    s1 = stage1_batch(x, pg, pu, k_in, k_ff)
    hs, y = stage2_batch(x, wg_t, wu_t, wd, [r[5] for r in s1])
    res = ForwardResult()
    for b, (s_in, g_hat, u_hat, h_hat, key, mask, t) in enumerate(s1):
        res.tokens.append(TokenResult(s_in, g_hat, u_hat, h_hat, key, mask, t, hs[b], y[b]))
    return res


def dense_ffn(x: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """The dense SwiGLU FFN (PrunePath, §2.1, Eq. (1)) for x [B][d]."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return (silu(x @ wg_t.T) * (x @ wu_t.T)) @ wd


# --------------------------------------------------------------------------
# Acceptance helpers shared by the parity tests.
# --------------------------------------------------------------------------

def mask_diff(tok: TokenResult, gpu_mask: np.ndarray, band: float = 1e-6):
    """Compare a GPU mask with the oracle's.  Channels whose oracle score lies
    within ``band`` (relative) of the k-th threshold t are excused.

    Returns (n_excused, n_unexcused, differing channel ids)."""
    a = set(np.asarray(tok.mask).tolist())
    b = set(np.asarray(gpu_mask).tolist())
    diff = sorted(a ^ b)
    if not diff:
        return 0, 0, diff
    t = tok.t
    exc = 0
    for j in diff:
        if np.isfinite(t) and abs(abs(tok.h_hat[j]) - t) <= band * t:
            exc += 1
    return exc, len(diff) - exc, diff


# --------------------------------------------------------------------------
# Quality of a mask and of an output (plain definitions; the pages give no
# numbers for them, so the values are diagnostics, not parity targets).
# --------------------------------------------------------------------------

def mask_overlap(mask_a: np.ndarray, mask_b: np.ndarray) -> int:
    """Number of channels kept by both masks (index arrays or 0/1 vectors)."""
    a, b = np.asarray(mask_a), np.asarray(mask_b)
    if a.dtype == np.uint8 or a.dtype == bool:
        return int(np.count_nonzero((a != 0) & (b != 0)))
    return len(set(a.tolist()) & set(b.tolist()))


def rel_l2_error(y: np.ndarray, y_ref: np.ndarray) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 (the numerator alone when y_ref is 0)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = float(np.sqrt(np.sum((y - y_ref) ** 2)))
    den = float(np.sqrt(np.sum(y_ref ** 2)))
    return num / den if den > 0 else num


# --------------------------------------------------------------------------
# Quantized Stage-2 weights (Prox, Abstract: the method is compatible with
# quantization).  Each row of W_gate^T, W_up^T (the weights of one channel)
# and of W_down (the output direction of one channel) gets one fp32 scale,
# with the rule of the int8 proxy: s = fl32(max |row| / 127),
# q = clamp(rne(fl32(w / s)), -127, 127); the row's weights become s * q.
# Stage 1 is unchanged (its proxy comes from the bf16 weights); Stage 2
# computes the kept channels with the quantized rows.
# --------------------------------------------------------------------------

@dataclass
class QWeights:
    qg: np.ndarray       # [F][d] int8 codes of W_gate^T rows
    sg: np.ndarray       # [F] fp32
    qu: np.ndarray
    su: np.ndarray
    qd: np.ndarray       # [F][d] int8 codes of W_down rows
    sd: np.ndarray
    wg_t: np.ndarray     # [F][d] float64 s * q (dequantized rows)
    wu_t: np.ndarray
    wd: np.ndarray


def quantize_rows_int8(w_rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """int8 codes and fp32 scales, one scale per row of w_rows [F][d]."""
    q, s = quantize_int8_pc(np.asarray(w_rows).T)      # the per-column rule on the transpose
    return np.ascontiguousarray(q.T), s


def build_qweights(wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray) -> QWeights:
    out = {}
    for name, w in (("g", wg_t), ("u", wu_t), ("d", wd)):
        q, s = quantize_rows_int8(w)
        out["q" + name], out["s" + name] = q, s
        out[name] = q.astype(np.float64) * s.astype(np.float64)[:, None]
    return QWeights(out["qg"], out["sg"], out["qu"], out["su"], out["qd"], out["sd"], out["g"], out["u"], out["d"])


def oracle_forward_q8(x: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd: np.ndarray, kind: str, k_in: int,
                      k_ff: int, proxies: Optional[Tuple[Proxy, Proxy]] = None,
                      qw: Optional[QWeights] = None) -> ForwardResult:
    """The forward with quantized Stage-2 weights: Stage 1 from the proxy of
    the bf16 weights, Stage 2 (stage2_batch) on the dequantized rows."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    wg_t, wu_t, wd = (np.asarray(a, dtype=np.float64) for a in (wg_t, wu_t, wd))
    if not (0 <= k_in <= x.shape[1] and 0 <= k_ff <= wg_t.shape[0]):
        raise ValueError("k out of range")
    if proxies is None:
        proxies = (build_proxy(wg_t.T, kind), build_proxy(wu_t.T, kind))
    if qw is None:
        qw = build_qweights(wg_t, wu_t, wd)
    s1 = stage1_batch(x, proxies[0], proxies[1], k_in, k_ff)
    hs, y = stage2_batch(x, qw.wg_t, qw.wu_t, qw.wd, [r[5] for r in s1])
    res = ForwardResult()
    for b, (s_in, g_hat, u_hat, h_hat, key, mask, t) in enumerate(s1):
        res.tokens.append(TokenResult(s_in, g_hat, u_hat, h_hat, key, mask, t, hs[b], y[b]))
    return res


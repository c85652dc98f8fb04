"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin ties a part of the oracle to the mathematics or to an independent
route: a closed form worked by hand, a special case that reduces to a library
routine (torch, not numpy), brute force over all subsets on tiny inputs, and
exact invariants.  The last section plants mistakes in the oracle and checks
that some pin catches each of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import prox_oracle as O
from prox_workloads import bf16_round, bf16_to_f32, gen_small, gen_ties

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


def _case(d, F, B, seed, kind="small"):
    c = gen_small(d, F, B, seed) if kind == "small" else gen_ties(d, F, B, seed)
    return _f64(c["x"]), _f64(c["wg_t"]), _f64(c["wu_t"]), _f64(c["wd"])


# ---------------------------------------------------------------------------
# P1. With every channel kept (k_ff = F) the method is the dense SwiGLU FFN
# (PrunePath, §2.1, Eq. (1); all units active recovers the dense FFN, §2.2,
# Eq. (2)).  Reference: torch float64 silu/linear, not the oracle's numpy.
# ---------------------------------------------------------------------------

def _torch_dense(x, wg_t, wu_t, wd):
    X, G, U, D = (torch.from_numpy(a) for a in (x, wg_t, wu_t, wd))
    h = torch.nn.functional.silu(torch.nn.functional.linear(X, G)) * torch.nn.functional.linear(X, U)
    return (h @ D).numpy()


def check_dense_identity(kind, d, F, B, k_in, seed):
    x, wg, wu, wd = _case(d, F, B, seed)
    y = O.oracle_forward(x, wg, wu, wd, kind, k_in, F).y
    ref = _torch_dense(x, wg, wu, wd)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(y - ref)) <= 1e-12 * scale


@pytest.mark.parametrize("kind", ["int8", "int4", "exact"])
@pytest.mark.parametrize("k_in_frac", [0.0, 0.5, 1.0])
def test_p1_dense_identity(kind, k_in_frac):
    d, F = 256, 96
    check_dense_identity(kind, d, F, 3, int(d * k_in_frac), seed=11)


# ---------------------------------------------------------------------------
# P2. Exact proxy (W~ = W) and no input sparsity: the mask is the top-k of the
# dense |h| (Prox, Abstract: the mask is the one the intermediate induces).
# Reference: torch stable descending sort of the float64 |h| from torch.
# Channels whose |h| lies within fp32 rounding (2^-23 relative) of the k-th
# value may be ordered differently by the fp32 ranking key, and are excused.
# ---------------------------------------------------------------------------

def check_exact_mask(d, F, k_ff, seed, kind="small"):
    x, wg, wu, wd = _case(d, F, 2, seed, kind)
    res = O.oracle_forward(x, wg, wu, wd, "exact", d, k_ff)
    X, G, U = (torch.from_numpy(a) for a in (x, wg, wu))
    h = torch.nn.functional.silu(X @ G.T) * (X @ U.T)
    for b, tok in enumerate(res.tokens):
        hb = h[b].abs()
        order = torch.sort(hb, descending=True, stable=True).indices[:k_ff]
        ref = set(order.tolist())
        got = set(tok.mask.tolist())
        if k_ff == 0:
            assert got == set()
            continue
        t = float(hb[order[-1]])
        for j in ref ^ got:
            assert abs(float(hb[j]) - t) <= 2.0 ** -23 * t, (j, float(hb[j]), t)


@pytest.mark.parametrize("k_ff", [0, 1, 17, 48, 95, 96])
def test_p2_exact_proxy_mask(k_ff):
    check_exact_mask(128, 96, k_ff, seed=5)


def test_p2_exact_proxy_mask_ties():
    # dyadic weights/inputs: many exactly equal |h|; ties go to the lower index
    check_exact_mask(16, 64, 20, seed=3, kind="ties")


# ---------------------------------------------------------------------------
# P3. Brute force on tiny inputs: every subset of the right size is tried;
# exactly one dominates all outside it (|v| larger, or equal and lower
# index).  Scores and y by scalar loops with exactly rounded sums (fsum).
# ---------------------------------------------------------------------------

def _brute_select(vals, k):
    n = len(vals)
    winners = []
    for S in itertools.combinations(range(n), k):
        inside, ok = set(S), True
        for j in S:
            for jj in range(n):
                if jj in inside:
                    continue
                if not (abs(vals[j]) > abs(vals[jj]) or (abs(vals[j]) == abs(vals[jj]) and j < jj)):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            winners.append(S)
    assert len(winners) == 1
    return list(winners[0])


def _silu_scalar(z):
    return z / (1.0 + math.exp(-z))


def check_brute_force(d, F, k_in, k_ff, kind, seed, data="small"):
    x, wg, wu, wd = _case(d, F, 1, seed, data)
    x = x[0]
    res = O.oracle_forward(x[None], wg, wu, wd, kind, k_in, k_ff)
    tok = res.tokens[0]
    # independent proxy values: scalar s * q (or the weight itself)
    pg, pu = O.build_proxy(wg.T, kind), O.build_proxy(wu.T, kind)

    def wtil(p, w_t, i, j):
        if kind == "exact":
            return float(w_t[j, i])
        s = p.s[j] if kind == "int8" else p.s[i // 128, j]
        return float(s) * float(p.q[i, j])

    s_in = _brute_select([float(v) for v in x], k_in)
    assert list(tok.s_in) == s_in
    keys = []
    for j in range(F):
        gh = math.fsum(float(x[i]) * wtil(pg, wg, i, j) for i in s_in)
        uh = math.fsum(float(x[i]) * wtil(pu, wu, i, j) for i in s_in)
        hh = _silu_scalar(gh) * uh
        assert abs(hh - tok.h_hat[j]) <= 1e-13 * max(1e-300, abs(hh)) + 1e-300
        keys.append(float(np.float32(abs(hh))))
    m = _brute_select(keys, k_ff)
    assert list(tok.mask) == m
    y = []
    for c in range(d):
        terms = []
        for j in m:
            g = math.fsum(float(x[i]) * float(wg[j, i]) for i in range(d))
            u = math.fsum(float(x[i]) * float(wu[j, i]) for i in range(d))
            terms.append(_silu_scalar(g) * u * float(wd[j, c]))
        y.append(math.fsum(terms))
    y = np.array(y)
    scale = max(np.max(np.abs(y)), 1e-300)
    assert np.max(np.abs(tok.y - y)) <= 1e-12 * scale


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("kind", ["int8", "exact"])
def test_p3_brute_force_random(seed, kind):
    check_brute_force(10, 9, 5, 4, kind, seed)


@pytest.mark.parametrize("seed", range(4))
def test_p3_brute_force_ties(seed):
    # tie-heavy data exercises "lower index wins" in both selections
    check_brute_force(10, 10, 4, 5, "int8", seed, data="ties")


def test_p3_brute_force_int4():
    # int4 needs d = 128; brute force over the channel subsets only (F small)
    x, wg, wu, wd = _case(128, 8, 1, 21)
    res = O.oracle_forward(x, wg, wu, wd, "int4", 77, 3)
    tok = res.tokens[0]
    pg, pu = O.build_proxy(wg.T, "int4"), O.build_proxy(wu.T, "int4")
    order = sorted(range(128), key=lambda i: (-abs(x[0, i]), i))[:77]
    assert list(tok.s_in) == sorted(order)
    keys = []
    for j in range(8):
        gh = math.fsum(float(x[0, i]) * float(pg.s[0, j]) * float(pg.q[i, j]) for i in order)
        uh = math.fsum(float(x[0, i]) * float(pu.s[0, j]) * float(pu.q[i, j]) for i in order)
        keys.append(float(np.float32(abs(_silu_scalar(gh) * uh))))
    assert list(tok.mask) == _brute_select(keys, 3)


# ---------------------------------------------------------------------------
# P4. Quantiser: worked values and invariants.
# ---------------------------------------------------------------------------

def test_p4_int8_worked_values():
    # column max 127 * 2^-7 gives s = 2^-7 exactly, so codes are w * 2^7;
    # the half-way codes 2.5, 3.5, -2.5 round to even: 2, 4, -2.
    col = np.array([127, -64, 3, 0, -127, 1, 2.5, 3.5, -2.5], dtype=np.float64) / 128.0
    q, s = O.quantize_int8_pc(col[:, None])
    assert s[0] == np.float32(2.0 ** -7)
    assert q[:, 0].tolist() == [127, -64, 3, 0, -127, 1, 2, 4, -2]


def test_p4_int4_worked_values():
    g0 = np.zeros(128)
    g0[:6] = np.array([7, -3, 2.5, 1.5, -0.5, 0.25]) / 8.0     # max 7/8 -> s = 1/8
    g1 = np.zeros(128)
    g1[0] = -0.4375                                           # max 7/16 -> s = 1/16
    g1[1] = 0.09375                                           # 1.5 -> 2
    q, s = O.quantize_int4_g128(np.concatenate([g0, g1])[:, None])
    assert s[:, 0].tolist() == [0.125, 0.0625]
    assert q[:6, 0].tolist() == [7, -3, 2, 2, 0, 0]
    assert q[128:130, 0].tolist() == [-7, 2]


def test_p4_zero_column():
    w = np.zeros((256, 3))
    w[:, 1] = 0.5
    q, s = O.quantize_int8_pc(w)
    assert s[0] == 0 and s[2] == 0 and not q[:, 0].any() and not q[:, 2].any()
    q4, s4 = O.quantize_int4_g128(w)
    assert not q4[:, 0].any() and (s4[:, 0] == 0).all()


@pytest.mark.parametrize("seed", [0, 1])
def test_p4_invariants(seed):
    _, wg, _, _ = _case(256, 64, 1, seed)
    w = wg.T
    for kind, qmax in (("int8", 127), ("int4", 7)):
        p = O.build_proxy(w, kind)
        assert np.abs(p.q).max() <= qmax
        if kind == "int8":
            s_full = np.broadcast_to(p.s[None, :].astype(np.float64), w.shape)
            assert (np.abs(p.q).max(axis=0) == qmax).all()
        else:
            s_full = np.repeat(p.s.astype(np.float64), 128, axis=0)
            assert (np.abs(p.q.reshape(2, 128, -1)).max(axis=1) == qmax).all()
        # |w/s - q| <= 1/2 plus the fp32 rounding of w/s (at most qmax * 2^-24)
        err = np.abs(w - s_full * p.q)
        assert (err <= s_full * (0.5 + qmax * 2.0 ** -23)).all()


# ---------------------------------------------------------------------------
# P5. Whole-forward invariants.
# ---------------------------------------------------------------------------

def test_p5_channel_permutation():
    # permuting channels (columns of W_gate/W_up, rows of W_down; PrunePath,
    # §2.2) permutes the mask and leaves y unchanged
    x, wg, wu, wd = _case(256, 128, 2, 9)
    perm = np.random.default_rng(0).permutation(128)
    a = O.oracle_forward(x, wg, wu, wd, "int8", 150, 40)
    b = O.oracle_forward(x, wg[perm], wu[perm], wd[perm], "int8", 150, 40)
    for ta, tb in zip(a.tokens, b.tokens):
        assert sorted(perm[tb.mask].tolist()) == ta.mask.tolist()
    assert np.max(np.abs(a.y - b.y)) <= 1e-12 * np.max(np.abs(a.y))


def test_p5_scaling():
    # ranking only: W_up * 2^e scales h~ and y exactly, the mask is unchanged;
    # W_down * c scales y only
    x, wg, wu, wd = _case(256, 128, 2, 10)
    a = O.oracle_forward(x, wg, wu, wd, "int8", 120, 50)
    b = O.oracle_forward(x, wg, wu * 4.0, wd, "int8", 120, 50)
    c = O.oracle_forward(x, wg, wu, wd * 3.0, "int8", 120, 50)
    for ta, tb, tc in zip(a.tokens, b.tokens, c.tokens):
        assert ta.mask.tolist() == tb.mask.tolist() == tc.mask.tolist()
        assert np.array_equal(tb.h_hat, 4.0 * ta.h_hat)
    assert np.array_equal(b.y, 4.0 * a.y)
    assert np.max(np.abs(c.y - 3.0 * a.y)) <= 1e-13 * np.max(np.abs(c.y))


def test_p5_batch_independence():
    # each token alone gives its own row of the batch (matrix products of
    # different shapes may round in a different order: 1e-13 relative)
    x, wg, wu, wd = _case(128, 64, 4, 12)
    a = O.oracle_forward(x, wg, wu, wd, "int8", 64, 20)
    for b in range(4):
        s = O.oracle_forward(x[b:b + 1], wg, wu, wd, "int8", 64, 20)
        assert s.tokens[0].mask.tolist() == a.tokens[b].mask.tolist()
        assert np.max(np.abs(s.tokens[0].h_hat - a.tokens[b].h_hat)) <= 1e-13 * np.max(np.abs(a.tokens[b].h_hat))
        assert np.max(np.abs(s.y[0] - a.y[b])) <= 1e-13 * np.max(np.abs(a.y[b]))


def test_p5_nested_masks():
    x, wg, wu, wd = _case(128, 64, 1, 13, "ties")
    prev = set()
    for k in range(65):
        m = set(O.oracle_forward(x, wg, wu, wd, "int8", 70, k).tokens[0].mask.tolist())
        assert prev <= m and len(m) == k
        prev = m


def test_p5_edge_cases():
    x, wg, wu, wd = _case(128, 64, 1, 14)
    r0 = O.oracle_forward(x, wg, wu, wd, "int8", 64, 0)
    assert r0.tokens[0].mask.size == 0 and not r0.y.any()
    # no input kept: every score is 0, so the first k channels win
    r1 = O.oracle_forward(x, wg, wu, wd, "int8", 0, 10)
    assert r1.tokens[0].mask.tolist() == list(range(10))
    assert not r1.tokens[0].h_hat.any()
    # all inputs kept == the proxy pre-activation over the dense x
    r2 = O.oracle_forward(x, wg, wu, wd, "int8", 128, 10)
    pg = O.build_proxy(wg.T, "int8")
    assert np.allclose(r2.tokens[0].g_hat, x[0] @ pg.w_tilde, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        O.oracle_forward(x, wg, wu, wd, "int8", 129, 10)
    with pytest.raises(ValueError):
        O.oracle_forward(x * np.inf, wg, wu, wd, "int8", 10, 10)


# ---------------------------------------------------------------------------
# P6. A d = 4, F = 4 example worked by hand.
#
#   x = [2, -1, 0.5, 4], k_in = 2  ->  S_in = {0, 3}   (|4| > |2| > |-1| > |0.5|)
#   W_gate = Qg / 128, W_up = Qu / 128 with each column reaching 127, so the
#   int8 proxy is exact: s_j = 2^-7 and q = Q.
#   g~_j = (2 Qg[0,j] + 4 Qg[3,j]) / 128 = [246, -4, -60, 2] / 128
#   u~_j = (2 Qu[0,j] + 4 Qu[3,j]) / 128 = [132, 294, -20, 512] / 128
#   |h~| = |silu(g~) u~| ~ [1.7289, 0.03533, 0.02819, 0.03149]  ->  M = {0, 1}
#   exact (dense x): g = [245, -129.5] / 128, u = [5, 291.5] / 128 on M
#   y = silu(g0) u0 * Wd[0] + silu(g1) u1 * Wd[1]
# ---------------------------------------------------------------------------

QG = np.array([[127, 0, 10, -127], [1, 127, 0, 5], [0, 3, 127, 0], [-2, -1, -20, 64]], float)
QU = np.array([[64, 127, -8, 2], [127, 0, 0, 0], [0, -5, 127, 1], [1, 10, -1, 127]], float)
WD = np.array([[1, 0, -1, 0.5], [0, 2, 0, -1], [3, 3, 3, 3], [-1, 1, -1, 1]], float)
XH = np.array([[2, -1, 0.5, 4]], float)


def test_p6_hand_example():
    wg_t, wu_t = (QG / 128).T, (QU / 128).T
    for kind in ("int8", "exact"):
        tok = O.oracle_forward(XH, wg_t, wu_t, WD, kind, 2, 2).tokens[0]
        assert tok.s_in.tolist() == [0, 3]
        assert tok.g_hat.tolist() == [246 / 128, -4 / 128, -60 / 128, 2 / 128]
        assert tok.u_hat.tolist() == [132 / 128, 294 / 128, -20 / 128, 512 / 128]
        sil = lambda z: z / (1 + math.exp(-z))  # noqa: E731
        hh = [sil(a / 128) * b / 128 for a, b in ((246, 132), (-4, 294), (-60, -20), (2, 512))]
        assert np.allclose(tok.h_hat, hh, rtol=1e-15, atol=0)
        assert tok.mask.tolist() == [0, 1]
        h0 = sil(245 / 128) * 5 / 128
        h1 = sil(-129.5 / 128) * 291.5 / 128
        y = [h0 * WD[0, c] + h1 * WD[1, c] for c in range(4)]
        assert np.allclose(tok.y, y, rtol=1e-15, atol=1e-300)
    q, s = O.quantize_int8_pc(QG / 128)
    assert (s == np.float32(2.0 ** -7)).all() and np.array_equal(q, QG.astype(np.int8))


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin above.
# ---------------------------------------------------------------------------

def _caught(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_mutant_tie_break_reversed(monkeypatch):
    def bad(keys, k):
        n = keys.shape[0]
        order = np.lexsort((-np.arange(n), -np.asarray(keys)))
        return np.sort(order[:k])
    monkeypatch.setattr(O, "select_topk", bad)
    assert _caught(lambda: check_brute_force(10, 10, 4, 5, "int8", 0, data="ties"))


def test_mutant_wrong_activation(monkeypatch):
    monkeypatch.setattr(O, "silu", lambda z: np.asarray(z) / (1.0 + np.exp(np.asarray(z))))
    assert _caught(lambda: check_dense_identity("int8", 64, 32, 1, 32, 0))


def test_mutant_signed_ranking(monkeypatch):
    orig = O.stage1_batch

    def bad(x, pg, pu, k_in, k_ff):
        out = []
        for s_in, g, u, h, key, mask, t in orig(x, pg, pu, k_in, k_ff):
            mask = O.select_topk(h.astype(np.float32), k_ff)     # ranks h~, not |h~|
            out.append((s_in, g, u, h, key, mask, t))
        return out
    monkeypatch.setattr(O, "stage1_batch", bad)
    assert _caught(lambda: check_exact_mask(128, 96, 17, 5))


def test_mutant_input_sparsity_dropped(monkeypatch):
    orig = O.stage1_batch
    monkeypatch.setattr(O, "stage1_batch",
                        lambda x, pg, pu, k_in, k_ff: orig(x, pg, pu, np.atleast_2d(x).shape[1], k_ff))
    assert _caught(test_p6_hand_example)


def test_mutant_round_half_away(monkeypatch):
    def bad(w32, amax32, qmax):
        s = (amax32 / np.float32(qmax)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = (w32 / s).astype(np.float32)
        q = np.where(s > 0, np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -qmax, qmax), 0)
        return q.astype(np.int8), s
    monkeypatch.setattr(O, "_quantize_block", bad)
    assert _caught(test_p4_int8_worked_values)


def test_mutant_down_transposed(monkeypatch):
    orig = O.stage2_batch
    monkeypatch.setattr(O, "stage2_batch", lambda x, wg, wu, wd, m: orig(x, wg, wu, np.ascontiguousarray(wd.T), m))
    assert _caught(lambda: check_dense_identity("int8", 64, 64, 1, 32, 0))


# ---------------------------------------------------------------------------
# P7. bf16 bit patterns -> values, from the format's definition (bf16 is the
# top 16 bits of an IEEE binary32: 1 sign, 8 exponent, 7 fraction bits).
# ---------------------------------------------------------------------------

def test_p7_bf16_bits_hand_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x7F7F, 0x7F80, 0x3EAB],
                    dtype=np.uint16)
    v = O.bf16_bits_to_f64(bits)
    assert v.dtype == np.float64
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 0.0 and not np.signbit(v[2])
    assert v[3] == 0.0 and np.signbit(v[3])                      # -0 keeps its sign
    assert v[4] == 2.0 ** -133                                    # smallest subnormal: 1 * 2^(-126 - 7)
    assert v[5] == 127 * 2.0 ** -133                              # largest subnormal
    assert v[6] == 2.0 ** -126                                    # smallest normal
    assert v[7] == (1 + 127 / 128) * 2.0 ** 127                   # largest finite bf16
    assert np.isinf(v[8]) and v[8] > 0
    assert v[9] == (1 + 0x2B / 128) * 2.0 ** (0x7D - 127)         # 0x3EAB: exponent 125, fraction 43
    # 2-D input keeps its shape
    assert O.bf16_bits_to_f64(bits.reshape(2, 5)).shape == (2, 5)


# ---------------------------------------------------------------------------
# P8. int4 group-128 proxy with several groups: every W~[i, j] is the scalar
# product of the scale of row i's group, s[i // 128, j], and the code q[i, j];
# brute force over the channel subsets on a two-group input (d = 256).
# ---------------------------------------------------------------------------

def check_int4_two_groups(seed, d=256, F=7, k_in=150, k_ff=3):
    x, wg, wu, wd = _case(d, F, 1, seed)
    # give the two groups very different scales so a wrong group is visible
    wg[:, 128:] *= 8.0
    wu[:, :128] *= 0.25
    res = O.oracle_forward(x, wg, wu, wd, "int4", k_in, k_ff)
    tok = res.tokens[0]
    pg, pu = O.build_proxy(wg.T, "int4"), O.build_proxy(wu.T, "int4")
    for p in (pg, pu):
        assert p.s.shape == (d // 128, F)
        for i in range(0, d, 37):
            for j in range(F):
                assert p.w_tilde[i, j] == float(p.s[i // 128, j]) * float(p.q[i, j]), (i, j)
    order = sorted(range(d), key=lambda i: (-abs(x[0, i]), i))[:k_in]
    assert list(tok.s_in) == sorted(order)
    keys = []
    for j in range(F):
        gh = math.fsum(float(x[0, i]) * float(pg.s[i // 128, j]) * float(pg.q[i, j]) for i in order)
        uh = math.fsum(float(x[0, i]) * float(pu.s[i // 128, j]) * float(pu.q[i, j]) for i in order)
        hh = _silu_scalar(gh) * uh
        assert abs(hh - tok.h_hat[j]) <= 1e-12 * abs(hh) + 1e-300, j
        keys.append(float(np.float32(abs(hh))))
    assert list(tok.mask) == _brute_select(keys, k_ff)


@pytest.mark.parametrize("seed", range(3))
def test_p8_int4_two_groups(seed):
    check_int4_two_groups(seed)


# ---------------------------------------------------------------------------
# P9. The threshold t is |h~| of the k-th channel in the ranking (the last one
# kept), not of the first one dropped.  Hand example of P6: |h~| ranks
# channels 0, 1, 3, 2, so with k = 2 the threshold is |h~_1|; with k = 1 it
# is |h~_0|; with k = F it is the smallest, |h~_2|.
# ---------------------------------------------------------------------------

def check_threshold_hand():
    wg_t, wu_t = (QG / 128).T, (QU / 128).T
    sil = lambda z: z / (1 + math.exp(-z))  # noqa: E731
    hh = [abs(sil(a / 128) * b / 128) for a, b in ((246, 132), (-4, 294), (-60, -20), (2, 512))]
    for k, j in ((1, 0), (2, 1), (3, 3), (4, 2)):
        tok = O.oracle_forward(XH, wg_t, wu_t, WD, "int8", 2, k).tokens[0]
        assert math.isclose(tok.t, hh[j], rel_tol=1e-14), (k, tok.t, hh[j])
    assert math.isnan(O.oracle_forward(XH, wg_t, wu_t, WD, "int8", 2, 0).tokens[0].t)


def test_p9_threshold_is_kth():
    check_threshold_hand()


def test_p9_threshold_random_is_smallest_kept():
    # on tie-free data t equals the smallest |h~| among the kept channels
    x, wg, wu, wd = _case(256, 200, 3, 41)
    for k in (1, 57, 199, 200):
        for tok in O.oracle_forward(x, wg, wu, wd, "int8", 180, k).tokens:
            assert tok.t == float(np.min(np.abs(tok.h_hat[tok.mask])))


# ---------------------------------------------------------------------------
# P10. The mask acceptance band is relative to t: a differing channel is
# excused when | |h~_j| - t | <= band * t.  Hand-built results at both edges
# of the band, at a small and a large t (an absolute band would swap the
# verdicts at both).
# ---------------------------------------------------------------------------

def _tok(h_hat, mask, t):
    h = np.asarray(h_hat, dtype=np.float64)
    return O.TokenResult(np.arange(0), h, h, h, np.abs(h).astype(np.float32),
                         np.asarray(mask, dtype=np.int64), float(t), None, None)


def check_band_edges():
    band = 1e-6
    for t in (1e-3, 1.0, 1e3):
        inside, outside = t * (1 - 0.5 * band), t * (1 - 4 * band)
        # oracle keeps {0, 1} (channel 1 is the k-th, at t); the GPU swapped 1 for 2
        tok = _tok([5 * t, t, inside], [0, 1], t)
        exc, unexc, diff = O.mask_diff(tok, np.array([0, 2]), band)
        assert (exc, unexc, diff) == (2, 0, [1, 2]), (t, exc, unexc)
        tok = _tok([5 * t, t, outside], [0, 1], t)
        exc, unexc, diff = O.mask_diff(tok, np.array([0, 2]), band)
        assert (exc, unexc) == (1, 1), (t, exc, unexc)
        # a channel far from t is never excused
        tok = _tok([5 * t, t, 0.5 * t], [0, 1], t)
        assert O.mask_diff(tok, np.array([1, 2]), band)[1] == 2
    # identical masks: nothing to excuse
    assert O.mask_diff(_tok([1.0, 2.0], [1], 2.0), np.array([1]), band) == (0, 0, [])


def test_p10_mask_band_relative():
    check_band_edges()


# ---------------------------------------------------------------------------
# P11. The ranking key.  The pages fix no precision for the magnitude
# ranking; both sides rank fp32(|h~|).  Ranking the float64 |h~| instead can
# change the mask only among channels whose |h~| lies within fp32 rounding
# (2^-24 relative) of t, i.e. well inside the acceptance band: brute force
# of both rankings on random and tie-heavy data.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,data", [("int8", "small"), ("int4", "small"), ("int8", "ties")])
def test_p11_fp32_key_vs_fp64_ranking(kind, data):
    d = 256 if kind == "int4" else 96
    x, wg, wu, wd = _case(d, 300, 4, 17, data)
    for k in (1, 90, 299):
        for tok in O.oracle_forward(x, wg, wu, wd, kind, d // 2, k).tokens:
            a = np.abs(tok.h_hat)
            order64 = np.lexsort((np.arange(a.size), -a))[:k]
            diff = set(order64.tolist()) ^ set(tok.mask.tolist())
            for j in diff:
                assert abs(a[j] - tok.t) <= 2.0 ** -24 * tok.t, (j, a[j], tok.t)
            assert np.array_equal(tok.key, a.astype(np.float32))


# ---------------------------------------------------------------------------
# Planted mistakes in the parts P7-P10 pin.
# ---------------------------------------------------------------------------

def test_mutant_int4_scales_tiled(monkeypatch):
    # scale of row i taken as s[i % G] instead of s[i // 128]
    def bad(w, kind):
        if kind != "int4":
            return orig(w, kind)
        q, s = O.quantize_int4_g128(w)
        s_rows = np.tile(s.astype(np.float64), (w.shape[0] // s.shape[0], 1))
        return O.Proxy(kind, q, s, q.astype(np.float64) * s_rows)
    orig = O.build_proxy
    monkeypatch.setattr(O, "build_proxy", bad)
    assert _caught(lambda: check_int4_two_groups(0))


def test_mutant_threshold_next_channel(monkeypatch):
    # t taken at the first dropped channel instead of the k-th kept one
    orig = O.stage1_batch

    def bad(x, pg, pu, k_in, k_ff):
        out = []
        for s_in, g, u, h, key, mask, t in orig(x, pg, pu, k_in, k_ff):
            order = np.lexsort((np.arange(key.shape[0]), -key))
            if k_ff < key.shape[0]:
                t = float(abs(h[order[k_ff]]))
            out.append((s_in, g, u, h, key, mask, t))
        return out
    monkeypatch.setattr(O, "stage1_batch", bad)
    assert _caught(check_threshold_hand)


def test_mutant_band_absolute(monkeypatch):
    def bad(tok, gpu_mask, band=1e-6):
        a, b = set(np.asarray(tok.mask).tolist()), set(np.asarray(gpu_mask).tolist())
        diff = sorted(a ^ b)
        exc = sum(1 for j in diff if abs(abs(tok.h_hat[j]) - tok.t) <= band)
        return exc, len(diff) - exc, diff
    monkeypatch.setattr(O, "mask_diff", bad)
    assert _caught(check_band_edges)


def test_mutant_bf16_shift(monkeypatch):
    def bad(bits):
        b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return b.view(np.float32).astype(np.float64)
    monkeypatch.setattr(O, "bf16_bits_to_f64", bad)
    assert _caught(test_p7_bf16_bits_hand_values)


# ---------------------------------------------------------------------------
# P12. Quality diagnostics: closed forms.
# ---------------------------------------------------------------------------

def test_p12_mask_overlap_and_error_closed_forms():
    a = np.array([1, 4, 7, 9])
    assert O.mask_overlap(a, a) == 4
    assert O.mask_overlap(a, np.array([0, 2, 3])) == 0
    assert O.mask_overlap(a, np.array([4, 9, 10])) == 2
    va, vb = np.zeros(12, np.uint8), np.zeros(12, np.uint8)
    va[[1, 4, 7]] = 1
    vb[[4, 7, 8]] = 1
    assert O.mask_overlap(va, vb) == 2
    y = np.array([3.0, 4.0])
    assert O.rel_l2_error(y, y) == 0.0
    assert O.rel_l2_error(2 * y, y) == 1.0                 # ||y|| / ||y||
    assert O.rel_l2_error(y + np.array([0.0, 5.0]), y) == 1.0
    assert O.rel_l2_error(y, np.zeros(2)) == 5.0            # y_ref = 0: the numerator


def test_p12_exact_mode_full_k_is_dense():
    # the exact-mask mode keeping every channel is the dense FFN (P1 for the
    # exact kind, every input kept)
    x, wg, wu, wd = _case(128, 64, 2, 31)
    res = O.oracle_forward(x, wg, wu, wd, "exact", 128, 64)
    assert O.rel_l2_error(res.y, _torch_dense(x, wg, wu, wd)) <= 1e-13


# ---------------------------------------------------------------------------
# P13. Quantized Stage-2 weights.
# ---------------------------------------------------------------------------

def test_p13_row_quantizer_worked_values():
    # row max 127 * 2^-7: s = 2^-7, codes = w * 2^7, ties to even; one scale
    # per ROW (a second row with its own scale)
    r0 = np.array([127, -64, 3, 2.5, -2.5, 3.5, 0, 1], dtype=np.float64) / 128.0
    r1 = np.array([0, 0, 7, -7, 1.5, 0.5, 0, 0], dtype=np.float64) / 16.0      # max 7/16: s = 7/16/127
    q, s = O.quantize_rows_int8(np.stack([r0, r1]))
    assert s[0] == np.float32(2.0 ** -7)
    assert q[0].tolist() == [127, -64, 3, 2, -2, 4, 0, 1]
    assert s[1] == np.float32(np.float32(7 / 16) / np.float32(127))
    assert q[1, 2] == 127 and q[1, 3] == -127
    assert q.shape == (2, 8) and s.shape == (2,)


def _exact_codes_case(d, F, B, seed):
    # weights that are exactly s * q with s = 2^-7 and every row reaching 127:
    # the row quantizer reproduces them, so the quantized forward is the
    # bf16 forward
    r = np.random.default_rng(seed)
    mats = []
    for _ in range(3):
        q = r.integers(-127, 128, size=(F, d)).astype(np.float64)
        q[:, 0] = 127
        mats.append(q / 128.0)
    x = _f64(bf16_round(r.laplace(size=(B, d)).astype(np.float32)))
    return x, mats[0], mats[1], mats[2]


def check_q8_reduces_to_bf16():
    x, wg, wu, wd = _exact_codes_case(96, 64, 2, 4)
    qw = O.build_qweights(wg, wu, wd)
    for a, b in ((qw.wg_t, wg), (qw.wu_t, wu), (qw.wd, wd)):
        assert np.array_equal(a, b)
    a = O.oracle_forward(x, wg, wu, wd, "int8", 60, 20)
    b = O.oracle_forward_q8(x, wg, wu, wd, "int8", 60, 20, qw=qw)
    assert [t.mask.tolist() for t in a.tokens] == [t.mask.tolist() for t in b.tokens]
    assert np.max(np.abs(a.y - b.y)) <= 1e-13 * np.max(np.abs(a.y))


def test_p13_exact_codes_reduce_to_bf16():
    check_q8_reduces_to_bf16()


def test_p13_q8_stage2_is_dequantized_rows():
    # y by scalar loops over the kept channels with s * q rows (fsum)
    x, wg, wu, wd = _case(16, 12, 1, 8)
    res = O.oracle_forward_q8(x, wg, wu, wd, "int8", 9, 5)
    tok = res.tokens[0]
    qw = O.build_qweights(wg, wu, wd)
    for c in range(16):
        terms = []
        for j in tok.mask:
            g = math.fsum(float(x[0, i]) * float(qw.sg[j]) * float(qw.qg[j, i]) for i in range(16))
            u = math.fsum(float(x[0, i]) * float(qw.su[j]) * float(qw.qu[j, i]) for i in range(16))
            terms.append(_silu_scalar(g) * u * float(qw.sd[j]) * float(qw.qd[j, c]))
        assert abs(math.fsum(terms) - tok.y[c]) <= 1e-12 * max(np.max(np.abs(tok.y)), 1e-300)
    # the mask is the one Stage 1 ranks from the bf16 weights' proxy
    assert tok.mask.tolist() == O.oracle_forward(x, wg, wu, wd, "int8", 9, 5).tokens[0].mask.tolist()


def test_mutant_q8_per_column_scales(monkeypatch):
    # one scale per column (the proxy's orientation) instead of per row
    def bad(w_rows):
        q, s = O.quantize_int8_pc(np.asarray(w_rows))
        return q, s
    monkeypatch.setattr(O, "quantize_rows_int8", bad)
    assert _caught(test_p13_row_quantizer_worked_values)

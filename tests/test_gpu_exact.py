"""GPU parity of the exact-mask mode (PROX_PROXY_EXACT_BF16: every input kept,
channels ranked by the exact |h| from the bf16 weights) against the oracle's
"exact" kind, and of the quality diagnostics against their plain definitions.

The proxy-quality figures (mask recall of the int8 / int4 proxies against
the exact mask, relative y error against the dense FFN) are printed per
workload as diagnostics: the pages give no number for them, so they are
"parity unpinned"; only their definitions are checked.
"""

import numpy as np
import pytest
import torch

from prox_workloads import gen_small, gen_ties, gen_weights, gen_x, pct_count, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(d, F, B, seed, kind="exact", data="small"):
    from _gpu_common import Case
    c = gen_small(d, F, B, seed) if data == "small" else gen_ties(d, F, B, seed)
    return Case(c["x"], c["wg_t"], c["wu_t"], c["wd"], kind)


def _report(label, st):
    print(f"[exact] {label}: excused={st['excused']} unexcused={st['unexcused']} "
          f"key_bits_differ={st['key_bits_differ']} max_rel_h={st['max_rel_h']:.2e} "
          f"max_rel_y={st['max_rel_y']:.2e}", flush=True)


@pytest.mark.parametrize("d,F,B", [(1024, 1000, 1), (2560, 777, 2), (384, 2304, 3), (512, 1376, 8)])
def test_exact_small(d, F, B):
    c = _case(d, F, B, seed=d + F + B)
    for sp in (0, 50, 70, 90):
        k_ff = pct_count(F, 100 - sp)
        label = f"d={d} F={F} B={B} sp={sp}"
        _report(label, c.check(d, k_ff, label=label))


def test_exact_edges_and_ties():
    import free_ffn_activation_prox_amd as P
    c = _case(512, 600, 2, seed=5)
    for k_ff in (0, 1, 599, 600):
        c.check(512, k_ff, label=f"edge k_ff={k_ff}")
    y, m, i = P.ffn_forward(c.dx, c.weights, c.proxy, 512, 0)
    assert not y.any().item() and not m.any().item()
    with pytest.raises(P.ProxError):
        P.ffn_forward(c.dx, c.weights, c.proxy, 511, 10)          # exact mode keeps every input
    t = _case(256, 520, 3, seed=6, data="ties")
    for k_ff in (3, 200, 519):
        _report(f"ties k_ff={k_ff}", t.check(256, k_ff, label=f"ties k_ff={k_ff}"))


def test_exact_full_k_is_dense():
    # every channel kept: the dense SwiGLU FFN (oracle's dense_ffn)
    import free_ffn_activation_prox_amd as P
    from oracle import prox_oracle as O
    c = _case(1024, 1500, 2, seed=7)
    y, _, _ = P.ffn_forward(c.dx, c.weights, c.proxy, 1024, 1500)
    ref = O.dense_ffn(c.x, c.wg, c.wu, c.wd)
    err = np.max(np.abs(y.cpu().numpy() - ref)) / np.max(np.abs(ref))
    assert err <= 1e-4, err


def _fullsize_case(name):
    from _gpu_common import Case
    wl = workloads()[name]
    d, F = wl.layers[0].d, wl.layers[0].F
    w = gen_weights(wl.config_id, 0, d, F)
    return Case(gen_x(wl, 0), w["wg_t"], w["wu_t"], w["wd"], "exact"), wl


@pytest.mark.parametrize("name", ["c1", "c2_s70", "c4_b1_s70", "c4_b8_s70"])
def test_exact_fullsize(name):
    c, wl = _fullsize_case(name)
    print(f"[exact] case {name}", flush=True)
    for sp in sorted({wl.sparsity_pct, 90}):
        k_ff = pct_count(wl.layers[0].F, 100 - sp)
        label = f"{name} sp={sp}"
        _report(label, c.check(c.d, k_ff, label=label))


def test_quality_kernel_matches_definitions():
    import free_ffn_activation_prox_amd as P
    from oracle import prox_oracle as O
    r = np.random.default_rng(3)
    B, F, d = 5, 3000, 777
    ma = (r.random((B, F)) < 0.3).astype(np.uint8)
    mb = (r.random((B, F)) < 0.4).astype(np.uint8)
    mb[0] = ma[0]                                   # identical masks
    mb[1] = 0                                       # nothing in common
    y_ref = r.standard_normal((B, d)).astype(np.float32)
    y = (y_ref + 1e-3 * r.standard_normal((B, d))).astype(np.float32)
    y[2] = y_ref[2]                                 # no error
    y_ref[3] = 0.0                                  # reference 0: the numerator
    dev = "cuda"
    ov, err = P.quality(torch.from_numpy(ma).to(dev), torch.from_numpy(mb).to(dev),
                        torch.from_numpy(y).to(dev), torch.from_numpy(y_ref).to(dev))
    ov, err = ov.cpu().numpy(), err.cpu().numpy()
    for b in range(B):
        assert ov[b] == O.mask_overlap(ma[b], mb[b]), b
        ref = O.rel_l2_error(y[b], y_ref[b])
        assert abs(err[b] - ref) <= 1e-12 * max(ref, 1e-300), (b, err[b], ref)
    assert ov[0] == ma[0].sum() and ov[1] == 0 and err[2] == 0.0


@pytest.mark.parametrize("name", ["c1", "c2_s50", "c2_s70", "c2_s90", "c3_b1", "c4_b1_s70"])
def test_proxy_quality_report(name):
    # diagnostics, parity unpinned: recall of the proxy mask against the exact
    # mask, and the relative y error of both against the dense FFN
    import free_ffn_activation_prox_amd as P
    from _gpu_common import to_dev
    wl = workloads()[name]
    d, F = wl.layers[0].d, wl.layers[0].F
    w = gen_weights(wl.config_id, 0, d, F)
    W = P.Weights(to_dev(w["wg_t"]), to_dev(w["wu_t"]), to_dev(w["wd"]))
    x = to_dev(gen_x(wl, 0, batch=4))
    k_in, k_ff = wl.k_in(), wl.k_ff()
    exact = P.build_proxy(W, "exact")
    proxy = P.build_proxy(W, wl.proxy)
    yp, mp, _ = P.ffn_forward(x, W, proxy, k_in, k_ff)
    ye, me, _ = P.ffn_forward(x, W, exact, d, k_ff)
    yd, _, _ = P.ffn_forward(x, W, exact, d, F)
    ov, err_p = P.quality(mp, me, yp, yd)
    _, err_e = P.quality(me, me, ye, yd)
    recall = ov.cpu().numpy() / k_ff
    ep, ee = err_p.cpu().numpy(), err_e.cpu().numpy()
    print(f"[quality] {name}: {wl.proxy} keep {wl.keep_pct}% sparsity {wl.sparsity_pct}%: mask recall vs exact "
          f"{recall.mean():.4f} (min {recall.min():.4f}); rel y error vs dense: proxy {ep.mean():.4f}, "
          f"exact {ee.mean():.4f}", flush=True)
    assert np.all((recall > 0) & (recall <= 1)) and np.all(np.isfinite(ep)) and np.all(ee <= ep + 1e-9)

"""GPU parity of large batches (prefill: more than 64 tokens per call, run as
consecutive 64-token sub-batches of the matrix-core path) against the oracle,
every token to the full bar; a full-size prefill of the Llama-2-7B layer."""

import numpy as np
import pytest
import torch

from prox_workloads import gen_small, gen_weights, gen_x, pct_count, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(label, st):
    print(f"[prefill] {label}: excused={st['excused']} unexcused={st['unexcused']} "
          f"max_rel_y={st['max_rel_y']:.2e}", flush=True)


@pytest.mark.parametrize("kind", ["int8", "int4"])
@pytest.mark.parametrize("B", [65, 100, 200, 512])
def test_prefill_small(kind, B):
    from _gpu_common import Case
    d, F = 512, 900
    g = gen_small(d, F, B, 300 + B)
    c = Case(g["x"], g["wg_t"], g["wu_t"], g["wd"], kind)
    for keep, sp in ((60, 70), (100, 50)):
        k_in, k_ff = pct_count(d, keep), pct_count(F, 100 - sp)
        label = f"{kind} B={B} keep={keep} sp={sp}"
        _report(label, c.check(k_in, k_ff, label=label))


def test_prefill_tokens_independent_of_the_batch():
    # a token's outputs do not depend on which sub-batch it lands in
    import free_ffn_activation_prox_amd as P
    from _gpu_common import Case
    d, F, B = 512, 900, 130
    g = gen_small(d, F, B, 7)
    c = Case(g["x"], g["wg_t"], g["wu_t"], g["wd"], "int8")
    y, m, i = P.ffn_forward(c.dx, c.weights, c.proxy, 300, 270)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(B)).cuda()
    yp, mp, ip = P.ffn_forward(c.dx[perm].contiguous(), c.weights, c.proxy, 300, 270)
    assert torch.equal(mp, m[perm]) and torch.equal(ip, i[perm])
    assert (yp - y[perm]).abs().max().item() <= 1e-4 * y.abs().max().item()


def test_prefill_fullsize_c2():
    from _gpu_common import Case
    wl = workloads()["c2_p512"]
    d, F = wl.layers[0].d, wl.layers[0].F
    w = gen_weights(wl.config_id, 0, d, F)
    x = gen_x(wl, 0, batch=256)
    print("[prefill] case c2 layer, 256 tokens", flush=True)
    c = Case(x, w["wg_t"], w["wu_t"], w["wd"], wl.proxy)
    _report("c2 layer, 256 tokens", c.check(wl.k_in(), wl.k_ff(), label="c2 prefill"))

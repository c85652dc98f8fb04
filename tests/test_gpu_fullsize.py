"""GPU parity at the full sizes of the measured workloads, in the launch
configuration the bench times (same entry point, same planner).

Every token is compared with the oracle in full.  Batches of 4 or more
tokens take the matrix-core path; there the batch must also be equivariant
under a permutation of its tokens, bit for bit.
"""

import numpy as np
import pytest
import torch

from prox_workloads import gen_weights, gen_x, workloads

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_cache = {}


def _layer(cfg_id, layer, d, F, kind):
    from _gpu_common import Case
    key = (cfg_id, layer)
    if key not in _cache:
        _cache.clear()
        w = gen_weights(cfg_id, layer, d, F)
        xb = np.zeros((1, d), dtype=np.uint16)
        _cache[key] = Case(xb, w["wg_t"], w["wu_t"], w["wd"], kind)
    return _cache[key]


def _with_x(case, x_bits):
    from _gpu_common import to_dev
    from oracle import prox_oracle as O
    case.xb = x_bits
    case.x = O.bf16_bits_to_f64(x_bits)
    case.B = x_bits.shape[0]
    case.dx = to_dev(x_bits)
    return case


def _run(name, layer=0, tokens=None):
    wl = workloads()[name]
    shp = wl.layers[layer]
    c = _layer(wl.config_id, layer, shp.d, shp.F, wl.proxy)
    c.check_proxy()
    _with_x(c, gen_x(wl, layer))
    st = c.check(wl.k_in(layer), wl.k_ff(layer), tokens=tokens, label=f"{name} L{layer}")
    print(f"[fullsize] {name} L{layer}: {st}", flush=True)
    return c, wl


@pytest.mark.parametrize("name", ["c2_s0", "c2_s50", "c2_s70", "c2_s90"])
def test_c2_llama7b_layer(name):
    _run(name)


@pytest.mark.parametrize("name", ["c4_b1_s50", "c4_b1_s70"])
def test_c4_70b_layer(name):
    _run(name)


@pytest.mark.parametrize("name", ["c4_b8_s50", "c4_b8_s70"])
def test_c4_70b_batch8(name):
    c, wl = _run(name)
    _permuted(c, wl, 0)


def test_c3_llama3_8b_stack_every_layer_batch1():
    # all 32 layers of the stack, one token each: proxy bytes, kept inputs,
    # mask and y against the oracle, layer by layer
    for layer in range(workloads()["c3_b1"].n_layers):
        print(f"[fullsize] c3_b1 layer {layer} start", flush=True)
        _run("c3_b1", layer)


@pytest.mark.parametrize("name,layer", [("c3_b4", 0), ("c3_b16", 0), ("c3_b4", 1), ("c3_b16", 1)])
def test_c3_llama3_8b_stack(name, layer):
    c, wl = _run(name, layer)
    _permuted(c, wl, layer)


@pytest.mark.parametrize("layer", [0, 1])
def test_c5_mixed_stack(layer):
    c, wl = _run("c5", layer)
    _permuted(c, wl, layer)


def _permuted(c, wl, layer):
    import free_ffn_activation_prox_amd as P
    k_in, k_ff = wl.k_in(layer), wl.k_ff(layer)
    perm = torch.from_numpy(np.random.default_rng(layer).permutation(c.B)).to(c.dx.device)
    y, m, i = P.ffn_forward(c.dx, c.weights, c.proxy, k_in, k_ff)
    yp, mp, ip = P.ffn_forward(c.dx[perm].contiguous(), c.weights, c.proxy, k_in, k_ff)
    assert torch.equal(mp, m[perm]) and torch.equal(ip, i[perm]), "permuted batch: masks differ"
    assert torch.equal(yp, y[perm]), "permuted batch: y differs"

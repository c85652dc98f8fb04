"""GPU parity of the quantized Stage-2 weights (int8 rows of W_gate^T, W_up^T
and W_down with fp32 row scales; prox_build_qweights / prox_ffn_forward_q8)
against the oracle (quantize_rows_int8, oracle_forward_q8): codes and scales
bit-exact; kept inputs and masks as for the bf16 Stage 2 (Stage 1 is the
same); y against the oracle's Stage 2 on the dequantized rows, on the GPU's
own mask, to the same two bars.
"""

import pytest
import torch

from prox_workloads import gen_small, gen_weights, gen_x, pct_count, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(label, st):
    print(f"[q8] {label}: excused={st['excused']} unexcused={st['unexcused']} max_rel_y={st['max_rel_y']:.2e}",
          flush=True)


@pytest.mark.parametrize("kind", ["int8", "int4"])
@pytest.mark.parametrize("d,F,B", [(1024, 1000, 1), (2560, 777, 2), (384, 2304, 3), (512, 1376, 8), (768, 900, 16)])
def test_q8_small(kind, d, F, B):
    from _gpu_common import Case
    g = gen_small(d, F, B, d + F + B + 1)
    c = Case(g["x"], g["wg_t"], g["wu_t"], g["wd"], kind).use_q8()
    c.check_qweights()
    for keep, sp in ((60, 70), (100, 50), (50, 90)):
        k_in, k_ff = pct_count(d, keep), pct_count(F, 100 - sp)
        label = f"{kind} d={d} F={F} B={B} keep={keep} sp={sp}"
        _report(label, c.check(k_in, k_ff, label=label))


def test_q8_edges():
    from _gpu_common import Case
    import free_ffn_activation_prox_amd as P
    g = gen_small(512, 600, 2, 9)
    c = Case(g["x"], g["wg_t"], g["wu_t"], g["wd"], "int8").use_q8()
    for k_in, k_ff in ((0, 10), (512, 1), (1, 600), (512, 600), (300, 0)):
        c.check(k_in, k_ff, label=f"edge {k_in}/{k_ff}")
    ex = P.build_proxy(c.weights, "exact")
    with pytest.raises(P.ProxError):
        P.ffn_forward(c.dx, c.gq, ex, 512, 10)        # exact mode has no quantized Stage 2


@pytest.mark.parametrize("name", ["c2_s50", "c2_s70", "c2_s90", "c4_b1_s70", "c4_b8_s70"])
def test_q8_fullsize(name):
    from _gpu_common import Case
    wl = workloads()[name]
    d, F = wl.layers[0].d, wl.layers[0].F
    w = gen_weights(wl.config_id, 0, d, F)
    print(f"[q8] case {name}", flush=True)
    c = Case(gen_x(wl, 0), w["wg_t"], w["wu_t"], w["wd"], wl.proxy).use_q8()
    c.check_qweights()
    _report(name, c.check(wl.k_in(), wl.k_ff(), label=name))

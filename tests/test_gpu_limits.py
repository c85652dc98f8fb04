"""GPU parity at the limits the header advertises: d_ff = 32768 (the most
channels one selection block ranks; the channel index fills 15 bits) and
d_model = 16384 (four 4096-column parts per Stage-2 thread), on both the
single-token path and the matrix-core path, at k_ff = d_ff - 1, d_ff and 30 %
of d_ff.  Every token is compared with the oracle to the full bar.
"""

import pytest
import torch

from prox_workloads import gen_small, pct_count

pytestmark = pytest.mark.gpu

MAX_D_FF = 32768
MAX_D_MODEL = 16384


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(d, F, B, seed, kind):
    from _gpu_common import Case
    c = gen_small(d, F, B, seed)
    return Case(c["x"], c["wg_t"], c["wu_t"], c["wd"], kind)


def _report(label, st):
    print(f"[limits] {label}: excused={st['excused']} unexcused={st['unexcused']} "
          f"max_rel_y={st['max_rel_y']:.2e}", flush=True)


@pytest.mark.parametrize("kind", ["int8", "int4"])
@pytest.mark.parametrize("B", [1, 2, 8])
def test_max_d_ff(kind, B):
    import free_ffn_activation_prox_amd as P
    d, F = 256, MAX_D_FF
    assert P.proxy_bytes(d, F, kind) > 0 and P.proxy_bytes(d, F + 1, kind) == 0
    print(f"[limits] case d_ff={F} {kind} B={B}", flush=True)
    c = _case(d, F, B, seed=101 + B, kind=kind)
    c.check_proxy()
    for k_ff in (F - 1, F, pct_count(F, 30)):
        label = f"d_ff={F} {kind} B={B} k_ff={k_ff}"
        _report(label, c.check(pct_count(d, 60), k_ff, label=label))


@pytest.mark.parametrize("kind", ["int8", "int4"])
@pytest.mark.parametrize("B", [1, 8])
def test_max_d_model(kind, B):
    import free_ffn_activation_prox_amd as P
    d, F = MAX_D_MODEL, 640
    assert P.proxy_bytes(d, F, kind) > 0 and P.proxy_bytes(d + 8, F, kind) == 0
    print(f"[limits] case d_model={d} {kind} B={B}", flush=True)
    c = _case(d, F, B, seed=202 + B, kind=kind)
    c.check_proxy()
    for k_in, k_ff in ((pct_count(d, 60), F - 1), (d, F), (pct_count(d, 60), pct_count(F, 30))):
        label = f"d_model={d} {kind} B={B} k_in={k_in} k_ff={k_ff}"
        _report(label, c.check(k_in, k_ff, label=label))

"""The allocation-free forward (prox_ffn_forward_noalloc) against the forward
with a caller workspace (prox_ffn_forward): the same y, mask and idx bit for
bit, on calls in a row whose sizes shrink (the scratch array keeps the last
call's contents), on the single-token and the matrix-core paths; and one case
against the oracle to the parity bar.
"""

import numpy as np
import pytest
import torch

from prox_workloads import gen_small, pct_count

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(d, F, B, seed, kind):
    from _gpu_common import Case
    c = gen_small(d, F, B, seed)
    return Case(c["x"], c["wg_t"], c["wu_t"], c["wd"], kind)


def _both(c, k_in, k_ff):
    import free_ffn_activation_prox_amd as P
    ref = P.ffn_forward(c.dx, c.weights, c.proxy, k_in, k_ff)
    dev = c.dx.device
    y = torch.full((c.B, c.d), float("nan"), dtype=torch.float32, device=dev)
    mask = torch.full((c.B, c.F), 7, dtype=torch.uint8, device=dev)
    idx = torch.full((c.B, max(k_ff, 1)), -5, dtype=torch.int32, device=dev)
    got = P.ffn_forward_noalloc(c.dx, c.weights, c.proxy, k_in, k_ff, y=y, mask=mask, idx=idx)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("sizes", [
    # (d, F, B, kind): the second call of each pair is smaller
    ((4096, 11008, 1, "int8"), (1024, 1000, 2, "int4")),
    ((1024, 3000, 16, "int4"), (512, 700, 4, "int8")),
])
def test_noalloc_matches_workspace_forward(sizes):
    import free_ffn_activation_prox_amd as P
    assert P.noalloc_scratch_bytes() == 32 << 20
    for n, (d, F, B, kind) in enumerate(sizes):
        print(f"[noalloc] call {n}: d={d} F={F} B={B} {kind}", flush=True)
        assert P.workspace_bytes(d, F, B, kind) <= P.noalloc_scratch_bytes()
        c = _case(d, F, B, seed=70 + n, kind=kind)
        k_in, k_ff = pct_count(d, 60), pct_count(F, 30)
        (yr, mr, ir), (yg, mg, ig) = _both(c, k_in, k_ff)
        assert torch.equal(mr, mg) and torch.equal(ir, ig), f"call {n}: mask/idx differ"
        assert torch.equal(yr, yg), f"call {n}: y differs"


def test_noalloc_against_oracle():
    from _gpu_common import BAND, Y_TIGHT
    from oracle import prox_oracle as O
    c = _case(2048, 1500, 3, seed=77, kind="int4")
    k_in, k_ff = pct_count(2048, 60), pct_count(1500, 30)
    _, (y, mask, idx) = _both(c, k_in, k_ff)
    y, mask = y.cpu().numpy(), mask.cpu().numpy()
    pg, pu = c.oracle_proxies()
    s1 = O.stage1_batch(c.x, pg, pu, k_in, k_ff)
    gms = [np.flatnonzero(mask[b]) for b in range(c.B)]
    _, yref = O.stage2_batch(c.x, c.wg, c.wu, c.wd, gms)
    for b in range(c.B):
        tok = O.TokenResult(*s1[b], None, None)
        assert O.mask_diff(tok, gms[b], BAND)[1] == 0
        assert np.max(np.abs(y[b] - yref[b])) <= Y_TIGHT * np.max(np.abs(yref[b]))

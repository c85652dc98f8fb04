"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases span several proxy tiles (256 channels), several Stage-2 column
chunks (2048 columns) and ragged tails; edge cases cover k = 0, k = all, tie-
heavy inputs, many tokens with divergent masks.  Full-size cases run the
shapes of the measured workloads (see test_gpu_fullsize.py).
"""

import numpy as np
import pytest
import torch

from prox_workloads import gen_small, gen_ties, pct_count

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(d, F, B, seed, kind, data="small"):
    from _gpu_common import Case
    c = gen_small(d, F, B, seed) if data == "small" else gen_ties(d, F, B, seed)
    return Case(c["x"], c["wg_t"], c["wu_t"], c["wd"], kind)


def _report(label, st):
    print(f"[parity] {label}: excused={st['excused']} unexcused={st['unexcused']} "
          f"key_bits_differ={st['key_bits_differ']} max_rel_h={st['max_rel_h']:.2e} "
          f"max_rel_y={st['max_rel_y']:.2e}", flush=True)


def test_tiny_workload_c1():
    # d=512, F=1376 (F not a multiple of the 256-channel tile), int8, keep 50 %, sparsity 50 %
    from _gpu_common import Case
    from prox_workloads import gen_weights, gen_x, workloads
    wl = workloads()["c1"]
    w = gen_weights(1, 0, 512, 1376)
    c = Case(gen_x(wl, 0), w["wg_t"], w["wu_t"], w["wd"], "int8")
    c.check_proxy()
    st = c.check(wl.k_in(), wl.k_ff(), label="c1")
    _report("c1", st)


@pytest.mark.parametrize("kind", ["int8", "int4"])
@pytest.mark.parametrize("d,F,B", [(1024, 1000, 3), (2560, 777, 2), (384, 2304, 1)])
def test_small_shapes(kind, d, F, B):
    c = _case(d, F, B, seed=d + F, kind=kind)
    c.check_proxy()
    for keep, sp in ((60, 70), (50, 50), (100, 90)):
        k_in, k_ff = pct_count(d, keep), pct_count(F, 100 - sp)
        st = c.check(k_in, k_ff, label=f"{kind} d={d} F={F} B={B} keep={keep} sp={sp}")
        _report(f"{kind} d={d} F={F} B={B} keep={keep} sp={sp}", st)


@pytest.mark.parametrize("kind", ["int8", "int4"])
def test_edge_k(kind):
    d, F = 512, 600
    c = _case(d, F, 2, seed=3, kind=kind)
    for k_in, k_ff in ((0, 10), (d, 1), (1, F), (d, F), (300, 0), (0, 0), (d, F - 1)):
        c.check(k_in, k_ff, label=f"{kind} k_in={k_in} k_ff={k_ff}")


def test_k_ff_zero_gives_zero_y():
    c = _case(256, 300, 2, seed=4, kind="int8")
    y, mask, idx = c.run_gpu(100, 0, taps=False)
    assert not y.any().item() and not mask.any().item()


def test_ties():
    # dyadic inputs and weights: many equal |x| and equal codes
    c = _case(256, 520, 3, seed=5, kind="int8", data="ties")
    c.check_proxy()
    for k_in, k_ff in ((100, 200), (37, 3), (255, 519)):
        st = c.check(k_in, k_ff, label=f"ties k_in={k_in} k_ff={k_ff}")
        _report(f"ties {k_in}/{k_ff}", st)


def test_tiny_dims():
    c = _case(8, 1, 1, seed=6, kind="int8")
    c.check(4, 1, label="d=8 F=1")
    c = _case(128, 3, 2, seed=7, kind="int4")
    c.check(64, 2, label="d=128 F=3 int4")


def test_ragged_d_and_many_tokens():
    # d = 2056 leaves a partial 2048-column chunk; 3 tokens with divergent masks
    c = _case(2056, 700, 3, seed=8, kind="int8")
    st = c.check(pct_count(2056, 60), pct_count(700, 30), label="d=2056 B=3")
    _report("d=2056 B=3", st)


def test_batch_row_equals_single():
    # 3 tokens: the per-token path (4+ tokens take the matrix-core path)
    c = _case(1024, 1024, 3, seed=9, kind="int8")
    import free_ffn_activation_prox_amd as P
    yb, mb, _ = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 300)
    for b in range(3):
        y1, m1, _ = P.ffn_forward(c.dx[b:b + 1].contiguous(), c.weights, c.proxy, 600, 300)
        assert torch.equal(m1[0], mb[b])
        # the Stage-2 work split depends on the batch, so only the fp32 summation
        # order of y differs
        assert (y1[0] - yb[b]).abs().max().item() <= 1e-5 * yb[b].abs().max().item()


def test_repeatable():
    c = _case(1024, 1500, 2, seed=10, kind="int4")
    import free_ffn_activation_prox_amd as P
    a = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450)
    b = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_stale_workspace_still_exact():
    # The workspace is scratch: whatever it holds on entry (the Stage-1
    # arrival counters included), the call gives the same outputs bit for bit.
    c = _case(1024, 2000, 3, seed=11, kind="int8")
    import free_ffn_activation_prox_amd as P
    ws = P.alloc_workspace(1024, 2000, 3, "int8")
    ref = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 700, workspace=ws)
    noise = np.random.default_rng(5).integers(0, 256, ws.numel(), dtype=np.uint8)
    for fill in ("ones", "random"):
        if fill == "ones":
            ws.fill_(255)
        else:
            ws.copy_(torch.from_numpy(noise).to(ws.device))
        y, m, i = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 700, workspace=ws)
        assert torch.equal(m, ref[1]) and torch.equal(i, ref[2]) and torch.equal(y, ref[0]), fill
        again = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 700, workspace=ws)
        for u, v in zip(again, ref):
            assert torch.equal(u, v), fill


def _pattern_case(d, F, n_patterns, seed, kind="int8"):
    # Channels copy one of a few weight rows, so their ranking keys coincide in
    # large groups: the threshold bin then holds hundreds or thousands of
    # exactly equal keys, and the lower index must win among them.
    from _gpu_common import Case
    from prox_workloads import bf16_round
    r = np.random.default_rng([seed, 4242, d, F])
    pats = {n: r.standard_normal((n_patterns, d), dtype=np.float32) * np.float32(0.05)
            for n in ("wg_t", "wu_t")}
    pick = r.integers(0, n_patterns, F)
    wg = bf16_round(pats["wg_t"][pick])
    wu = bf16_round(pats["wu_t"][pick])
    wd = bf16_round(r.standard_normal((F, d), dtype=np.float32) * np.float32(0.02))
    x = bf16_round(r.laplace(0.0, 1.0, size=(2, d)).astype(np.float32))
    return Case(x, wg, wu, wd, kind)


@pytest.mark.parametrize("F,n_patterns", [(2048, 3), (4096, 3), (8192, 3)])
def test_many_equal_keys(F, n_patterns):
    # F=2048: ~680 equal keys per value (ranked by histogram + index order);
    # F=4096, 8192: ~1365 / ~2730 per value, more than the candidate list
    # holds (the path that ranks every key with one block scan)
    import free_ffn_activation_prox_amd as P
    from oracle import prox_oracle as O
    d = 256
    c = _pattern_case(d, F, n_patterns, seed=F)
    for sp in (50, 70, 90):
        k_in, k_ff = pct_count(d, 60), pct_count(F, 100 - sp)
        st = c.check(k_in, k_ff, label=f"patterns F={F} sp={sp}")
        _report(f"patterns F={F} sp={sp}", st)
        assert st["key_bits_differ"] == 0
        # equal keys: the selection must match the oracle's exactly
        _, mask, _ = P.ffn_forward(c.dx, c.weights, c.proxy, k_in, k_ff)
        pg, pu = c.oracle_proxies()
        for b in range(c.B):
            omask = O.stage1_token(c.x[b], pg, pu, k_in, k_ff)[5]
            assert np.array_equal(np.flatnonzero(mask[b].cpu().numpy()), np.asarray(omask)), (F, sp, b)



@pytest.mark.parametrize("B", [1, 8])
def test_measurement_events(B):
    # the measurement hook leaves the outputs unchanged and gives positive
    # phase times
    import free_ffn_activation_prox_amd as P
    c = _case(1024, 1500, B, seed=12, kind="int8")
    ref = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(P.N_PHASES + 1)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    out = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450, events=ev)
    torch.cuda.synchronize()
    for u, v in zip(out, ref):
        assert torch.equal(u, v)
    times = [ev[p].elapsed_time(ev[p + 1]) for p in range(P.N_PHASES)]
    assert all(0.0 < t < 1000.0 for t in times), times


@pytest.mark.parametrize("B", [1, 8])
def test_kernel_events(B):
    # event mode 1: each phase's kernels carry a start/stop pair; outputs are
    # unchanged, every phase interval is positive and the phases, run back to
    # back, fit inside the boundary events of the same call (mode 0)
    import free_ffn_activation_prox_amd as P
    c = _case(1024, 1500, B, seed=13, kind="int8")
    ref = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * P.N_PHASES)]
    for e in kev:
        e.record()
    torch.cuda.synchronize()
    out = P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450, events=kev, kernel_events=True)
    torch.cuda.synchronize()
    for u, v in zip(out, ref):
        assert torch.equal(u, v)
    ktimes = [kev[2 * p].elapsed_time(kev[2 * p + 1]) for p in range(P.N_PHASES)]
    assert all(0.0 < t < 1000.0 for t in ktimes), ktimes
    # phase p ends before phase p + 1 starts (stream order)
    for p in range(P.N_PHASES - 1):
        assert kev[2 * p + 1].elapsed_time(kev[2 * p + 2]) >= 0.0
    # a later plain call is not timed by the pairs (the library forgets them)
    P.ffn_forward(c.dx, c.weights, c.proxy, 600, 450)
    torch.cuda.synchronize()
    assert [kev[2 * p].elapsed_time(kev[2 * p + 1]) for p in range(P.N_PHASES)] == ktimes


@pytest.mark.parametrize("B,kind", [(1, "int4"), (2, "int8"), (8, "int4"), (8, "int8")])
def test_graph_replay(B, kind):
    # one forward captured in a HIP graph and replayed several times with new
    # x and eager work between the replays; every replay equals an eager call
    # bit for bit (int4 splits proxy tiles across blocks, so the per-tile
    # arrival counters must be left clear by every call)
    import free_ffn_activation_prox_amd as P
    d, F = 1024, 1000
    c = _case(d, F, B, seed=60 + B, kind=kind)
    k_in, k_ff = pct_count(d, 60), pct_count(F, 30)
    dev = c.dx.device
    xbuf = c.dx.clone()
    y = torch.empty(B, d, dtype=torch.float32, device=dev)
    mask = torch.empty(B, F, dtype=torch.uint8, device=dev)
    idx = torch.empty(B, k_ff, dtype=torch.int32, device=dev)
    ws = P.alloc_workspace(d, F, B, kind)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        P.ffn_forward(xbuf, c.weights, c.proxy, k_in, k_ff, y=y, mask=mask, idx=idx, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.ffn_forward(xbuf, c.weights, c.proxy, k_in, k_ff, y=y, mask=mask, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(B)
    for rep in range(4):
        xnew = (torch.randn(B, d, generator=gen) * 2.0).to(torch.bfloat16).to(dev)
        xbuf.copy_(xnew)
        g.replay()
        torch.cuda.synchronize()
        ye, me, ie = P.ffn_forward(xnew, c.weights, c.proxy, k_in, k_ff)
        torch.cuda.synchronize()
        assert torch.equal(mask, me) and torch.equal(idx, ie), f"replay {rep}: mask differs"
        assert torch.equal(y, ye), f"replay {rep}: y differs"


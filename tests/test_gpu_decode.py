"""GPU checks of the decode-step harness (free_ffn_activation_prox_amd.decode)
against the decode oracle (oracle/decode_oracle.py) on a small Llama-shaped
stack (2 layers, d 256, F 640, 4 query / 2 key-value heads).

* dense FFN: every step's output against the oracle's block with the same
  bf16 rounding of the projections' inputs, relative L2 error <= 2e-2 (about
  ten bf16 roundings of 2^-9 on the way: projections' outputs, rotary
  embedding, attention weights, FFN products);
* Prox FFN in place: each layer's FFN, on the bf16 input the block gave it,
  against the Prox oracle (mask to the 1e-6 band, y to 1e-4 of max|y|);
* exact mode keeping every channel equals the dense FFN to the same 2e-2.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SHAPE = dict(n_layers=2, d=256, F=640, n_heads=4, n_kv=2)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _build(ffn, k_in=None, k_ff=None):
    from free_ffn_activation_prox_amd.decode import DecodeHarness, DecoderShape, random_layers
    from prox_workloads import gen_weights
    sh = DecoderShape(**SHAPE)
    layers = random_layers(sh, lambda l: gen_weights(77, l, sh.d, sh.F, std=0.05), seed=3, std=0.05)
    return sh, layers, DecodeHarness(sh, layers, max_ctx=16, ffn=ffn, proxy="int8", k_in=k_in, k_ff=k_ff)


def _oracle_layers(layers):
    from oracle import decode_oracle as D
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    return [D.LayerWeights(f(L["wq"]), f(L["wk"]), f(L["wv"]), f(L["wo"]), f(L["g_attn"]), f(L["g_ffn"]),
                           f(L["wg_t"]), f(L["wu_t"]), f(L["wd"])) for L in layers]


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _x0(d, seed=0):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal((1, d)).astype(np.float32)).cuda()


def test_decode_dense_block_matches_oracle():
    from oracle import decode_oracle as D
    sh, layers, h = _build("dense")
    o = D.DecoderOracle(_oracle_layers(layers), sh.n_heads, sh.n_kv, ffn="dense")
    x = _x0(sh.d)
    for step in range(6):
        xin = x.cpu().numpy()[0].astype(np.float64)
        y = h.step(x)
        ref = o.step(xin, step, rnd=_bf16)
        err = np.linalg.norm(y.cpu().numpy()[0] - ref) / np.linalg.norm(ref)
        print(f"[decode] dense step {step}: rel L2 error {err:.2e}", flush=True)
        assert err <= 2e-2, (step, err)
        x = y


def test_decode_prox_ffn_in_context():
    from oracle import prox_oracle as O
    from prox_workloads import pct_count
    d, F = SHAPE["d"], SHAPE["F"]
    k_in, k_ff = pct_count(d, 60), pct_count(F, 30)
    sh, layers, h = _build("prox", k_in, k_ff)
    h.taps = {}
    x = _x0(d, 1)
    for _ in range(4):
        x = h.step(x)
    ol = _oracle_layers(layers)
    n = 0
    for i, (f_in, f_out, m) in enumerate(zip(h.taps["ffn_in"], h.taps["ffn_out"], h.taps["mask"])):
        L = ol[i % sh.n_layers]
        xin = f_in.float().cpu().numpy().astype(np.float64)
        res = O.oracle_forward(xin, L.wg_t, L.wu_t, L.wd, "int8", k_in, k_ff).tokens[0]
        gm = np.flatnonzero(m.cpu().numpy()[0])
        assert O.mask_diff(res, gm, 1e-6)[1] == 0, i
        yref = O.oracle_stage2(xin, L.wg_t, L.wu_t, L.wd, [gm])[0]
        err = np.max(np.abs(f_out.cpu().numpy()[0] - yref)) / np.max(np.abs(yref))
        assert err <= 1e-4, (i, err)
        n += 1
    assert n == 4 * sh.n_layers


def test_decode_exact_full_k_is_dense():
    d, F = SHAPE["d"], SHAPE["F"]
    _, _, hd_ = _build("dense")
    _, _, he = _build("exact", d, F)
    xd = xe = _x0(d, 2)
    for step in range(4):
        xd, xe = hd_.step(xd), he.step(xe)
        err = (torch.linalg.norm(xd - xe) / torch.linalg.norm(xd)).item()
        assert err <= 2e-2, (step, err)


def test_decode_q8_runs_close_to_bf16_prox():
    # int8 Stage-2 rows: the same masks most of the time and an output close to
    # the bf16-row Prox FFN (row quantization error ~ 2^-8 of a row's max)
    from prox_workloads import pct_count
    d, F = SHAPE["d"], SHAPE["F"]
    k_in, k_ff = pct_count(d, 60), pct_count(F, 30)
    _, _, hp = _build("prox", k_in, k_ff)
    _, _, hq = _build("q8", k_in, k_ff)
    x = _x0(d, 4)
    yp, yq = hp.step(x), hq.step(x)
    err = (torch.linalg.norm(yp - yq) / torch.linalg.norm(yp)).item()
    print(f"[decode] q8 vs bf16 rows, one step: rel L2 {err:.2e}", flush=True)
    assert err <= 5e-2

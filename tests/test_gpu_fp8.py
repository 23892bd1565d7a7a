"""GPU parity of the FP8 E4M3 experts (dynamic per-token / per-row activation scales, per-channel
weight scales) and of the FP8 quantiser, against the CPU oracle's fp8 contract."""
import numpy as np
import pytest
import torch

import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import codecs, router

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_quant_fp8_bitwise_against_oracle():
    rng = np.random.default_rng(12)
    rows = []
    rows.append(rng.standard_normal(5120) * 3.0)                      # typical activations
    rows.append(rng.standard_normal(5120) * 1e-3)                     # small values, subnormal codes
    rows.append(np.zeros(5120))                                       # all-zero row
    ties = codecs.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))     # grid points 0..416
    mids = (ties[:-1] + ties[1:]) / 2                                 # exact ties when amax = 448
    r = np.zeros(5120)
    r[0] = 448.0
    r[1:1 + len(mids)] = mids
    r[200:200 + len(mids)] = -mids
    rows.append(r)
    z = rng.standard_normal(2560) * 0.25
    z[7] = -0.0
    rows.append(np.concatenate([z, z]))
    for _ in range(27):
        rows.append(rng.standard_normal(5120) * 10.0 ** rng.uniform(-3, 3))
    x = torch.tensor(np.stack(rows), dtype=torch.float32).to(torch.bfloat16)
    codes, scales = bm.quant_fp8(x.cuda())
    torch.cuda.synchronize()
    want_c, want_s = codecs.quant_rows_fp8(x.float().numpy())
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    got = codes.cpu().numpy()
    assert np.array_equal(got, want_c), np.argwhere(got != want_c)[:5]
    # 2560-wide rows (the h width)
    c2, s2 = bm.quant_fp8(x[:, :2560].contiguous().cuda())
    w2c, w2s = codecs.quant_rows_fp8(x[:, :2560].float().numpy())
    assert np.array_equal(c2.cpu().numpy(), w2c) and np.array_equal(s2.cpu().numpy(), w2s)


def test_quant_fp8_every_bf16_value():
    """Every finite bf16 value of magnitude at most 448 (both signs, zeros and subnormals), quantised
    in rows whose amax is 448 (scale 1): each code is the E4M3 rounding of the value itself, against
    the oracle bit for bit; and the same values in rows of other amax (general fp32 products)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                 # finite patterns only
    vals = codecs.bf16_bits_to_f64(bits)
    vals = vals[np.abs(vals) <= 448.0]
    per = 2559
    n_rows = -(-len(vals) // per)
    rows = np.zeros((n_rows, 2560))
    rows[:, 0] = 448.0
    flat = np.zeros(n_rows * per)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(n_rows, per)
    for scale in (1.0, 3.0 / 7.0, 1e-3 * 1.7):
        x = torch.tensor(rows * scale, dtype=torch.float32).to(torch.bfloat16)
        codes, scales = bm.quant_fp8(x.cuda())
        torch.cuda.synchronize()
        want_c, want_s = codecs.quant_rows_fp8(x.float().numpy())
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32)), scale
        got = codes.cpu().numpy()
        assert np.array_equal(got, want_c), (scale, np.argwhere(got != want_c)[:5])
    _say("every bf16 value quantised:", len(vals))


@pytest.mark.parametrize("cols", [2560, 4096])
def test_quant_fp8_many_rows_bitwise_sampled(cols):
    """Prefill-sized row counts (16384 or more rows of up to 4096 values) take the quantiser that
    runs one wave per row; its codes and scales on 256 sampled rows (first, last, special rows and
    random ones) against the oracle, bit for bit."""
    rng = np.random.default_rng(14)
    n = 16384 + 37
    x = rng.standard_normal((n, cols)) * (10.0 ** rng.uniform(-3, 3, size=(n, 1)))
    x[5] = 0.0                                           # all-zero row
    x[9, :] = 0.0
    x[9, 3] = -0.0
    x[9, 11] = 448.0                                     # amax exactly 448: scale 1
    x[n - 1] *= 1e-30                                    # tiny amax, large inverse scale
    xb = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
    _say("quantising", n, "rows of", cols)
    codes, scales = bm.quant_fp8(xb.cuda())
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, 5, 9, n - 2, n - 1], rng.choice(n, 251, replace=False)]))
    want_c, want_s = codecs.quant_rows_fp8(xb[pick].float().numpy())
    got_c, got_s = codes.cpu().numpy()[pick], scales.cpu().numpy()[pick]
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(got_c, want_c), np.argwhere(got_c != want_c)[:5]


@pytest.fixture(scope="module")
def beam_fp8():
    _say("generating Beam FP8 weights on cuda:0")
    d = synthgen.make_inputs("fp8_prefill", device="cuda", T=1)
    torch.cuda.synchronize()
    return d


def _run(name, weights, T=None):
    wl = synthgen.WORKLOADS[name]
    d = synthgen.make_inputs(wl, device="cuda", T=T, with_experts=False)
    T = d["T"]
    cfg = bm.WorkloadCfg.of(wl.shape, "bf16", "fp8")
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    out = bm.forward(d["x"], weights["w_router"], d["bias"], weights["w_gate_up"],
                     weights["w_down"], cfg, w_gate_up_scale=weights["w_gate_up_scale"],
                     w_down_scale=weights["w_down_scale"], topk_ids_out=ids)
    torch.cuda.synchronize()
    d["w_router"] = weights["w_router"]
    return wl, d, out, ids


@pytest.mark.parametrize("name,T,n_check", [("fp8_decode", None, 32), ("fp8_decode", 77, 77),
                                            ("fp8_prefill", None, 10), ("fp8_decode", 300, 10)])
def test_fp8_forward_parity(beam_fp8, name, T, n_check):
    wl, d, out, ids = _run(name, beam_fp8, T)
    T = d["T"]
    _say("fp8 forward", name, "T =", T)
    sh = wl.shape
    r = router.route(d["x"].cpu(), d["w_router"].cpu(), d["bias"].cpu(), sh.n_groups,
                     sh.topk_groups, sh.topk, sh.routed_scale)
    ids_c = ids.cpu().numpy()
    rc = parity.check_routing(ids_c, _weights_for(r, ids_c), r)
    assert not rc["failures"], rc
    toks = np.arange(T) if T <= n_check else np.sort(np.random.default_rng(T).choice(
        T, n_check, replace=False))
    get = parity.expert_loader(beam_fp8["w_gate_up"], beam_fp8["w_down"], sh.d_ff,
                               beam_fp8["w_gate_up_scale"], beam_fp8["w_down_scale"])
    err, rms = parity.check_outputs(out.cpu().numpy()[toks], d["x"], ids_c, r, sh.routed_scale,
                                    get, "fp8", toks)
    _say(name, T, "fp8 max|err|/rms", err)
    assert err <= parity.TOL["fp8"]


def _weights_for(r, ids_c):
    """Oracle weights in the GPU's id order (the routing check compares per expert id)."""
    return router.weights(r.s, ids_c.astype(np.int64), 2.5)

"""CPU tests of the every-row checker (fullcheck.py) itself: a float32 emulation of the expert path
(torch CPU, FP32 accumulation and activation, the oracle's quantiser) stands in for the device. A
faithful emulation must pass with its admissible rounding differences counted; a planted mistake in
one h element, and a wrong slot order, must fail. No GPU and no HIP code is involved."""
import numpy as np
import torch

import pytest

import fullcheck
from oracle import codecs


def bf16(t):
    return t.to(torch.bfloat16).to(torch.float32)


def quant32(rows):
    q, s = codecs.quant_rows_fp8(rows.numpy())
    return q, s


def run(contract, T=300, E=8, K=2, H=512, F=256, seed=0, corrupt=False, shuffle=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    ids = np.stack([np.random.default_rng(seed + t).choice(E, K, replace=False) for t in range(T)])
    w = np.random.default_rng(seed).uniform(0.1, 1, size=(T, K))
    exs, raw = {}, {}
    for e in range(E):
        if contract == "bf16":
            gu = (torch.randn(2 * F, H, generator=g) * 0.05).to(torch.bfloat16)
            dn = (torch.randn(H, F, generator=g) * 0.05).to(torch.bfloat16)
            raw[e] = (gu.float(), dn.float(), None, None)
            exs[e] = fullcheck.expert_f64(gu, dn, F)
        else:
            gu = torch.randn(2 * F, H, generator=g) * 0.05
            dn = torch.randn(H, F, generator=g) * 0.05
            sgu = gu.abs().amax(1) / 448
            sdn = dn.abs().amax(1) / 448
            qgu = (gu / sgu[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
            qdn = (dn / sdn[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
            raw[e] = (torch.from_numpy(fullcheck.LUT_E4M3[qgu.numpy()]).float(),
                      torch.from_numpy(fullcheck.LUT_E4M3[qdn.numpy()]).float(), sgu, sdn)
            exs[e] = fullcheck.expert_f64(qgu, qdn, F, sgu, sdn)
    # emulated GPU pass (float32 everywhere, rows grouped by expert in token order)
    flat = ids.ravel()
    order = np.concatenate([np.nonzero(flat == e)[0] for e in range(E)])
    off = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]).astype(np.int32)
    xf = x.float()
    if contract == "fp8":
        xq, xs = quant32(xf)
        xd = torch.from_numpy(fullcheck.LUT_E4M3[xq]).float()
    hs = []
    hq_all, hs_all = [], []
    Y = torch.zeros(T * K, H)
    for e in range(E):
        sl = order[off[e]:off[e + 1]]
        gu, dn, sgu, sdn = raw[e]
        if contract == "bf16":
            a = xf[sl // K] @ gu.T
        else:
            a = (xd[sl // K] @ gu.T) * torch.from_numpy(xs[sl // K])[:, None] * sgu[None, :]
        gg, uu = bf16(a[:, :F]), bf16(a[:, F:])
        h = bf16(gg / (1 + torch.exp(-gg)) * uu)
        if corrupt and e == 3:
            h[5, 7] = h[5, 7] * 1.5
        hs.append(h)
        if contract == "bf16":
            y = h @ dn.T
        else:
            q, s = quant32(h)
            hq_all.append(q)
            hs_all.append(s)
            y = (torch.from_numpy(fullcheck.LUT_E4M3[q]).float() @ dn.T) * torch.from_numpy(s)[:, None] * sdn[None, :]
        Y[sl] = torch.from_numpy(w.ravel()[sl]).float()[:, None] * y
    out = Y.view(T, K, H)[:, 0].clone()
    for k in range(1, K):
        out = out + Y.view(T, K, H)[:, k]
    if shuffle:   # two rows of expert 2 swapped in the slot list
        a0 = off[2]
        order[a0], order[a0 + 1] = order[a0 + 1], order[a0]
    st = {"expert_off": off, "sorted_slot": order.astype(np.int32),
          "h": torch.cat(hs).to(torch.bfloat16), "y": Y}
    if contract == "fp8":
        st.update(hq=np.concatenate(hq_all), hs=np.concatenate(hs_all), xq=xq, xs=xs)
    stats = fullcheck.check_batch(out, x, ids.astype(np.int64), w, st, lambda e: exs[e], contract, E)
    return stats


@pytest.mark.parametrize("contract", ["bf16", "fp8"])
def test_faithful_fp32_emulation_passes(contract):
    stats = run(contract)
    assert stats["tokens_checked"] == 300 and stats["rows_checked"] == 600
    assert stats["err_y_vs_own_h"] <= 1e-4 and stats["err_out_vs_own_h"] <= 1e-4
    assert stats["err_out_pure"] <= {"bf16": 1e-2, "fp8": 5e-2}[contract]
    assert stats["h_other_rounding_elements"] > 0   # the FP32 path does take other admissible roundings


def test_planted_y_error_fails():
    # a Y row off by a little more than FP32 accumulation can explain
    import fullcheck as fc
    orig = fc.check_expert_rows

    def skewed(*a, **k):
        res = orig(*a, **k)
        res["y_hyb"] = res["y_hyb"] * (1 + 1e-4)
        return res
    fc.check_expert_rows = skewed
    try:
        with pytest.raises(AssertionError, match="Y outside its bound"):
            run("bf16")
    finally:
        fc.check_expert_rows = orig


def test_planted_h_error_fails():
    with pytest.raises(AssertionError, match="no admissible rounding"):
        run("bf16", corrupt=True)


def test_wrong_slot_order_fails():
    with pytest.raises(AssertionError, match="moe_align order"):
        run("bf16", shuffle=True)


def test_admissible_interval_widens_under_cancellation():
    # g well inside a bf16 interval: one value; u tiny next to its error bound: several
    g = np.array([0.70312]); u = np.array([3.67e-4])
    lo, hi = fullcheck.admissible_h(g, u, np.array([1e-7]), np.array([2.5e-5]))
    h = codecs.bf16_round(fullcheck.silu(codecs.bf16_round(g)) * codecs.bf16_round(u))
    assert lo[0] < h[0] < hi[0]
    lo2, hi2 = fullcheck.admissible_h(g, u, np.array([1e-9]), np.array([1e-12]))
    assert lo2[0] == hi2[0] == h[0]

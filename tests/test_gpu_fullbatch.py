"""Every-row GPU parity at the benchmark's batch sizes, through the workspace inspection hook.

Prefill (T = 8192, bf16 and FP8) is checked on every token and every sorted row; the skewed batch
(T = 32768) on every row of four hot experts (about 6.5K rows each, so every full 320-row block, its
first and last 16-row sub-tiles and the partial last block) and four cold ones, plus sampled tokens
end to end. See fullcheck.py for the rules (admissible roundings, near-flip tokens)."""
import json
import os

import numpy as np
import pytest
import torch

import fullcheck
import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import router

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _say(*a):
    parity.say(*a)


def _forward(name, W, T=None, skew_delta=None):
    wl = synthgen.WORKLOADS[name]
    d = synthgen.make_inputs(wl, device="cuda", T=T, with_experts=False, skew_delta=skew_delta)
    T = d["T"]
    sh = wl.shape
    cfg = bm.WorkloadCfg.of(sh, wl.x_dtype, wl.w_dtype)
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, sh.topk), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, sh.topk), dtype=torch.float32, device="cuda")
    kw = {}
    if wl.w_dtype == "fp8":
        kw = dict(w_gate_up_scale=W["w_gate_up_scale"], w_down_scale=W["w_down_scale"])
    out = bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg,
                     topk_ids_out=ids, topk_w_out=tw, workspace=ws, **kw)
    torch.cuda.synchronize()
    r = router.route(d["x"].cpu(), W["w_router"].cpu(), d["bias"].cpu(), sh.n_groups,
                     sh.topk_groups, sh.topk, sh.routed_scale)
    ids_c = ids.cpu().numpy().astype(np.int64)
    rc = parity.check_routing(ids_c, router.weights(r.s, ids_c, sh.routed_scale), r)
    assert not rc["failures"] and not rc["order_bad"], rc
    _say(name, "T", T, "near-tie tokens", len(rc["near_ties"]))
    w_o = router.weights(r.s, ids_c, sh.routed_scale)
    return wl, cfg, d, ws, out, ids_c, w_o


def _loader(W, d_ff):
    cache = {}

    def get(e):
        if e not in cache:
            if len(cache) > 8:
                cache.clear()
            fp8 = "w_gate_up_scale" in W
            cache[e] = fullcheck.expert_f64(
                W["w_gate_up"][e], W["w_down"][e], d_ff,
                W["w_gate_up_scale"][e] if fp8 else None, W["w_down_scale"][e] if fp8 else None)
        return cache[e]
    return get


def _assert_stats(stats, contract, T):
    # (each Y row and each token's out is checked inside check_batch against the elementwise bound
    # of the down projection of the GPU's own h)
    assert stats["err_out_pure"] <= parity.TOL[contract], stats
    assert stats["near_flip_tokens"] <= max(2, T // 50), stats


@pytest.fixture(scope="module")
def beam_bf16():
    _say("generating Beam bf16 weights on cuda:0")
    d = synthgen.make_inputs("prefill", device="cuda", T=1)
    torch.cuda.synchronize()
    return d


def test_prefill_bf16_every_token(beam_bf16):
    wl, cfg, d, ws, out, ids, w_o = _forward("prefill", beam_bf16)
    st = fullcheck.read_state(ws, cfg, wl.T, False)
    stats = fullcheck.check_batch(out, d["x"], ids, w_o, st, _loader(beam_bf16, 2560), "bf16",
                                  256, say=_say)
    assert stats["tokens_checked"] == wl.T and stats["rows_checked"] == wl.T * 8
    _assert_stats(stats, "bf16", wl.T)
    assert stats["near_flip_tokens"] == 0


def test_skew_bf16_whole_experts(beam_bf16):
    delta = json.load(open(os.path.join(GOLD, "skew_bias.json")))["delta"]
    wl, cfg, d, ws, out, ids, w_o = _forward("skew", beam_bf16, skew_delta=delta)
    T = wl.T
    hot = synthgen.hot_set(16, 256, 0)
    cold = [e for e in range(256) if e not in hot][:4]
    sel = set(hot[:4]) | set(cold)
    counts = np.bincount(ids.ravel(), minlength=256)
    _say("skew rows of the checked experts", {e: int(counts[e]) for e in sorted(sel)})
    assert min(counts[e] for e in hot[:4]) > 320 * 10 and min(counts[e] for e in cold) > 320
    # sampled tokens: the first and last token of each checked hot expert's blocks 0 and 1, and more
    st0 = fullcheck.read_state(ws, cfg, T, False, rows=[0], with_y=False)
    off, ss = st0["expert_off"], st0["sorted_slot"]
    toks = set()
    for e in hot[:4]:
        for b in (0, 1):
            lo = off[e] + 320 * b
            toks |= {int(ss[lo]) // 8, int(ss[lo + 319]) // 8, int(ss[lo + 15]) // 8,
                     int(ss[lo + 304]) // 8}
    toks |= set(np.random.default_rng(5).choice(T, 4, replace=False).tolist())
    # rows to copy: every row of the checked experts and of the sampled tokens
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in sorted(sel)] +
                          [np.nonzero(np.isin(ss // 8, sorted(toks)))[0]])
    rows = np.unique(rows)
    st = fullcheck.read_state(ws, cfg, T, False, rows=rows)
    # h / hq / hs were copied for `rows` only: index them through a remap
    pos = np.full(T * 8, -1, dtype=np.int64)
    pos[rows] = np.arange(len(rows))
    h_sub = st["h"]

    class _H:   # st["h"][global sorted rows] -> the copied sub-array
        def __getitem__(self, idx):
            return h_sub[torch.as_tensor(pos[np.asarray(idx)])]
    st["h"] = _H()
    stats = fullcheck.check_batch(out, d["x"], ids, w_o, st, _loader(beam_bf16, 2560), "bf16",
                                  256, expert_sel=sel, token_sel=sorted(toks), say=_say)
    assert stats["tokens_checked"] >= len(toks)
    _assert_stats(stats, "bf16", T)


@pytest.fixture(scope="module")
def beam_fp8():
    _say("generating Beam FP8 weights on cuda:0")
    d = synthgen.make_inputs("fp8_prefill", device="cuda", T=1)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("name,T", [("fp8_decode", None), ("fp8_decode", 300),
                                    ("fp8_prefill", None)])
def test_fp8_every_token(beam_fp8, name, T):
    wl, cfg, d, ws, out, ids, w_o = _forward(name, beam_fp8, T=T)
    T = d["T"]
    st = fullcheck.read_state(ws, cfg, T, True)
    stats = fullcheck.check_batch(out, d["x"], ids, w_o, st, _loader(beam_fp8, 2560), "fp8", 256,
                                  say=_say)
    assert stats["tokens_checked"] == T
    _assert_stats(stats, "fp8", T)

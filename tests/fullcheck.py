"""Every-row parity of the expert path, through the library's workspace inspection hook (tests only).

After a forward, the workspace holds the GPU's intermediate arrays (beam_moe_workspace_region): the
slot order of the sorted rows, the activation h of every row after its bf16 rounding point, and for
FP8 experts the E4M3 codes and scales of x and h, plus every slot's weighted expert output. These
checks compare each of them with the CPU oracle, row by row:

  * moe_align: the GPU's sorted rows of each expert are exactly that expert's slots in token order.
  * x quantisation (FP8): codes and scales equal the oracle's bit for bit.
  * h: every element equals the oracle's bf16 value, or one that an FP32 computation of the same
    steps could produce. The oracle takes g and u exactly (float64); an FP32 dot product of the
    same operands lies within delta = C_ACC * 2^-24 * ||a|| * ||b|| of it (Cauchy-Schwarz bounds
    the sum of |products| by ||a|| ||b||; C_ACC = 16 is about a hundred times the RMS rounding error
    of FP32 accumulation over these lengths, and far below the worst-case (n-1) * 2^-24 bound, which
    would admit both neighbours of almost every value). bf16 rounding is monotonic, so bf16(g) lies
    in [bf16(g - delta), bf16(g + delta)] (usually one or two values; more where cancellation makes
    g small next to ||a|| ||b||); the SiLU product then carries at most 8 * 2^-24 relative error
    (the exponential, one add, one divide, one multiply in FP32), and its range over those
    intervals bounds h. Any GPU value outside fails. The elements that differ from the oracle's
    own rounding are counted and reported.
  * h quantisation (FP8): the GPU's codes and scales equal the oracle's quantisation of the GPU's own
    h, bit for bit.
  * down: every slot's weighted output lies inside the elementwise bound of FP32 accumulation (and,
    for FP8, of the FP8 instructions' per-block summation) of the oracle's down projection of the
    GPU's h (codes and scales for FP8).
  * out, against the oracle computed from the inputs alone (pure), at the block's bar. A token one of
    whose h rows has a different FP8 scale than the pure oracle's (the row's largest |h| took the
    other admissible bf16 rounding, so every code of the row is re-scaled) is a near-flip token:
    counted, reported, bounded, and compared against the oracle recomputed from the GPU's h.
"""
from __future__ import annotations

import numpy as np
import torch

import routing_grouped_expert_fp32_amd as bm
from oracle import codecs, router

U32 = 2.0 ** -24
C_ACC = 16.0
LUT_E4M3 = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
# FP8 matrix instructions do not sum their products exactly: measured on gfx950, the result of one
# 128-deep (or 32-deep) E4M3 MFMA lies within 6.0e-4 of its largest |product| of the exact sum
# (4M random and planted results); 2^-10 is that bound with a margin of 1.6
FP8_BLOCK = 128
FP8_BLOCK_REL = 2.0 ** -10


def block_max(a):
    """max over each FP8_BLOCK-wide block of the columns of a [n][K] -> [n][K / FP8_BLOCK]"""
    n, k = a.shape
    return a.reshape(n, k // FP8_BLOCK, FP8_BLOCK).max(axis=2)


def silu(z):
    return z / (1.0 + np.exp(-z))


def read_state(ws, cfg, T, fp8, rows=None, with_y=True, dense=False):
    """Copies the inspected arrays to the host. rows: optional sorted-row indices to copy (h, hq,
    hs); y is indexed by slot and copied whole unless with_y is False. dense: the workspace of
    beam_dense_mlp_forward (cfg gives hidden, d_ff, w_dtype)."""
    def view(region, dt):
        return bm.workspace_view(ws, cfg, T, region, dt, dense=dense)
    st = {}
    st["expert_off"] = view("expert_off", torch.int32).cpu().numpy()
    st["sorted_slot"] = view("sorted_slot", torch.int32).cpu().numpy()
    F, H = cfg.d_ff, cfg.hidden
    h = view("h", torch.bfloat16).view(-1, F)
    st["h"] = (h if rows is None else h[torch.as_tensor(rows, device=h.device)]).cpu()
    if fp8:
        hq = view("hq", torch.uint8).view(-1, F)
        hs = view("hs", torch.float32)
        if rows is not None:
            idx = torch.as_tensor(rows, device=hq.device)
            hq, hs = hq[idx], hs[idx]
        st["hq"] = hq.cpu().numpy()
        st["hs"] = hs.cpu().numpy()
        st["xq"] = view("xq", torch.uint8).view(T, H).cpu().numpy()
        st["xs"] = view("xs", torch.float32).cpu().numpy()
    if with_y:
        st["y"] = view("y", torch.float32).view(-1, H).cpu()
    return st


def expert_f64(w_gate_up_e, w_down_e, d_ff, gu_scale_e=None, dn_scale_e=None):
    """Float64 gate / up / down of one expert (decoded codes for FP8) plus scales."""
    if gu_scale_e is None:
        gu = w_gate_up_e.to("cpu", torch.float64).numpy()
        dn = w_down_e.to("cpu", torch.float64).numpy()
        return {"gate": gu[:d_ff], "up": gu[d_ff:], "down": dn}
    gu = LUT_E4M3[w_gate_up_e.cpu().numpy()]
    dn = LUT_E4M3[w_down_e.cpu().numpy()]
    s = gu_scale_e.cpu().numpy().astype(np.float64)
    return {"gate": gu[:d_ff], "up": gu[d_ff:], "down": dn, "gate_scale": s[:d_ff],
            "up_scale": s[d_ff:], "down_scale": dn_scale_e.cpu().numpy().astype(np.float64)}


# SiLU is decreasing below its minimum at z0 (silu'(z0) = 0) and increasing above it
_Z0 = -1.2784645427610738
_SILU_MIN = _Z0 / (1.0 + np.exp(-_Z0))


def _silu_range(lo, hi):
    a, b = silu(lo), silu(hi)
    smin = np.where((lo < _Z0) & (hi > _Z0), _SILU_MIN, np.minimum(a, b))
    return smin, np.maximum(a, b)


def admissible_h(g, u, dg, du):
    """Interval [lo, hi] of the bf16 values an FP32 evaluation of bf16(silu(bf16(g)) * bf16(u)) can
    produce when g and u carry absolute errors up to dg, du (elementwise arrays). bf16 rounding is
    monotonic, so bf16(g) lies in [bf16(g - dg), bf16(g + dg)] and likewise u; the product's range
    over those intervals, widened by the product's own FP32 error (8 * 2^-24 relative), bounds h."""
    glo, ghi = codecs.bf16_round(g - dg), codecs.bf16_round(g + dg)
    ulo, uhi = codecs.bf16_round(u - du), codecs.bf16_round(u + du)
    slo, shi = _silu_range(glo, ghi)
    p = np.stack([slo * ulo, slo * uhi, shi * ulo, shi * uhi])
    pmin, pmax = p.min(axis=0), p.max(axis=0)
    dh = 8 * U32 * np.maximum(np.abs(pmin), np.abs(pmax))
    return codecs.bf16_round(pmin - dh), codecs.bf16_round(pmax + dh)


def check_expert_rows(x_rows, ex, contract, h_gpu, hq_gpu=None, hs_gpu=None):
    """One expert's rows: x_rows [n][H] float64 (bf16 token values), h_gpu [n][F] float64 (the GPU's
    h). Returns a dict: y_hyb [n][H] (down of the GPU's h), h_pure [n][F], flips (elements that took
    the other admissible rounding), and for FP8 scale_flip (rows whose pure scale differs), y_pure
    ({row: y} for the rows whose pure codes differ from the GPU's). Raises AssertionError on any
    inadmissible value."""
    n = x_rows.shape[0]
    if contract == "bf16":
        g = x_rows @ ex["gate"].T
        u = x_rows @ ex["up"].T
        nx = np.linalg.norm(x_rows, axis=1)[:, None]
        dg = C_ACC * U32 * nx * np.linalg.norm(ex["gate"], axis=1)[None, :]
        du = C_ACC * U32 * nx * np.linalg.norm(ex["up"], axis=1)[None, :]
    elif contract == "fp8":
        qx, sx = codecs.quant_rows_fp8(x_rows)
        xd = LUT_E4M3[qx]
        sx = sx.astype(np.float64)[:, None]
        nx = np.linalg.norm(xd, axis=1)[:, None]
        ag = xd @ ex["gate"].T
        au = xd @ ex["up"].T
        sg, su = sx * ex["gate_scale"][None, :], sx * ex["up_scale"][None, :]
        g, u = sg * ag, su * au
        # each FP8 MFMA sums its block of 128 code products to within FP8_BLOCK_REL of the block's
        # largest |product| (bounded by max|x| * max|w| over the block), then the blocks are added
        # in FP32, then two scale multiplies
        mx = block_max(np.abs(xd))
        dg = sg * (FP8_BLOCK_REL * (mx @ block_max(np.abs(ex["gate"])).T)
                   + C_ACC * U32 * nx * np.linalg.norm(ex["gate"], axis=1)[None, :]) + 4 * U32 * np.abs(g)
        du = su * (FP8_BLOCK_REL * (mx @ block_max(np.abs(ex["up"])).T)
                   + C_ACC * U32 * nx * np.linalg.norm(ex["up"], axis=1)[None, :]) + 4 * U32 * np.abs(u)
    else:
        raise ValueError(contract)
    gh, uh = codecs.bf16_round(g), codecs.bf16_round(u)
    h_pure = codecs.bf16_round(silu(gh) * uh)
    mism = h_gpu != h_pure
    flips = int(mism.sum())
    if flips:
        ii, jj = np.nonzero(mism)
        got = h_gpu[ii, jj]
        lo, hi = admissible_h(g[ii, jj], u[ii, jj], dg[ii, jj], du[ii, jj])
        ok = (got >= lo) & (got <= hi)
        if not ok.all():
            k = int(np.argmin(ok))
            raise AssertionError(
                f"h[{ii[k]}][{jj[k]}] = {got[k]!r} is no admissible rounding: oracle g {g[ii[k], jj[k]]!r}"
                f" u {u[ii[k], jj[k]]!r} h {h_pure[ii[k], jj[k]]!r} ({int((~ok).sum())} such elements)")
    res = {"h_pure": h_pure, "flips": flips, "flip_rows": np.nonzero(mism.any(axis=1))[0]}
    nd = np.linalg.norm(ex["down"], axis=1)[None, :]
    if contract == "bf16":
        res["y_hyb"] = h_gpu @ ex["down"].T
        # the bf16 MFMA sums exactly rounded products in FP32
        res["dy"] = C_ACC * U32 * np.linalg.norm(h_gpu, axis=1)[:, None] * nd + 2 * U32 * np.abs(res["y_hyb"])
        rows = res["flip_rows"]
        res["y_pure"] = dict(zip(rows.tolist(), list(h_pure[rows] @ ex["down"].T)))
        res["scale_flip"] = np.zeros(n, dtype=bool)
        return res
    # FP8: the GPU's codes of its own h, bit for bit
    q_own, s_own = codecs.quant_rows_fp8(h_gpu)
    assert np.array_equal(s_own.view(np.uint32), hs_gpu.view(np.uint32)), "h scales"
    assert np.array_equal(q_own, hq_gpu), "h codes"
    sd = ex["down_scale"][None, :]
    hd = LUT_E4M3[hq_gpu]
    sh = hs_gpu.astype(np.float64)[:, None] * sd
    res["y_hyb"] = sh * (hd @ ex["down"].T)
    res["dy"] = sh * (FP8_BLOCK_REL * (block_max(np.abs(hd)) @ block_max(np.abs(ex["down"])).T)
                      + C_ACC * U32 * np.linalg.norm(hd, axis=1)[:, None] * nd) \
        + 4 * U32 * np.abs(res["y_hyb"])
    rows = res["flip_rows"]
    res["scale_flip"] = np.zeros(n, dtype=bool)
    res["y_pure"] = {}
    if len(rows):
        qp, sp = codecs.quant_rows_fp8(h_pure[rows])
        res["scale_flip"][rows] = sp != hs_gpu[rows]
        diff = np.nonzero((qp != hq_gpu[rows]).any(axis=1) | (sp != hs_gpu[rows]))[0]
        if len(diff):
            yp = sp[diff].astype(np.float64)[:, None] * sd * (LUT_E4M3[qp[diff]] @ ex["down"].T)
            res["y_pure"] = dict(zip(rows[diff].tolist(), list(yp)))
    return res


def rel(a, b, rms):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))) / rms)


def check_batch(out_gpu, x, ids, w_oracle, st, get_expert, contract, n_experts, expert_sel=None,
                token_sel=None, say=None, y_parts=1, routed=False):
    """Every-row check of one forward. out_gpu [T][H] (torch or numpy), x [T][H] torch (bf16), ids
    [T][K] int64 (the GPU's routes), w_oracle [T][K] float64 (oracle weights for those routes), st from
    read_state, get_expert(e) -> expert_f64 dict. expert_sel / token_sel: if given, only the rows of
    those experts plus every row of those tokens are checked (out only for tokens all of whose slots
    were checked). routed: a call over a local expert range; ids hold local expert indices and -1
    for slots outside the range, and out sums only the local slots (exactly zero for a token with
    none; tokens_checked counts the others). Each slot's output and each token's out must lie within
    the elementwise bound of the down projection of the GPU's own h (FP32 accumulation; for FP8 also
    the per-block bound of the FP8 instructions); out must meet the block's bar against the pure oracle on every token that
    is not a near-flip token. Returns a stats dict; raises AssertionError on a failure."""
    if say is None:
        import parity
        say = parity.say
    T, K = ids.shape
    H = x.shape[1]
    TK = T * K
    flat = ids.ravel()
    off, ss = st["expert_off"], st["sorted_slot"]
    x64 = x.to("cpu", torch.float64).numpy()
    fp8 = contract == "fp8"
    if fp8:   # x quantisation, every token, bit for bit
        qx, sx = codecs.quant_rows_fp8(x64)
        assert np.array_equal(sx.view(np.uint32), st["xs"].view(np.uint32)), "x scales"
        assert np.array_equal(qx, st["xq"]), "x codes"
    tok_mask = np.zeros(T, dtype=bool)
    if token_sel is not None:
        tok_mask[np.asarray(token_sel)] = True
    # which sorted rows of each expert are checked
    picks = {}
    for e in range(n_experts):
        slots = ss[off[e]:off[e + 1]]
        assert np.array_equal(slots, np.nonzero(flat == e)[0]), f"moe_align order of expert {e}"
        if len(slots) == 0:
            continue
        if expert_sel is None or e in expert_sel:
            picks[e] = np.arange(len(slots))
        else:
            p = np.nonzero(tok_mask[slots // K])[0]
            if len(p):
                picks[e] = p
    n_chk = sum(len(p) for p in picks.values())
    pos = np.full(TK, -1, dtype=np.int64)           # slot -> row of the arrays below
    Yh = np.empty((n_chk, H))                       # weighted output from the GPU's own h
    DY = np.empty((n_chk, H))                       # its elementwise bound
    pure_rows = {}                                  # slot -> weighted pure output where it differs
    near_flip_slots = []
    flips = flip_rows = 0
    at = 0
    for i_e, (e, pick) in enumerate(sorted(picks.items())):
        rows = off[e] + pick
        sl = ss[off[e]:off[e + 1]][pick]
        ex = get_expert(e)
        hr = st["h"][torch.as_tensor(rows)].to(torch.float64).numpy()
        res = check_expert_rows(x64[sl // K], ex, contract, hr,
                                st["hq"][rows] if fp8 else None, st["hs"][rows] if fp8 else None)
        wv = w_oracle.ravel()[sl][:, None]
        n = len(sl)
        pos[sl] = np.arange(at, at + n)
        Yh[at:at + n] = wv * res["y_hyb"]
        DY[at:at + n] = np.abs(wv) * res["dy"]
        for i, yp in res["y_pure"].items():
            pure_rows[int(sl[i])] = wv[i, 0] * yp
        near_flip_slots += sl[res["scale_flip"]].tolist()
        flips += res["flips"]
        flip_rows += len(res["flip_rows"])
        at += n
        if i_e % 32 == 31:
            say(f"  experts checked: {i_e + 1}/{len(picks)}, rows {at}")
    # every checked slot's Y row against the down projection of its own h, element by element (with
    # a K-split down GEMM the rows hold partial sums: only out is checked then)
    err_y = ratio_y = None
    if y_parts == 1:
        chk = np.nonzero(pos >= 0)[0]
        Yg = st["y"][torch.as_tensor(chk)].to(torch.float64).numpy()
        Yo, Db = Yh[pos[chk]], DY[pos[chk]]
        excess = np.abs(Yg - Yo) - Db - 2 * U32 * np.abs(Yo)
        assert (excess <= 0).all(), f"Y outside its bound at slot {chk[np.argmax(excess.max(axis=1))]}"
        rms_y = float(np.sqrt(np.mean(Yo ** 2)))
        err_y = rel(Yg, Yo, rms_y)
        ratio_y = float(np.max(np.abs(Yg - Yo) / (Db + 1e-300)))
        del Yg, Yo, Db, excess
    # out over the tokens all of whose slots were checked, k order from slot k = 0 (routed: every
    # token, over its local slots)
    if routed:   # a token with no local slot must come out exactly zero
        has = (ids >= 0).any(axis=1)
        none = np.nonzero(~has)[0]
        if len(none):
            o0 = out_gpu[torch.as_tensor(none)] if isinstance(out_gpu, torch.Tensor) else out_gpu[none]
            assert not np.asarray(o0.cpu() if isinstance(o0, torch.Tensor) else o0).any(), \
                "out of a token with no local slot"
        full = np.nonzero(has)[0]
        Yh = np.concatenate([Yh, np.zeros((1, H))])
        DY = np.concatenate([DY, np.zeros((1, H))])
        pos = np.where(pos >= 0, pos, len(Yh) - 1)
    else:
        full = np.nonzero((pos.reshape(T, K) >= 0).all(axis=1))[0]
    og = np.asarray(out_gpu[torch.as_tensor(full)].cpu() if isinstance(out_gpu, torch.Tensor)
                    else out_gpu[full], dtype=np.float64)
    o_h = np.zeros((len(full), H))
    o_b = np.zeros((len(full), H))
    o_p = np.zeros((len(full), H))
    for k in range(K):
        r = pos[full * K + k]
        c = Yh[r]
        o_h = o_h + c
        o_b = o_b + DY[r] + 8 * y_parts * U32 * np.abs(c)
        for i, s_ in enumerate((full * K + k).tolist()):
            if s_ in pure_rows:
                c[i] = pure_rows[s_]
        o_p = o_p + c
    assert (np.abs(og - o_h) <= o_b).all(), "out outside the bound of its own h"
    rms = float(np.sqrt(np.mean(o_p ** 2)))
    near_tok = sorted(set(s_ // K for s_ in near_flip_slots))
    flagged = np.isin(full, near_tok)
    err_hyb = rel(og, o_h, rms)
    err_pure = rel(og[~flagged], o_p[~flagged], rms) if (~flagged).any() else 0.0
    err_flag_pure = rel(og[flagged], o_p[flagged], rms) if flagged.any() else 0.0
    tok_err = np.max(np.abs(og - o_p), axis=1) / rms
    stats = {"rows_checked": int(n_chk), "h_other_rounding_elements": flips,
             "h_rows_with_other_roundings": flip_rows, "rows_codes_differ": len(pure_rows),
             "tokens_checked": len(full), "near_flip_tokens": len(near_tok),
             "err_y_vs_own_h": err_y, "max_y_err_over_bound": ratio_y,
             "err_out_vs_own_h": err_hyb, "err_out_pure": err_pure,
             "err_near_flip_vs_pure": err_flag_pure,
             "tokens_err_over_1e-2": int((tok_err > 1e-2).sum())}
    say("every-row check", contract, stats)
    return stats

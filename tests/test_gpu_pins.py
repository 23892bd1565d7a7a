"""GPU pins that need no tolerance argument: exact tie rules of the selection, the identical-experts
closed form, permutation equivariance, and exhaustive checks of the kernels' bf16 and E4M3
rounding routines against the oracle codecs.

Tie rules ([V] §MoE and residual stream; [H] §专家混合: 4 of 8 groups by the sum of their two best
biased scores, then the top 8 experts of those groups; ties, which the pages leave open, go to the
lower group and the lower expert index). With W_r = 0 every score is sigmoid(0) = 1/2 exactly, so
b = 1/2 + bias is exact in FP32 and in float64 when the bias lies on a 2^-10 grid: GPU and oracle
see the same numbers and every tie is a true tie, so the ids must agree exactly, in order. Identical
router rows give bit-identical FP32 logits on the GPU (each output of the router GEMM is computed the
same way), so copied rows plant ties with real scores too.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import codecs, experts, router

pytestmark = pytest.mark.gpu
SH = synthgen.BEAM_SHAPE


def _say(*a):
    parity.say(*a)


def _cfg():
    return bm.WorkloadCfg.of(SH, "bf16", "bf16")


def _route_exact(x, w_r, bias):
    ids, w = bm.route(x, w_r, bias, _cfg())
    torch.cuda.synchronize()
    r = router.route(x.cpu(), w_r.cpu(), bias.cpu(), SH.n_groups, SH.topk_groups, SH.topk,
                     SH.routed_scale)
    return ids.cpu().numpy(), w.cpu().numpy(), r


@pytest.mark.parametrize("T", [5, 100, 1100])
def test_all_ties(T):
    """W_r = 0, bias = 0: every expert scores 1/2, so groups 0-3 and experts 0-7 are chosen, in
    index order, each with weight 2.5 / 8."""
    x = synthgen.normal((T, SH.hidden), 1.0, 0, 1, "cuda", torch.bfloat16)
    w_r = torch.zeros((SH.n_experts, SH.hidden), dtype=torch.float32, device="cuda")
    bias = torch.zeros(SH.n_experts, dtype=torch.float32, device="cuda")
    ids, w, r = _route_exact(x, w_r, bias)
    assert (ids == np.arange(8)[None, :]).all(), ids[:2]
    assert (w == np.float32(2.5 / 8)).all()
    assert (r.ids == np.arange(8)[None, :]).all()


@pytest.mark.parametrize("T", [5, 100, 1100])
def test_planted_ties_on_an_exact_grid(T):
    """W_r = 0 and biases drawn from a handful of values on a 2^-10 grid: many equal scores inside
    and across groups and equal group scores; the GPU's ids must equal the oracle's exactly, in
    order, for 24 different bias vectors (the fused select-and-align launch, the partial-logit path
    and the one-pass router)."""
    x = synthgen.normal((T, SH.hidden), 1.0, 0, 1, "cuda", torch.bfloat16)
    w_r = torch.zeros((SH.n_experts, SH.hidden), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(T)
    n_group_ties = 0
    for trial in range(24):
        levels = rng.choice(np.arange(-16, 17), size=rng.integers(2, 6), replace=False)
        b = rng.choice(levels, size=SH.n_experts).astype(np.float64) * 2.0 ** -10
        bias = torch.tensor(b, dtype=torch.float32, device="cuda")
        ids, w, r = _route_exact(x, w_r, bias)
        assert np.array_equal(ids, r.ids.astype(np.int32)), (trial, ids[0], r.ids[0])
        assert np.all(np.abs(w - 2.5 / 8) == 0)
        gs = np.sort(r.group_score[0])[::-1]
        n_group_ties += int(gs[SH.topk_groups - 1] == gs[SH.topk_groups])
    _say("bias vectors with a tie at the group cut:", n_group_ties, "of 24")
    assert n_group_ties > 0


@pytest.mark.parametrize("T", [40, 200, 1100])
def test_ties_from_identical_router_rows(T):
    """Real scores with planted ties: groups 1 and 5 are copies of group 0 (equal group scores), and
    inside groups 2 and 6 every even expert's router row is copied to the next one. The GPU must pick
    the lower group and the lower expert index, exactly as the oracle."""
    x = synthgen.normal((T, SH.hidden), 1.0, 3, 1, "cuda", torch.bfloat16)
    w_r = synthgen.normal((SH.n_experts, SH.hidden), 0.02, 3, 2, "cuda")
    gs = SH.n_experts // SH.n_groups
    for g in (1, 5):
        w_r[g * gs:(g + 1) * gs] = w_r[0:gs]
    for g in (2, 6):
        for e in range(g * gs, (g + 1) * gs, 2):
            w_r[e + 1] = w_r[e]
    bias = torch.zeros(SH.n_experts, dtype=torch.float32, device="cuda")
    ids, w, r = _route_exact(x, w_r, bias)
    mism = [t for t in range(T) if not np.array_equal(ids[t], r.ids[t])]
    assert not mism, [(t, ids[t], r.ids[t]) for t in mism[:3]]
    chosen_groups = set((r.ids // gs).ravel().tolist())
    assert 0 in chosen_groups or not ({1, 5} & chosen_groups)   # a copy never beats group 0
    ties = int(sum(len(np.unique(r.b[t][r.ids[t]])) < SH.topk for t in range(T)))
    _say("tokens", T, "with tied experts among the chosen:", ties)
    assert ties > 0


@pytest.mark.parametrize("T", [64, 600])
def test_identical_experts_closed_form(T):
    """Every expert the same MLP: out = 2.5 * MLP(x) for any routing (bf16 contract, every token;
    T = 64 takes the decode kernels, T = 600 the tiled ones)."""
    d = synthgen.make_inputs("decode", device="cuda", T=T, with_experts=False)
    gu0 = synthgen.normal((2 * SH.d_ff, SH.hidden), 0.02, 0, 4, "cuda", torch.bfloat16)
    dn0 = synthgen.normal((SH.hidden, SH.d_ff), 0.02, 0, 5, "cuda", torch.bfloat16)
    wgu = gu0.unsqueeze(0).expand(SH.n_experts, -1, -1).contiguous()
    wdn = dn0.unsqueeze(0).expand(SH.n_experts, -1, -1).contiguous()
    out = bm.forward(d["x"], d["w_router"], d["bias"], wgu, wdn, _cfg())
    torch.cuda.synchronize()
    ex = experts.split_expert(gu0.cpu(), dn0.cpu(), SH.d_ff)
    ref = 2.5 * experts.expert_mlp(d["x"].cpu(), ex, "bf16")
    err, rms = parity.rel_err(out.cpu().numpy(), ref)
    _say("identical experts T", T, "max|err|/rms", err)
    assert err <= parity.TOL["bf16"]
    del wgu, wdn


@pytest.mark.parametrize("T", [32, 300])
def test_permutation_equivariance(T):
    """Permuting the tokens permutes the routes and the output, bit for bit (every token's routing
    and expert rows are computed independently of its position)."""
    W = synthgen.make_inputs("decode", device="cuda", T=1)
    d = synthgen.make_inputs("decode", device="cuda", T=T, with_experts=False)
    perm = torch.from_numpy(np.random.default_rng(T).permutation(T)).cuda()
    ids1 = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    ids2 = torch.empty_like(ids1)
    o1 = bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], _cfg(),
                    topk_ids_out=ids1)
    o2 = bm.forward(d["x"][perm].contiguous(), W["w_router"], d["bias"], W["w_gate_up"],
                    W["w_down"], _cfg(), topk_ids_out=ids2)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids1[perm])
    assert torch.equal(o2.view(torch.int32), o1[perm].view(torch.int32))
    del W


def _chunks(lo, hi, step):
    return [(a, min(a + step, hi)) for a in range(lo, hi, step)]


def _gpu_convert(bits_np, dtype):
    src = torch.from_numpy(bits_np.view(np.float32)).cuda()
    out = bm.convert(src, dtype)
    torch.cuda.synchronize()
    return out.view(torch.int16 if dtype == bm.BEAM_BF16 else torch.uint8).cpu().numpy()


def test_bf16_rounding_exhaustive():
    """The kernels' fp32 -> bf16 rounding against the oracle's bf16_round on every fp32 bit pattern
    in the oracle's domain: zero and every normal magnitude up to the largest bf16 (NaN, infinities,
    fp32 subnormals and magnitudes past the largest bf16 are outside it)."""
    hi_ok = np.float32((2.0 - 2.0 ** -7) * 2.0 ** 127)   # the largest bf16

    def oracle_bits(bits):
        v = bits.view(np.float32)
        a = np.abs(v)
        keep = (a == 0) | ((a >= np.float32(2.0 ** -126)) & (a <= hi_ok))
        r = codecs.bf16_round(v[keep].astype(np.float64)).astype(np.float32)
        return keep, (r.view(np.uint32) >> 16).astype(np.uint16)

    n_checked = 0
    chunks = _chunks(0, 1 << 32, 1 << 25)
    with cf.ThreadPoolExecutor(8) as pool:
        for i in range(0, len(chunks), 8):
            batch = [np.arange(lo, hi, dtype=np.uint64).astype(np.uint32) for lo, hi in chunks[i:i + 8]]
            futs = [pool.submit(oracle_bits, b) for b in batch]
            for bits, fut in zip(batch, futs):
                got = _gpu_convert(bits, bm.BEAM_BF16).view(np.uint16)
                keep, want = fut.result()
                g = got[keep]
                if not np.array_equal(g, want):
                    k = int(np.argmax(g != want))
                    raise AssertionError(
                        f"fp32 {bits[keep][k]:#010x}: GPU {g[k]:#06x} oracle {want[k]:#06x}")
                n_checked += int(keep.sum())
            if i % 32 == 0:
                _say("  bf16 patterns checked so far", n_checked)
    _say("bf16 rounding: fp32 patterns checked", n_checked)
    assert n_checked > 4_200_000_000


def test_e4m3_rounding_exhaustive():
    """The kernels' fp32 -> E4M3 encoder against the oracle's e4m3_encode on every fp32 value of
    magnitude below 1024 (both signs, zero and subnormals included), which spans every code, every
    rounding boundary, the saturation band 448..464 and beyond; larger magnitudes (which saturate
    by a single comparison) on a sample."""
    def oracle_codes(bits):
        return codecs.e4m3_encode(bits.view(np.float32).astype(np.float64))

    top = int(np.float32(1024.0).view(np.uint32))
    n_checked = 0
    chunks = [(lo, hi, sign) for sign in (0, 1 << 31) for lo, hi in _chunks(0, top, 1 << 25)]
    with cf.ThreadPoolExecutor(8) as pool:
        for i in range(0, len(chunks), 8):
            batch = [(np.arange(lo, hi, dtype=np.uint64) | sign).astype(np.uint32)
                     for lo, hi, sign in chunks[i:i + 8]]
            futs = [pool.submit(oracle_codes, b) for b in batch]
            for bits, fut in zip(batch, futs):
                got = _gpu_convert(bits, bm.BEAM_FP8_E4M3)
                want = fut.result()
                if not np.array_equal(got, want):
                    k = int(np.argmax(got != want))
                    raise AssertionError(
                        f"fp32 {bits[k]:#010x}: GPU {got[k]:#04x} oracle {want[k]:#04x}")
                n_checked += len(bits)
            if i % 16 == 0:
                _say("  E4M3 values checked so far", n_checked)
    big = np.random.default_rng(3).integers(top, int(np.float32(3e38).view(np.uint32)), 1 << 20,
                                            dtype=np.uint64).astype(np.uint32)
    big = np.concatenate([big, big | np.uint32(1 << 31)])
    assert np.array_equal(_gpu_convert(big, bm.BEAM_FP8_E4M3), oracle_codes(big))
    _say("E4M3 encoder: fp32 values checked", n_checked + len(big))


def test_fp8_instruction_summation_bound():
    """The bound the every-row FP8 checks assume for the FP8 matrix instruction (fullcheck.FP8_BLOCK_
    REL): each 16x16x128 E4M3 MFMA result lies within 2^-10 of its largest |product| of the exact
    sum (with the accumulator input added). Random finite codes over the whole range, codes of the
    magnitudes the kernels see (activations and weights scaled to +-448), and planted tiles with one
    large product among many small ones; exact sums in float64 on the host. Also shows that the
    instruction does not simply return the FP32 rounding of the exact sum."""
    import fullcheck
    rng = np.random.default_rng(11)
    lut = fullcheck.LUT_E4M3
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    scaled = np.array([c for c in finite if 6 <= (c >> 3) & 15 <= 14], dtype=np.uint8)
    n = 2048
    worst, n_fp32_exact, total = 0.0, 0, 0
    for kind in ("all", "scaled", "planted", "scaled+c"):
        pool = finite if kind == "all" else scaled
        a = rng.choice(pool, size=(n, 16, 128))
        b = rng.choice(pool, size=(n, 16, 128))
        c = np.zeros((n, 16, 16), dtype=np.float32)
        if kind == "planted":
            a[:] = 0x38
            b[:] = 0x38                                       # 1.0 x 1.0 everywhere ...
            k = rng.integers(0, 128, size=n)
            a[np.arange(n), :, k] = (7 + rng.integers(0, 9, size=(n, 16))) << 3   # ... but one 2^j
            b[np.arange(n), :, k] = (7 + rng.integers(0, 9, size=(n, 16))) << 3
        if kind == "scaled+c":
            c = rng.uniform(-1e6, 1e6, size=(n, 16, 16)).astype(np.float32)
        d = fp_tiles = bm.fp8_dot_tiles(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(),
                                        torch.from_numpy(c).cuda()).cpu().numpy().astype(np.float64)
        del fp_tiles
        av, bv = lut[a], lut[b]
        exact = np.einsum("tik,tjk->tij", av, bv) + c
        maxp = np.max(np.abs(av)[:, :, None, :] * np.abs(bv)[:, None, :, :], axis=3)
        worst = max(worst, float(np.max(np.abs(d - exact) / maxp)))
        n_fp32_exact += int(np.sum(d == exact.astype(np.float32)))
        total += d.size
    _say("FP8 MFMA: worst |error| / largest |product|", worst, "; results equal to the FP32 rounding",
         "of the exact sum:", n_fp32_exact, "of", total)
    assert worst <= fullcheck.FP8_BLOCK_REL
    assert n_fp32_exact < total

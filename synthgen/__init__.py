"""Seeded, counter-based synthetic inputs for the Beam routed-MoE block.

Every element of every tensor is a pure function of (seed, tensor id, flat index), computed with
integer hashing, one table lookup and correctly rounded IEEE operations only. The same bits
therefore come out on the CPU and on a GPU, so the CPU oracle and the HIP path can both be fed
from here (the GPU copy is generated on the device; any slice can be regenerated on the host).

This module holds none of the block's arithmetic: no routing, no expert math, no activation
quantisation. The FP8 *weights* are checkpoint data; they are produced here with torch's own
float8_e4m3fn cast, per output channel, as an input-preparation step.

Distributions (workload recipes of the five configurations the block is measured on):
  normal(sigma):   z = Q[h >> 16] * sigma in fp32, Q = fp32 table of standard-normal quantiles at
                   (j + 0.5) / 65536 (Wichura AS241 via Python's statistics.NormalDist), |z| <= 4.32.
  uniform(lo, hi): u = (h >> 8) * 2^-24 in [0, 1); v = fp32(lo + (hi - lo) * u), fp64 arithmetic.
  h = hash32((hash32(lo32(i) ^ key) + (hi32(i) * C) mod 2^32)), key = f(seed, tensor id),
  hash32 = the "lowbias32" integer finaliser (xorshift-multiply, constants 0x7feb352d / 0x846ca68b).
"""
from __future__ import annotations

import statistics
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "TENSOR_IDS", "BeamShape", "Workload", "WORKLOADS", "normal", "uniform", "fp8_rows",
    "hot_set", "make_inputs", "normal_table", "make_dense", "DENSE_D_FF",
]

TENSOR_IDS = dict(x=1, w_router=2, bias=3, w_gate_up=4, w_down=5, hot_set=6, dense_gate_up=7,
                  dense_down=8, residual=9)

_M32 = 0xFFFFFFFF


def _mul32(x, c: int):
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32), without int64 overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _hash32(x):
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    return x ^ (x >> 16)


def _hash32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    return x ^ (x >> 16)


def _key(seed: int, tid: int) -> int:
    k = _hash32_int((seed ^ 0x3C6EF372) & _M32)
    return _hash32_int(k ^ ((tid * 0x9E3779B9) & _M32))


def _bits(numel: int, seed: int, tid: int, offset: int, device) -> torch.Tensor:
    """32-bit hash values (in int64) for flat indices offset .. offset+numel-1."""
    i = torch.arange(offset, offset + numel, dtype=torch.int64, device=device)
    k = _key(seed, tid)
    h = _hash32((i & _M32) ^ k)
    return _hash32((h + _mul32(i >> 32, 0x632BE5AB)) & _M32)


_QTABLE_CACHE: dict = {}


def normal_table(device="cpu") -> torch.Tensor:
    """fp32 standard-normal quantiles at (j + 0.5) / 65536, j = 0..65535."""
    dev = torch.device(device)
    key = (dev.type, dev.index)
    if key not in _QTABLE_CACHE:
        if ("cpu", None) not in _QTABLE_CACHE:
            nd = statistics.NormalDist()
            q = np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)], dtype=np.float64)
            _QTABLE_CACHE[("cpu", None)] = torch.from_numpy(q.astype(np.float32))
        _QTABLE_CACHE[key] = _QTABLE_CACHE[("cpu", None)].to(dev)
    return _QTABLE_CACHE[key]


def normal(shape, sigma: float, seed: int, tid: int, device="cpu", dtype=torch.float32,
           offset: int = 0) -> torch.Tensor:
    """N(0, sigma^2) samples (16-bit quantile resolution), rounded to `dtype` (fp32 or bf16, RNE)."""
    n = int(np.prod(shape)) if len(shape) else 1
    h = _bits(n, seed, tid, offset, device)
    z = normal_table(device)[h >> 16]
    if sigma != 1.0:
        z = z * torch.tensor(sigma, dtype=torch.float32, device=device)
    return z.to(dtype).reshape(shape)


def uniform(shape, lo: float, hi: float, seed: int, tid: int, device="cpu",
            offset: int = 0) -> torch.Tensor:
    """U(lo, hi) samples as fp32."""
    n = int(np.prod(shape)) if len(shape) else 1
    h = _bits(n, seed, tid, offset, device)
    u = (h >> 8).to(torch.float64) * (2.0 ** -24)
    v = u * (hi - lo)
    v = v + lo
    return v.to(torch.float32).reshape(shape)


def fp8_rows(rows: int, cols: int, sigma: float, seed: int, tid: int, device="cpu",
             offset: int = 0):
    """FP8 E4M3FN checkpoint rows: fp32 N(0, sigma^2) weights quantised per row (output channel)
    with scale = amax / 448 and torch's own saturating cast. Returns (codes uint8 [rows][cols],
    scales fp32 [rows]). Rows with amax = 0 get scale 1."""
    w = normal((rows, cols), sigma, seed, tid, device, torch.float32, offset)
    amax = w.abs().amax(dim=1)
    s = amax / torch.tensor(448.0, dtype=torch.float32, device=device)
    s = torch.where(amax > 0, s, torch.ones_like(s))
    q = (w / s[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s


def hot_set(n_hot: int, n_experts: int, seed: int) -> list:
    """n_hot distinct expert ids, drawn without replacement: the experts with the smallest hash."""
    h = _bits(n_experts, seed, TENSOR_IDS["hot_set"], 0, "cpu")
    order = torch.argsort(h * n_experts + torch.arange(n_experts), stable=True)
    return sorted(int(e) for e in order[:n_hot])


@dataclass(frozen=True)
class BeamShape:
    hidden: int = 5120
    n_experts: int = 256
    n_groups: int = 8
    topk_groups: int = 4
    topk: int = 8
    d_ff: int = 2560
    routed_scale: float = 2.5


TINY_SHAPE = BeamShape(hidden=512, n_experts=32, n_groups=8, topk_groups=2, topk=4, d_ff=256)
BEAM_SHAPE = BeamShape()


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    shape: BeamShape
    x_dtype: str            # "f32" | "bf16"
    w_dtype: str            # "f32" | "bf16" | "fp8"
    bias: str               # "uniform" | "zero" | "skew"
    seed: int = 0
    sigma_w: float = 0.02
    n_hot: int = 16
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 64, TINY_SHAPE, "f32", "f32", "uniform",
                     notes="tiny MoE, FP32 throughout"),
    "decode": Workload("decode", 32, BEAM_SHAPE, "bf16", "bf16", "uniform",
                       notes="Beam MoE layer, decode batch T=32"),
    "prefill": Workload("prefill", 8192, BEAM_SHAPE, "bf16", "bf16", "zero",
                        notes="Beam MoE layer, prefill batch T=8192, bias 0"),
    "skew": Workload("skew", 32768, BEAM_SHAPE, "bf16", "bf16", "skew",
                     notes="T=32768, 16 hot experts take ~40% of the slots"),
    "fp8_decode": Workload("fp8_decode", 32, BEAM_SHAPE, "bf16", "fp8", "uniform",
                           notes="FP8 E4M3 experts, T=32"),
    "fp8_prefill": Workload("fp8_prefill", 8192, BEAM_SHAPE, "bf16", "fp8", "zero",
                            notes="FP8 E4M3 experts, T=8192"),
}


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_bias(wl: Workload, device="cpu", skew_delta: float | None = None) -> torch.Tensor:
    E = wl.shape.n_experts
    if wl.bias == "uniform":
        return uniform((E,), -0.1, 0.1, wl.seed, TENSOR_IDS["bias"], device)
    b = torch.zeros(E, dtype=torch.float32, device=device)
    if wl.bias == "skew":
        if skew_delta is None:
            raise ValueError("the skewed workload needs its bias offset delta")
        b[hot_set(wl.n_hot, E, wl.seed)] = float(np.float32(skew_delta))
    return b


def make_inputs(wl: Workload | str, device="cpu", T: int | None = None, with_experts=True,
                skew_delta: float | None = None, experts: list | None = None) -> dict:
    """Builds the inputs of one workload on `device`.

    x [T][H] (x_dtype), w_router [E][H] fp32, bias [E] fp32, and (if with_experts)
    w_gate_up [E][2F][H] and w_down [E][H][F] in w_dtype (fp8: uint8 codes plus fp32 scales
    w_gate_up_scale [E][2F], w_down_scale [E][H]). `experts` restricts generation to a subset of
    experts (dict of per-expert tensors instead of stacked ones), for host-side spot checks.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    sh = wl.shape
    T = wl.T if T is None else T
    H, E, F = sh.hidden, sh.n_experts, sh.d_ff
    out = {"workload": wl, "T": T}
    out["x"] = normal((T, H), 1.0, wl.seed, TENSOR_IDS["x"], device, _torch_dtype(wl.x_dtype))
    out["w_router"] = normal((E, H), wl.sigma_w, wl.seed, TENSOR_IDS["w_router"], device)
    out["bias"] = make_bias(wl, device, skew_delta)
    if not with_experts:
        return out
    fp8 = wl.w_dtype == "fp8"

    def gen(e):
        gu_off, dn_off = e * 2 * F * H, e * H * F
        tid_gu, tid_dn = TENSOR_IDS["w_gate_up"], TENSOR_IDS["w_down"]
        if fp8:
            return (fp8_rows(2 * F, H, wl.sigma_w, wl.seed, tid_gu, device, gu_off)
                    + fp8_rows(H, F, wl.sigma_w, wl.seed, tid_dn, device, dn_off))
        dt = _torch_dtype(wl.w_dtype)
        return (normal((2 * F, H), wl.sigma_w, wl.seed, tid_gu, device, dt, gu_off), None,
                normal((H, F), wl.sigma_w, wl.seed, tid_dn, device, dt, dn_off), None)

    if experts is None:
        wdt = torch.uint8 if fp8 else _torch_dtype(wl.w_dtype)
        out["w_gate_up"] = torch.empty((E, 2 * F, H), dtype=wdt, device=device)
        out["w_down"] = torch.empty((E, H, F), dtype=wdt, device=device)
        if fp8:
            out["w_gate_up_scale"] = torch.empty((E, 2 * F), dtype=torch.float32, device=device)
            out["w_down_scale"] = torch.empty((E, H), dtype=torch.float32, device=device)
        for e in range(E):
            gu, gus, dn, dns = gen(e)
            out["w_gate_up"][e].copy_(gu)
            out["w_down"][e].copy_(dn)
            if fp8:
                out["w_gate_up_scale"][e].copy_(gus)
                out["w_down_scale"][e].copy_(dns)
            del gu, gus, dn, dns
    else:
        parts = {e: gen(e) for e in experts}
        out["w_gate_up_e"] = {e: p[0] for e, p in parts.items()}
        out["w_down_e"] = {e: p[2] for e, p in parts.items()}
        if fp8:
            out["w_gate_up_scale_e"] = {e: p[1] for e, p in parts.items()}
            out["w_down_scale_e"] = {e: p[3] for e, p in parts.items()}
    return out


def expected_distinct_experts(T: int, E: int = 256, K: int = 8) -> float:
    """Uniform-routing expectation of the number of experts touched by T tokens (for reports)."""
    return E * (1.0 - (1.0 - K / E) ** T)


def skew_hot_fraction_target() -> tuple:
    """Share of slots the skewed workload aims to put on its hot experts, with its tolerance."""
    return 0.40, 0.005


def nbytes_gib(t: torch.Tensor) -> float:
    return t.numel() * t.element_size() / 2 ** 30



# Beam's dense MLP layers (the first three): d_ff 20480
DENSE_D_FF = 20480


def make_dense(T: int, hidden: int = 5120, d_ff: int = DENSE_D_FF, w_dtype: str = "bf16",
               device="cpu", seed: int = 0, sigma_w: float = 0.02) -> dict:
    """Inputs of one dense SwiGLU layer: x [T][hidden] bf16 N(0,1) (the same stream as the MoE
    workloads' x), w_gate_up [2 d_ff][hidden] and w_down [hidden][d_ff] N(0, sigma_w^2) in bf16, or
    as FP8 E4M3 codes with per-row scales (w_gate_up_scale, w_down_scale)."""
    out = {"T": T, "hidden": hidden, "d_ff": d_ff}
    out["x"] = normal((T, hidden), 1.0, seed, TENSOR_IDS["x"], device, torch.bfloat16)
    if w_dtype == "fp8":
        out["w_gate_up"], out["w_gate_up_scale"] = fp8_rows(
            2 * d_ff, hidden, sigma_w, seed, TENSOR_IDS["dense_gate_up"], device)
        out["w_down"], out["w_down_scale"] = fp8_rows(
            hidden, d_ff, sigma_w, seed, TENSOR_IDS["dense_down"], device)
    else:
        out["w_gate_up"] = normal((2 * d_ff, hidden), sigma_w, seed, TENSOR_IDS["dense_gate_up"],
                                  device, torch.bfloat16)
        out["w_down"] = normal((hidden, d_ff), sigma_w, seed, TENSOR_IDS["dense_down"], device,
                               torch.bfloat16)
    return out

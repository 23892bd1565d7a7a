"""Python binding of libbeam_moe.so, the Beam routed-MoE block on MI355X (gfx950).

Argument marshalling only: every step of the block runs in the library's HIP kernels. torch
supplies device memory and the current stream. The functions mirror the C ABI in
include/beam_moe.h (same names, same argument meaning). If the shared library is missing the
import still works, but every call raises: there is no CPU fallback.

Sources of the method (cited by tag and section in the library):
  [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API"
  [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持"
  [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可"
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "BEAM_F32", "BEAM_BF16", "BEAM_FP8_E4M3", "Cfg", "make_cfg", "lib", "lib_path", "route",
    "forward", "workspace_bytes", "route_workspace_bytes", "BeamError", "timing_enable",
    "timing_collect", "STAGES", "status_string", "quant_fp8", "forward_routed", "dense_mlp",
    "dense_workspace_bytes", "residual_boundary", "forward_boundary", "workspace_region",
    "workspace_view", "WS_REGIONS", "convert", "dense_workspace_region", "fp8_dot_tiles",
    "forward_noalloc",
]

BEAM_F32, BEAM_BF16, BEAM_FP8_E4M3 = 0, 1, 2
_DT_CODE = {torch.float32: BEAM_F32, torch.bfloat16: BEAM_BF16, torch.uint8: BEAM_FP8_E4M3,
            torch.float8_e4m3fn: BEAM_FP8_E4M3}
STAGES = ["router_logits", "router_select", "moe_align", "quant_x_fp8", "gate_up", "quant_h_fp8",
          "down", "combine"]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libbeam_moe.so")


class BeamError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


class Cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("x_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


def make_cfg(hidden=5120, n_experts=256, n_groups=8, topk_groups=4, topk=8, d_ff=2560,
             routed_scale=2.5, x_dtype=BEAM_BF16, w_dtype=BEAM_BF16, out_dtype=BEAM_F32) -> Cfg:
    return Cfg(hidden, n_experts, n_groups, topk_groups, topk, d_ff, routed_scale, x_dtype,
               w_dtype, out_dtype)


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded shared library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with "
                               "`python -m routing_grouped_expert_fp32_amd.build` "
                               "(there is no fallback path)")
        L = ctypes.CDLL(lib_path)
        vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32
        cfgp = ctypes.POINTER(Cfg)
        L.beam_moe_route.argtypes = [vp, vp, vp, vp, vp, i64, cfgp, vp, sz, vp]
        L.beam_moe_route.restype = i32
        L.beam_moe_forward.argtypes = [vp, vp, vp, vp, vp, vp, i64, cfgp, vp, vp, vp, vp, vp, sz,
                                       vp]
        L.beam_moe_forward.restype = i32
        L.beam_moe_workspace_bytes.argtypes = [cfgp, i64]
        L.beam_moe_workspace_bytes.restype = sz
        L.beam_moe_route_workspace_bytes.argtypes = [cfgp, i64]
        L.beam_moe_route_workspace_bytes.restype = sz
        L.beam_status_string.argtypes = [i32]
        L.beam_status_string.restype = ctypes.c_char_p
        L.beam_moe_version.argtypes = []
        L.beam_moe_version.restype = i32
        L.beam_moe_timing_enable.argtypes = [i32]
        L.beam_moe_timing_enable.restype = None
        L.beam_moe_timing_stages.argtypes = [ctypes.c_uint32]
        L.beam_moe_timing_stages.restype = None
        L.beam_moe_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(i32), i32]
        L.beam_moe_timing_collect.restype = i32
        L.beam_moe_stage_name.argtypes = [i32]
        L.beam_moe_stage_name.restype = ctypes.c_char_p
        L.beam_moe_forward_routed.argtypes = [vp, vp, vp, vp, vp, vp, i64, cfgp, i32, i32, vp,
                                              vp, vp, sz, vp]
        L.beam_moe_forward_routed.restype = i32
        L.beam_dense_mlp_forward.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, vp,
                                             sz, vp]
        L.beam_dense_mlp_forward.restype = i32
        L.beam_dense_mlp_workspace_bytes.argtypes = [i32, i32, i32, i64]
        L.beam_dense_mlp_workspace_bytes.restype = sz
        f32 = ctypes.c_float
        L.beam_residual_boundary.argtypes = [vp, i32, vp, vp, vp, vp, vp, i64, i32, i32, f32, vp]
        L.beam_residual_boundary.restype = i32
        L.beam_moe_forward_boundary.argtypes = [vp, vp, vp, vp, vp, i64, cfgp, vp, vp, vp, vp, vp,
                                                i32, f32, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_forward_boundary.restype = i32
        L.beam_moe_quant_fp8.argtypes = [vp, i64, i32, vp, vp, vp]
        L.beam_moe_quant_fp8.restype = i32
        L.beam_moe_workspace_region.argtypes = [cfgp, i64, i32, ctypes.POINTER(sz),
                                                ctypes.POINTER(sz)]
        L.beam_moe_workspace_region.restype = i32
        L.beam_dense_mlp_workspace_region.argtypes = [i32, i32, i32, i64, i32,
                                                      ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.beam_dense_mlp_workspace_region.restype = i32
        L.beam_moe_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, cfgp, vp, vp, vp, vp,
                                               vp]
        L.beam_moe_forward_noalloc.restype = i32
        L.beam_moe_fp8_dot_tiles.argtypes = [vp, vp, vp, vp, i64, vp]
        L.beam_moe_fp8_dot_tiles.restype = i32
        L.beam_moe_convert.argtypes = [vp, i64, i32, vp, vp]
        L.beam_moe_convert.restype = i32
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    try:
        return lib().beam_status_string(status).decode()
    except RuntimeError:
        return "library not loaded"


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_bytes(cfg: Cfg, T: int) -> int:
    return int(lib().beam_moe_workspace_bytes(ctypes.byref(cfg), T))


def route_workspace_bytes(cfg: Cfg, T: int) -> int:
    return int(lib().beam_moe_route_workspace_bytes(ctypes.byref(cfg), T))


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def route(x, w_router, bias, cfg: Cfg, topk_ids=None, topk_w=None, workspace=None, stream=None):
    """beam_moe_route: returns (topk_ids int32 [T][K], topk_w fp32 [T][K])."""
    T = x.shape[0]
    if topk_ids is None:
        topk_ids = torch.empty((T, cfg.topk), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, cfg.topk), dtype=torch.float32, device=x.device)
    nbytes = route_workspace_bytes(cfg, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check_dev(x, w_router, bias, topk_ids, topk_w, workspace)
    rc = lib().beam_moe_route(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_ids), _ptr(topk_w),
                              T, ctypes.byref(cfg), _ptr(workspace), workspace.numel(),
                              _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_route")
    return topk_ids, topk_w


def forward(x, w_router, bias, w_gate_up, w_down, cfg: Cfg, out=None, w_gate_up_scale=None,
            w_down_scale=None, topk_ids_out=None, topk_w_out=None, workspace=None, stream=None):
    """beam_moe_forward: returns out [T][H] (fp32 unless cfg.out_dtype is bf16)."""
    T = x.shape[0]
    if out is None:
        odt = torch.bfloat16 if cfg.out_dtype == BEAM_BF16 else torch.float32
        out = torch.empty((T, cfg.hidden), dtype=odt, device=x.device)
    nbytes = workspace_bytes(cfg, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check_dev(x, w_router, bias, w_gate_up, w_down, out, w_gate_up_scale, w_down_scale,
               topk_ids_out, topk_w_out, workspace)
    rc = lib().beam_moe_forward(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up),
                                _ptr(w_down), _ptr(out), T, ctypes.byref(cfg),
                                _ptr(w_gate_up_scale), _ptr(w_down_scale), _ptr(topk_ids_out),
                                _ptr(topk_w_out), _ptr(workspace), workspace.numel(),
                                _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_forward")
    return out


def forward_noalloc(x, w_router, bias, w_gate_up, w_down, cfg: Cfg, out=None, w_gate_up_scale=None,
                    w_down_scale=None, topk_ids_out=None, topk_w_out=None, stream=None):
    """beam_moe_forward_noalloc: beam_moe_forward on the library's own per-GPU workspace."""
    T = x.shape[0]
    if out is None:
        odt = torch.bfloat16 if cfg.out_dtype == BEAM_BF16 else torch.float32
        out = torch.empty((T, cfg.hidden), dtype=odt, device=x.device)
    _check_dev(x, w_router, bias, w_gate_up, w_down, out, w_gate_up_scale, w_down_scale,
               topk_ids_out, topk_w_out)
    rc = lib().beam_moe_forward_noalloc(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up),
                                        _ptr(w_down), _ptr(out), T, ctypes.byref(cfg),
                                        _ptr(w_gate_up_scale), _ptr(w_down_scale),
                                        _ptr(topk_ids_out), _ptr(topk_w_out), _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_forward_noalloc")
    return out


def forward_routed(x, topk_ids, topk_w, w_gate_up, w_down, cfg: Cfg, expert_begin: int = 0,
                   expert_end: int | None = None, out=None, w_gate_up_scale=None,
                   w_down_scale=None, workspace=None, stream=None):
    """beam_moe_forward_routed: out [T][H] from given routes over experts [expert_begin,
    expert_end); w_gate_up / w_down (and the FP8 scales) hold only those experts."""
    T = x.shape[0]
    if expert_end is None:
        expert_end = cfg.n_experts
    if out is None:
        odt = torch.bfloat16 if cfg.out_dtype == BEAM_BF16 else torch.float32
        out = torch.empty((T, cfg.hidden), dtype=odt, device=x.device)
    nbytes = workspace_bytes(cfg, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check_dev(x, topk_ids, topk_w, w_gate_up, w_down, out, w_gate_up_scale, w_down_scale,
               workspace)
    rc = lib().beam_moe_forward_routed(_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gate_up),
                                       _ptr(w_down), _ptr(out), T, ctypes.byref(cfg),
                                       int(expert_begin), int(expert_end), _ptr(w_gate_up_scale),
                                       _ptr(w_down_scale), _ptr(workspace), workspace.numel(),
                                       _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_forward_routed")
    return out


def dense_workspace_bytes(hidden: int, d_ff: int, w_dtype: int, T: int) -> int:
    return int(lib().beam_dense_mlp_workspace_bytes(hidden, d_ff, w_dtype, T))


def dense_mlp(x, w_gate_up, w_down, out=None, out_dtype=BEAM_F32, w_gate_up_scale=None,
              w_down_scale=None, workspace=None, stream=None):
    """beam_dense_mlp_forward: out [T][hidden] = down(silu(gate x) * up x) for bf16 x."""
    T, H = x.shape
    F = w_gate_up.shape[0] // 2
    wdt = _DT_CODE[w_gate_up.dtype]
    if out is None:
        odt = torch.bfloat16 if out_dtype == BEAM_BF16 else torch.float32
        out = torch.empty((T, H), dtype=odt, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(dense_workspace_bytes(H, F, wdt, T), 16), dtype=torch.uint8,
                                device=x.device)
    _check_dev(x, w_gate_up, w_down, out, w_gate_up_scale, w_down_scale, workspace)
    rc = lib().beam_dense_mlp_forward(_ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(out), T, H, F,
                                      wdt, out_dtype, _ptr(w_gate_up_scale), _ptr(w_down_scale),
                                      _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_dense_mlp_forward")
    return out


def residual_boundary(y, h, gamma_post, gamma_next, depth_n: int, eps: float, h_out=None,
                      x_next=None, stream=None):
    """beam_residual_boundary: returns (h_out, x_next), both bf16 [T][hidden]."""
    T, H = h.shape
    if h_out is None:
        h_out = torch.empty_like(h)
    if x_next is None:
        x_next = torch.empty_like(h)
    _check_dev(y, h, gamma_post, gamma_next, h_out, x_next)
    rc = lib().beam_residual_boundary(_ptr(y), _DT_CODE[y.dtype], _ptr(h), _ptr(gamma_post),
                                      _ptr(gamma_next), _ptr(h_out), _ptr(x_next), T, H,
                                      int(depth_n), float(eps), _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_residual_boundary")
    return h_out, x_next


def forward_boundary(x, w_router, bias, w_gate_up, w_down, cfg: Cfg, h, gamma_post, gamma_next,
                     depth_n: int, eps: float, h_out=None, x_next=None, w_gate_up_scale=None,
                     w_down_scale=None, topk_ids_out=None, topk_w_out=None, workspace=None,
                     stream=None):
    """beam_moe_forward_boundary: the MoE block with its combine fused into the following
    norm -> residual -> norm boundary; returns (h_out, x_next)."""
    T = x.shape[0]
    if h_out is None:
        h_out = torch.empty_like(h)
    if x_next is None:
        x_next = torch.empty_like(h)
    nbytes = workspace_bytes(cfg, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check_dev(x, w_router, bias, w_gate_up, w_down, h, gamma_post, gamma_next, h_out, x_next,
               w_gate_up_scale, w_down_scale, topk_ids_out, topk_w_out, workspace)
    rc = lib().beam_moe_forward_boundary(
        _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, ctypes.byref(cfg),
        _ptr(w_gate_up_scale), _ptr(w_down_scale), _ptr(h), _ptr(gamma_post), _ptr(gamma_next),
        int(depth_n), float(eps), _ptr(h_out), _ptr(x_next), _ptr(topk_ids_out), _ptr(topk_w_out),
        _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_forward_boundary")
    return h_out, x_next


def quant_fp8(src, codes=None, scales=None, stream=None):
    """beam_moe_quant_fp8 on bf16 rows src [rows][cols]: returns (codes uint8, scales fp32)."""
    rows, cols = src.shape
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=src.device)
    _check_dev(src, codes, scales)
    rc = lib().beam_moe_quant_fp8(_ptr(src), rows, cols, _ptr(codes), _ptr(scales),
                                  _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_quant_fp8")
    return codes, scales


def convert(src, dst_dtype: int, dst=None, stream=None):
    """beam_moe_convert: fp32 [n] -> bf16 (BEAM_BF16, returned as torch.bfloat16) or E4M3 codes
    (BEAM_FP8_E4M3, returned as uint8) with the kernels' rounding routines."""
    n = src.numel()
    if dst is None:
        dt = torch.bfloat16 if dst_dtype == BEAM_BF16 else torch.uint8
        dst = torch.empty(src.shape, dtype=dt, device=src.device)
    _check_dev(src, dst)
    rc = lib().beam_moe_convert(_ptr(src), n, dst_dtype, _ptr(dst), _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_convert")
    return dst


def fp8_dot_tiles(a, b, c, stream=None):
    """beam_moe_fp8_dot_tiles on uint8 codes a, b [n][16][128] and fp32 c [n][16][16]: returns d."""
    d = torch.empty_like(c)
    _check_dev(a, b, c, d)
    rc = lib().beam_moe_fp8_dot_tiles(_ptr(a), _ptr(b), _ptr(c), _ptr(d), a.shape[0],
                                      _stream(stream))
    if rc != 0:
        raise BeamError(rc, "beam_moe_fp8_dot_tiles")
    return d


WS_REGIONS = {"expert_off": 0, "sorted_slot": 1, "h": 2, "hq": 3, "hs": 4, "xq": 5, "xs": 6,
              "y": 7}


def workspace_region(cfg: Cfg, T: int, region: str) -> tuple:
    """beam_moe_workspace_region: (byte offset, bytes) of an intermediate array in a forward's
    workspace (names as in WS_REGIONS)."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib().beam_moe_workspace_region(ctypes.byref(cfg), T, WS_REGIONS[region],
                                         ctypes.byref(off), ctypes.byref(n))
    if rc != 0:
        raise BeamError(rc, "beam_moe_workspace_region")
    return off.value, n.value


def dense_workspace_region(hidden: int, d_ff: int, w_dtype: int, T: int, region: str) -> tuple:
    """beam_dense_mlp_workspace_region: (byte offset, bytes) of an intermediate array."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib().beam_dense_mlp_workspace_region(hidden, d_ff, w_dtype, T, WS_REGIONS[region],
                                               ctypes.byref(off), ctypes.byref(n))
    if rc != 0:
        raise BeamError(rc, "beam_dense_mlp_workspace_region")
    return off.value, n.value


def workspace_view(workspace, cfg: Cfg, T: int, region: str, dtype, dense: bool = False):
    """A flat torch view (no copy) of one intermediate array inside a forward's workspace (of
    beam_dense_mlp_forward when dense is set; cfg then gives hidden, d_ff and w_dtype)."""
    if dense:
        off, n = dense_workspace_region(cfg.hidden, cfg.d_ff, cfg.w_dtype, T, region)
    else:
        off, n = workspace_region(cfg, T, region)
    return workspace[off:off + n].view(dtype)


def timing_enable(on: bool = True, stages=None) -> None:
    """Turn stage timing on or off; `stages` (names from STAGES) limits which stages record events
    (None: all)."""
    mask = 0xFFFFFFFF if stages is None else sum(1 << STAGES.index(n) for n in stages)
    lib().beam_moe_timing_stages(mask)
    lib().beam_moe_timing_enable(1 if on else 0)


def timing_collect() -> dict:
    """{stage name: (total ms, launches)} of the calls made since timing was enabled."""
    n = len(STAGES)
    tot = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    lib().beam_moe_timing_collect(tot, cnt, n)
    return {STAGES[i]: (tot[i], cnt[i]) for i in range(n)}


@dataclass
class WorkloadCfg:
    """Helper: cfg of a synthgen workload shape."""

    @staticmethod
    def of(shape, x_dtype: str, w_dtype: str, out_dtype: str = "f32") -> Cfg:
        code = {"f32": BEAM_F32, "bf16": BEAM_BF16, "fp8": BEAM_FP8_E4M3}
        return make_cfg(shape.hidden, shape.n_experts, shape.n_groups, shape.topk_groups,
                        shape.topk, shape.d_ff, shape.routed_scale, code[x_dtype], code[w_dtype],
                        code[out_dtype])

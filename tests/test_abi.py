"""The C-ABI library loads, exports every symbol include/beam_moe.h declares, and rejects bad
arguments with the documented status before any launch (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import routing_grouped_expert_fp32_amd as bm

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "beam_moe.h")

OK, NULL, ALIGN, SHAPE, DTYPE, UNSUP, WS, ALIAS, LAUNCH, DEVICE = range(10)


def _declared():
    text = open(HEADER).read()
    return re.findall(r"BEAM_API\s+[\w\s\*]+?\b(beam_\w+)\s*\(", text)


def test_header_declares_entry_points():
    names = _declared()
    for n in ["beam_moe_route", "beam_moe_forward", "beam_moe_workspace_bytes",
              "beam_moe_route_workspace_bytes", "beam_status_string", "beam_moe_version",
              "beam_moe_forward_routed", "beam_moe_quant_fp8"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = bm.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.beam_moe_version() >= 100
    for s in range(10):
        assert bm.status_string(s) not in ("", "unknown status")


def _cfg(**kw):
    return bm.make_cfg(**kw)


# fake, aligned device addresses: validation rejects the call before anything dereferences them
A = [(i + 1) << 40 for i in range(12)]   # 1 TiB apart: no accidental overlap


def _gpu_visible():
    """True where HIP could see a GPU (the kernel driver's device node exists, or torch sees one).
    Calls that pass validation with fake addresses would then reach a kernel launch, so the tests
    that make them run only where the library must answer BEAM_ERR_DEVICE instead."""
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def _fwd(cfg, T=32, x=A[0], wr=A[1], bias=A[2], wgu=A[3], wd=A[4], out=A[5], gus=None, ds=None,
         ids=None, w=None, ws=A[8], ws_bytes=1 << 38):
    lib = bm.lib()
    return lib.beam_moe_forward(x, wr, bias, wgu, wd, out, T,
                                ctypes.byref(cfg) if cfg is not None else None, gus, ds, ids, w,
                                ws, ws_bytes, None)


def _route(cfg, T=32, x=A[0], wr=A[1], bias=A[2], ids=A[6], w=A[7], ws=A[8], ws_bytes=1 << 38):
    return bm.lib().beam_moe_route(x, wr, bias, ids, w, T,
                                   ctypes.byref(cfg) if cfg is not None else None, ws, ws_bytes,
                                   None)


def test_null_cfg_and_pointers():
    assert _fwd(None) == NULL
    assert _route(None) == NULL
    c = _cfg()
    assert _fwd(c, x=None) == NULL
    assert _fwd(c, wd=None) == NULL
    assert _fwd(c, ws=None) == NULL
    assert _route(c, ids=None) == NULL


def test_shape_errors():
    assert _fwd(_cfg(n_groups=7)) == SHAPE                 # 256 % 7
    assert _fwd(_cfg(topk_groups=9)) == SHAPE              # more kept groups than groups
    assert _fwd(_cfg(topk=200)) == SHAPE                   # K > Gk * E / G
    assert _fwd(_cfg(routed_scale=0.0)) == SHAPE
    assert _fwd(_cfg(routed_scale=float("nan"))) == SHAPE
    assert _fwd(_cfg(), T=-1) == SHAPE
    assert _route(_cfg(), T=-5) == SHAPE


def test_dtype_errors():
    assert _fwd(_cfg(x_dtype=7)) == DTYPE
    assert _fwd(_cfg(out_dtype=bm.BEAM_FP8_E4M3)) == DTYPE
    assert _fwd(_cfg(x_dtype=bm.BEAM_F32, w_dtype=bm.BEAM_BF16)) == DTYPE
    assert _fwd(_cfg(x_dtype=bm.BEAM_BF16, w_dtype=bm.BEAM_F32)) == DTYPE
    assert _fwd(_cfg(), gus=A[9]) == DTYPE                 # scales only with fp8 weights


def test_unsupported_shapes():
    assert _fwd(_cfg(hidden=5000)) == UNSUP
    assert _fwd(_cfg(d_ff=2500)) == UNSUP
    assert _fwd(_cfg(n_experts=512, n_groups=8)) == UNSUP
    assert _fwd(_cfg(topk=17, topk_groups=8)) == UNSUP
    big_T = (1 << 31) // 5120 + 1                          # bf16 x of 4 GiB or more
    assert _fwd(_cfg(), T=big_T) == UNSUP
    assert _fwd(_cfg(), T=big_T - 1, ws_bytes=0) == WS      # one token less passes the size check


def test_zero_tokens_is_a_noop():
    assert _fwd(_cfg(), T=0) == OK
    assert _route(_cfg(), T=0) == OK
    assert _fwd(_cfg(), T=0, x=None, out=None, ws=None) == OK


def test_alignment():
    assert _fwd(_cfg(), x=A[0] + 2) == ALIGN
    assert _fwd(_cfg(), out=A[5] + 8) == ALIGN
    assert _fwd(_cfg(), ids=A[6] + 4) == ALIGN
    assert _route(_cfg(), w=A[7] + 4) == ALIGN


def test_workspace_size():
    c = _cfg()
    need = bm.workspace_bytes(c, 32)
    assert need > 0
    assert _fwd(c, ws_bytes=need - 1) == WS
    assert bm.workspace_bytes(_cfg(n_groups=7), 32) == 0
    rneed = bm.route_workspace_bytes(c, 32)
    assert 0 < rneed < need
    assert _route(c, ws_bytes=rneed - 1) == WS


def test_aliasing():
    c = _cfg()
    assert _fwd(c, out=A[0]) == ALIAS                      # out on top of x
    assert _fwd(c, out=A[8]) == ALIAS                      # out inside the workspace
    assert _fwd(c, ids=A[5]) == ALIAS                      # routing copy on top of out
    assert _route(c, ids=A[7], w=A[7]) == ALIAS


def test_valid_call_without_gpu_reports_device():
    """A fully valid call on a machine with no gfx950 device fails loudly, it never falls back."""
    if _gpu_visible():
        pytest.skip("a GPU is present")
    assert _fwd(_cfg()) == DEVICE
    assert _route(_cfg()) == DEVICE


def test_quant_fp8_validation():
    q = bm.lib().beam_moe_quant_fp8
    assert q(A[0], -1, 5120, A[1], A[2], None) == SHAPE
    assert q(A[0], 4, 0, A[1], A[2], None) == SHAPE
    assert q(A[0], 4, 100, A[1], A[2], None) == UNSUP           # cols % 8
    assert q(A[0], 0, 5120, None, None, None) == OK             # no rows: no-op
    assert q(None, 4, 5120, A[1], A[2], None) == NULL
    assert q(A[0] + 2, 4, 5120, A[1], A[2], None) == ALIGN
    assert q(A[0], 4, 5120, A[0], A[2], None) == ALIAS          # codes on top of the source


def _routed(cfg, T=32, x=A[0], ids=A[6], w=A[7], wgu=A[3], wd=A[4], out=A[5], begin=0, end=256,
            gus=None, ds=None, ws=A[8], ws_bytes=1 << 38):
    return bm.lib().beam_moe_forward_routed(x, ids, w, wgu, wd, out, T,
                                            ctypes.byref(cfg) if cfg is not None else None,
                                            begin, end, gus, ds, ws, ws_bytes, None)


def test_forward_routed_validation():
    c = _cfg()
    assert "beam_moe_forward_routed" in _declared()
    assert _routed(None) == NULL
    assert _routed(c, ids=None) == NULL
    assert _routed(c, w=None) == NULL
    assert _routed(c, begin=-1) == SHAPE
    assert _routed(c, begin=5, end=4) == SHAPE
    assert _routed(c, end=257) == SHAPE
    assert _routed(c, T=-1) == SHAPE
    assert _routed(c, T=0, x=None, out=None, ws=None) == OK
    assert _routed(c, gus=A[9]) == DTYPE
    fp8 = _cfg(w_dtype=bm.BEAM_FP8_E4M3)
    assert _routed(fp8) == NULL                              # fp8 needs both scale arrays
    assert _routed(c, ids=A[6] + 4) == ALIGN
    assert _routed(c, ws_bytes=bm.workspace_bytes(c, 32) - 1) == WS
    assert _routed(c, out=A[6]) == ALIAS                     # out on top of the routes
    assert _routed(c, out=A[8]) == ALIAS                     # out inside the workspace


def test_forward_routed_without_gpu_reports_device():
    if _gpu_visible():
        pytest.skip("a GPU is present")
    assert _routed(_cfg()) == DEVICE
    assert _routed(_cfg(), begin=32, end=64) == DEVICE
    assert _routed(_cfg(), begin=7, end=7) == DEVICE         # empty range: valid (zeros)


def test_forward_routed_empty_range_needs_no_weights():
    if _gpu_visible():
        pytest.skip("a GPU is present")
    assert _routed(_cfg(), begin=9, end=9, wgu=None, wd=None) == DEVICE   # passes validation
    assert _routed(_cfg(), begin=9, end=10, wgu=None) == NULL


def _dense(T=32, x=A[0], wgu=A[3], wd=A[4], out=A[5], H=5120, F=20480, wdt=bm.BEAM_BF16,
           odt=bm.BEAM_F32, gus=None, ds=None, ws=A[8], ws_bytes=1 << 38):
    return bm.lib().beam_dense_mlp_forward(x, wgu, wd, out, T, H, F, wdt, odt, gus, ds, ws,
                                           ws_bytes, None)


def test_dense_mlp_validation():
    names = _declared()
    assert "beam_dense_mlp_forward" in names and "beam_dense_mlp_workspace_bytes" in names
    assert _dense(T=-1) == SHAPE
    assert _dense(H=0) == SHAPE
    assert _dense(wdt=bm.BEAM_F32) == DTYPE
    assert _dense(odt=bm.BEAM_FP8_E4M3) == DTYPE
    assert _dense(gus=A[9]) == DTYPE                        # scales only with fp8 weights
    assert _dense(H=5000) == UNSUP
    assert _dense(F=20000) == UNSUP
    assert _dense(H=65536, F=65536) == UNSUP                # hidden * d_ff >= 2^31
    assert _dense(T=(1 << 31) // 5120 + 1) == UNSUP         # bf16 x of 4 GiB or more
    assert _dense(T=0, x=None, out=None, ws=None) == OK
    assert _dense(x=None) == NULL
    assert _dense(wdt=bm.BEAM_FP8_E4M3) == NULL             # fp8 needs both scale arrays
    assert _dense(out=A[5] + 4) == ALIGN
    need = bm.dense_workspace_bytes(5120, 20480, bm.BEAM_BF16, 32)
    assert need > 0 and bm.dense_workspace_bytes(5000, 20480, bm.BEAM_BF16, 32) == 0
    assert _dense(ws_bytes=need - 1) == WS
    assert _dense(out=A[0]) == ALIAS


def test_dense_mlp_without_gpu_reports_device():
    if _gpu_visible():
        pytest.skip("a GPU is present")
    assert _dense() == DEVICE


def _bnd(y=A[0], ydt=bm.BEAM_F32, h=A[1], gp=A[2], gn=A[3], ho=A[4], xn=A[5], T=32, H=5120,
         n=7, eps=1e-6):
    return bm.lib().beam_residual_boundary(y, ydt, h, gp, gn, ho, xn, T, H, n, ctypes.c_float(eps),
                                           None)


def _fbnd(cfg, T=32, h=A[9], ho=A[10], xn=A[11], n=7, eps=1e-6, ws_bytes=1 << 38):
    return bm.lib().beam_moe_forward_boundary(A[0], A[1], A[2], A[3], A[4], T,
                                              ctypes.byref(cfg) if cfg is not None else None,
                                              None, None, h, A[5], A[6], n, ctypes.c_float(eps),
                                              ho, xn, None, None, A[8], ws_bytes, None)


def test_boundary_validation():
    names = _declared()
    assert "beam_residual_boundary" in names and "beam_moe_forward_boundary" in names
    assert _bnd(T=-1) == SHAPE
    assert _bnd(n=0) == SHAPE
    assert _bnd(eps=-1.0) == SHAPE
    assert _bnd(eps=float("nan")) == SHAPE
    assert _bnd(ydt=bm.BEAM_FP8_E4M3) == DTYPE
    assert _bnd(H=5000) == UNSUP
    assert _bnd(H=16384 + 256) == UNSUP                    # above the boundary kernel's width
    assert _bnd(T=0, y=None, h=None, ho=None, xn=None) == OK
    assert _bnd(y=None) == NULL
    assert _bnd(gn=None) == NULL
    assert _bnd(xn=A[5] + 2) == ALIGN
    assert _bnd(xn=A[0]) == ALIAS                          # x_next on top of y
    assert _bnd(ho=A[5]) == ALIAS                          # h_out on top of x_next
    assert _bnd(ho=A[1] + 1024) == ALIAS                   # h_out partly over h
    c = _cfg()
    assert _fbnd(None) == NULL
    assert _fbnd(_cfg(x_dtype=bm.BEAM_F32, w_dtype=bm.BEAM_F32)) == DTYPE
    assert _fbnd(c, n=0) == SHAPE
    assert _fbnd(c, h=None) == NULL
    assert _fbnd(c, ws_bytes=bm.workspace_bytes(c, 32) - 1) == WS
    assert _fbnd(c, xn=A[8]) == ALIAS                      # x_next inside the workspace


def test_boundary_without_gpu_reports_device():
    if _gpu_visible():
        pytest.skip("a GPU is present")
    assert _bnd() == DEVICE
    assert _bnd(ho=A[1]) == DEVICE                         # in place: valid
    assert _fbnd(_cfg()) == DEVICE


def test_workspace_region_and_convert_validation():
    lib = bm.lib()
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    cfg = _cfg()
    # regions of a bf16 forward; FP8 regions only with FP8 experts
    T = 100
    seen = []
    for reg in range(8):
        rc = lib.beam_moe_workspace_region(ctypes.byref(cfg), T, reg, ctypes.byref(off),
                                           ctypes.byref(n))
        if reg in (3, 4, 5, 6):
            assert rc == UNSUP
            continue
        assert rc == OK and off.value % 256 == 0 and n.value > 0
        seen.append((off.value, off.value + n.value))
    total = bm.workspace_bytes(cfg, T)
    seen.sort()
    assert all(a[1] <= b[0] for a, b in zip(seen, seen[1:])) and seen[-1][1] <= total
    f8 = _cfg(w_dtype=bm.BEAM_FP8_E4M3)
    for reg in range(8):
        assert lib.beam_moe_workspace_region(ctypes.byref(f8), T, reg, ctypes.byref(off),
                                             ctypes.byref(n)) == OK
        assert off.value + n.value <= bm.workspace_bytes(f8, T)
    assert lib.beam_moe_workspace_region(ctypes.byref(cfg), T, 8, ctypes.byref(off),
                                         ctypes.byref(n)) == UNSUP
    assert lib.beam_moe_workspace_region(ctypes.byref(cfg), -1, 0, ctypes.byref(off),
                                         ctypes.byref(n)) == SHAPE
    assert lib.beam_moe_workspace_region(ctypes.byref(cfg), T, 0, None, ctypes.byref(n)) == NULL
    # expected sizes of the regions
    sizes = {0: 4 * 257, 1: 4 * T * 8, 2: 2 * T * 8 * 2560, 7: 4 * T * 8 * 5120}
    for reg, want in sizes.items():
        lib.beam_moe_workspace_region(ctypes.byref(cfg), T, reg, ctypes.byref(off), ctypes.byref(n))
        assert n.value == want, (reg, n.value, want)
    # conversion: argument checks before any launch
    assert lib.beam_moe_convert(A[0], -1, bm.BEAM_BF16, A[1], None) == SHAPE
    assert lib.beam_moe_convert(A[0], 16, bm.BEAM_F32, A[1], None) == DTYPE
    assert lib.beam_moe_convert(A[0], 0, bm.BEAM_BF16, A[1], None) == OK
    assert lib.beam_moe_convert(None, 16, bm.BEAM_BF16, A[1], None) == NULL
    assert lib.beam_moe_convert(A[0] + 4, 16, bm.BEAM_BF16, A[1], None) == ALIGN
    assert lib.beam_moe_convert(A[0], 16, bm.BEAM_BF16, A[0] + 16, None) == ALIAS
    if not _gpu_visible():
        assert lib.beam_moe_convert(A[0], 16, bm.BEAM_FP8_E4M3, A[1], None) == DEVICE


HOSTCHECK = os.path.join(os.path.dirname(__file__), "hostcheck")
CSRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "routing_grouped_expert_fp32_amd",
                    "csrc")


@pytest.fixture(scope="module")
def hostcheck_binary(tmp_path_factory):
    """The host dispatcher and validation (api.cpp, host_rules.cpp) built for the CPU with
    AddressSanitizer and UndefinedBehaviorSanitizer, linked against stubs of the HIP runtime and of
    every kernel launcher (tests/hostcheck/stubs.cpp); no GPU code is built or run."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("hostcheck") / "hostcheck")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_rules.cpp"),
            os.path.join(HOSTCHECK, "stubs.cpp"), os.path.join(HOSTCHECK, "driver.cpp")]
    sanitizers = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-fno-omit-frame-pointer", *sanitizers,
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *srcs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


@pytest.mark.parametrize("mode", ["plain", "sync"])
def test_host_dispatch_under_sanitizers(hostcheck_binary, mode):
    """Every entry point over 7 cfgs x 13 batch sizes (0 .. 32768) plus the dense layer, with each
    launch's buffers checked against the arguments and the workspace, and the validation errors,
    under ASan/UBSan; `sync` runs with BEAM_MOE_SYNC_CHECK=1 (one stream synchronisation per
    launch)."""
    import subprocess
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("BEAM_MOE_SYNC_CHECK", None)
    args = [hostcheck_binary] + (["--sync"] if mode == "sync" else [])
    res = subprocess.run(args, capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-4000:])
    m = re.search(r"hostcheck: (\d+) checks, 0 failed, (\d+) launches checked", res.stdout)
    assert m and int(m.group(2)) > 1000, res.stdout

"""Host-side checks of the C ABI (CPU only: no GPU call is made).

The library must load and export every function include/igemm_conv.h
declares; the acceptance gate must decline exactly what the page's rules and
the library's stated limits decline, before any HIP call.  Fake, aligned,
non-overlapping pointer values are used: a declined call never dereferences
them.
"""
import glob
import itertools
import os
import re

import pytest
import torch

import implicit_gemm_nhwc_amd as igc
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def setup_module(_):
    if not os.path.exists(igc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert "conv2d_fwd" in names and "conv2d_fwd_nk" in names and len(names) >= 8
    lib = igc.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_reason_names():
    assert igc.conv2d_abi_version() == 5
    for code, name in igc.REASONS.items():
        assert igc.conv2d_reason_string(code) == name
    assert igc.conv2d_reason_string(999) == "unknown"


X, W, Y, SRC, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
BASE = dict(in_shape=(2, 9, 9, 32), filt_shape=(3, 3, 32, 48), out_shape=(2, 9, 9, 48),
            filter_is_fcrs=False, stride=1, padding=1, dilation=1, groups=1, dtype=0)


def test_element_gather_goes_to_tiled_kernel():
    """C_in * element bytes not a multiple of 16: accepted, on the tiled
    kernel's element gather whatever C_out (the vector kernels need whole
    16-byte channel vectors)."""
    for c, f, dt in ((3, 64, 0), (12, 16, 1), (8, 256, 2), (1, 3, 0)):
        name = igc.conv2d_fwd_kernel_name((1, 32, 32, c), (3, 3, c, f), (1, 32, 32, f),
                                          filter_is_fcrs=False, dtype=dt, stride=1, padding=1)
        assert name == "igemm_fwd_kernel", (c, f, dt, name)
    assert igc.conv2d_workspace_bytes((3, 3, 3, 64), False, 0) == 64 * (64 + 8) * 2


def _check(**kw):
    args = {**BASE, **kw}
    inp = args.pop("input", X)
    flt = args.pop("filter", W)
    out = args.pop("output", Y)
    return igc.conv2d_fwd_check(inp, flt, out, **args)


def test_base_case_accepted():
    assert _check() == 0
    assert _check(source=SRC, beta=0.5) == 0
    assert _check(source=Y, beta=1.0) == 0            # in-place residual
    assert _check(workspace=WS, workspace_bytes=48 * 328 * 2) == 0


@pytest.mark.parametrize("kw,reason", [
    (dict(dtype=3), "dtype"),
    (dict(dtype=-1), "dtype"),
    (dict(stride=3), "stride"),
    (dict(stride=(1, 2)), "stride"),
    (dict(dilation=2), "dilation"),
    (dict(dilation=(1, 2)), "dilation"),
    (dict(padding=3, out_shape=(2, 13, 13, 48)), "padding"),
    (dict(padding=(0, 1)), "padding"),
    (dict(groups=2), "groups"),
    (dict(groups=0), "groups"),
    (dict(filt_shape=(3, 3, 16, 48)), "shape"),
    (dict(filt_shape=(0, 3, 32, 48)), "shape"),
    (dict(in_shape=(-1, 9, 9, 32)), "shape"),
    (dict(out_shape=(2, 9, 9, 47)), "output_shape"),
    (dict(out_shape=(2, 8, 9, 48)), "output_shape"),
    (dict(in_shape=(1, 1, 1, 32), filt_shape=(5, 5, 32, 48), padding=1,
          out_shape=(1, 0, 0, 48)), "output_shape"),
    # any C_in: the tiled kernel's element gather takes C_in * E % 16 != 0
    (dict(in_shape=(2, 9, 9, 12), filt_shape=(3, 3, 12, 48)), "ok"),
    (dict(dtype=2, in_shape=(2, 9, 9, 8), filt_shape=(3, 3, 8, 48)), "ok"),
    (dict(in_shape=(2, 9, 9, 3), filt_shape=(3, 3, 3, 48)), "ok"),
    (dict(input=X + 8), "alignment"),
    (dict(output=Y + 2), "alignment"),
    (dict(source=SRC + 4), "alignment"),
    (dict(input=0), "null_pointer"),
    (dict(output=0), "null_pointer"),
    (dict(output=X + 1024), "overlap"),
    (dict(output=W), "overlap"),
    (dict(source=Y + 64), "overlap"),
    (dict(workspace=Y + 256, workspace_bytes=1 << 20), "overlap"),
    (dict(workspace=WS, workspace_bytes=100), "workspace"),
    # the transpose writes the workspace before the GEMM reads the source
    (dict(source=SRC, beta=0.5, workspace=SRC + 256, workspace_bytes=1 << 20), "overlap"),
    (dict(source=SRC, beta=0.5, workspace=SRC - 48 * 328 * 2 + 16,
          workspace_bytes=48 * 328 * 2), "overlap"),
    (dict(workspace=X + 4096, workspace_bytes=1 << 20), "overlap"),
    (dict(workspace=W + 64, workspace_bytes=1 << 20), "overlap"),
    (dict(in_shape=(300000, 100, 100, 32), out_shape=(300000, 100, 100, 48)), "size_limit"),
])
def test_decline_paths(kw, reason):
    assert igc.REASONS[_check(**kw)] == reason


def test_declined_call_enqueues_nothing():
    # No GPU here: a declined conv2d_fwd must return 0 before any HIP call.
    assert igc.conv2d_fwd(X, W, Y, **{**BASE, "stride": 3}) == 0
    assert igc.conv2d_fwd(X, W, Y, **{**BASE, "groups": 2}) == 0
    assert igc.conv2d_fwd_nk(X, W, BASE["filt_shape"], Y, filter_is_fcrs=False, stride=1,
                             padding=1, dtype=5, in_shape=BASE["in_shape"],
                             out_shape=BASE["out_shape"]) == 0
    lib = igc.lib()
    assert lib.conv2d_filter_to_nk(W, 0, igc._i64((3, 3, 32, 48)), 7, WS, 1 << 20, None) == 0
    assert lib.conv2d_filter_to_nk(W, 0, igc._i64((3, 3, 32, 48)), 0, WS, 10, None) == 0
    assert lib.conv2d_filter_to_nk(W, 0, igc._i64((3, 3, 32, 48)), 0, WS + 4, 1 << 20, None) == 0


def test_empty_output_is_handled_without_launch():
    # N = 0: accepted, nothing to compute, no HIP call.
    args = dict(BASE, in_shape=(0, 9, 9, 32), out_shape=(0, 9, 9, 48))
    assert _check(**args) == 0
    inp, flt, out = X, W, Y
    assert igc.conv2d_fwd(inp, flt, out, **args) == 1


def test_workspace_and_pitch():
    # K rounded up to whole 128-byte k-tiles, plus a 16-byte zero pad per row
    assert igc.conv2d_nk_row_pitch((3, 3, 16, 16), False, 0) == 192 + 8     # 144 -> 3*64
    assert igc.conv2d_nk_row_pitch((64, 64, 3, 3), True, 0) == 576 + 8
    assert igc.conv2d_nk_row_pitch((5, 5, 256, 256), False, 2) == 6400         # C_out > 64: no pad
    assert igc.conv2d_nk_row_pitch((5, 5, 256, 64), False, 2) == 6400 + 16
    assert igc.conv2d_nk_row_pitch((3, 3, 16, 16), False, 2) == 256 + 16    # 144 -> 2*128
    assert igc.conv2d_workspace_bytes((3, 3, 128, 3), False, 0) == 3 * 1160 * 2
    assert igc.conv2d_workspace_bytes((256, 128, 3, 3), True, 1) == 256 * 1152 * 2
    assert igc.conv2d_workspace_bytes((3, 3, 16, 16), False, 9) == 0


DT_NAMES = {0: ("bfloat16", "bfloat16", "bfloat16"), 1: ("float16", "float16", "float16"),
            2: ("float8_e4m3fn", "float8_e4m3fn", "bfloat16"), 3: ("float32",) * 3}


def test_gate_matches_oracle_gate():
    """The C gate and the oracle's reading of the page agree on every
    combination (shapes chosen so the library's own limits never bind)."""
    n = 0
    for dt, st, dil, pad, groups, (h, k, c, f), fcrs in itertools.product(
            [0, 1, 2, 3], [(1, 1), (2, 2), (3, 3), (1, 2)], [(1, 1), (2, 2)],
            [(0, 0), (1, 1), (2, 2), (3, 3), (1, 0)], [1, 2],
            [(9, 3, 32, 48), (5, 5, 16, 3), (2, 5, 64, 8), (7, 1, 32, 1)], [False, True]):
        ho = oracle.out_size(h, k, st[0], pad[0])
        wo = oracle.out_size(h, k, st[1], pad[1])
        in_shape = (2, h, h, c)
        filt = (f, c, k, k) if fcrs else (k, k, c, f)
        out_shape = (2, max(ho, 0), max(wo, 0), f)
        names = DT_NAMES[dt]
        want = oracle.gate_accepts(names[0], names[1], names[2], in_shape, filt, fcrs,
                                   out_shape, st, dil, pad, groups)
        got = _check(in_shape=in_shape, filt_shape=filt, out_shape=out_shape,
                     filter_is_fcrs=fcrs, stride=st, dilation=dil, padding=pad,
                     groups=groups, dtype=dt)
        assert (got == 0) == want, (dt, st, dil, pad, groups, h, k, c, f, fcrs, got)
        n += 1
    assert n > 1000


def test_kernel_selection():
    """The kernel each named workload goes to, the declined and empty cases."""
    import datagen
    want = {"tiny_3x3_16c": "igemm_fwd_band_kernel",
            "resnet_3x3_64c_n32": "igemm_fwd_band_kernel",
            "strided_3x3_s2_128to256_n32": "igemm_fwd_wide_kernel",
            "fp8_5x5_256c_residual_n16": "igemm_fwd_patch_kernel",
            "rgb_3x3_128to3_512px": "igemm_fwd_tapfold_kernel"}
    dts = {"bfloat16": torch.bfloat16, "float16": torch.float16,
           "float8_e4m3fn": torch.float8_e4m3fn}
    for name, spec in datagen.WORKLOADS.items():
        r, s_, c, f = spec["R"], spec["S"], spec["C"], spec["F"]
        w_shape = (f, c, r, s_) if spec["fcrs"] else (r, s_, c, f)
        got = igc.conv2d_fwd_kernel_name(
            (spec["N"], spec["H"], spec["W"], c), w_shape,
            (spec["N"],) + tuple(spec["out_hw"]) + (f,), filter_is_fcrs=spec["fcrs"],
            dtype=dts[spec["dtype"]], stride=spec["stride"], padding=spec["pad"])
        assert got == want[name], (name, got)
    # declined (stride 3), empty batch, and a wide layer with C_out = 65
    assert igc.conv2d_fwd_kernel_name((1, 8, 8, 16), (3, 3, 16, 16), (1, 3, 3, 16),
                                      filter_is_fcrs=False, dtype=torch.bfloat16, stride=3,
                                      padding=1) is None
    assert igc.conv2d_fwd_kernel_name((0, 8, 8, 16), (3, 3, 16, 16), (0, 8, 8, 16),
                                      filter_is_fcrs=False, dtype=torch.bfloat16,
                                      padding=1) == "none"
    assert igc.conv2d_fwd_kernel_name((2, 8, 8, 64), (3, 3, 64, 65), (2, 8, 8, 65),
                                      filter_is_fcrs=False, dtype=torch.float16,
                                      padding=1) == "igemm_fwd_wide_kernel"


def test_patch_kernel_selection():
    """The patch-resident kernel takes stride-1 layers with C_out > 64 (a
    multiple of 4), a spatial filter and C_in a whole number of 128-byte
    chunks, when 256-pixel (else 128-pixel) tiles of one image, at least
    3/4 of their slots used, give every CU a workgroup; the wide kernel
    takes the rest."""
    def name(n, h, w, c, f, r, s, st, p, dt):
        ho, wo = (h + 2 * p - r) // st + 1, (w + 2 * p - s) // st + 1
        return igc.conv2d_fwd_kernel_name((n, h, w, c), (r, s, c, f), (n, ho, wo, f),
                                          filter_is_fcrs=False, dtype=dt, stride=st, padding=p)
    bf, f8 = torch.bfloat16, torch.float8_e4m3fn
    patch, wide = "igemm_fwd_patch_kernel", "igemm_fwd_wide_kernel"
    assert name(16, 64, 64, 256, 256, 5, 5, 1, 2, f8) == patch
    assert name(16, 64, 64, 64, 256, 3, 3, 1, 1, bf) == patch       # one 128-byte chunk
    assert name(16, 64, 66, 128, 128, 1, 3, 1, 0, f8) == patch      # 1 x 3
    assert name(16, 64, 64, 64, 256, 3, 3, 2, 1, bf) == wide        # stride 2
    assert name(16, 64, 64, 64, 256, 1, 1, 1, 0, bf) == wide        # no spatial filter
    assert name(16, 64, 64, 96, 256, 3, 3, 1, 1, bf) == wide        # 192-byte pixels
    assert name(16, 64, 64, 64, 130, 3, 3, 1, 1, bf) == wide        # C_out % 4 != 0
    # 128 tiles of 256 pixels, 256 of 128 pixels: the 128-pixel plan
    assert name(8, 64, 64, 64, 128, 3, 3, 1, 1, bf) == patch
    assert name(4, 64, 64, 64, 128, 3, 3, 1, 1, bf) == wide         # 128 tiles even of 128 pixels
    assert name(64, 7, 7, 64, 256, 3, 3, 1, 1, bf) == wide          # 49-pixel images
    # 50 x 50: 256-pixel tiles leave the last round a quarter full, 100-pixel
    # ones (2 x 50) fill 500 tiles
    assert name(20, 50, 50, 64, 256, 3, 3, 1, 1, bf) == patch
    assert name(5, 50, 50, 64, 256, 3, 3, 1, 1, bf) == wide         # too few tiles either way
    # the patch kernel takes no grouped or mapped launch: the general
    # entry's fast path may use it, the transposed phases never
    p = igc.conv_params(stride=1, pad_begin=1)
    assert igc.conv2d_fwd_general_kernel_name((16, 64, 64, 64), (3, 3, 64, 256),
                                              (16, 64, 64, 256), p, filter_is_fcrs=False,
                                              dtype=0) == patch


# ------------------------------------------------------------ fused epilogue
SC, BI = 0x60000000, 0x60001000
OUT_BYTES = 2 * 9 * 9 * 48 * 2


@pytest.mark.parametrize("kw,reason", [
    (dict(), "ok"),
    (dict(scale=SC, bias=BI, activation="relu"), "ok"),
    (dict(activation="silu"), "ok"),
    (dict(bias=BI), "ok"),
    (dict(activation=3), "epilogue"),
    (dict(activation=-1), "epilogue"),
    (dict(scale=SC + 2), "epilogue"),
    (dict(bias=BI + 1, activation="relu"), "epilogue"),
    (dict(scale=Y + 64), "epilogue"),                      # inside the output
    (dict(bias=Y + OUT_BYTES - 4), "epilogue"),            # last word overlaps
    (dict(bias=Y - 48 * 4 + 4), "epilogue"),               # runs into the output
    (dict(bias=Y - 48 * 4), "ok"),                         # ends where it starts
])
def test_epilogue_check(kw, reason):
    code = igc.conv2d_epilogue_check(Y, out_shape=BASE["out_shape"], **kw)
    assert igc.REASONS[code] == reason


def test_epilogue_declined_call_enqueues_nothing():
    # a bad epilogue declines before any HIP call, on both entry points; a
    # bad convolution declines whatever the epilogue
    assert igc.conv2d_fwd_epilogue(X, W, Y, activation=7, **BASE) == 0
    assert igc.conv2d_fwd_epilogue(X, W, Y, scale=Y, **BASE) == 0
    assert igc.conv2d_fwd_epilogue(X, W, Y, bias=SC, activation="relu",
                                   **{**BASE, "stride": 3}) == 0
    assert igc.conv2d_fwd_nk_epilogue(X, W, BASE["filt_shape"], Y, filter_is_fcrs=False,
                                      stride=1, padding=1, dtype=0, bias=BI + 2,
                                      in_shape=BASE["in_shape"],
                                      out_shape=BASE["out_shape"]) == 0
    # empty output with a valid epilogue: handled, nothing launched
    args = dict(BASE, in_shape=(0, 9, 9, 32), out_shape=(0, 9, 9, 48))
    assert igc.conv2d_fwd_epilogue(X, W, Y, scale=SC, activation="silu", **args) == 1


# --------------------------------------------------------- im2col ablation
def test_im2col_bytes_and_declines():
    # 2 x 9 x 9 x 32 bf16, 3x3 stride 1 pad 1: M = 162, K = 288 -> Kp = 320
    assert igc.conv2d_im2col_bytes((2, 9, 9, 32), 3, 3, stride=1, padding=1,
                                   dtype=torch.bfloat16) == 162 * 320 * 2
    # fp8, 5x5 stride 2 pad 2 on 16 x 16 x 16: Ho = 8, K = 400 -> Kp = 512
    assert igc.conv2d_im2col_bytes((1, 16, 16, 16), 5, 5, stride=2, padding=2,
                                   dtype=torch.float8_e4m3fn) == 64 * 512
    for kw in (dict(stride=3), dict(padding=3), dict(dtype=7)):
        args = dict(stride=1, padding=1, dtype=torch.bfloat16)
        args.update(kw)
        assert igc.conv2d_im2col_bytes((2, 9, 9, 32), 3, 3, **args) == 0
    assert igc.conv2d_im2col_bytes((2, 9, 9, 12), 3, 3, stride=1, padding=1,
                                   dtype=torch.bfloat16) == 0        # vector width
    lib = igc.lib()
    call = lambda x, a, nb, st=1: lib.conv2d_im2col(  # noqa: E731
        x, igc._i64((2, 9, 9, 32)), igc._rs(3, 3), igc._pair(st), igc._pair(1), 0, a, nb, None)
    need = 162 * 320 * 2
    assert call(X, WS, need - 1) == 0          # too small
    assert call(X + 8, WS, need) == 0          # misaligned input
    assert call(X, WS + 4, need) == 0          # misaligned output
    assert call(X, X + 4096, need) == 0        # overlaps the input
    assert call(X, 0, need) == 0               # null output
    assert call(X, WS, need, st=3) == 0        # stride


# ----------------------------------------------------- transposed convolution
TBASE = dict(in_shape=(2, 9, 9, 32), filt_shape=(3, 3, 48, 32), out_shape=(2, 9, 9, 48),
             stride=1, padding=1, dilation=1, dtype=0)


def _tcheck(**kw):
    args = {**TBASE, **kw}
    return igc.conv2d_transposed_check(args.pop("input", X), args.pop("filter", W),
                                       args.pop("output", Y), **args)


def test_transposed_workspace_bytes():
    # equivalent forward filter RSCF {3, 3, 32, 48}: K = 288 -> 320 (+8 for C_out <= 64)
    ws = igc.conv2d_transposed_workspace_bytes
    assert ws((2, 9, 9, 32), (3, 3, 48, 32), stride=1, padding=1,
              dtype=torch.bfloat16) == 48 * 328 * 2
    assert ws((2, 9, 9, 32), (3, 3, 48, 32), stride=1, padding=1, dtype=9) == 0

    def al(v):
        return (v + 255) // 256 * 256
    # stride 2, R = 3, p = 1: row / column phase 0 takes tap 1, phase 1 taps
    # 0 and 2; NK rows of K = 32, 64, 64, 128 elements (+8 pad), each matrix
    # 256-byte aligned, and nothing else (no phase buffers)
    want = 0
    for jh, jw in ((1, 1), (1, 2), (2, 1), (2, 2)):
        k = jh * jw * 32
        want += al(48 * ((k + 63) // 64 * 64 + 8) * 2)
    assert ws((2, 9, 9, 32), (3, 3, 48, 32), stride=2, padding=1,
              dtype=torch.bfloat16) == want
    # stride 3, R = 2, p = 0: phase 2 of each axis has no tap (K = 0: rows of
    # the 8-element pad alone)
    want = 0
    for jh, jw in itertools.product((1, 1, 0), (1, 1, 0)):
        k = jh * jw * 32
        want += al(48 * ((k + 63) // 64 * 64 + 8) * 2)
    assert ws((2, 9, 9, 32), (2, 2, 48, 32), stride=3, padding=0,
              dtype=torch.bfloat16) == want
    # dilation 2 at stride 1: one phase, all 9 taps
    assert ws((2, 9, 9, 32), (3, 3, 48, 32), stride=1, dilation=2, padding=1,
              dtype=torch.bfloat16) == 48 * 328 * 2


@pytest.mark.parametrize("kw,reason", [
    (dict(), "ok"),
    (dict(source=SRC, beta=0.5, scale=SC, activation="silu"), "ok"),
    (dict(padding=0, out_shape=(2, 11, 11, 48)), "ok"),
    (dict(filt_shape=(5, 5, 48, 32), padding=2), "ok"),
    (dict(filt_shape=(4, 4, 48, 32), padding=1, out_shape=(2, 10, 10, 48)), "ok"),
    (dict(stride=2, out_shape=(2, 17, 17, 48)), "ok"),
    (dict(stride=2, padding=2, filt_shape=(4, 4, 48, 32), out_shape=(2, 16, 16, 48)), "ok"),
    (dict(stride=3, out_shape=(2, 25, 25, 48)), "ok"),
    (dict(stride=(2, 1), out_shape=(2, 17, 9, 48)), "ok"),
    (dict(stride=2, filt_shape=(1, 1, 48, 32), padding=0, out_shape=(2, 17, 17, 48)), "ok"),
    (dict(dilation=2, out_shape=(2, 11, 11, 48)), "ok"),
    (dict(dilation=(3, 1), stride=2, out_shape=(2, 21, 17, 48)), "ok"),
    (dict(padding=3, out_shape=(2, 5, 5, 48)), "ok"),
    (dict(filt_shape=(5, 5, 48, 32), padding=1, out_shape=(2, 11, 11, 48)), "ok"),
    (dict(filt_shape=(3, 5, 48, 32), out_shape=(2, 9, 11, 48)), "ok"),
    (dict(padding=(1, 0), out_shape=(2, 9, 11, 48)), "ok"),
    (dict(stride=2, out_shape=(2, 18, 18, 48)), "output_shape"),
    (dict(stride=2, out_shape=(2, 17, 17, 48), workspace=WS, workspace_bytes=1024), "workspace"),
    (dict(stride=(0, 1)), "stride"),
    (dict(dilation=(1, 0)), "dilation"),
    (dict(padding=(-1, 1)), "padding"),
    (dict(padding=6), "output_shape"),                           # Ho = 11 - 12 < 1
    (dict(dilation=2), "output_shape"),                          # Ho is 11
    (dict(filt_shape=(3, 3, 48, 16)), "shape"),
    (dict(in_shape=(2, 9, 9, 12), filt_shape=(3, 3, 48, 12)), "ok"),   # any C: element gather
    (dict(in_shape=(1, 1 << 29, 2, 32), stride=(2, 1),
          out_shape=(1, (1 << 30) - 1, 2, 48)), "size_limit"),  # extent 2^30
    (dict(out_shape=(2, 9, 9, 47)), "output_shape"),
    (dict(out_shape=(2, 10, 10, 48)), "output_shape"),
    (dict(dtype=5), "dtype"),
    (dict(output=X + 64), "overlap"),
    (dict(activation=9), "epilogue"),
])
def test_transposed_decline_paths(kw, reason):
    assert igc.REASONS[_tcheck(**kw)] == reason


def test_transposed_out_hw_matches_oracle_rule():
    for h, r, st, p, d in itertools.product([1, 5, 9], [1, 2, 3, 5], [1, 2, 3], [0, 1, 2], [1, 2]):
        ho, _ = igc.transposed_out_hw(h, h, r, r, stride=st, padding=p, dilation=d)
        assert ho == (h - 1) * st + d * (r - 1) + 1 - 2 * p


def test_transposed_declined_call_enqueues_nothing():
    assert igc.conv2d_transposed_fwd(X, W, Y, **{**TBASE, "stride": (0, 1)}) == 0
    assert igc.conv2d_transposed_fwd(X, W, Y, **{**TBASE, "dilation": 2}) == 0   # output shape
    args = dict(TBASE, in_shape=(0, 9, 9, 32), out_shape=(0, 9, 9, 48))
    assert igc.conv2d_transposed_fwd(X, W, Y, **args) == 1


def test_workspace_beside_source_accepted():
    # a workspace that ends exactly where the source starts does not overlap it
    nk = 48 * 328 * 2
    assert _check(source=SRC, beta=0.5, workspace=SRC - nk, workspace_bytes=nk) == 0


# ------------------------------------------------------ pointer-free query
def test_query_matches_pointer_gate():
    """conv2d_fwd_query gives the shape/parameter reason conv2d_fwd_check
    gives for well-formed pointers, for accepted and declined problems."""
    cases = [dict(), dict(stride=3), dict(dilation=2), dict(padding=(0, 1)), dict(groups=2),
             dict(dtype=7), dict(filt_shape=(3, 3, 16, 48)), dict(out_shape=(2, 9, 9, 47)),
             dict(in_shape=(2, 9, 9, 12), filt_shape=(3, 3, 12, 48)),
             dict(in_shape=(300000, 100, 100, 32), out_shape=(300000, 100, 100, 48)),
             dict(in_shape=(0, 9, 9, 32), out_shape=(0, 9, 9, 48))]
    for kw in cases:
        args = {**BASE, **kw}
        q = igc.conv2d_fwd_query(args["in_shape"], args["filt_shape"], args["out_shape"],
                                 filter_is_fcrs=args["filter_is_fcrs"], dtype=args["dtype"],
                                 stride=args["stride"], padding=args["padding"],
                                 dilation=args["dilation"], groups=args["groups"])
        assert q == _check(**kw), kw
    # pointer rules are not the query's: a misaligned input passes it
    assert igc.conv2d_fwd_query(BASE["in_shape"], BASE["filt_shape"], BASE["out_shape"],
                                filter_is_fcrs=False, dtype=0, padding=1) == 0
    assert igc.REASONS[_check(input=X + 8)] == "alignment"


# --------------------------------------------- epilogue against the workspace
NK_BYTES = 48 * 328 * 2


@pytest.mark.parametrize("kw,reason", [
    (dict(scale=SC, bias=BI), "ok"),
    (dict(scale=WS + 64), "epilogue"),                     # inside the workspace
    (dict(bias=WS + NK_BYTES - 4, activation="relu"), "epilogue"),
    (dict(bias=WS + NK_BYTES), "ok"),                       # just past its end
    (dict(scale=WS - 48 * 4), "ok"),                        # ends where it starts
    (dict(scale=WS - 48 * 4 + 4), "epilogue"),
])
def test_epilogue_against_workspace(kw, reason):
    code = igc.conv2d_fwd_epilogue_check(X, W, Y, workspace=WS, workspace_bytes=NK_BYTES,
                                         **BASE, **kw)
    assert igc.REASONS[code] == reason
    if reason != "ok":
        assert igc.conv2d_fwd_epilogue(X, W, Y, workspace=WS, workspace_bytes=NK_BYTES,
                                       **BASE, **kw) == 0


def test_filter_to_nk_declines_nk_of_2gib():
    # NK matrix of 2^31 bytes or more: the transpose's 32-bit indices would
    # overflow, so the call is declined (no GPU here: it must not launch)
    lib = igc.lib()
    big = (1, 1, 1 << 16, 1 << 15)            # K = 65536, C_out = 32768 -> 2^32 bytes bf16
    assert lib.conv2d_filter_to_nk(W, 0, igc._i64(big), 0, WS, 1 << 40, None) == 0
    just = (1, 1, 1 << 14, 1 << 16)           # 2^30 elements -> 2^31 bytes
    assert lib.conv2d_filter_to_nk(W, 0, igc._i64(just), 0, WS, 1 << 40, None) == 0


# ------------------------------------------------------- binding checks
def _cpu(shape, dt=torch.bfloat16):
    return torch.zeros(shape, dtype=dt)


def test_binding_rejects_host_tensors():
    x, w, y = _cpu((1, 4, 4, 16)), _cpu((3, 3, 16, 8)), _cpu((1, 4, 4, 8))
    with pytest.raises(igc.InvalidArgument, match="GPU tensor"):
        igc.conv2d_fwd(x, w, y, filter_is_fcrs=False, padding=1)
    with pytest.raises(igc.InvalidArgument, match="GPU tensor"):
        igc.conv2d_fwd_nk(x, _cpu(1000, torch.uint8), w.shape, y, filter_is_fcrs=False,
                          padding=1)
    with pytest.raises(igc.InvalidArgument, match="GPU tensor"):
        igc.conv2d_filter_to_nk(w, _cpu(1000, torch.uint8), filter_is_fcrs=False)
    with pytest.raises(igc.InvalidArgument, match="GPU tensor"):
        igc.conv2d_im2col(x, 3, 3, _cpu(100000, torch.uint8), padding=1)
    with pytest.raises(igc.InvalidArgument, match="GPU tensor"):
        igc.conv2d_transposed_fwd(x, _cpu((3, 3, 8, 16)), y, padding=1)
    # a host tensor mixed with raw device pointers is caught too
    with pytest.raises(igc.InvalidArgument, match="GPU tensor"):
        igc.conv2d_fwd(X, W, Y, source=_cpu((2, 9, 9, 48)), beta=1.0, **BASE)


class _FakeCuda:
    """Stands in for a GPU tensor in the binding's checks on a machine
    without a GPU: the binding only reads these attributes before calling
    into the library."""

    def __init__(self, shape, dtype, contiguous=True, device="cuda:0", ptr=0x70000000):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = torch.device(device)
        self._contig = contiguous
        self._ptr = ptr

    def is_contiguous(self):
        return self._contig

    def numel(self):
        n = 1
        for v in self.shape:
            n *= v
        return n

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()

    def data_ptr(self):
        return self._ptr


def test_binding_checks_tensor_properties(monkeypatch):
    monkeypatch.setattr(igc.torch, "Tensor", _FakeCuda)
    ok = dict(input=_FakeCuda((1, 4, 4, 16), torch.bfloat16, ptr=X),
              filter=_FakeCuda((3, 3, 16, 8), torch.bfloat16, ptr=W),
              output=_FakeCuda((1, 4, 4, 8), torch.bfloat16, ptr=Y))

    def call(**kw):
        args = {**ok, **kw}
        return igc.conv2d_fwd_epilogue(args.pop("input"), args.pop("filter"),
                                       args.pop("output"), filter_is_fcrs=False, padding=1,
                                       stream=0, **args)
    bad = [
        (dict(input=_FakeCuda((1, 4, 4, 16), torch.bfloat16, contiguous=False)), "contiguous"),
        (dict(filter=_FakeCuda((3, 3, 16, 8), torch.float16)), "filter dtype"),
        (dict(output=_FakeCuda((1, 4, 4, 8), torch.float16)), "output dtype"),
        (dict(input=_FakeCuda((1, 4, 4, 16), torch.float32)), "input dtype"),
        (dict(source=_FakeCuda((1, 4, 4, 4), torch.bfloat16, ptr=SRC)), "source"),
        (dict(source=_FakeCuda((1, 4, 4, 8), torch.float16, ptr=SRC)), "source"),
        (dict(output=_FakeCuda((1, 4, 4, 8), torch.bfloat16, device="cuda:1")), "on cuda:1"),
        (dict(scale=_FakeCuda((8,), torch.float16, ptr=SC)), "float32"),
        (dict(bias=_FakeCuda((7,), torch.float32, ptr=BI)), "C_out"),
        (dict(workspace=_FakeCuda((10,), torch.uint8, ptr=WS), workspace_bytes=4096),
         "workspace"),
    ]
    for kw, msg in bad:
        with pytest.raises(igc.InvalidArgument, match=msg):
            call(**kw)
    # explicit shapes larger than the buffers they describe
    with pytest.raises(igc.InvalidArgument, match="input holds"):
        igc.conv2d_fwd(ok["input"], ok["filter"], ok["output"], filter_is_fcrs=False,
                       padding=1, in_shape=(2, 4, 4, 16), out_shape=(2, 4, 4, 8), stream=0)
    with pytest.raises(igc.InvalidArgument, match="NK matrix holds"):
        igc.conv2d_fwd_nk(ok["input"], _FakeCuda((100,), torch.uint8, ptr=WS), (3, 3, 16, 8),
                          ok["output"], filter_is_fcrs=False, padding=1, stream=0)


# ------------------------------------------------ general convolution
GBASE = dict(in_shape=(2, 20, 21, 32), filt_shape=(3, 3, 16, 8), filter_is_fcrs=False,
             stride=(3, 2), dilation=(2, 1), pad_begin=(1, 0), pad_end=(2, 3), groups=2,
             dtype=0)


def _gen(**kw):
    """(in_shape, filt_shape, out_shape, params, fcrs, dtype) with the output
    shape from the oracle's size rule unless given."""
    a = {**GBASE, **kw}
    fcrs = a["filter_is_fcrs"]
    if fcrs:
        f, _, r, s = a["filt_shape"]
    else:
        r, s, _, f = a["filt_shape"]
    st = a["stride"] if isinstance(a["stride"], tuple) else (a["stride"],) * 2
    dl = a["dilation"] if isinstance(a["dilation"], tuple) else (a["dilation"],) * 2
    pb = a["pad_begin"] if isinstance(a["pad_begin"], tuple) else (a["pad_begin"],) * 2
    pe = a["pad_end"] if isinstance(a["pad_end"], tuple) else (a["pad_end"],) * 2
    n, h, w, _ = a["in_shape"]
    ho = oracle.out_size_general(h, r, st[0], dl[0], pb[0], pe[0]) if min(st + dl) > 0 else 1
    wo = oracle.out_size_general(w, s, st[1], dl[1], pb[1], pe[1]) if min(st + dl) > 0 else 1
    out = a.get("out_shape", (n, max(ho, 0), max(wo, 0), f))
    p = igc.conv_params(stride=st, dilation=dl, pad_begin=pb, pad_end=pe, groups=a["groups"])
    return a["in_shape"], a["filt_shape"], out, p, fcrs, a["dtype"]


def _gcheck(input=X, filter=W, output=Y, source=None, workspace=None, workspace_bytes=0,
            scale=None, bias=None, activation=None, **kw):
    i, f, o, p, fcrs, dt = _gen(**kw)
    return igc.conv2d_fwd_general_check(input, filter, output, p, filter_is_fcrs=fcrs,
                                        source=source, scale=scale, bias=bias,
                                        activation=activation, workspace=workspace,
                                        workspace_bytes=workspace_bytes, dtype=dt, in_shape=i,
                                        filt_shape=f, out_shape=o)


def test_general_base_case_accepted_and_kernel():
    assert _gcheck() == 0
    i, f, o, p, fcrs, dt = _gen()
    assert o == (2, 7, 11, 8)      # (20+1+2-2*2-1)//3+1, (21+0+3-1*2-1)//2+1
    assert igc.conv2d_fwd_general_query(i, f, o, p, filter_is_fcrs=fcrs, dtype=dt) == 0
    assert igc.conv2d_fwd_general_kernel_name(i, f, o, p, filter_is_fcrs=fcrs,
                                              dtype=dt) == "igemm_fwd_kernel"
    assert _gcheck(source=SRC, workspace=WS, workspace_bytes=1 << 20, scale=0x60000000,
                   bias=0x60001000, activation="silu") == 0
    assert _gcheck(source=Y) == 0                                   # in place


@pytest.mark.parametrize("kw", [
    dict(stride=1, dilation=1, pad_begin=1, pad_end=1, groups=1, filt_shape=(3, 3, 32, 48)),
    dict(stride=2, dilation=1, pad_begin=2, pad_end=2, groups=1, filt_shape=(5, 5, 32, 3)),
    dict(stride=1, dilation=1, pad_begin=0, pad_end=0, groups=1, filt_shape=(1, 1, 32, 128)),
])
def test_general_page_problems_take_conv2d_fwd_kernels(kw):
    """Inside the page's gate the general entry runs what conv2d_fwd runs."""
    i, f, o, p, fcrs, dt = _gen(**kw)
    st, pad = p.stride[0], p.pad_begin[0]
    name = igc.conv2d_fwd_general_kernel_name(i, f, o, p, filter_is_fcrs=fcrs, dtype=dt)
    assert name is not None and name == igc.conv2d_fwd_kernel_name(
        i, f, o, filter_is_fcrs=fcrs, dtype=dt, stride=st, padding=pad)


@pytest.mark.parametrize("kw,reason", [
    (dict(dtype=3), "dtype"),
    (dict(stride=(0, 1)), "stride"),
    (dict(dilation=(1, 0)), "dilation"),
    (dict(pad_begin=(-1, 0)), "padding"),
    (dict(pad_end=(0, -2)), "padding"),
    (dict(groups=0), "groups"),
    (dict(groups=3, in_shape=(2, 20, 21, 48), filt_shape=(3, 3, 16, 8)), "groups"),
    (dict(groups=4), "shape"),                      # 4 * 16 != 32 input channels
    (dict(filt_shape=(0, 3, 16, 8)), "shape"),
    (dict(in_shape=(2, 20, 21, -32)), "shape"),
    (dict(out_shape=(2, 7, 11, 9)), "output_shape"),
    (dict(out_shape=(2, 8, 11, 8)), "output_shape"),
    (dict(in_shape=(1, 2, 2, 32), dilation=4, pad_begin=0, pad_end=0,
          out_shape=(1, 0, 0, 8)), "output_shape"),
    (dict(in_shape=(2, 20, 21, 8), filt_shape=(3, 3, 4, 8)), "ok"),       # Cg = 4
    (dict(dtype=2, in_shape=(2, 20, 21, 16), filt_shape=(3, 3, 8, 8)), "ok"),
    (dict(groups=32, in_shape=(2, 20, 21, 32), filt_shape=(3, 3, 1, 32)), "ok"),   # depthwise
    (dict(input=X + 8), "alignment"),
    (dict(input=0), "null_pointer"),
    (dict(output=X + 1024), "overlap"),
    (dict(source=Y + 64), "overlap"),
    (dict(workspace=WS, workspace_bytes=100), "workspace"),
    (dict(workspace=X + 64, workspace_bytes=1 << 20), "overlap"),
    (dict(activation="gelu"), "epilogue"),
    (dict(scale=Y + 4), "epilogue"),
    (dict(scale=WS + 64, workspace=WS, workspace_bytes=1 << 20), "epilogue"),
])
def test_general_decline_paths(kw, reason):
    assert igc.REASONS[_gcheck(**kw)] == reason


@pytest.mark.parametrize("kw,reason", [
    (dict(dilation=(1 << 29, 1), in_shape=(1, 1 << 29, 4, 32), pad_begin=0, pad_end=0,
          filt_shape=(1, 3, 16, 8)), "ok"),
    (dict(dilation=(1 << 28, 1), in_shape=(1, (1 << 29) + 5, 4, 32), pad_begin=0,
          pad_end=0, filt_shape=(3, 3, 16, 8)), "ok"),
    (dict(dilation=(1 << 29, 1), in_shape=(1, (1 << 30) + 5, 4, 32), pad_begin=0,
          pad_end=0, filt_shape=(3, 3, 16, 8)), "size_limit"),    # H >= 2^30
    # H + pt + pb = 20 + pt + 2 against 2^30 (a large stride keeps M small)
    (dict(pad_begin=((1 << 30) - 22, 0), stride=(1 << 20, 2)), "size_limit"),
    (dict(pad_begin=((1 << 30) - 23, 0), stride=(1 << 20, 2)), "ok"),
])
def test_general_coordinate_limits(kw, reason):
    i, f, o, p, fcrs, dt = _gen(**kw)
    assert igc.REASONS[igc.conv2d_fwd_general_query(i, f, o, p, filter_is_fcrs=fcrs,
                                                    dtype=dt)] == reason


def test_general_input_bytes_use_all_channels():
    # the input holds N*H*W*C_in elements (all groups): an output right after
    # a 2x20x21x16 input would still overlap the 32-channel one
    assert igc.REASONS[_gcheck(output=X + 2 * 20 * 21 * 16 * 2)] == "overlap"
    assert _gcheck(output=X + 2 * 20 * 21 * 32 * 2) == 0


def test_general_declined_call_enqueues_nothing():
    i, f, o, p, fcrs, dt = _gen(groups=4)
    assert igc.conv2d_fwd_general(X, W, Y, p, filter_is_fcrs=fcrs, dtype=dt, in_shape=i,
                                  filt_shape=f, out_shape=o) == 0
    i, f, o, p, fcrs, dt = _gen(in_shape=(0, 20, 21, 32), out_shape=(0, 7, 11, 8))
    assert igc.conv2d_fwd_general(X, W, Y, p, filter_is_fcrs=fcrs, dtype=dt, in_shape=i,
                                  filt_shape=f, out_shape=o) == 1   # empty: nothing to do


def test_general_gate_against_oracle_sizes():
    """Over a grid of parameters the general gate accepts exactly the
    problems whose oracle output is non-empty (vector width and limits not
    binding), and the page gate accepts the subset the page allows."""
    n = 0
    for (sh, sw), (dh, dw), (pt, pl, pb, pr), g, fcrs in itertools.product(
            [(1, 1), (2, 2), (3, 1), (1, 4)], [(1, 1), (2, 3)],
            [(0, 0, 0, 0), (1, 1, 1, 1), (2, 0, 1, 3), (3, 3, 3, 3)], [1, 2, 4],
            [False, True]):
        cg, f, r, s = 16, 8, 3, 2
        in_shape = (1, 9, 7, cg * g)
        filt = (f, cg, r, s) if fcrs else (r, s, cg, f)
        ho = oracle.out_size_general(9, r, sh, dh, pt, pb)
        wo = oracle.out_size_general(7, s, sw, dw, pl, pr)
        out = (1, max(ho, 0), max(wo, 0), f)
        p = igc.conv_params(stride=(sh, sw), dilation=(dh, dw), pad_begin=(pt, pl),
                            pad_end=(pb, pr), groups=g)
        got = igc.conv2d_fwd_general_query(in_shape, filt, out, p, filter_is_fcrs=fcrs,
                                           dtype=0)
        assert (got == 0) == (ho >= 1 and wo >= 1), (sh, sw, dh, dw, pt, pl, pb, pr, g)
        page = oracle.gate_accepts("bfloat16", "bfloat16", "bfloat16", in_shape, filt, fcrs,
                                   out, (sh, sw), (dh, dw), (pt, pl), g) and pt == pb and \
            pl == pr
        name = igc.conv2d_fwd_general_kernel_name(in_shape, filt, out, p, filter_is_fcrs=fcrs,
                                                  dtype=0)
        fast = g == 1 and (dh, dw) == (1, 1) and sh == sw
        # several groups of 16 bf16 channels (32 bytes, one MFMA k-step):
        # super-groups on the band kernel
        sgroups = g > 1 and (dh, dw) == (1, 1) and sh == sw and sh <= 2
        if got == 0 and not page:
            if fast:   # the forward kernels with per-side padding, never the tap-fold one
                assert name in ("igemm_fwd_band_kernel", "igemm_fwd_wide_kernel",
                                "igemm_fwd_patch_kernel", "igemm_fwd_resident_kernel",
                                "igemm_fwd_kernel"), name
            elif sgroups:
                assert name == "igemm_fwd_band_kernel"
            else:
                assert name == "igemm_fwd_kernel"
        n += 1
    assert n == 192


def _nk_bytes(r, s, c, f, dt):
    return f * igc.conv2d_nk_row_pitch((r, s, c, f), False, dt) * (1 if dt == 2 else 2)


@pytest.mark.parametrize("dt", [0, 1, 2])
def test_general_workspace_bytes(dt):
    """The general entry's workspace: the plain NK matrix (C_out rows of
    R*S*Cg) on the tiled path, and C_out rows of R*S*q*Cg (block-diagonal
    super-groups of q) on the super-group path, with q a divisor of the
    groups, q * Fg <= 64 and q * Cg * element bytes a power-of-two multiple
    of 32 (64 for fp8); a smaller workspace is declined."""
    e = 1 if dt == 2 else 2
    # tiled path (dilation 2): the plain matrix
    i, f, o, p, fcrs, _ = _gen(dtype=dt)
    assert igc.conv2d_fwd_general_workspace_bytes(i, f, o, p, filter_is_fcrs=fcrs,
                                                  dtype=dt) == _nk_bytes(3, 3, 16, 8, dt)
    # 32 groups of 8 -> 8 channels, 3x3, 28x28: super-groups
    i, f, o, p, fcrs, _ = _gen(dtype=dt, in_shape=(4, 28, 28, 256), filt_shape=(3, 3, 8, 256),
                               stride=1, dilation=1, pad_begin=1, pad_end=1, groups=32)
    assert igc.conv2d_fwd_general_kernel_name(i, f, o, p, filter_is_fcrs=fcrs,
                                              dtype=dt) == "igemm_fwd_band_kernel"
    got = igc.conv2d_fwd_general_workspace_bytes(i, f, o, p, filter_is_fcrs=fcrs, dtype=dt)
    ksb = 64 if dt == 2 else 32
    allowed = {_nk_bytes(3, 3, q * 8, q * 8, dt) // (q * 8) * 256
               for q in (1, 2, 4, 8) if (q * 8 * e) % ksb == 0}
    assert got in allowed, (got, allowed)
    assert _gcheck(workspace=WS, workspace_bytes=got, dtype=dt, in_shape=i, filt_shape=f,
                   out_shape=o, stride=1, dilation=1, pad_begin=1, pad_end=1, groups=32) == 0
    assert igc.REASONS[_gcheck(workspace=WS, workspace_bytes=got - 16, dtype=dt, in_shape=i,
                               filt_shape=f, out_shape=o, stride=1, dilation=1, pad_begin=1,
                               pad_end=1, groups=32)] == "workspace"
    # declined problem: 0
    i, f, o, p, fcrs, _ = _gen(dtype=dt, groups=4)
    assert igc.conv2d_fwd_general_workspace_bytes(i, f, o, p, filter_is_fcrs=fcrs,
                                                  dtype=dt) == 0


@pytest.mark.parametrize("n,h,c,f,r,st,p,dt,want", [
    (32, 224, 8, 96, 4, 4, 0, 0, "igemm_fwd_wide_kernel"),      # 4x4 stride-4 patchify
    (2, 25, 64, 48, 3, 3, 1, 0, "igemm_fwd_band_kernel"),
    (2, 20, 96, 16, 3, 3, 1, 0, "igemm_fwd_resident_kernel"),
    (2, 25, 64, 128, 3, 3, 1, 1, "igemm_fwd_wide_kernel"),
    (4, 64, 16, 64, 4, 4, 0, 1, "igemm_fwd_band_kernel"),
])
def test_general_equal_strides_beyond_two(n, h, c, f, r, st, p, dt, want):
    """One group, unit dilation, equal strides above 2 (outside the page's
    gate even with equal padding): accepted and run on the forward kernels,
    not the tiled fallback."""
    ho = (h + 2 * p - r) // st + 1
    prm = igc.conv_params(stride=st, pad_begin=p)
    shapes = ((n, h, h, c), (r, r, c, f), (n, ho, ho, f), prm)
    assert igc.conv2d_fwd_general_query(*shapes, filter_is_fcrs=False, dtype=dt) == 0
    assert igc.conv2d_fwd_general_kernel_name(*shapes, filter_is_fcrs=False, dtype=dt) == want


@pytest.mark.parametrize("g,cg,fg,dt,want", [
    (32, 8, 8, 0, "igemm_fwd_band_kernel"),        # ResNeXt-like
    (64, 1, 2, 0, "igemm_fwd_band_kernel"),        # depthwise, multiplier 2
    (16, 1, 2, 2, "igemm_fwd_kernel"),             # fp8 depthwise: 16 * 1 byte < 64
    (2, 64, 128, 0, "igemm_fwd_kernel"),           # Fg > 64
    (4, 24, 16, 0, "igemm_fwd_kernel"),            # q * 48 bytes never a power of two
    (8, 16, 16, 2, "igemm_fwd_band_kernel"),       # fp8: q = 4 -> 64 bytes, 64 channels
])
def test_general_supergroup_selection(g, cg, fg, dt, want):
    i, f, o, p, fcrs, _ = _gen(dtype=dt, in_shape=(2, 20, 21, g * cg),
                               filt_shape=(3, 3, cg, g * fg), stride=1, dilation=1,
                               pad_begin=1, pad_end=1, groups=g)
    assert igc.conv2d_fwd_general_kernel_name(i, f, o, p, filter_is_fcrs=fcrs,
                                              dtype=dt) == want


@pytest.mark.parametrize("shape,want", [
    (dict(in_shape=(32, 56, 56, 64), filt=(3, 3, 64, 64), st=1, p=1, dt=0), True),    # band
    (dict(in_shape=(2, 16, 16, 16), filt=(3, 3, 16, 16), st=1, p=1, dt=0), True),     # band
    (dict(in_shape=(32, 56, 56, 128), filt=(3, 3, 128, 256), st=2, p=1, dt=1), False),  # wide
    (dict(in_shape=(1, 64, 64, 128), filt=(3, 3, 128, 3), st=1, p=1, dt=0), False),   # tap-fold
    (dict(in_shape=(32, 56, 56, 64), filt=(3, 3, 64, 64), st=3, p=1, dt=0), False),   # declined
    (dict(in_shape=(2, 16, 16, 64), filt=(3, 3, 64, 64), st=1, p=1, dt=2), False),    # fp8
    (dict(in_shape=(2, 16, 16, 16), filt=(3, 3, 16, 12), st=1, p=1, dt=0), False),    # F % 8
])
def test_filter_in_kernel_query(shape, want):
    """The band kernel transposes a bf16 / fp16 stored filter itself (RSCF:
    C_out a multiple of 8); every other problem reads an NK matrix made by a
    transpose launch."""
    n, h, w, _ = shape["in_shape"]
    r, s, _, f = shape["filt"]
    st, p = shape["st"], shape["p"]
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    got = igc.conv2d_fwd_filter_in_kernel(shape["in_shape"], shape["filt"], (n, ho, wo, f),
                                          filter_is_fcrs=False, dtype=shape["dt"], stride=st,
                                          padding=p)
    assert got == want
    if want:
        assert igc.conv2d_fwd_kernel_name(shape["in_shape"], shape["filt"], (n, ho, wo, f),
                                          filter_is_fcrs=False, dtype=shape["dt"], stride=st,
                                          padding=p) == "igemm_fwd_band_kernel"


@pytest.mark.parametrize("shape,kernel", [
    # stride 1, dilation dividing the padding before each axis and the
    # extents: dilation phases on the band kernel
    (dict(in_shape=(32, 56, 56, 64), filt=(3, 3, 64, 64), dil=2, pb=2, pe=2), "band"),
    (dict(in_shape=(2, 24, 18, 32), filt=(3, 3, 32, 32), dil=3, pb=3, pe=3), "band"),
    (dict(in_shape=(2, 20, 20, 32), filt=(3, 3, 32, 32), dil=2, pb=0, pe=0), "band"),
    (dict(in_shape=(1, 16, 15, 32), filt=(3, 3, 32, 16), dil=(2, 1), pb=(2, 1), pe=(2, 1)),
     "band"),
    # an extent or a padding the dilation does not divide: the tiled kernel
    (dict(in_shape=(1, 17, 16, 32), filt=(3, 3, 32, 16), dil=2, pb=2, pe=2), "tiled"),
    (dict(in_shape=(1, 16, 16, 32), filt=(3, 3, 32, 16), dil=2, pb=1, pe=3), "tiled"),
    (dict(in_shape=(1, 16, 16, 32), filt=(3, 3, 32, 16), dil=2, pb=2, pe=1), "tiled"),  # Ho 15
    # C_out > 64: no band kernel
    (dict(in_shape=(1, 16, 16, 32), filt=(3, 3, 32, 96), dil=2, pb=2, pe=2), "tiled"),
])
def test_general_dilation_phase_selection(shape, kernel):
    n, h, w, c = shape["in_shape"]
    r, s, _, f = shape["filt"]
    p = igc.conv_params(stride=1, dilation=shape["dil"], pad_begin=shape["pb"],
                        pad_end=shape["pe"])
    ho, wo = igc.out_hw_general(h, w, r, s, p)
    name = igc.conv2d_fwd_general_kernel_name(shape["in_shape"], shape["filt"], (n, ho, wo, f),
                                              p, filter_is_fcrs=False, dtype=0)
    assert name == {"band": "igemm_fwd_band_kernel", "tiled": "igemm_fwd_kernel"}[kernel]
    # the plain NK matrix either way
    assert igc.conv2d_fwd_general_workspace_bytes(
        shape["in_shape"], shape["filt"], (n, ho, wo, f), p, filter_is_fcrs=False,
        dtype=0) == igc.conv2d_workspace_bytes(shape["filt"], False, 0)

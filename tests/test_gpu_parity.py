"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (from the arithmetic: fp32 accumulation of exactly-rounded inputs,
one final rounding to bf16/fp16 with a relative error of at most 2^-9 / 2^-11):
  max|gpu - ref| <= 1e-2 * max|ref|  for bf16 / fp16 inputs,
  max|gpu - ref| <= 4e-2 * max|ref|  for fp8 e4m3fn inputs (bf16 output),
over the whole tensor, with every output finite.  Where the exact result is
representable in the output type (delta filters, all-ones border counts) the test asks for exact
bits.  Bitwise checks compare two GPU calls (layouts, residual forms,
in-place, determinism).
"""
import itertools
import os
import sys
import zlib

import numpy as np
import pytest
import torch

import datagen
import implicit_gemm_nhwc_amd as igc
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"bfloat16": 1e-2, "float16": 1e-2, "float8_e4m3fn": 4e-2}


def setup_module(_):
    if not os.path.exists(igc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    t = t.detach().cpu().contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16)
    return t.view(torch.uint8)


def _assert_close(got, ref, tol, what=""):
    g = got.detach().cpu().to(torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"non-finite GPU output {what}"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    if scale == 0.0:
        assert err == 0.0, what
    else:
        assert err <= tol * scale, f"{what}: max|err| {err:.4g} > {tol} * {scale:.4g}"
    return err, scale


def _run(x, w, *, fcrs, stride, pad, src=None, beta=0.0, ws=True):
    """conv2d_fwd on device copies; returns the output tensor (on device)."""
    xd, wd = x.to(DEV), w.to(DEV)
    sd = None if src is None else src.to(DEV)
    if fcrs:
        f, _, r, s = w.shape
    else:
        r, s, _, f = w.shape
    n, h, wi, _ = x.shape
    ho, wo = igc.out_hw(h, wi, r, s, stride, pad)
    out = torch.empty((n, ho, wo, f), dtype=datagen.OUT_DTYPES[_name(x.dtype)], device=DEV)
    wsd = None
    if ws:
        nb = igc.conv2d_workspace_bytes(w.shape, fcrs, x.dtype)
        wsd = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    rc = igc.conv2d_fwd(xd, wd, out, filter_is_fcrs=fcrs, stride=stride, padding=pad,
                        source=sd, beta=beta, workspace=wsd)
    assert rc == 1, f"conv2d_fwd returned {rc}"
    torch.cuda.synchronize()
    return out


def _name(dtype):
    return {torch.bfloat16: "bfloat16", torch.float16: "float16",
            torch.float8_e4m3fn: "float8_e4m3fn"}[dtype]


# ------------------------------------------------------------------ NK
@pytest.mark.parametrize("dtype", ["bfloat16", "float16", "float8_e4m3fn"])
@pytest.mark.parametrize("fcrs", [False, True])
@pytest.mark.parametrize("r,s,c,f", [(3, 3, 16, 16), (3, 3, 64, 64), (5, 5, 32, 3),
                                     (1, 1, 48, 17), (3, 2, 128, 5), (3, 3, 3, 16),
                                     (7, 7, 3, 64), (1, 3, 12, 5), (3, 3, 1, 1)])
def test_filter_to_nk_bit_exact(dtype, fcrs, r, s, c, f):
    _say(f"NK transpose {dtype} fcrs={fcrs} R{r} S{s} C{c} F{f}")
    _, w, _ = datagen.make_case(N=1, H=1, W=1, C=c, F=f, R=r, S=s, dtype=dtype, fcrs=fcrs,
                                x_dist=("normal", 1.0), w_dist=("normal", 1.0), seed=3)
    pitch = igc.conv2d_nk_row_pitch(w.shape, fcrs, w.dtype)
    nk = torch.full((f, pitch), 0x55 if dtype == "float8_e4m3fn" else 0x5555,
                    dtype=torch.uint8 if dtype == "float8_e4m3fn" else torch.int16,
                    device=DEV)
    assert igc.conv2d_filter_to_nk(w.to(DEV), nk, filter_is_fcrs=fcrs) == 1
    torch.cuda.synchronize()
    want = _bits(oracle.filter_to_nk(w, fcrs, k_pad=pitch))
    assert torch.equal(nk.cpu().view(want.dtype), want)


# ----------------------------------------------------- named workloads
@pytest.mark.parametrize("name", datagen.WORKLOAD_ORDER)
def test_workload_parity(name):
    spec, x, w, src = datagen.make_workload(name)
    _say(f"workload {name}: {spec['dtype']} N{spec['N']} {spec['H']}x{spec['W']} "
         f"C{spec['C']}->{spec['F']} {spec['R']}x{spec['S']} st{spec['stride']} "
         f"p{spec['pad']} fcrs={spec['fcrs']} residual={src is not None}")
    out = _run(x, w, fcrs=spec["fcrs"], stride=spec["stride"], pad=spec["pad"], src=src,
               beta=spec["beta"])
    tol = TOL[spec["dtype"]]
    # the whole output tensor against the oracle (the fp8 5x5 workload's
    # 214.7 GFLOP take the oracle a few seconds on the host's cores)
    ref = oracle.conv2d(x, w, filter_is_fcrs=spec["fcrs"], stride=spec["stride"],
                        padding=spec["pad"], source=src, beta=spec["beta"])
    err, scale = _assert_close(out, ref, tol, name)
    _say(f"  max|err|/max|ref| = {err / max(scale, 1e-300):.3e}")


def test_fp8_workload_fcrs_variant_bitwise():
    """The fp8 workload's filter stored FCRS gives the same bits as RSCF."""
    spec, x, w, src = datagen.make_workload("fp8_5x5_256c_residual_n16")
    _say("fp8 workload, RSCF vs FCRS")
    wf = w.view(torch.uint8).permute(3, 2, 0, 1).contiguous().view(w.dtype)
    a = _run(x, w, fcrs=False, stride=1, pad=2, src=src, beta=0.5)
    b = _run(x, wf, fcrs=True, stride=1, pad=2, src=src, beta=0.5)
    assert torch.equal(_bits(a), _bits(b))


# ------------------------------------------------------ kernel paths
# One case per kernel variant the dispatcher can pick, each checked to go
# where it is meant to (conv2d_fwd_kernel_name) and against the oracle over
# the whole output.  The "single" cases give a wave a single block of output
# pixels, so the epilogue may read the final MFMA's accumulators first.
PATH_CASES = [
    # id, dtype, N, H, W, C, F, R, S, stride, pad, residual, kernel
    # (a 1x1 filter: with a spatial filter this layer takes the patch kernel)
    ("wide256_bf16_tap", "bfloat16", 16, 64, 64, 64, 256, 1, 1, 1, 0, False, "wide"),
    ("wide256_fp16_walk", "float16", 16, 64, 64, 48, 192, 3, 3, 1, 1, True, "wide"),
    ("wide256_fp8_walk", "float8_e4m3fn", 16, 64, 64, 80, 256, 3, 3, 1, 1, False, "wide"),
    ("wide128_bf16_walk_s2_f160", "bfloat16", 4, 30, 30, 96, 160, 3, 3, 2, 1, True, "wide"),
    ("wide128_fp8_tap", "float8_e4m3fn", 2, 20, 20, 128, 96, 3, 3, 1, 1, False, "wide"),
    # more 128 x 128 tiles than CUs (384): 128 x 128 tiles; with fewer the
    # cases above take 128 x 64 tiles in three stages
    ("wide128_bf16_many_tiles", "bfloat16", 12, 64, 64, 64, 96, 3, 3, 1, 1, True, "wide"),
    # 128 x 128 tiles between 1.25 and 2 per CU (368) and C_out a multiple of
    # 256: 256 x 128 tiles of 8 waves, tap-aligned and walked k-tiles
    ("wide256x128_bf16_tap_s2", "bfloat16", 30, 56, 56, 128, 256, 3, 3, 2, 1, True, "wide"),
    ("wide256x128_fp8_walk_s2", "float8_e4m3fn", 30, 56, 56, 80, 256, 3, 3, 2, 1, False, "wide"),
    ("band_u1_bf16", "bfloat16", 2, 20, 20, 16, 48, 3, 3, 1, 1, False, "band"),
    ("band_u2_fp16_tm1", "float16", 2, 20, 20, 32, 24, 5, 5, 1, 2, True, "band"),
    ("band_u1_fp8", "float8_e4m3fn", 2, 20, 20, 64, 64, 3, 3, 1, 1, False, "band"),
    ("band_u2_fp8_resid", "float8_e4m3fn", 2, 20, 20, 128, 32, 3, 3, 1, 1, True, "band"),
    ("band_u4_bf16_s2", "bfloat16", 2, 28, 28, 64, 64, 3, 3, 2, 1, False, "band"),
    ("band_lds_epilogue", "bfloat16", 2, 20, 20, 64, 20, 3, 3, 1, 1, True, "band"),
    # one accumulator block per wave: the epilogue reads the last MFMA first
    ("band_fp8_single_block", "float8_e4m3fn", 1, 8, 8, 64, 16, 3, 3, 1, 1, False, "band"),
    # tap-fold kernel: C_out * R * S <= 32 (3x3 up to 3 channels, 5x5 one,
    # 1x3 eight), strides 1 and 2, paddings 0..2, several strips and row
    # segments, partial last strip and segment
    ("tapfold_bf16_rgb", "bfloat16", 2, 40, 70, 128, 3, 3, 3, 1, 1, False, "tapfold"),
    ("tapfold_fp16_s2_resid", "float16", 2, 33, 41, 64, 2, 3, 3, 2, 1, True, "tapfold"),
    ("tapfold_fp8_p0", "float8_e4m3fn", 1, 30, 50, 64, 3, 3, 3, 1, 0, False, "tapfold"),
    ("tapfold_bf16_5x5_f1", "bfloat16", 2, 20, 20, 32, 1, 5, 5, 1, 2, True, "tapfold"),
    ("tapfold_bf16_1x3_f8", "bfloat16", 1, 17, 300, 32, 8, 1, 3, 1, 0, False, "tapfold"),
    ("tapfold_fp8_s2_p2_resid", "float8_e4m3fn", 2, 19, 23, 128, 3, 3, 3, 2, 2, True, "tapfold"),
    ("tapfold_fp16_c256", "float16", 1, 9, 9, 256, 1, 3, 3, 1, 1, False, "tapfold"),
    # rows of at most eight 1 KB blocks go through the loader registers (the
    # cases above but c256 and the fp8 one below): three output rows per
    # workgroup (five input rows through the two-slot ring); fp8 with
    # C_in = 256 (four k-steps) keeps the load-to-LDS ring
    ("tapfold_bf16_rgb_th3_resid", "bfloat16", 4, 128, 128, 128, 3, 3, 3, 1, 1, True, "tapfold"),
    ("tapfold_fp8_c256_ring", "float8_e4m3fn", 2, 20, 40, 256, 3, 3, 3, 1, 1, False, "tapfold"),
    ("resident_c48", "bfloat16", 2, 20, 20, 48, 32, 3, 3, 1, 1, False, "resident"),
    ("resident_fp16_c48", "float16", 2, 10, 10, 48, 24, 3, 3, 1, 1, True, "resident"),
    ("resident_fp8_single", "float8_e4m3fn", 1, 4, 4, 48, 16, 3, 3, 1, 1, True, "resident"),
    ("fallback_tiled", "bfloat16", 1, 12, 12, 96, 64, 5, 5, 1, 2, True, "tiled"),
    ("fallback_tiled_fp16", "float16", 1, 12, 12, 96, 64, 5, 5, 1, 2, True, "tiled"),
    ("fallback_tiled_fp8", "float8_e4m3fn", 1, 12, 12, 48, 64, 5, 5, 1, 2, False, "tiled"),
    ("fallback_tiled_fp8_single", "float8_e4m3fn", 1, 4, 4, 208, 16, 5, 5, 1, 2, True, "tiled"),
    ("wide_fp8_single", "float8_e4m3fn", 1, 4, 4, 64, 96, 3, 3, 1, 1, True, "wide"),
    # C_in * E not a multiple of 16: the tiled kernel's element gather (taps
    # spanning a 16-byte chunk of k), any C_out
    ("eg_bf16_c3", "bfloat16", 2, 20, 22, 3, 64, 3, 3, 1, 1, False, "tiled"),
    ("eg_fp16_c12_s2", "float16", 1, 17, 19, 12, 24, 3, 3, 2, 1, True, "tiled"),
    ("eg_fp8_c8", "float8_e4m3fn", 2, 15, 15, 8, 96, 3, 3, 1, 1, True, "tiled"),
    ("eg_bf16_c1_f3_5x5", "bfloat16", 1, 30, 31, 1, 3, 5, 5, 1, 2, False, "tiled"),
    ("eg_bf16_c20_f130", "bfloat16", 1, 14, 13, 20, 130, 3, 3, 1, 0, True, "tiled"),
    ("eg_fp8_c3_s2", "float8_e4m3fn", 1, 33, 31, 3, 16, 3, 3, 2, 2, False, "tiled"),
    ("wide256_fp8_resid", "float8_e4m3fn", 16, 64, 64, 64, 256, 3, 3, 1, 1, True, "wide"),
    # patch-resident kernel: stride 1, C_in a whole number of 128-byte
    # chunks, at least one 256-pixel tile per CU.  One chunk; three chunks
    # (two patch swaps) with C_out = 160 (channel rows past C_out masked);
    # ragged 60 x 60 output (partial tiles) with C_out = 192; a 1 x 3
    # filter without padding; 7 x 7 (padding 2: a ragged 62 x 62 output)
    # with C_out = 256 (two filter stages beside the larger patch)
    ("patch_bf16_3x3_one_chunk", "bfloat16", 16, 64, 64, 64, 256, 3, 3, 1, 1, False, "patch"),
    ("patch_fp16_5x5_three_chunks_f160", "float16", 16, 64, 64, 192, 160, 5, 5, 1, 2, True,
     "patch"),
    ("patch_fp8_3x3_two_chunks", "float8_e4m3fn", 16, 64, 64, 256, 256, 3, 3, 1, 1, True, "patch"),
    ("patch_bf16_ragged_f192", "bfloat16", 16, 60, 60, 128, 192, 3, 3, 1, 1, True, "patch"),
    ("patch_fp8_1x3_f128", "float8_e4m3fn", 16, 64, 66, 128, 128, 1, 3, 1, 0, False, "patch"),
    ("patch_bf16_7x7_two_stages", "bfloat16", 16, 64, 64, 64, 256, 7, 7, 1, 2, False, "patch"),
    # 128-pixel tiles (256-pixel ones would leave half the CUs idle): 64 and
    # 128 output channels per wave
    ("patch128_bf16_f128_resid", "bfloat16", 8, 64, 64, 64, 128, 3, 3, 1, 1, True, "patch"),
    ("patch128_fp8_f256", "float8_e4m3fn", 8, 64, 64, 128, 256, 3, 3, 1, 1, False, "patch"),
]
_KERNEL = {"wide": "igemm_fwd_wide_kernel", "band": "igemm_fwd_band_kernel",
           "patch": "igemm_fwd_patch_kernel",
           "tapfold": "igemm_fwd_tapfold_kernel",
           "resident": "igemm_fwd_resident_kernel", "tiled": "igemm_fwd_kernel"}


@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: c[0])
def test_kernel_paths(case):
    cid, dt, n, h, w, c, f, r, s, st, p, resid, kern = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    _say(f"path {cid}: {dt} N{n} {h}x{w} C{c}->{f} {r}x{s} st{st} p{p} residual={resid}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(cid.encode()) % 1000)
    got_kernel = igc.conv2d_fwd_kernel_name(x.shape, wt.shape, (n, ho, wo, f),
                                            filter_is_fcrs=False, dtype=x.dtype, stride=st,
                                            padding=p)
    assert got_kernel == _KERNEL[kern], (cid, got_kernel)
    beta = 0.5 if resid else 0.0
    out = _run(x, wt, fcrs=False, stride=st, pad=p, src=src, beta=beta)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p, source=src,
                        beta=beta)
    _assert_close(out, ref, TOL[dt], cid)


# ------------------------------------------------------ randomized sweep
def _sweep_cases():
    rng = np.random.default_rng(2024)
    dtypes = ["bfloat16", "float16", "float8_e4m3fn"]
    couts = [1, 2, 3, 4, 5, 8, 15, 16, 17, 33, 64, 100, 130]
    cases = []
    for i, (dt, fcrs, st, p, resid) in enumerate(itertools.product(
            dtypes, [False, True], [1, 2], [0, 1, 2], [False, True])):
        f = couts[i % len(couts)]
        c = int(rng.choice([16, 32, 48, 64, 128] if dt != "float8_e4m3fn" else [16, 32, 64, 128]))
        r = int(rng.choice([1, 2, 3, 5]))
        s = int(rng.choice([1, 3, 5]))
        h = int(rng.integers(max(r, 3), 19))
        w = int(rng.integers(max(s, 3), 19))
        n = int(rng.integers(1, 3))
        cases.append((dt, fcrs, st, p, resid, n, h, w, c, f, r, s))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_sweep(case):
    dt, fcrs, st, p, resid, n, h, w, c, f, r, s = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    _say(f"sweep {case} -> out {n}x{ho}x{wo}x{f}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=fcrs,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(repr(case).encode()) % 1000)
    beta = -0.75 if resid else 0.0
    out = _run(x, wt, fcrs=fcrs, stride=st, pad=p, src=src, beta=beta)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=st, padding=p, source=src, beta=beta)
    _assert_close(out, ref, TOL[dt], str(case))


def _patch_sweep_cases():
    """Random layers the patch-resident kernel takes (stride 1, C_out > 64 and
    a multiple of 4, C_in a whole number of 128-byte chunks, enough tiles:
    draws the host-side kernel query sends elsewhere are skipped), with
    ragged sizes, 1 x 2 up to 5 x 5 filters, every padding, residuals and
    RSCF / FCRS filters; at most 30 GFLOP each for the oracle."""
    rng = np.random.default_rng(77)
    tdt = {"bfloat16": torch.bfloat16, "float16": torch.float16,
           "float8_e4m3fn": torch.float8_e4m3fn}
    cases = []
    for i in range(400):
        if len(cases) == 14:
            break
        dt = ["bfloat16", "float16", "float8_e4m3fn"][len(cases) % 3]
        e = 1 if dt == "float8_e4m3fn" else 2
        c = int(rng.choice([128, 256])) // e
        f = int(rng.choice([68, 100, 128, 132, 192, 256]))
        r = int(rng.integers(1, 6))
        s = int(rng.integers(1 if r > 1 else 2, 6))
        p = int(rng.integers(0, 3))
        n = int(rng.choice([8, 12, 16]))
        h = int(rng.integers(40, 80))
        w = int(rng.integers(40, 80))
        resid = bool(rng.integers(0, 2))
        fcrs = bool(rng.integers(0, 2))
        ho, wo = oracle.out_size(h, r, 1, p), oracle.out_size(w, s, 1, p)
        if 2 * n * ho * wo * f * r * s * c > 30e9:
            continue
        ws = (f, c, r, s) if fcrs else (r, s, c, f)
        if igc.conv2d_fwd_kernel_name((n, h, w, c), ws, (n, ho, wo, f), filter_is_fcrs=fcrs,
                                      dtype=tdt[dt], stride=1,
                                      padding=p) != "igemm_fwd_patch_kernel":
            continue
        cases.append((dt, fcrs, p, resid, n, h, w, c, f, r, s))
    return cases


@pytest.mark.parametrize("case", _patch_sweep_cases(), ids=lambda c: "-".join(map(str, c)))
def test_patch_random_sweep(case):
    dt, fcrs, p, resid, n, h, w, c, f, r, s = case
    ho, wo = oracle.out_size(h, r, 1, p), oracle.out_size(w, s, 1, p)
    _say(f"patch sweep {case} -> out {n}x{ho}x{wo}x{f}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=fcrs,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(repr(case).encode()) % 1000)
    assert igc.conv2d_fwd_kernel_name(x.shape, wt.shape, (n, ho, wo, f), filter_is_fcrs=fcrs,
                                      dtype=x.dtype, stride=1,
                                      padding=p) == "igemm_fwd_patch_kernel", case
    beta = -0.75 if resid else 0.0
    out = _run(x, wt, fcrs=fcrs, stride=1, pad=p, src=src, beta=beta)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=1, padding=p, source=src, beta=beta)
    _assert_close(out, ref, TOL[dt], str(case))


@pytest.mark.parametrize("dt", ["bfloat16", "float8_e4m3fn"])
@pytest.mark.parametrize("m_extra", [1, 15, 17, 255, 257])
def test_pixel_tails(dt, m_extra):
    """M just past tile multiples: M = Wo = 256 + m_extra (one row, 1x3 filter)."""
    n, h, w = 1, 1, 258 + m_extra
    _say(f"pixel tail {dt} M={256 + m_extra}")
    x, wt, _ = datagen.make_case(N=n, H=h, W=w, C=32, F=40, R=1, S=3, dtype=dt, fcrs=False,
                                 x_dist=("normal", 1.0), w_dist=("normal", 1.0), seed=7)
    out = _run(x, wt, fcrs=False, stride=1, pad=0, src=None)
    assert out.shape[2] == 256 + m_extra
    ref = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=0)
    _assert_close(out, ref, TOL[dt])


# ------------------------------------------------------ exact special cases
@pytest.mark.parametrize("dt", ["bfloat16", "float16", "float8_e4m3fn"])
@pytest.mark.parametrize("k,st", [(1, 1), (3, 1), (5, 1), (3, 2)])
def test_centered_delta_bit_exact(dt, k, st):
    p = (k - 1) // 2
    c = 32
    _say(f"delta {dt} k{k} st{st}")
    x, _, _ = datagen.make_case(N=2, H=9, W=11, C=c, F=c, R=1, S=1, dtype=dt, fcrs=False,
                                x_dist=("normal", 2.0), w_dist=("normal", 1.0), seed=11)
    w = torch.zeros((k, k, c, c), dtype=torch.float32)
    for ci in range(c):
        w[p, p, ci, ci] = 1.0
    w = w.to(x.dtype)
    out = _run(x, w, fcrs=False, stride=st, pad=p)
    # exact in bf16/fp16; "+ 0.0" because a sum that starts at +0 turns -0 into +0
    want = (x[:, ::st, ::st, :].to(torch.float32) + 0.0).to(out.dtype)
    assert torch.equal(_bits(out), _bits(want))


def test_fp8_every_code_through_delta():
    """Every finite e4m3fn code passes through a 1x1 identity filter into bf16
    bit-exactly (the two NaN codes are replaced by +-0: a NaN would spread to
    its whole pixel through NaN * 0; -0 comes out as +0, as in IEEE sums
    started at +0)."""
    _say("fp8 all codes via identity")
    codes = torch.arange(256, dtype=torch.int64)
    codes[0x7F], codes[0xFF] = 0x00, 0x80
    x = codes.to(torch.uint8).reshape(1, 1, 16, 16).view(torch.float8_e4m3fn).contiguous()
    w = torch.eye(16, dtype=torch.float32).reshape(1, 1, 16, 16).to(torch.float8_e4m3fn)
    out = _run(x, w, fcrs=False, stride=1, pad=0)
    want = (x.to(torch.float32) + 0.0).to(torch.bfloat16)   # -0 sums to +0
    assert torch.equal(_bits(out), _bits(want))


@pytest.mark.parametrize("k,st,p", [(3, 1, 1), (3, 2, 1), (5, 1, 2), (5, 2, 2), (3, 1, 0),
                                    (2, 2, 2)])
def test_all_ones_border_exact(k, st, p):
    n, h, w, c, f = 2, 13, 10, 16, 20
    _say(f"all-ones k{k} st{st} p{p}")
    x = torch.ones((n, h, w, c), dtype=torch.bfloat16)
    wt = torch.ones((k, k, c, f), dtype=torch.bfloat16)
    out = _run(x, wt, fcrs=False, stride=st, pad=p)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p)
    np.testing.assert_array_equal(out.cpu().to(torch.float64).numpy(), ref)


# --------------------------------------------------------------- invariants
@pytest.mark.parametrize("dt", ["bfloat16", "float16", "float8_e4m3fn"])
def test_layouts_bitwise_equal(dt):
    _say(f"layouts {dt}")
    x, w, _ = datagen.make_case(N=2, H=14, W=9, C=64, F=48, R=3, S=3, dtype=dt, fcrs=False,
                                x_dist=("normal", 1.0), w_dist=("normal", 0.2), seed=13)
    wb = _bits(w)
    wf = wb.permute(3, 2, 0, 1).contiguous().view(w.dtype)
    a = _run(x, w, fcrs=False, stride=1, pad=1)
    b = _run(x, wf, fcrs=True, stride=1, pad=1)
    assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("dt", ["bfloat16", "float16", "float8_e4m3fn"])
def test_residual_forms(dt):
    _say(f"residual forms {dt}")
    x, w, src = datagen.make_case(N=2, H=10, W=12, C=32, F=36, R=3, S=3, dtype=dt, fcrs=True,
                                  x_dist=("normal", 1.0), w_dist=("normal", 0.3),
                                  src_dist=("normal", 1.0), out_hw=(10, 12), seed=17)
    plain = _run(x, w, fcrs=True, stride=1, pad=1)
    zero = _run(x, w, fcrs=True, stride=1, pad=1, src=src, beta=0.0)
    assert torch.equal(_bits(plain), _bits(zero))        # beta = 0: D == conv
    d = _run(x, w, fcrs=True, stride=1, pad=1, src=src, beta=1.0)
    ref = oracle.conv2d(x, w, filter_is_fcrs=True, stride=1, padding=1, source=src, beta=1.0)
    _assert_close(d, ref, TOL[dt])
    # in place: source == output
    inplace = src.to(DEV).clone()
    rc = igc.conv2d_fwd(x.to(DEV), w.to(DEV), inplace, filter_is_fcrs=True, stride=1,
                        padding=1, source=inplace, beta=1.0)
    assert rc == 1
    torch.cuda.synchronize()
    assert torch.equal(_bits(inplace), _bits(d))


def test_fwd_nk_and_nullptr_workspace_match_fwd():
    _say("fwd_nk / NULL workspace")
    x, w, _ = datagen.make_case(N=2, H=17, W=15, C=64, F=64, R=3, S=3, dtype="bfloat16",
                                fcrs=True, x_dist=("normal", 1.0), w_dist=("normal", 0.1),
                                seed=19)
    a = _run(x, w, fcrs=True, stride=2, pad=1)
    b = _run(x, w, fcrs=True, stride=2, pad=1, ws=False)
    assert torch.equal(_bits(a), _bits(b))
    nk = torch.empty(igc.conv2d_workspace_bytes(w.shape, True, w.dtype), dtype=torch.uint8,
                     device=DEV)
    assert igc.conv2d_filter_to_nk(w.to(DEV), nk, filter_is_fcrs=True) == 1
    c = torch.empty_like(a)
    assert igc.conv2d_fwd_nk(x.to(DEV), nk, w.shape, c, filter_is_fcrs=True, stride=2,
                             padding=1) == 1
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(c))


def test_deterministic():
    _say("determinism")
    x, w, _ = datagen.make_case(N=4, H=28, W=28, C=128, F=256, R=3, S=3, dtype="float16",
                                fcrs=False, x_dist=("uniform", 1.0), w_dist=("uniform", 1.0),
                                seed=23)
    a = _run(x, w, fcrs=False, stride=1, pad=1)
    b = _run(x, w, fcrs=False, stride=1, pad=1)
    assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("f", [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 33, 63, 65, 129])
def test_store_masks_guard_bands(f):
    """Output inside a larger buffer: the guard bands on both sides must keep
    their sentinel bits (no store past co >= C_out or m >= M)."""
    n, h, w, c = 1, 7, 13, 32
    _say(f"guard bands C_out={f}")
    x, wt, _ = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=3, S=3, dtype="bfloat16",
                                 fcrs=False, x_dist=("normal", 1.0), w_dist=("normal", 0.2),
                                 seed=29)
    numel = n * h * w * f
    guard = 4096
    buf = torch.full((guard + numel + guard,), -12345, dtype=torch.int16, device=DEV)
    out = buf[guard:guard + numel].view(torch.bfloat16).view(n, h, w, f)
    nb = igc.conv2d_workspace_bytes(wt.shape, False, wt.dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    rc = igc.conv2d_fwd(x.to(DEV), wt.to(DEV), out, filter_is_fcrs=False, stride=1, padding=1,
                        workspace=ws)
    assert rc == 1
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:guard] == -12345) and torch.all(b[guard + numel:] == -12345)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=1)
    _assert_close(out, ref, 1e-2)


# ---------------------------------------------------------- degenerate cases
def test_empty_batch_and_zero_channels():
    _say("empty batch / C_in = 0")
    x = torch.empty((0, 8, 8, 16), dtype=torch.bfloat16, device=DEV)
    w = torch.ones((3, 3, 16, 8), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0, 8, 8, 8), dtype=torch.bfloat16, device=DEV)
    assert igc.conv2d_fwd(x, w, out, filter_is_fcrs=False, stride=1, padding=1) == 1
    # C_in = 0: K = 0, the result is beta * source (or zeros)
    x0 = torch.empty((1, 6, 6, 0), dtype=torch.bfloat16, device=DEV)
    w0 = torch.empty((3, 3, 0, 8), dtype=torch.bfloat16, device=DEV)
    src = torch.randn((1, 6, 6, 8), device=DEV).to(torch.bfloat16)
    out0 = torch.full((1, 6, 6, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    assert igc.conv2d_fwd(x0, w0, out0, filter_is_fcrs=False, stride=1, padding=1,
                          source=src, beta=2.0) == 1
    torch.cuda.synchronize()
    assert torch.equal(out0.float(), 2.0 * src.float())
    out1 = torch.full((1, 6, 6, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    assert igc.conv2d_fwd(x0, w0, out1, filter_is_fcrs=False, stride=1, padding=1) == 1
    torch.cuda.synchronize()
    assert torch.all(out1.float() == 0)


# ------------------------------------------ filter transposed in the kernel
# id, dtype, N, H, W, C, F, R, S, stride, pad, residual
FILTER_IN_KERNEL = [
    ("bf16_f64", "bfloat16", 2, 17, 15, 64, 64, 3, 3, 1, 1, True),
    ("fp16_f40_zero_row_s2", "float16", 2, 19, 18, 32, 40, 3, 3, 2, 1, False),
    ("fp16_f24_5x5", "float16", 2, 20, 20, 32, 24, 5, 5, 1, 2, True),
    ("bf16_f16_1x1", "bfloat16", 2, 16, 18, 64, 16, 1, 1, 1, 0, False),
    ("bf16_f32_1x3", "bfloat16", 1, 13, 30, 32, 32, 1, 3, 1, 1, True),
    # blocks of more than one round per thread (RSCF: 2 per round)
    ("bf16_f48_c128_rounds", "bfloat16", 1, 12, 14, 128, 48, 3, 3, 1, 1, False),
    # the NK path only: C_out not a multiple of 8 (RSCF), R*S = 6 (FCRS), fp8
    ("bf16_f5", "bfloat16", 1, 12, 13, 16, 5, 3, 3, 1, 1, False),
    ("bf16_2x3", "bfloat16", 1, 12, 13, 32, 16, 2, 3, 1, 1, False),
    ("fp8_f24", "float8_e4m3fn", 2, 14, 16, 64, 24, 3, 3, 1, 1, True),
]


def _in_kernel(dt, fcrs, f, r, s):
    return dt != "float8_e4m3fn" and ((r * s in (1, 9)) if fcrs else f % 8 == 0)


@pytest.mark.parametrize("fcrs", [False, True])
@pytest.mark.parametrize("case", FILTER_IN_KERNEL, ids=lambda c: c[0])
def test_filter_in_kernel_matches_nk_path(case, fcrs):
    """conv2d_fwd on the band kernel transposes a bf16 / fp16 stored filter
    into LDS itself (RSCF with C_out a multiple of 8, FCRS with R*S of 1 or
    9): the same bits as the NK path (conv2d_filter_to_nk, then
    conv2d_fwd_nk), the oracle's values, and the workspace left untouched.
    Other filters take the NK path inside conv2d_fwd."""
    cid, dt, n, h, w, c, f, r, s, st, p, resid = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    _say(f"filter in kernel {cid} fcrs={fcrs}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=fcrs,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(cid.encode()) % 1000)
    assert igc.conv2d_fwd_kernel_name(x.shape, wt.shape, (n, ho, wo, f), filter_is_fcrs=fcrs,
                                      dtype=x.dtype, stride=st,
                                      padding=p) == "igemm_fwd_band_kernel"
    fused = _in_kernel(dt, fcrs, f, r, s)
    assert igc.conv2d_fwd_filter_in_kernel(x.shape, wt.shape, (n, ho, wo, f),
                                           filter_is_fcrs=fcrs, dtype=x.dtype, stride=st,
                                           padding=p) == fused
    beta = 0.5 if resid else 0.0
    xd, wd = x.to(DEV), wt.to(DEV)
    sd = None if src is None else src.to(DEV)
    nkb = igc.conv2d_workspace_bytes(wt.shape, fcrs, wt.dtype)
    ws = torch.full((nkb,), 0x5A, dtype=torch.uint8, device=DEV)
    a = torch.empty((n, ho, wo, f), dtype=datagen.OUT_DTYPES[dt], device=DEV)
    assert igc.conv2d_fwd(xd, wd, a, filter_is_fcrs=fcrs, stride=st, padding=p, source=sd,
                          beta=beta, workspace=ws) == 1
    nk = torch.empty(nkb, dtype=torch.uint8, device=DEV)
    assert igc.conv2d_filter_to_nk(wd, nk, filter_is_fcrs=fcrs) == 1
    b = torch.empty_like(a)
    assert igc.conv2d_fwd_nk(xd, nk, wt.shape, b, filter_is_fcrs=fcrs, stride=st, padding=p,
                             source=sd, beta=beta) == 1
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))
    if fused:
        assert bool((ws == 0x5A).all())
    ref = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=st, padding=p, source=src, beta=beta)
    _assert_close(a, ref, TOL[dt], cid)

"""GPU parity of the transposed convolution (page "conv_transposed_gpu":
NHWC input, RSFC filter) through conv2d_transposed_fwd, against the fp64
oracle (oracle.conv2d_transposed, a scatter-form implementation pinned by
hand-worked cases, brute force and the adjoint identity with conv2d).
Tolerances as for the forward convolution.
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
from test_gpu_parity import TOL, _assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def setup_module(_):
    if not os.path.exists(igc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # dtype, N, H, W, C, F, R, stride, pad, residual/epilogue
    ("bfloat16", 2, 20, 18, 32, 48, 3, 1, 1, False),
    ("float16", 2, 16, 16, 64, 96, 3, 1, 0, True),
    ("float8_e4m3fn", 2, 14, 15, 64, 32, 5, 1, 2, True),
    ("bfloat16", 1, 12, 12, 128, 130, 1, 1, 0, False),
    ("bfloat16", 2, 17, 9, 32, 16, 2, 1, 0, True),
    ("float16", 1, 24, 24, 64, 64, 4, 1, 1, False),
    ("bfloat16", 8, 32, 32, 256, 128, 3, 1, 1, True),
    # stride 2: four phase convolutions and the interleave
    ("bfloat16", 2, 16, 12, 32, 48, 4, 2, 1, False),     # the 2x upsampler
    ("float16", 2, 11, 13, 64, 96, 3, 2, 1, True),
    ("float8_e4m3fn", 1, 10, 9, 64, 32, 2, 2, 0, True),
    ("bfloat16", 1, 9, 10, 32, 20, 5, 2, 2, True),       # C_out not a multiple of 8
    ("bfloat16", 2, 8, 8, 64, 130, 3, 2, 0, False),
    ("float16", 1, 12, 12, 32, 16, 6, 2, 2, True),
    # even R: the four phases share one shape and run as one grouped launch
    # (band kernel above for R = 4, 2, 6; wide kernel here)
    ("bfloat16", 2, 10, 12, 64, 96, 4, 2, 1, True),
    ("float8_e4m3fn", 1, 8, 8, 128, 256, 2, 2, 0, False),
    # 128-byte channel chunks and enough 128-pixel tiles over the four phases
    # (256): the grouped, mapped launch of the patch kernel, 128 and 256
    # output channels per workgroup (the first is the benchmark's upsampler)
    ("bfloat16", 8, 32, 32, 256, 128, 4, 2, 1, True),
    ("float8_e4m3fn", 8, 32, 32, 128, 256, 4, 2, 1, False),
    ("bfloat16", 8, 32, 32, 64, 256, 4, 2, 1, True),
    # 192-byte pixels: enough 128 x 128 tiles over the four phases (512) for
    # the grouped wide launch to keep 128 x 128 tiles (smaller ones take
    # 128 x 64)
    ("bfloat16", 8, 32, 32, 96, 256, 4, 2, 1, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_transposed_matches_oracle(case):
    dt, n, h, w, c, f, r, st, p, fused = case
    ho, wo = (h - 1) * st - 2 * p + r, (w - 1) * st - 2 * p + r
    _say(f"transposed {case} -> out {n}x{ho}x{wo}x{f}")
    seed = zlib.crc32(repr(case).encode()) % 1000
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype=dt, fcrs=False,
                                     x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                     src_dist=("normal", 1.0) if fused else None,
                                     out_hw=(ho, wo), seed=seed)
    # an RSFC filter [R, S, F, C]: the seeded RSCF draw [R, S, C, F] re-laid out
    wt = wfwd.permute(0, 1, 3, 2).contiguous()
    kw, okw = {}, {}
    if fused:
        g = torch.Generator().manual_seed(seed + 1)
        scale = (torch.rand(f, generator=g) + 0.5).float()
        bias = torch.randn(f, generator=g).float()
        kw = dict(source=src.to(DEV), beta=0.5, scale=scale.to(DEV), bias=bias.to(DEV),
                  activation="silu")
        okw = dict(source=src, beta=0.5, scale=scale, bias=bias, act="silu")
    out = igc.conv2d_transposed(x.to(DEV), wt.to(DEV), stride=st, padding=p, **kw)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (n, ho, wo, f)
    ref = oracle.conv2d_transposed(x, wt, stride=st, padding=p, **okw)
    _assert_close(out, ref, TOL[dt], str(case))


def test_transposed_stride2_in_place_and_workspace():
    # source == output (in place) with a caller workspace, against the
    # library-allocated, separate-source call: bitwise equal
    n, h, w, c, f, r, st, p = 2, 12, 10, 64, 64, 4, 2, 1
    ho, wo = (h - 1) * st - 2 * p + r, (w - 1) * st - 2 * p + r
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype="bfloat16",
                                     fcrs=False, x_dist=("normal", 1.0),
                                     w_dist=("normal", 0.1), src_dist=("normal", 1.0),
                                     out_hw=(ho, wo), seed=5)
    wt = wfwd.permute(0, 1, 3, 2).contiguous().to(DEV)
    xd, sd = x.to(DEV), src.to(DEV)
    a = torch.empty((n, ho, wo, f), dtype=torch.bfloat16, device=DEV)
    assert igc.conv2d_transposed_fwd(xd, wt, a, stride=st, padding=p, source=sd, beta=-1.5,
                                     activation="relu") == 1
    b = sd.clone()
    ws = torch.empty(igc.conv2d_transposed_workspace_bytes(x.shape, wt.shape, stride=st,
                                                           padding=p, dtype=x.dtype),
                     dtype=torch.uint8, device=DEV)
    assert igc.conv2d_transposed_fwd(xd, wt, b, stride=st, padding=p, source=b, beta=-1.5,
                                     activation="relu", workspace=ws) == 1
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.conv2d_transposed(x, wt.cpu(), stride=st, padding=p, source=src, beta=-1.5,
                                   act="relu")
    _assert_close(a, ref, TOL["bfloat16"], "in place")


def _tr_sweep():
    rng = np.random.default_rng(91)
    cases = []
    for i, (dt, st, r) in enumerate(itertools.product(
            ["bfloat16", "float16", "float8_e4m3fn"], [1, 2], [2, 3, 4, 5])):
        p = int(rng.integers(0, r))
        f = int(rng.choice([3, 8, 24, 64, 96, 136]))
        c = int(rng.choice([16, 32, 64] if dt != "float8_e4m3fn" else [16, 64, 128]))
        h, w = int(rng.integers(3, 14)), int(rng.integers(3, 14))
        cases.append((dt, int(rng.integers(1, 3)), h, w, c, f, r, st, p, bool(i % 2)))
    return cases


@pytest.mark.parametrize("case", _tr_sweep(), ids=lambda c: "-".join(map(str, c)))
def test_transposed_random_sweep(case):
    dt, n, h, w, c, f, r, st, p, fused = case
    ho, wo = (h - 1) * st - 2 * p + r, (w - 1) * st - 2 * p + r
    if ho < 1 or wo < 1:
        pytest.skip("empty output")
    code = igc.conv2d_transposed_check(0x10000000, 0x20000000, 0x30000000, stride=st, padding=p,
                                       dtype=igc.dtype_code(getattr(torch, dt)),
                                       in_shape=(n, h, w, c), filt_shape=(r, r, f, c),
                                       out_shape=(n, ho, wo, f))
    assert code == 0, igc.REASONS[code]
    _say(f"transposed sweep {case} -> out {n}x{ho}x{wo}x{f}")
    seed = zlib.crc32(repr(case).encode()) % 1000
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype=dt, fcrs=False,
                                     x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                     src_dist=("normal", 1.0) if fused else None,
                                     out_hw=(ho, wo), seed=seed)
    wt = wfwd.permute(0, 1, 3, 2).contiguous()
    kw, okw = {}, {}
    if fused:
        kw = dict(source=src.to(DEV), beta=-0.5, activation="relu")
        okw = dict(source=src, beta=-0.5, act="relu")
    out = igc.conv2d_transposed(x.to(DEV), wt.to(DEV), stride=st, padding=p, **kw)
    torch.cuda.synchronize()
    ref = oracle.conv2d_transposed(x, wt, stride=st, padding=p, **okw)
    _assert_close(out, ref, TOL[dt], str(case))


# Strides, dilations, paddings and filter shapes per axis: phases of
# different shapes (one launch each), phases without taps (epilogue only),
# dilated phases (the tiled kernel), negative phase paddings (large p).
# dtype, N, H, W, C, F, (R, S), stride, dilation, padding, fused
GENERAL = [
    ("bfloat16", 2, 9, 11, 32, 48, (3, 3), 1, 2, 1, True),          # dilation, stride 1
    ("float16", 1, 10, 8, 64, 24, (3, 2), 2, (2, 1), (1, 0), True),  # dilated phases
    ("bfloat16", 2, 7, 6, 32, 40, (3, 3), 3, 1, 1, False),           # stride 3
    ("float8_e4m3fn", 1, 6, 7, 64, 32, (2, 2), 3, 1, 0, True),       # phases without taps
    ("bfloat16", 1, 8, 9, 32, 72, (4, 3), (2, 3), 1, (1, 0), True),  # per-axis stride, R != S
    ("float16", 2, 12, 10, 32, 16, (3, 3), 1, 1, 3, False),          # p > R - 1: cropping
    ("bfloat16", 1, 9, 9, 64, 96, (5, 5), 2, 1, 4, True),            # negative phase padding
    ("bfloat16", 2, 10, 10, 32, 8, (1, 1), 2, 1, 0, True),           # 1x1 stride 2: zeros + epilogue
    ("float8_e4m3fn", 2, 8, 8, 128, 136, (2, 2), 2, 1, 0, True),     # wide kernel, grouped phases
    ("float16", 1, 7, 9, 64, 64, (3, 5), (3, 2), (2, 1), (2, 1), False),
    # C * E not a multiple of 16: element-wise flip, phases on the element gather
    ("bfloat16", 2, 9, 8, 12, 40, (4, 4), 2, 1, 1, True),                # grouped phases
    ("float8_e4m3fn", 1, 7, 7, 3, 16, (3, 3), 1, 1, 1, False),
    ("float16", 1, 6, 7, 20, 96, (3, 3), 3, 1, 0, True),
]


@pytest.mark.parametrize("case", GENERAL, ids=lambda c: "-".join(map(str, c)))
def test_transposed_general_matches_oracle(case):
    dt, n, h, w, c, f, (r, s), st, dil, p, fused = case
    ho, wo = igc.transposed_out_hw(h, w, r, s, stride=st, padding=p, dilation=dil)
    _say(f"transposed general {case} -> out {n}x{ho}x{wo}x{f}")
    seed = zlib.crc32(repr(case).encode()) % 1000
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                     x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                     src_dist=("normal", 1.0) if fused else None,
                                     out_hw=(ho, wo), seed=seed)
    wt = wfwd.permute(0, 1, 3, 2).contiguous()       # RSFC [R, S, F, C]
    kw, okw = {}, {}
    if fused:
        g = torch.Generator().manual_seed(seed + 1)
        scale = (torch.rand(f, generator=g) + 0.5).float()
        bias = torch.randn(f, generator=g).float()
        kw = dict(source=src.to(DEV), beta=0.75, scale=scale.to(DEV), bias=bias.to(DEV),
                  activation="relu")
        okw = dict(source=src, beta=0.75, scale=scale, bias=bias, act="relu")
    out = igc.conv2d_transposed(x.to(DEV), wt.to(DEV), stride=st, padding=p, dilation=dil, **kw)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (n, ho, wo, f)
    ref = oracle.conv2d_transposed(x, wt, stride=st, padding=p, dilation=dil, **okw)
    _assert_close(out, ref, TOL[dt], str(case))


def test_transposed_in_place_general():
    """source == output through the output map (stride 3, phases launched
    one by one): equal bits to a separate source."""
    n, h, w, c, f, r, st, p = 1, 7, 8, 32, 24, 4, 3, 1
    ho, wo = igc.transposed_out_hw(h, w, r, r, stride=st, padding=p)
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype="bfloat16",
                                     fcrs=False, x_dist=("normal", 1.0),
                                     w_dist=("normal", 0.1), src_dist=("normal", 1.0),
                                     out_hw=(ho, wo), seed=8)
    wt = wfwd.permute(0, 1, 3, 2).contiguous().to(DEV)
    xd, sd = x.to(DEV), src.to(DEV)
    a = igc.conv2d_transposed(xd, wt, stride=st, padding=p, source=sd, beta=-1.0)
    b = sd.clone()
    assert igc.conv2d_transposed_fwd(xd, wt, b, stride=st, padding=p, source=b, beta=-1.0) == 1
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))

"""The kernel paths again, on the LDS-poison debug build of the library
(libigemmconv_ldspoison.so, built from the same sources with IGC_LDS_POISON):
every workgroup first fills its LDS with 0xFF bytes, a NaN in every element
type.  A fragment or epilogue read that runs ahead of its data -- a missing
s_waitcnt or barrier around the direct-to-LDS requests -- then turns outputs
into NaN instead of plausible stale values, and the comparison against the
oracle (which also requires every output to be finite) fails.  One case per
kernel variant, plus the transposed, general and fused-epilogue paths, and
the band kernel's in-kernel filter transpose (whose rows would otherwise
be found in LDS from an earlier launch of the same problem)."""
import os
import sys
import zlib

import pytest
import torch

import datagen
import implicit_gemm_nhwc_amd as igc
import oracle
from test_gpu_parity import FILTER_IN_KERNEL, PATH_CASES, TOL, _assert_close, _run

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def setup_module(_):
    if not os.path.exists(igc.POISON_LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_poison_build_is_the_poison_build():
    assert igc.lib().conv2d_build_flags() == 0
    with igc.using_library(igc.POISON_LIB_PATH) as L:
        assert L.conv2d_build_flags() & 1
        assert igc.lib() is L
    assert igc.lib().conv2d_build_flags() == 0


@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: c[0])
def test_kernel_paths_poisoned(case):
    cid, dt, n, h, w, c, f, r, s, st, p, resid, kern = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    _say(f"poison path {cid}: {dt} N{n} {h}x{w} C{c}->{f} {r}x{s} st{st} p{p} residual={resid}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(cid.encode()) % 1000)
    beta = 0.5 if resid else 0.0
    with igc.using_library(igc.POISON_LIB_PATH):
        out = _run(x, wt, fcrs=False, stride=st, pad=p, src=src, beta=beta)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p, source=src,
                        beta=beta)
    _assert_close(out, ref, TOL[dt], cid)


# dtype, N, H, W, C, F, (R, S), stride, dilation, padding: grouped band,
# wide and patch phases, one-by-one phases, dilated (tiled) phases
TRANSPOSED = [
    ("bfloat16", 2, 10, 9, 32, 48, (4, 4), 2, 1, 1),
    ("bfloat16", 8, 32, 32, 256, 128, (4, 4), 2, 1, 1),
    ("float8_e4m3fn", 1, 8, 8, 128, 136, (2, 2), 2, 1, 0),
    ("float16", 1, 7, 6, 32, 40, (3, 3), 3, 1, 1),
    ("bfloat16", 1, 9, 8, 64, 24, (3, 2), 2, (2, 1), (1, 0)),
]


@pytest.mark.parametrize("case", TRANSPOSED, ids=lambda c: "-".join(map(str, c)))
def test_transposed_poisoned(case):
    dt, n, h, w, c, f, (r, s), st, dil, p = case
    ho, wo = igc.transposed_out_hw(h, w, r, s, stride=st, padding=p, dilation=dil)
    _say(f"poison transposed {case}")
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                     x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                     src_dist=("normal", 1.0), out_hw=(ho, wo),
                                     seed=zlib.crc32(repr(case).encode()) % 1000)
    wt = wfwd.permute(0, 1, 3, 2).contiguous()
    with igc.using_library(igc.POISON_LIB_PATH):
        out = igc.conv2d_transposed(x.to(DEV), wt.to(DEV), stride=st, padding=p, dilation=dil,
                                    source=src.to(DEV), beta=0.5)
        torch.cuda.synchronize()
    ref = oracle.conv2d_transposed(x, wt, stride=st, padding=p, dilation=dil, source=src,
                                   beta=0.5)
    _assert_close(out, ref, TOL[dt], str(case))


def test_general_and_epilogue_poisoned():
    """A grouped, dilated, strided general problem with the fused epilogue."""
    _say("poison general")
    x, wt, src = datagen.make_case(N=2, H=19, W=17, C=64, F=48, R=3, S=3, dtype="float16",
                                   fcrs=False, x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0), out_hw=(9, 8), seed=31, filt_c=16)
    g = torch.Generator().manual_seed(32)
    scale = (torch.rand(48, generator=g) + 0.5).float()
    bias = torch.randn(48, generator=g).float()
    kw = dict(stride=(2, 2), dilation=(2, 1), pad_begin=(1, 0), pad_end=(2, 0), groups=4)
    with igc.using_library(igc.POISON_LIB_PATH):
        out = igc.conv2d_general(x.to(DEV), wt.to(DEV), filter_is_fcrs=False, source=src.to(DEV),
                                 beta=0.25, scale=scale.to(DEV), bias=bias.to(DEV),
                                 activation="silu", **kw)
        torch.cuda.synchronize()
    assert tuple(out.shape) == (2, 9, 8, 48)
    ref = oracle.conv2d_general(x, wt, filter_is_fcrs=False, source=src, beta=0.25,
                                scale=scale, bias=bias, act="silu", **kw)
    _assert_close(out, ref, TOL["float16"], "general")


def test_supergroups_poisoned():
    """Grouped channels run as block-diagonal super-groups on the band
    kernel, with a residual source."""
    _say("poison super-groups")
    x, wt, src = datagen.make_case(N=2, H=16, W=15, C=128, F=128, R=3, S=3, dtype="bfloat16",
                                   fcrs=False, x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0), out_hw=(16, 15), seed=33, filt_c=8)
    kw = dict(stride=1, dilation=1, pad_begin=1, pad_end=1, groups=16)
    p = igc.conv_params(**kw)
    assert igc.conv2d_fwd_general_kernel_name(x.shape, wt.shape, (2, 16, 15, 128), p,
                                              filter_is_fcrs=False,
                                              dtype=x.dtype) == "igemm_fwd_band_kernel"
    with igc.using_library(igc.POISON_LIB_PATH):
        out = igc.conv2d_general(x.to(DEV), wt.to(DEV), filter_is_fcrs=False, source=src.to(DEV),
                                 beta=0.5, **kw)
        torch.cuda.synchronize()
    ref = oracle.conv2d_general(x, wt, filter_is_fcrs=False, source=src, beta=0.5, **kw)
    _assert_close(out, ref, TOL["bfloat16"], "super-groups")


@pytest.mark.parametrize("fcrs", [False, True])
@pytest.mark.parametrize("case", FILTER_IN_KERNEL, ids=lambda c: c[0])
def test_filter_in_kernel_poisoned(case, fcrs):
    cid, dt, n, h, w, c, f, r, s, st, p, resid = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    _say(f"poison filter in kernel {cid} fcrs={fcrs}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=fcrs,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(cid.encode()) % 1000)
    beta = 0.5 if resid else 0.0
    with igc.using_library(igc.POISON_LIB_PATH):
        out = _run(x, wt, fcrs=fcrs, stride=st, pad=p, src=src, beta=beta)
    ref = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=st, padding=p, source=src,
                        beta=beta)
    _assert_close(out, ref, TOL[dt], cid)


def test_dilation_phases_poisoned():
    """Dilation as phases on the band kernel (input views, output map, the
    stored filter transposed in the kernel), with a residual source."""
    _say("poison dilation phases")
    x, wt, src = datagen.make_case(N=2, H=16, W=20, C=64, F=48, R=3, S=3, dtype="bfloat16",
                                   fcrs=True, x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0), out_hw=(16, 20), seed=34)
    kw = dict(stride=1, dilation=2, pad_begin=2, pad_end=2, groups=1)
    p = igc.conv_params(**kw)
    assert igc.conv2d_fwd_general_kernel_name(x.shape, wt.shape, (2, 16, 20, 48), p,
                                              filter_is_fcrs=True,
                                              dtype=x.dtype) == "igemm_fwd_band_kernel"
    with igc.using_library(igc.POISON_LIB_PATH):
        out = igc.conv2d_general(x.to(DEV), wt.to(DEV), filter_is_fcrs=True, source=src.to(DEV),
                                 beta=0.5, **kw)
        torch.cuda.synchronize()
    ref = oracle.conv2d_general(x, wt, filter_is_fcrs=True, source=src, beta=0.5, **kw)
    _assert_close(out, ref, TOL["bfloat16"], "dilation phases")

"""GPU parity of the transposed convolution (page "conv_transposed_gpu":
NHWC input, RSFC filter) through conv2d_transposed_fwd, against the fp64
oracle (oracle.conv2d_transposed, a scatter-form implementation pinned by
hand-worked cases, brute force and the adjoint identity with conv2d).
Tolerances as for the forward convolution.
"""
import os
import sys
import zlib

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
    # dtype, N, H, W, C, F, R, pad, residual/epilogue, kernel it lands on
    ("bfloat16", 2, 20, 18, 32, 48, 3, 1, False, "band"),
    ("float16", 2, 16, 16, 64, 96, 3, 0, True, "wide"),
    ("float8_e4m3fn", 2, 14, 15, 64, 32, 5, 2, True, "band"),
    ("bfloat16", 1, 12, 12, 128, 130, 1, 0, False, "wide"),
    ("bfloat16", 2, 17, 9, 32, 16, 2, 0, True, "band"),
    ("float16", 1, 24, 24, 64, 64, 4, 1, False, "band"),
    ("bfloat16", 8, 32, 32, 256, 128, 3, 1, True, "wide"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_transposed_matches_oracle(case):
    dt, n, h, w, c, f, r, p, fused, kern = case
    ho, wo = h - 1 - 2 * p + r, w - 1 - 2 * p + r
    _say(f"transposed {case} -> out {n}x{ho}x{wo}x{f}")
    seed = zlib.crc32(repr(case).encode()) % 1000
    x, wfwd, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype=dt, fcrs=False,
                                     x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                     src_dist=("normal", 1.0) if fused else None,
                                     out_hw=(ho, wo), seed=seed)
    # an RSFC filter [R, S, F, C]: the seeded RSCF draw [R, S, C, F] re-laid out
    wt = wfwd.permute(0, 1, 3, 2).contiguous()
    # the equivalent forward problem is what decides the kernel
    assert igc.conv2d_fwd_kernel_name((n, h, w, c), (r, r, c, f), (n, ho, wo, f),
                                      filter_is_fcrs=False, dtype=x.dtype, stride=1,
                                      padding=r - 1 - p).endswith(
        {"band": "band_kernel", "wide": "wide_kernel"}[kern])
    kw = {}
    okw = {}
    if fused:
        g = torch.Generator().manual_seed(seed + 1)
        scale = (torch.rand(f, generator=g) + 0.5).float()
        bias = torch.randn(f, generator=g).float()
        kw = dict(source=src.to(DEV), beta=0.5, scale=scale.to(DEV), bias=bias.to(DEV),
                  activation="silu")
        okw = dict(source=src, beta=0.5, scale=scale, bias=bias, act="silu")
    out = igc.conv2d_transposed(x.to(DEV), wt.to(DEV), stride=1, padding=p, **kw)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (n, ho, wo, f)
    ref = oracle.conv2d_transposed(x, wt, stride=1, padding=p, **okw)
    _assert_close(out, ref, TOL[dt], str(case))

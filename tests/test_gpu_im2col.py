"""GPU checks of the materialised im2col route (the write-then-GEMM path the
fused gather replaces, kept for measurement):
  - conv2d_im2col is a bit copy: equal bit for bit to oracle.im2col;
  - conv2d_fwd_nk on the im2col matrix viewed as a 1x1 convolution computes
    the convolution: within the plain path's tolerance of the fp64 oracle.
"""
import os
import sys
import zlib

import pytest
import torch

import datagen
import implicit_gemm_nhwc_amd as igc
import oracle
from test_gpu_parity import TOL, _assert_close, _bits

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
    # dtype, N, H, W, C, F, R, S, stride, pad
    ("bfloat16", 2, 9, 11, 32, 16, 3, 3, 1, 1),
    ("float16", 1, 12, 10, 24, 40, 3, 3, 2, 1),
    ("float8_e4m3fn", 2, 10, 9, 16, 96, 5, 5, 1, 2),
    ("bfloat16", 1, 7, 7, 64, 3, 5, 5, 2, 2),
    ("float16", 3, 6, 5, 8, 130, 1, 1, 1, 0),
    ("bfloat16", 1, 5, 6, 128, 8, 2, 3, 2, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_im2col_bit_exact(case):
    dt, n, h, w, c, f, r, s, st, p = case
    _say(f"im2col {case}")
    x, _, _ = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                x_dist=("normal", 1.0), w_dist=("normal", 1.0),
                                seed=zlib.crc32(repr(case).encode()) % 1000)
    nbytes = igc.conv2d_im2col_bytes(x.shape, r, s, stride=st, padding=p, dtype=x.dtype)
    kp = igc.im2col_row_elems(r, s, c, x.dtype)
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    assert nbytes == n * ho * wo * kp * x.element_size()
    # a canary past the end must survive
    buf = torch.full((nbytes + 256,), 0x5A, dtype=torch.uint8, device=DEV)
    assert igc.conv2d_im2col(x.to(DEV), r, s, buf, stride=st, padding=p, a_bytes=nbytes) == 1
    torch.cuda.synchronize()
    want = _bits(oracle.im2col(x, r, s, stride=st, padding=p, k_pad=kp))
    got = buf[:nbytes].cpu().view(want.dtype).reshape(want.shape)
    assert torch.equal(got, want)
    assert torch.all(buf[nbytes:].cpu() == 0x5A)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_materialized_route_matches_oracle(case):
    dt, n, h, w, c, f, r, s, st, p = case
    _say(f"im2col + GEMM {case}")
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=True,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0), out_hw=(ho, wo),
                                   seed=zlib.crc32(repr(case).encode()) % 997)
    xd, wd, sd = x.to(DEV), wt.to(DEV), src.to(DEV)
    out = torch.empty((n, ho, wo, f), dtype=datagen.OUT_DTYPES[dt], device=DEV)
    nk = torch.empty(igc.conv2d_workspace_bytes(wt.shape, True, x.dtype), dtype=torch.uint8,
                     device=DEV)
    a = torch.empty(igc.conv2d_im2col_bytes(x.shape, r, s, stride=st, padding=p,
                                            dtype=x.dtype), dtype=torch.uint8, device=DEV)
    assert igc.conv2d_materialized(xd, wd, out, nk, a, filter_is_fcrs=True, stride=st,
                                   padding=p, source=sd, beta=0.5) == 1
    torch.cuda.synchronize()
    ref = oracle.conv2d(x, wt, filter_is_fcrs=True, stride=st, padding=p, source=src, beta=0.5)
    _assert_close(out, ref, TOL[dt], str(case))

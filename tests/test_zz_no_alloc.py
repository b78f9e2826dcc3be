"""conv2d_fwd_noalloc: conv2d_fwd with the NK matrix in the library's static
device scratch instead of a workspace, for callers that cannot allocate.

GPU: through the C ABI, two calls in a row (the second on a smaller problem
with a smaller NK matrix, so stale scratch contents of the first would show)
must give exactly the bits conv2d_fwd gives on the same inputs (the same
kernels run), and agree with the fp64 oracle.  CPU: a problem whose NK matrix
exceeds the scratch is declined before any HIP call.
"""
import os
import sys

import pytest
import torch

import datagen
import implicit_gemm_nhwc_amd as igc
import oracle

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
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.uint8)


# (id, dtype, N, H, W, C, F, R, S, stride, pad, residual) -- first the larger
# problems (patch kernel, 819 KB NK matrix; wide kernel, 590 KB), then
# smaller ones
CASES = [
    ("patch_fp8_5x5", "float8_e4m3fn", 16, 64, 64, 128, 256, 5, 5, 1, 2, True),
    ("wide_fp16_s2", "float16", 4, 28, 28, 128, 256, 3, 3, 2, 1, True),
    ("band_fp8_resid", "float8_e4m3fn", 1, 10, 12, 64, 24, 3, 3, 1, 1, True),
    ("band_bf16", "bfloat16", 1, 8, 8, 32, 16, 3, 3, 1, 1, False),
]


def _inputs(case):
    cid, dt, n, h, w, c, f, r, s, st, p, resid = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                   x_dist=("normal", 1.0), w_dist=("normal", 0.2),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=len(cid))
    return x, wt, src, (n, ho, wo, f)


@pytest.mark.gpu
def test_noalloc_matches_conv2d_fwd_on_calls_in_a_row():
    prev_nk = None
    for case in CASES:
        cid, dt, n, h, w, c, f, r, s, st, p, resid = case
        x, wt, src, oshape = _inputs(case)
        nk_bytes = igc.conv2d_workspace_bytes(wt.shape, False, wt.dtype)
        assert nk_bytes <= igc.NOALLOC_SCRATCH_BYTES
        if prev_nk is not None:
            assert nk_bytes < prev_nk      # each call smaller than the one before
        prev_nk = nk_bytes
        _say(f"noalloc {cid}: {dt} N{n} {h}x{w} C{c}->{f} {r}x{s} st{st} p{p} "
             f"residual={resid}, NK {nk_bytes} bytes")
        xd, wd = x.to(DEV), wt.to(DEV)
        sd = None if src is None else src.to(DEV)
        beta = 0.5 if resid else 0.0
        odt = datagen.OUT_DTYPES[dt]
        a = torch.full(oshape, 7.0, dtype=odt, device=DEV)
        assert igc.conv2d_fwd_noalloc(xd, wd, a, filter_is_fcrs=False, stride=st, padding=p,
                                      source=sd, beta=beta) == 1
        ws = torch.empty(nk_bytes, dtype=torch.uint8, device=DEV)
        b = torch.empty(oshape, dtype=odt, device=DEV)
        assert igc.conv2d_fwd(xd, wd, b, filter_is_fcrs=False, stride=st, padding=p,
                              source=sd, beta=beta, workspace=ws) == 1
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b)), cid
        ref = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p, source=src,
                            beta=beta)
        got = a.cpu().to(torch.float64).numpy()
        scale = float(abs(ref).max())
        assert float(abs(got - ref).max()) <= TOL[dt] * scale, cid


@pytest.mark.gpu
def test_noalloc_second_call_after_larger_one_is_exact():
    # the same small problem before and after a large one: identical bits
    small, large = CASES[-1], CASES[0]
    outs = []
    for case in (small, large, small):
        x, wt, src, oshape = _inputs(case)
        cid, dt, n, h, w, c, f, r, s, st, p, resid = case
        out = torch.empty(oshape, dtype=datagen.OUT_DTYPES[dt], device=DEV)
        assert igc.conv2d_fwd_noalloc(x.to(DEV), wt.to(DEV), out, filter_is_fcrs=False,
                                      stride=st, padding=p,
                                      source=None if src is None else src.to(DEV),
                                      beta=0.5 if resid else 0.0) == 1
        torch.cuda.synchronize()
        outs.append(_bits(out))
    assert torch.equal(outs[0], outs[2])


def test_noalloc_declines_beyond_scratch():
    # NK matrix of 5x5x512 -> 512 bf16 = 512 * 12800 * 2 bytes > 8 MiB: declined
    # before any HIP call (no GPU is needed for this check)
    shape = dict(in_shape=(1, 8, 8, 512), filt_shape=(5, 5, 512, 512),
                 out_shape=(1, 8, 8, 512), filter_is_fcrs=False, stride=1, padding=2,
                 dtype=0)
    assert igc.conv2d_workspace_bytes((5, 5, 512, 512), False, 0) > igc.NOALLOC_SCRATCH_BYTES
    assert igc.conv2d_fwd_noalloc(0x10000000, 0x20000000, 0x30000000, **shape) == 0
    # the same problem is accepted by conv2d_fwd's gate
    assert igc.conv2d_fwd_check(0x10000000, 0x20000000, 0x30000000, **shape) == 0
    # and a declined shape is declined here too
    assert igc.conv2d_fwd_noalloc(0x10000000, 0x20000000, 0x30000000,
                                  **{**shape, "stride": 3}) == 0

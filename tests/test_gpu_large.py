"""GPU parity at the largest sizes the kernels accept: tensors beyond 2^31
bytes in total, single images just under the 2^31-byte limit of a 32-bit
buffer offset, and pixel tiles that straddle image boundaries.

Inputs are drawn on the GPU from a seeded generator (no host copy of the
multi-GB tensors).  Reference values come from the fp64 oracle applied to
the 3x3 input window of each sampled output pixel, cut from the GPU tensor
with zeros where the window leaves the image: oracle.conv2d of that window
with padding 0 is, by the definition, the output at the pixel.  Sampled
pixels: every image corner and edge midpoint, the last pixel of each image
and the first of the next, and seeded random ones.
"""
import os
import sys

import numpy as np
import pytest
import torch

import implicit_gemm_nhwc_amd as igc
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def setup_module(_):
    if not os.path.exists(igc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pixels(n, ho, wo, count, seed):
    pix = set()
    for b in range(n):
        for oh in (0, ho // 2, ho - 1):
            for ow in (0, wo // 2, wo - 1):
                pix.add((b, oh, ow))
    rng = np.random.default_rng(seed)
    for _ in range(count):
        pix.add((int(rng.integers(0, n)), int(rng.integers(0, ho)), int(rng.integers(0, wo))))
    return sorted(pix)


def _windows(x, pix, r, s, st, p):
    """[len(pix), r, s, C] input windows (zeros outside the image), on the host."""
    n, h, w, c = x.shape
    out = torch.zeros((len(pix), r, s, c), dtype=x.dtype)
    for i, (b, oh, ow) in enumerate(pix):
        ih0, iw0 = oh * st - p, ow * st - p
        h0, h1 = max(ih0, 0), min(ih0 + r, h)
        w0, w1 = max(iw0, 0), min(iw0 + s, w)
        if h0 < h1 and w0 < w1:
            out[i, h0 - ih0:h1 - ih0, w0 - iw0:w1 - iw0] = x[b, h0:h1, w0:w1].cpu()
    return out


# id, N, H, W, C, F, stride, pad, kernel; 3x3 bf16 RSCF filters
LARGE = [
    # two 708 MB images per 32-bit span (the wide kernel's limit), 2.1 GB in
    # all, output 2.8 GB; 128-pixel tiles straddle the image boundaries
    ("wide_3x1920", 3, 1920, 1920, 96, 128, 1, 1, "igemm_fwd_wide_kernel"),
    # the patch kernel's per-image buffers: 943 MB input and output images
    ("patch_3x1920", 3, 1920, 1920, 128, 128, 1, 1, "igemm_fwd_patch_kernel"),
    # one image of 2,147,024,896 bytes, just under 2^31 (the band kernel's limit)
    ("band_5792sq", 1, 5792, 5792, 32, 8, 1, 1, "igemm_fwd_band_kernel"),
    # two 1.13 GB images exceed the wide kernel's span: the 64-bit fallback
    ("tiled_2x2100", 2, 2100, 2100, 128, 96, 2, 1, "igemm_fwd_kernel"),
]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: c[0])
def test_large_tensors(case):
    cid, n, h, w, c, f, st, p, kern = case
    ho, wo = oracle.out_size(h, 3, st, p), oracle.out_size(w, 3, st, p)
    assert igc.conv2d_fwd_kernel_name((n, h, w, c), (3, 3, c, f), (n, ho, wo, f),
                                      filter_is_fcrs=False, dtype=torch.bfloat16, stride=st,
                                      padding=p) == kern
    _say(f"large {cid}: N{n} {h}x{w} C{c}->{f} st{st} p{p}: input "
         f"{n * h * w * c * 2 / 2**30:.2f} GiB, output {n * ho * wo * f * 2 / 2**30:.2f} GiB")
    g = torch.Generator(device=DEV).manual_seed(7)
    x = torch.randn((n, h, w, c), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    wt = (torch.randn((3, 3, c, f), generator=g, device=DEV) / np.sqrt(9 * c)).to(torch.bfloat16)
    src = torch.randn((n, ho, wo, f), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty((n, ho, wo, f), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(igc.conv2d_workspace_bytes(wt.shape, False, wt.dtype), dtype=torch.uint8,
                     device=DEV)
    assert igc.conv2d_fwd(x, wt, out, filter_is_fcrs=False, stride=st, padding=p, source=src,
                          beta=0.5, workspace=ws) == 1
    torch.cuda.synchronize()
    pix = _pixels(n, ho, wo, 64, seed=n * 1000 + h)
    # the last pixel of each image and the first of the next
    for b in range(n - 1):
        pix += [(b, ho - 1, wo - 1), (b + 1, 0, 0)]
    win = _windows(x, pix, 3, 3, st, p)
    idx = torch.as_tensor([(b * ho + oh) * wo + ow for b, oh, ow in pix], device=DEV)
    src_pts = src.reshape(-1, f)[idx].cpu().reshape(len(pix), 1, 1, f)
    ref = oracle.conv2d(win, wt.cpu(), filter_is_fcrs=False, stride=1, padding=0,
                        source=src_pts, beta=0.5).reshape(len(pix), f)
    got = out.reshape(-1, f)[idx].cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    _say(f"  {len(pix)} pixels: max|err| {err:.3e}, max|ref| {scale:.3e}")
    assert err <= 1e-2 * scale
    assert torch.isfinite(out[:, ::97, ::89].float()).all()

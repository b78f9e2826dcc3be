"""GPU parity of the general forward convolution (conv2d_fwd_general: per-axis
stride, dilation, padding before / after each axis, channel groups) through
the C ABI, against the fp64 oracle (oracle.conv2d_general) over the whole
output tensor.  Tolerances as for conv2d_fwd: fp32 accumulation of exactly
rounded inputs and one rounding to the output type.  Each widened parameter
has its own sweep; a problem inside the page's gate must give conv2d_fwd's
bits."""
import os
import sys
import zlib

import numpy as np

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


# name, dtype, N, H, W, C_in, C_out, R, S, stride, dilation, pad_begin, pad_end, groups
CASES = [
    # dilation
    ("dil2_same_bf16", "bfloat16", 2, 17, 19, 64, 64, 3, 3, 1, 2, 2, 2, 1),
    ("dil3x1_fp16", "float16", 1, 23, 15, 32, 48, 3, 3, 1, (3, 1), (3, 1), (3, 1), 1),
    ("dil2_s2_fp8", "float8_e4m3fn", 2, 21, 20, 64, 40, 3, 3, 2, 2, 2, 1, 1),
    ("dil4_5x5_bf16", "bfloat16", 1, 30, 33, 16, 24, 5, 5, 1, 4, 8, 8, 1),
    # stride beyond 2 and per-axis strides
    ("s4_patchify_bf16", "bfloat16", 2, 32, 36, 16, 96, 4, 4, 4, 1, 0, 0, 1),
    ("s3_3x3_fp16", "float16", 2, 25, 26, 32, 32, 3, 3, 3, 1, 1, 1, 1),
    ("s1x2_fp8", "float8_e4m3fn", 1, 14, 31, 32, 24, 3, 3, (1, 2), 1, 1, 1, 1),
    ("s5x3_7x7_bf16", "bfloat16", 1, 40, 29, 16, 8, 7, 7, (5, 3), 1, 3, 3, 1),
    # asymmetric padding
    ("same_s2_even_bf16", "bfloat16", 2, 16, 16, 32, 64, 3, 3, 2, 1, 0, 1, 1),
    ("pad_tlbr_fp16", "float16", 1, 13, 17, 32, 20, 3, 2, 1, 1, (2, 0), (0, 3), 1),
    ("pad3_fp8", "float8_e4m3fn", 1, 15, 15, 16, 16, 7, 7, 2, 1, 3, 3, 1),
    # channel groups
    ("g2_bf16", "bfloat16", 2, 15, 14, 64, 64, 3, 3, 1, 1, 1, 1, 2),
    ("g32_resnext_bf16", "bfloat16", 2, 14, 14, 256, 256, 3, 3, 1, 1, 1, 1, 32),
    ("g4_s2_fp16", "float16", 1, 19, 17, 64, 32, 3, 3, 2, 1, 1, 1, 4),
    ("g2_fp8", "float8_e4m3fn", 1, 12, 13, 64, 48, 3, 3, 1, 1, 1, 1, 2),
    ("g2_fg3_bf16", "bfloat16", 1, 9, 11, 32, 6, 3, 3, 1, 1, 1, 1, 2),
    ("g2_wide_bf16", "bfloat16", 1, 10, 12, 128, 256, 1, 1, 1, 1, 0, 0, 2),
    ("g8_cg8_ragged_k_bf16", "bfloat16", 3, 23, 29, 64, 64, 3, 3, 1, 1, 1, 1, 8),
    # everything at once
    ("all_fp16", "float16", 2, 27, 22, 96, 48, 3, 2, (3, 2), (2, 3), (1, 0), (2, 3), 3),
    ("all_fp8", "float8_e4m3fn", 1, 26, 31, 64, 32, 5, 3, (2, 3), (2, 1), (4, 0), (1, 2), 2),
    # channel counts that are not whole 16-byte vectors: element gather
    ("stem_7x7_s2_p3_c3_bf16", "bfloat16", 2, 37, 41, 3, 64, 7, 7, 2, 1, 3, 3, 1),
    ("resnext_cg4_fp16", "float16", 2, 14, 15, 128, 128, 3, 3, 1, 1, 1, 1, 32),
    ("depthwise_bf16", "bfloat16", 2, 19, 18, 32, 32, 3, 3, 1, 1, 1, 1, 32),
    ("depthwise_x2_s2_fp8", "float8_e4m3fn", 1, 21, 22, 16, 32, 5, 5, 2, 1, 2, 2, 16),
    ("dil2_c12_fp16", "float16", 1, 16, 17, 12, 20, 3, 3, 1, 2, (2, 1), (2, 3), 1),
    # one group, unit dilation, stride 1 or 2, other paddings: the forward
    # kernels with per-side padding (band, wide, resident)
    ("fast_band_pad3_bf16", "bfloat16", 2, 20, 22, 64, 64, 3, 3, 1, 1, 3, 3, 1),
    ("fast_band_tl_fp8", "float8_e4m3fn", 2, 19, 17, 64, 40, 5, 5, 2, 1, (0, 4), (3, 1), 1),
    ("fast_wide_asym_fp16", "float16", 2, 15, 16, 128, 256, 3, 3, 2, 1, (0, 1), (2, 0), 1),
    ("fast_wide_big_pad_bf16", "bfloat16", 1, 12, 13, 64, 96, 3, 3, 1, 1, (5, 0), (0, 6), 1),
    ("fast_resident_bf16", "bfloat16", 2, 9, 11, 96, 16, 3, 3, 1, 1, (1, 0), (0, 2), 1),
    # equal strides beyond 2: the same forward kernels (their gathers take
    # any stride)
    ("fast_s3_band_bf16", "bfloat16", 2, 25, 26, 64, 48, 3, 3, 3, 1, 1, 1, 1),
    ("fast_s3_band_fp8", "float8_e4m3fn", 2, 25, 26, 64, 48, 3, 3, 3, 1, 1, 1, 1),
    ("fast_s3_resident_bf16", "bfloat16", 2, 20, 22, 96, 16, 3, 3, 3, 1, 1, 1, 1),
    ("fast_s3_wide_fp16", "float16", 2, 25, 26, 64, 128, 3, 3, 3, 1, 1, (0, 2), 1),
    ("fast_s4_patchify_wide_bf16", "bfloat16", 4, 64, 64, 8, 96, 4, 4, 4, 1, 0, 0, 1),
    ("fast_s4_band_fp16", "float16", 4, 64, 64, 16, 64, 4, 4, 4, 1, 0, 0, 1),
    # several groups, unit dilation, stride 1 or 2: super-groups on the band
    # kernel (block-diagonal NK matrix, pixel pitch C_in / C_out)
    ("sg_g32_many_tiles_bf16", "bfloat16", 3, 28, 30, 256, 256, 3, 3, 1, 1, 1, 1, 32),
    ("sg_g16_fp8", "float8_e4m3fn", 2, 17, 19, 256, 256, 3, 3, 1, 1, 1, 1, 16),
    ("sg_g4_asym_pad_fp16", "float16", 2, 21, 18, 128, 64, 3, 3, 2, 1, (0, 1), (2, 0), 4),
    ("sg_depthwise_x2_s2_bf16", "bfloat16", 2, 23, 20, 64, 128, 3, 3, 2, 1, 1, 1, 64),
    ("sg_depthwise_5x5_fp16", "float16", 1, 19, 33, 96, 96, 5, 5, 1, 1, 2, 2, 96),
    ("sg_g8_fg6_bf16", "bfloat16", 1, 15, 16, 128, 48, 3, 1, 1, 1, (1, 0), (1, 0), 8),
    # one group, stride 1, dilation dividing the padding before each axis
    # and the extents: dilation phases on the band kernel (input views of
    # every dh-th row / dw-th column, output map)
    ("dp_d2_same_bf16", "bfloat16", 2, 16, 20, 64, 48, 3, 3, 1, 2, 2, 2, 1),
    ("dp_d3_fp16", "float16", 2, 24, 18, 32, 32, 3, 3, 1, 3, 3, 3, 1),
    ("dp_d2_fp8", "float8_e4m3fn", 2, 20, 20, 64, 40, 3, 3, 1, 2, 2, 2, 1),
    ("dp_d2x1_bf16", "bfloat16", 1, 16, 15, 32, 16, 3, 3, 1, (2, 1), (2, 1), (2, 1), 1),
    ("dp_d1x3_fp16", "float16", 2, 13, 18, 32, 24, 3, 3, 1, (1, 3), (1, 3), (1, 3), 1),
    ("dp_d2_5x5_bf16", "bfloat16", 1, 20, 24, 32, 24, 5, 5, 1, 2, 4, 4, 1),
    ("dp_d2_valid_bf16", "bfloat16", 2, 20, 20, 32, 32, 3, 3, 1, 2, 0, 0, 1),
    ("dp_d4_f5_fp16", "float16", 1, 32, 32, 32, 5, 3, 3, 1, 4, 4, 4, 1),
]

ELEM = {"bfloat16": 2, "float16": 2, "float8_e4m3fn": 1}


def _dilation_phases(case):
    """Whether conv2d_fwd_general runs the case as dilation phases on the
    band kernel: one group, stride 1, dilation above 1 dividing the padding
    before each axis and the input and output extents, and the band
    kernel's channel rules (C_out <= 64, C_in * element bytes a
    power-of-two multiple of the MFMA k-step)."""
    _, dt, n, h, w, c, f, r, s, st, dil, pb, pe, g = case
    st, dil, pb, pe = _pair(st), _pair(dil), _pair(pb), _pair(pe)
    if g != 1 or st != (1, 1) or dil == (1, 1):
        return False
    b, ksb = c * ELEM[dt], 64 if ELEM[dt] == 1 else 32
    if f > 64 or b % ksb or (b // 16) & (b // 16 - 1):
        return False
    ho = oracle.out_size_general(h, r, 1, dil[0], pb[0], pe[0])
    wo = oracle.out_size_general(w, s, 1, dil[1], pb[1], pe[1])
    return (pb[0] % dil[0] == 0 and pb[1] % dil[1] == 0 and h % dil[0] == 0 and
            w % dil[1] == 0 and ho % dil[0] == 0 and wo % dil[1] == 0)


def _supergroup(case):
    """Whether conv2d_fwd_general runs the case as super-groups on the band
    kernel: several groups, unit dilation, equal strides of 1 or 2, and some
    q dividing the groups with q * Fg <= 64 and q * Cg * element bytes a
    power-of-two multiple of the MFMA k-step (32 bytes, 64 for fp8)."""
    _, dt, _, _, _, c, f, _, _, st, dil, _, _, g = case
    st, dil = _pair(st), _pair(dil)
    if g == 1 or dil != (1, 1) or st[0] != st[1] or st[0] > 2:
        return False
    cg, fg, e = c // g, f // g, ELEM[dt]
    ksb = 64 if e == 1 else 32
    for q in range(1, g + 1):
        b = q * cg * e
        if g % q == 0 and q * fg <= 64 and b % ksb == 0 and (b // 16) & (b // 16 - 1) == 0:
            return True
    return False


def _fast(case):
    _, _, _, _, _, _, _, _, _, st, dil, _, _, g = case
    st, dil = _pair(st), _pair(dil)
    return g == 1 and dil == (1, 1) and st[0] == st[1]


def _pair(v):
    return (v, v) if isinstance(v, int) else tuple(v)


def _draw(case, fcrs=False, resid=False):
    cid, dt, n, h, w, c, f, r, s, st, dil, pb, pe, g = case
    p = igc.conv_params(stride=st, dilation=dil, pad_begin=pb, pad_end=pe, groups=g)
    ho, wo = igc.out_hw_general(h, w, r, s, p)
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=fcrs,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(cid.encode()) % 1000,
                                   filt_c=c // g)
    return p, (n, ho, wo, f), x, wt, src


def _oracle(case, x, wt, fcrs, **kw):
    _, _, _, _, _, _, _, _, _, st, dil, pb, pe, g = case
    return oracle.conv2d_general(x, wt, filter_is_fcrs=fcrs, stride=_pair(st),
                                 dilation=_pair(dil), pad_begin=_pair(pb), pad_end=_pair(pe),
                                 groups=g, **kw)


def _run(x, wt, out_shape, p, fcrs, **kw):
    out = torch.empty(out_shape, dtype=datagen.OUT_DTYPES[str(x.dtype)[6:]], device=DEV)
    nb = igc.conv2d_fwd_general_workspace_bytes(x.shape, wt.shape, out_shape, p,
                                                filter_is_fcrs=fcrs, dtype=x.dtype)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    rc = igc.conv2d_fwd_general(x.to(DEV), wt.to(DEV), out, p, filter_is_fcrs=fcrs,
                                workspace=ws, **kw)
    assert rc == 1, f"conv2d_fwd_general returned {rc}"
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_general_parity(case):
    cid, dt = case[0], case[1]
    _say(f"general {cid}: {case[2:]}")
    p, oshape, x, wt, _ = _draw(case)
    name = igc.conv2d_fwd_general_kernel_name(x.shape, wt.shape, oshape, p, filter_is_fcrs=False,
                                              dtype=x.dtype)
    if _fast(case):
        want = {"fast_band_pad3_bf16": "igemm_fwd_band_kernel",
                "fast_band_tl_fp8": "igemm_fwd_band_kernel",
                "fast_wide_asym_fp16": "igemm_fwd_wide_kernel",
                "fast_wide_big_pad_bf16": "igemm_fwd_wide_kernel",
                "fast_resident_bf16": "igemm_fwd_resident_kernel",
                "fast_s3_band_bf16": "igemm_fwd_band_kernel",
                "fast_s3_band_fp8": "igemm_fwd_band_kernel",
                "fast_s3_resident_bf16": "igemm_fwd_resident_kernel",
                "fast_s3_wide_fp16": "igemm_fwd_wide_kernel",
                "fast_s4_patchify_wide_bf16": "igemm_fwd_wide_kernel",
                "fast_s4_band_fp16": "igemm_fwd_band_kernel"}.get(cid)
        assert name != "igemm_fwd_tapfold_kernel"
        if want:
            assert name == want, name
    elif _supergroup(case) or _dilation_phases(case):
        assert name == "igemm_fwd_band_kernel", name
    else:
        assert name == "igemm_fwd_kernel", name
    _say(f"  kernel {name}")
    out = _run(x, wt, oshape, p, False)
    ref = _oracle(case, x, wt, False)
    err, scale = _assert_close(out, ref, TOL[dt], cid)
    _say(f"  max|err|/max|ref| = {err / max(scale, 1e-300):.3e}")


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in (
    "dil2_s2_fp8", "g32_resnext_bf16", "g2_fg3_bf16", "all_fp16", "pad_tlbr_fp16",
    "g2_wide_bf16", "fast_band_tl_fp8", "fast_wide_asym_fp16", "sg_g16_fp8",
    "sg_depthwise_x2_s2_bf16", "sg_g8_fg6_bf16", "depthwise_bf16", "dp_d2_same_bf16",
    "dp_d2_fp8", "dp_d4_f5_fp16")], ids=lambda c: c[0])
def test_general_fcrs_residual_epilogue(case):
    """FCRS filter, a residual source and the fused scale / bias / SiLU, with
    groups offsetting the coefficients; FCRS bits equal RSCF bits."""
    cid, dt = case[0], case[1]
    _say(f"general epilogue {cid}")
    p, oshape, x, wt, src = _draw(case, fcrs=True, resid=True)
    f = oshape[3]
    gen = torch.Generator().manual_seed(zlib.crc32(cid.encode()) % 977)
    scale = (torch.rand(f, generator=gen) * 3.0 - 1.5).to(torch.float32)
    bias = torch.randn(f, generator=gen).to(torch.float32)
    kw = dict(source=src.to(DEV), beta=-0.75, scale=scale.to(DEV), bias=bias.to(DEV),
              activation="silu")
    out = _run(x, wt, oshape, p, True, **kw)
    ref = _oracle(case, x, wt, True, source=src, beta=-0.75, scale=scale, bias=bias,
                  act="silu")
    _assert_close(out, ref, TOL[dt], cid)
    # the same filter stored RSCF: identical bits
    w_rscf = wt.view(torch.uint8).permute(2, 3, 1, 0).contiguous().view(wt.dtype) \
        if wt.element_size() == 1 else wt.permute(2, 3, 1, 0).contiguous()
    out2 = _run(x, w_rscf, oshape, p, False, **kw)
    assert torch.equal(_bits(out), _bits(out2))


def test_general_groups_equal_separate_convolutions():
    """A grouped call gives, bit for bit, the concatenation of one ungrouped
    call per group on that group's channels."""
    case = ("g4_split", "bfloat16", 2, 13, 15, 64, 32, 3, 3, (2, 1), (1, 2), (1, 2), (0, 2), 4)
    _say("general groups vs per-group calls")
    p, oshape, x, wt, _ = _draw(case)
    out = _run(x, wt, oshape, p, False)
    g, cg, fg = 4, 16, 8
    p1 = igc.conv_params(stride=(2, 1), dilation=(1, 2), pad_begin=(1, 2), pad_end=(0, 2))
    for k in range(g):
        xs = x[..., k * cg:(k + 1) * cg].contiguous()
        ws_ = wt[..., k * fg:(k + 1) * fg].contiguous()
        part = _run(xs, ws_, oshape[:3] + (fg,), p1, False)
        assert torch.equal(_bits(out[..., k * fg:(k + 1) * fg].contiguous()), _bits(part)), k


@pytest.mark.parametrize("st,pad", [(1, 1), (2, 0), (2, 2), (1, 0)])
def test_general_page_problems_match_conv2d_fwd(st, pad):
    """Inside the page's gate conv2d_fwd_general runs conv2d_fwd's kernel:
    the same bits."""
    _say(f"general page problem st{st} p{pad}")
    x, wt, _ = datagen.make_case(N=2, H=19, W=21, C=64, F=48, R=3, S=3, dtype="bfloat16",
                                 fcrs=False, x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                 seed=11)
    p = igc.conv_params(stride=st, pad_begin=pad)
    ho, wo = igc.out_hw_general(19, 21, 3, 3, p)
    assert (ho, wo) == igc.out_hw(19, 21, 3, 3, st, pad)
    a = _run(x, wt, (2, ho, wo, 48), p, False)
    b = igc.conv2d(x.to(DEV), wt.to(DEV), filter_is_fcrs=False, stride=st, padding=pad)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))


def test_general_dilated_equals_zero_inserted_filter():
    """Dilation d equals the undilated convolution with d - 1 zero taps
    between the filter's taps: both calls within tolerance of the oracle of
    the dilated problem (their summation orders differ)."""
    _say("general dilation vs zero-inserted filter")
    case = ("dilz", "bfloat16", 1, 20, 22, 32, 16, 3, 3, 1, (2, 3), (2, 3), (2, 3), 1)
    p, oshape, x, wt, _ = _draw(case)
    a = _run(x, wt, oshape, p, False)
    wz = torch.zeros((5, 7, 32, 16), dtype=wt.dtype)
    wz[::2, ::3] = wt
    p2 = igc.conv_params(pad_begin=(2, 3))
    b = _run(x, wz, oshape, p2, False)
    ref = _oracle(case, x, wt, False)
    _assert_close(a, ref, TOL["bfloat16"], "dilated")
    _assert_close(b, ref, TOL["bfloat16"], "zero-inserted")


def test_supergroups_in_place_residual_and_repeat():
    """Super-groups with the output as its own residual source (each output
    element read once, by the lane that writes it), twice in a row on the
    same buffers: both calls match the oracle."""
    case = ("sg_inplace", "bfloat16", 2, 14, 13, 64, 64, 3, 3, 1, 1, 1, 1, 8)
    assert _supergroup(case)
    _say("general super-groups in place")
    p, oshape, x, wt, src = _draw(case, resid=True)
    y = src.to(DEV).clone()
    nb = igc.conv2d_fwd_general_workspace_bytes(x.shape, wt.shape, oshape, p,
                                                filter_is_fcrs=False, dtype=x.dtype)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    xd, wd = x.to(DEV), wt.to(DEV)
    ref = _oracle(case, x, wt, False, source=src, beta=1.0)
    for it in range(2):
        assert igc.conv2d_fwd_general(xd, wd, y, p, filter_is_fcrs=False, source=y, beta=1.0,
                                      workspace=ws) == 1
        torch.cuda.synchronize()
        _assert_close(y, ref, TOL["bfloat16"], f"in place {it}")
        ref = _oracle(case, x, wt, False, source=y.cpu(), beta=1.0)


GENERAL_FULL = [
    # the general layers the benchmark times, at their full sizes, compared
    # with the oracle over every output element
    ("dilated2_3x3_64c_n32", "bfloat16", 32, 56, 56, 64, 64, 3, 3, 1, 2, 2, 2, 1),
    ("grouped32_3x3_256c_n32", "bfloat16", 32, 28, 28, 256, 256, 3, 3, 1, 1, 1, 1, 32),
    ("patchify_4x4_s4_8to96_n32", "bfloat16", 32, 224, 224, 8, 96, 4, 4, 4, 1, 0, 0, 1),
]


@pytest.mark.parametrize("case", GENERAL_FULL, ids=lambda c: c[0])
def test_general_benchmark_layers_full_size(case):
    cid, dt = case[0], case[1]
    _say(f"general full size {cid}: {case[2:]}")
    p, oshape, x, wt, _ = _draw(case)
    out = _run(x, wt, oshape, p, False)
    ref = _oracle(case, x, wt, False)
    err, scale = _assert_close(out, ref, TOL[dt], cid)
    _say(f"  max|err|/max|ref| = {err / max(scale, 1e-300):.3e}")


def _sweep_general():
    """Seeded random general problems over the paths conv2d_fwd_general
    picks: super-groups (several groups, unit dilation, stride 1 or 2),
    dilation phases (one group, stride 1, dilation dividing the padding and
    the extents), the forward kernels (one group, unit dilation) and the
    tiled kernel (the rest)."""
    rng = np.random.default_rng(7)
    cases = []
    for i in range(36):
        dt = ["bfloat16", "float16", "float8_e4m3fn"][i % 3]
        kind = ["group", "dilate", "plain", "any"][(i // 3) % 4]
        r = int(rng.choice([1, 3, 5]))
        s_ = int(rng.choice([1, 3]))
        if kind == "group":
            g = int(rng.choice([2, 4, 8, 16, 32]))
            cg = int(rng.choice([1, 2, 4, 8, 16, 32]))
            fg = int(rng.choice([1, 2, 4, 8, 16]))
            st, dil = int(rng.choice([1, 2])), 1
        elif kind == "dilate":
            g, cg, fg = 1, int(rng.choice([16, 32, 64])), int(rng.choice([8, 16, 24, 40, 64]))
            st, dil = 1, int(rng.choice([2, 3]))
        elif kind == "plain":
            g, cg, fg = 1, int(rng.choice([16, 32, 64])), int(rng.choice([8, 16, 48, 64, 96]))
            st, dil = int(rng.choice([1, 2])), 1
        else:
            g = int(rng.choice([1, 2, 4]))
            cg, fg = int(rng.choice([3, 8, 16])), int(rng.choice([4, 8, 12]))
            st, dil = int(rng.choice([1, 2, 3])), int(rng.choice([1, 2]))
        if kind == "dilate":
            pb = dil * int(rng.integers(0, 2)) * (r // 2)
            pw = dil * int(rng.integers(0, 2)) * (s_ // 2)
            h = dil * int(rng.integers(4, 10))
            w = dil * int(rng.integers(4, 10))
            pad_b, pad_e = (pb, pw), (pb, pw)
        else:
            pad_b = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
            pad_e = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
            h, w = int(rng.integers(6, 20)), int(rng.integers(6, 20))
        n = int(rng.integers(1, 3))
        cases.append((f"sweep{i}_{kind}", dt, n, h, w, g * cg, g * fg, r, s_, st, dil, pad_b,
                      pad_e, g))
    return cases


@pytest.mark.parametrize("case", _sweep_general(), ids=lambda c: c[0])
def test_general_random_sweep(case):
    cid, dt = case[0], case[1]
    p, oshape, x, wt, _ = _draw(case)
    if oshape[1] < 1 or oshape[2] < 1:
        pytest.skip("empty output")
    name = igc.conv2d_fwd_general_kernel_name(x.shape, wt.shape, oshape, p, filter_is_fcrs=False,
                                              dtype=x.dtype)
    _say(f"general sweep {case[2:]} -> {oshape}, {name}")
    if _supergroup(case) or _dilation_phases(case):
        assert name == "igemm_fwd_band_kernel", name
    out = _run(x, wt, oshape, p, False)
    ref = _oracle(case, x, wt, False)
    _assert_close(out, ref, TOL[dt], cid)

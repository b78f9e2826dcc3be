"""Pins the oracle to facts other than itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix:
hand-worked examples, brute force written independently, closed forms,
special cases, invariants, or a library routine.  A plausible mistake in the
oracle (dropped term, wrong sign or index, transposed operand, wrong padding
side, flipped filter) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(shape):
    return RNG.standard_normal(shape)


def _brute(x, w, fcrs, st, p, src=None, beta=0.0):
    """Pure-Python convolution over an explicitly zero-padded copy, each sum
    correctly rounded by math.fsum.  Filter read with natural 4-D indexing.
    st and p are ints or (height, width) pairs."""
    sh, sw = (st, st) if isinstance(st, int) else st
    ph, pw = (p, p) if isinstance(p, int) else p
    n_, h, wd, c = x.shape
    if fcrs:
        f, _, r_, s_ = w.shape
        tap = lambda r, s, ci, co: w[co, ci, r, s]  # noqa: E731
    else:
        r_, s_, _, f = w.shape
        tap = lambda r, s, ci, co: w[r, s, ci, co]  # noqa: E731
    xp = np.zeros((n_, h + 2 * ph, wd + 2 * pw, c))
    xp[:, ph:ph + h, pw:pw + wd, :] = x
    ho = (h + 2 * ph - r_) // sh + 1
    wo = (wd + 2 * pw - s_) // sw + 1
    y = np.zeros((n_, ho, wo, f))
    for n, oh, ow, co in itertools.product(range(n_), range(ho), range(wo), range(f)):
        terms = [xp[n, oh * sh + r, ow * sw + s, ci] * tap(r, s, ci, co)
                 for r in range(r_) for s in range(s_) for ci in range(c)]
        v = math.fsum(terms)
        if src is not None:
            v = v + beta * src[n, oh, ow, co]
        y[n, oh, ow, co] = v
    return y


def _rel(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


# ----------------------------------------------------------------- golden
def _read_handworked():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "handworked_conv.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "case":
                cur = dict(name=vals[0], dims=[int(v) for v in vals[1:10]],
                           beta=float(vals[10]))
                cases.append(cur)
            elif vals == ["none"]:
                cur[tag] = None
            else:
                cur[tag] = np.array([float(v) for v in vals])
    return cases


@pytest.mark.parametrize("case", _read_handworked(), ids=lambda c: c["name"])
def test_handworked_examples(case):
    n, h, w, c, r, s, f, st, p = case["dims"]
    x = case["x"].reshape(n, h, w, c)
    wt = case["w"].reshape(r, s, c, f)
    ho = (h + 2 * p - r) // st + 1
    wo = (w + 2 * p - s) // st + 1
    src = None if case["src"] is None else case["src"].reshape(n, ho, wo, f)
    y = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p,
                      source=src, beta=case["beta"])
    np.testing.assert_array_equal(y.reshape(-1), case["y"])
    # the same filter stored FCRS must give the same bits
    y2 = oracle.conv2d(x, wt.transpose(3, 2, 0, 1).copy(), filter_is_fcrs=True,
                       stride=st, padding=p, source=src, beta=case["beta"])
    np.testing.assert_array_equal(y2, y)


# ------------------------------------------------------------- brute force
BRUTE_CASES = [
    # N H W C F R S st p fcrs residual
    (1, 5, 5, 1, 1, 3, 3, 1, 1, False, False),
    (2, 6, 7, 3, 2, 3, 3, 1, 1, True, False),
    (1, 7, 6, 2, 3, 5, 5, 1, 2, False, True),
    (2, 7, 7, 4, 2, 3, 3, 2, 1, True, True),
    (1, 6, 6, 2, 2, 2, 2, 2, 0, False, False),
    (1, 7, 5, 3, 1, 1, 1, 2, 0, True, False),
    (2, 4, 5, 2, 3, 3, 2, 1, 2, False, False),
    (1, 5, 7, 4, 2, 5, 3, 2, 2, True, True),
    (1, 3, 3, 1, 2, 5, 5, 1, 2, False, False),
    (1, 7, 7, 1, 1, 2, 3, 1, 0, True, False),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force_tiny(case):
    n, h, w, c, f, r, s, st, p, fcrs, resid = case
    x = _rand((n, h, w, c))
    wt = _rand((f, c, r, s) if fcrs else (r, s, c, f))
    ho = (h + 2 * p - r) // st + 1
    wo = (w + 2 * p - s) // st + 1
    src = _rand((n, ho, wo, f)) if resid else None
    beta = 0.75 if resid else 0.0
    y = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=st, padding=p,
                      source=src, beta=beta)
    yb = _brute(x, wt, fcrs, st, p, src, beta)
    assert y.shape == yb.shape
    assert _rel(y, yb) <= 1e-12


@pytest.mark.parametrize("st,p,fcrs", [((1, 2), (2, 0), False), ((2, 1), (0, 1), True),
                                       ((3, 1), (1, 2), False)])
def test_brute_force_anisotropic(st, p, fcrs):
    """Unequal height/width strides and paddings: the oracle is general even
    though the dispatcher only accepts equal pairs; pins that the height
    parameters act on R/H and the width parameters on S/W."""
    x = _rand((2, 7, 6, 3))
    wt = _rand((2, 3, 3, 2) if fcrs else (3, 3, 3, 2))
    y = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=st, padding=p)
    yb = _brute(x, wt, fcrs, st, p)
    assert y.shape == yb.shape
    assert _rel(y, yb) <= 1e-12


# ------------------------------------------------------ library routine
@pytest.mark.parametrize("n,h,w,c,f,r,s,st,p", [
    (2, 13, 11, 8, 6, 3, 3, 1, 1),
    (1, 16, 16, 16, 5, 5, 5, 2, 2),
    (3, 9, 12, 4, 7, 3, 2, 2, 0),
    (1, 20, 20, 24, 3, 3, 3, 1, 0),
])
def test_matches_torch_conv2d_f64(n, h, w, c, f, r, s, st, p):
    x = torch.randn(n, h, w, c, dtype=torch.float64)
    wf = torch.randn(f, c, r, s, dtype=torch.float64)
    ref = torch.nn.functional.conv2d(x.permute(0, 3, 1, 2), wf, stride=st,
                                     padding=p).permute(0, 2, 3, 1).numpy()
    y = oracle.conv2d(x, wf, filter_is_fcrs=True, stride=st, padding=p)
    assert _rel(y, ref) <= 1e-12
    y2 = oracle.conv2d(x, wf.permute(2, 3, 1, 0).contiguous(), filter_is_fcrs=False,
                       stride=st, padding=p)
    np.testing.assert_array_equal(y2, y)


# ----------------------------------------------------------- closed forms
@pytest.mark.parametrize("fcrs", [False, True])
def test_1x1_stride1_is_matmul(fcrs):
    n, h, w, c, f = 2, 5, 6, 7, 9
    x = _rand((n, h, w, c))
    wm = _rand((c, f))
    wt = wm.T.reshape(f, c, 1, 1).copy() if fcrs else wm.reshape(1, 1, c, f).copy()
    y = oracle.conv2d(x, wt, filter_is_fcrs=fcrs, stride=1, padding=0)
    ref = (x.reshape(n * h * w, c) @ wm).reshape(n, h, w, f)
    assert _rel(y, ref) <= 1e-13


@pytest.mark.parametrize("k,st", [(1, 1), (3, 1), (5, 1), (3, 2), (5, 2)])
def test_centered_delta_reproduces_input(k, st):
    p = (k - 1) // 2
    if p > 2:
        pytest.skip("padding above 2")
    n, h, w, c = 2, 7, 9, 5
    x = _rand((n, h, w, c))
    wt = np.zeros((k, k, c, c))
    for ci in range(c):
        wt[p, p, ci, ci] = 1.0
    y = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p)
    np.testing.assert_array_equal(y, x[:, ::st, ::st, :])


@pytest.mark.parametrize("r0,s0,st,p", [(0, 0, 1, 1), (2, 1, 1, 1), (0, 2, 1, 2),
                                       (4, 3, 1, 2), (1, 0, 2, 1), (2, 2, 2, 0)])
def test_off_center_delta_pins_orientation(r0, s0, st, p):
    """A single tap at (r0, s0) moves the input by (r0 - p, s0 - p): pins no
    filter flip, the padding side and R <-> H, S <-> W."""
    n, h, w, c, k = 1, 6, 7, 3, 5 if max(r0, s0) > 2 else 3
    x = _rand((n, h, w, c))
    wt = np.zeros((k, k, c, c))
    for ci in range(c):
        wt[r0, s0, ci, ci] = 1.0
    y = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p)
    ho, wo = y.shape[1:3]
    for oh in range(ho):
        for ow in range(wo):
            ih, iw = oh * st - p + r0, ow * st - p + s0
            want = x[0, ih, iw] if (0 <= ih < h and 0 <= iw < w) else np.zeros(c)
            np.testing.assert_array_equal(y[0, oh, ow], want)


@pytest.mark.parametrize("k,st,p", [(3, 1, 1), (3, 2, 1), (5, 1, 2), (5, 2, 2),
                                    (3, 1, 0), (2, 2, 2), (1, 1, 2)])
def test_all_ones_border_counts(k, st, p):
    n, h, w, c, f = 1, 7, 8, 6, 2
    x = np.ones((n, h, w, c))
    wt = np.ones((k, k, c, f))
    y = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p)

    def cnt(o, size):
        return sum(1 for r in range(k) if 0 <= o * st - p + r < size)

    for oh in range(y.shape[1]):
        for ow in range(y.shape[2]):
            assert np.all(y[0, oh, ow] == c * cnt(oh, h) * cnt(ow, w))


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("k,p", [(3, 1), (5, 2), (3, 0), (2, 1)])
def test_stride2_subsamples_stride1(k, p):
    x = _rand((2, 9, 8, 3))
    wt = _rand((k, k, 3, 4))
    y1 = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=p)
    y2 = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=2, padding=p)
    np.testing.assert_array_equal(y2, y1[:, ::2, ::2, :][:, :y2.shape[1], :y2.shape[2]])


def test_bilinear_in_input_and_filter():
    x1, x2 = _rand((2, 8, 7, 5)), _rand((2, 8, 7, 5))
    w1, w2 = _rand((3, 3, 5, 4)), _rand((3, 3, 5, 4))
    a, b = 0.75, -1.5
    cv = lambda x, w: oracle.conv2d(x, w, filter_is_fcrs=False, stride=1, padding=1)  # noqa: E731
    assert _rel(cv(a * x1 + b * x2, w1), a * cv(x1, w1) + b * cv(x2, w1)) <= 1e-12
    assert _rel(cv(x1, a * w1 + b * w2), a * cv(x1, w1) + b * cv(x1, w2)) <= 1e-12


def test_residual_identities():
    x, wt = _rand((2, 6, 6, 4)), _rand((3, 3, 4, 5))
    src = _rand((2, 6, 6, 5))
    y = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=1)
    d0 = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=1, source=src, beta=0.0)
    np.testing.assert_array_equal(d0, y)
    d1 = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=1, source=src, beta=1.0)
    np.testing.assert_array_equal(d1, y + src)
    dh = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=1, padding=1, source=src, beta=-0.5)
    np.testing.assert_array_equal(dh, y - 0.5 * src)


def test_points_equal_full():
    x, wt = _rand((2, 9, 10, 3)), _rand((4, 3, 3, 3))
    src = _rand((2, 5, 5, 4))
    y = oracle.conv2d(x, wt, filter_is_fcrs=True, stride=2, padding=1, source=src, beta=0.3)
    pix = [0, 7, 24, 25, 49]
    yp = oracle.conv2d_points(x, wt, pix, filter_is_fcrs=True, stride=2, padding=1,
                              source=src, beta=0.3)
    np.testing.assert_array_equal(yp, y.reshape(-1, 4)[pix])


def test_empty_and_degenerate():
    wt = _rand((3, 3, 4, 2))
    y = oracle.conv2d(np.zeros((0, 5, 5, 4)), wt, filter_is_fcrs=False, stride=1, padding=1)
    assert y.shape == (0, 5, 5, 2)
    y = oracle.conv2d(_rand((1, 5, 5, 0)), np.zeros((3, 3, 0, 2)), filter_is_fcrs=False,
                      stride=1, padding=1)
    np.testing.assert_array_equal(y, np.zeros((1, 5, 5, 2)))
    assert oracle.out_size(2, 5, 1, 1) == 0
    assert oracle.out_size(56, 3, 2, 1) == 28
    assert oracle.out_size(7, 3, 2, 0) == 3


# ----------------------------------------------------------- input decode
def test_fp8_e4m3fn_decode_all_codes():
    """torch's fp8 -> float64 upcast (the oracle's input path) against the OCP
    E4M3 definition: bias 7, subnormals at exponent 0, no infinities,
    S.1111.111 is NaN, largest finite 448."""
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        sign = -1.0 if b >> 7 else 1.0
        e, m = (b >> 3) & 0xF, b & 0x7
        if e == 15 and m == 7:
            assert math.isnan(got[b])
            continue
        want = sign * (m / 8.0) * 2.0 ** -6 if e == 0 else sign * (1 + m / 8.0) * 2.0 ** (e - 7)
        assert got[b] == want, (b, got[b], want)
    assert np.nanmax(np.abs(got)) == 448.0


def test_bf16_fp16_decode_samples():
    bits = torch.tensor([0x0000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=torch.int32)
    bf = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    want = [np.frombuffer(np.array([int(b) << 16], dtype=np.uint32).tobytes(), np.float32)[0]
            for b in bits.tolist()]
    np.testing.assert_array_equal(bf, np.array(want, dtype=np.float64))
    hb = torch.tensor([0x3C00, 0x0001, 0x7BFF, 0xC000], dtype=torch.int32).to(torch.int16)
    np.testing.assert_array_equal(hb.view(torch.float16).to(torch.float64).numpy(),
                                  [1.0, 2.0 ** -24, 65504.0, -2.0])


# ------------------------------------------------------------ NK transpose
@pytest.mark.parametrize("fcrs", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float8_e4m3fn])
def test_filter_to_nk_brute(fcrs, dtype):
    r, s, c, f = 3, 2, 5, 4
    shape = (f, c, r, s) if fcrs else (r, s, c, f)
    w = torch.randn(shape).clamp(-400, 400).to(dtype)
    k = r * s * c
    nk = oracle.filter_to_nk(w, fcrs, k_pad=k + 6)
    assert nk.shape == (f, k + 6) and nk.dtype == dtype
    nkb = nk.view(torch.uint8 if dtype == torch.float8_e4m3fn else torch.int16)
    wb = w.view(nkb.dtype)
    for co in range(f):
        for rr in range(r):
            for ss in range(s):
                for ci in range(c):
                    src = wb[co, ci, rr, ss] if fcrs else wb[rr, ss, ci, co]
                    assert nkb[co, (rr * s + ss) * c + ci] == src
        assert torch.all(nkb[co, k:] == 0)


# --------------------------------------------------------------- the gate
def _gate_cases():
    rows = []
    with open(os.path.join(GOLDEN, "gate_cases.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t = line.split()
            rows.append(dict(expect=bool(int(t[0])), dt=t[1], fdt=t[2], odt=t[3],
                             stride=(int(t[4]), int(t[5])), dil=(int(t[6]), int(t[7])),
                             pad=(int(t[8]), int(t[9])), groups=int(t[10]),
                             note=" ".join(t[11:])))
    return rows


@pytest.mark.parametrize("row", _gate_cases(), ids=lambda r: r["note"])
def test_gate_table(row):
    n, h, w, c, f, k = 2, 9, 9, 32, 48, 3
    st, p = row["stride"][0], row["pad"][0]
    ho = (h + 2 * p - k) // st + 1
    ok = oracle.gate_accepts(row["dt"], row["fdt"], row["odt"], (n, h, w, c),
                             (k, k, c, f), False, (n, ho, ho, f), row["stride"],
                             row["dil"], row["pad"], row["groups"])
    assert ok == row["expect"]


def test_gate_shape_rules():
    base = dict(dtype="bfloat16", filter_dtype="bfloat16", out_dtype="bfloat16",
                filter_is_fcrs=False, stride=(1, 1), dilation=(1, 1),
                padding=(1, 1), groups=1)
    g = lambda i, fd, o, **kw: oracle.gate_accepts(  # noqa: E731
        in_nhwc=i, filt_dims=fd, out_nhwc=o, **{**base, **kw})
    assert g((2, 8, 8, 16), (3, 3, 16, 4), (2, 8, 8, 4))
    assert not g((2, 8, 8, 16), (3, 3, 32, 4), (2, 8, 8, 4))        # C_in mismatch
    assert not g((2, 8, 8, 16), (3, 3, 16, 4), (2, 8, 8, 5))        # C_out mismatch
    assert not g((2, 8, 8, 16), (3, 3, 16, 4), (2, 7, 8, 4))        # wrong Ho
    assert g((2, 8, 8, 16), (4, 16, 3, 3), (2, 8, 8, 4), filter_is_fcrs=True)
    assert not g((1, 1, 1, 16), (5, 5, 16, 4), (1, 0, 0, 4))        # filter > padded input
    assert g((0, 8, 8, 16), (3, 3, 16, 4), (0, 8, 8, 4))            # empty batch


# ------------------------------------------------------ fused epilogue pins
def _read_epilogue_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "epilogue_cases.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "case":
                cur = dict(name=vals[0], dims=[int(v) for v in vals[1:10]],
                           beta=float(vals[10]), act=vals[11])
                cases.append(cur)
            elif vals == ["none"]:
                cur[tag] = None
            else:
                cur[tag] = np.array([float(v) for v in vals])
    return cases


@pytest.mark.parametrize("case", _read_epilogue_cases(), ids=lambda c: c["name"])
def test_epilogue_handworked(case):
    n, h, w, c, r, s, f, st, p = case["dims"]
    x = case["x"].reshape(n, h, w, c)
    wt = case["w"].reshape(r, s, c, f)
    ho = (h + 2 * p - r) // st + 1
    wo = (w + 2 * p - s) // st + 1
    src = None if case["src"] is None else case["src"].reshape(n, ho, wo, f)
    y = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=False, stride=st, padding=p,
                               source=src, beta=case["beta"], scale=case["scale"],
                               bias=case["bias"], act=case["act"])
    np.testing.assert_allclose(y.reshape(-1), case["y"], rtol=1e-15, atol=1e-15)


def _small_problem(seed, fcrs=False, n=2, h=6, w=5, c=3, f=4, r=3, s=3):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, h, w, c))
    wt = g.standard_normal((f, c, r, s) if fcrs else (r, s, c, f))
    return x, wt


@pytest.mark.parametrize("st,p", [(1, 0), (1, 1), (2, 1), (2, 2)])
def test_epilogue_none_is_conv2d(st, p):
    x, wt = _small_problem(1)
    ho = (6 + 2 * p - 3) // st + 1
    wo = (5 + 2 * p - 3) // st + 1
    src = np.random.default_rng(2).standard_normal((2, ho, wo, 4))
    for source, beta in ((None, 0.0), (src, -0.75)):
        a = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p,
                          source=source, beta=beta)
        b = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=False, stride=st, padding=p,
                                   source=source, beta=beta)
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("st", [1, 2])
def test_epilogue_bias_is_a_constant_input_channel(st):
    # an extra input channel of ones whose only weight b[co] sits on the
    # centre tap of a 3x3 filter at padding 1 (always inside the image) adds
    # exactly b[co] to every output
    x, wt = _small_problem(3)
    bias = np.array([0.5, -1.25, 3.0, 0.0])
    x1 = np.concatenate([x, np.ones(x.shape[:3] + (1,))], axis=3)
    w1 = np.concatenate([wt, np.zeros((3, 3, 1, 4))], axis=2)
    w1[1, 1, 3, :] = bias
    want = oracle.conv2d(x1, w1, filter_is_fcrs=False, stride=st, padding=1)
    got = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=False, stride=st, padding=1,
                                 bias=bias)
    assert _rel(got, want) < 1e-13


@pytest.mark.parametrize("fcrs", [False, True])
def test_epilogue_scale_folds_into_filter(fcrs):
    # scale[co] * conv(x, w) == conv(x, w with output channel co scaled)
    x, wt = _small_problem(4, fcrs=fcrs)
    scale = np.array([2.0, -0.5, 0.0, 1.5])
    wf = wt * (scale[:, None, None, None] if fcrs else scale[None, None, None, :])
    want = oracle.conv2d(x, wf, filter_is_fcrs=fcrs, stride=1, padding=1)
    got = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=fcrs, stride=1, padding=1,
                                 scale=scale)
    assert _rel(got, want) < 1e-13


def test_activation_identities():
    v = np.random.default_rng(5).standard_normal(1000) * 8
    r = oracle.activation(v, "relu")
    assert np.all(r >= 0)
    np.testing.assert_array_equal(r - oracle.activation(-v, "relu"), v)
    si = oracle.activation(v, "silu")
    # sigmoid(v) + sigmoid(-v) = 1, so silu(v) - silu(-v) = v
    assert np.max(np.abs(si - oracle.activation(-v, "silu") - v)) < 1e-12 * np.max(np.abs(v))
    big = oracle.activation(np.array([-800.0, -40.0, 40.0]), "silu")
    assert big[0] == 0.0 and abs(big[1]) < 1e-15 and abs(big[2] - 40.0) < 1e-15
    np.testing.assert_array_equal(oracle.activation(v, "none"), v)
    with pytest.raises(ValueError):
        oracle.activation(v, "gelu")


def test_epilogue_points_equal_full():
    x, wt = _small_problem(6)
    src = np.random.default_rng(7).standard_normal((2, 6, 5, 4))
    sc, bi = np.array([1.5, -2.0, 0.25, 1.0]), np.array([0.0, 1.0, -1.0, 0.5])
    full = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=False, stride=1, padding=1,
                                  source=src, beta=0.5, scale=sc, bias=bi, act="silu")
    pix = [0, 7, 29, 59, 31]
    pts = oracle.conv2d_epilogue_points(x, wt, pix, filter_is_fcrs=False, stride=1,
                                        padding=1, source=src, beta=0.5, scale=sc, bias=bi,
                                        act="silu")
    np.testing.assert_array_equal(pts, full.reshape(-1, 4)[pix])


# ------------------------------------------------------------ im2col pins
@pytest.mark.parametrize("n,h,w,c,r,s,st,p", [
    (1, 4, 5, 2, 3, 3, 1, 1), (2, 5, 4, 1, 2, 3, 2, 0), (1, 6, 6, 3, 5, 5, 2, 2),
    (1, 3, 3, 2, 1, 1, 1, 0), (2, 4, 4, 2, 3, 2, 1, 2)])
def test_im2col_brute_force(n, h, w, c, r, s, st, p):
    x = torch.randn(n, h, w, c, generator=torch.Generator().manual_seed(h * 7 + c),
                    dtype=torch.float32).to(torch.bfloat16)
    ho, wo = (h + 2 * p - r) // st + 1, (w + 2 * p - s) // st + 1
    a = oracle.im2col(x, r, s, stride=st, padding=p, k_pad=r * s * c + 3)
    assert tuple(a.shape) == (n * ho * wo, r * s * c + 3)
    xv = x.float().tolist()
    av = a.float().tolist()
    for nn in range(n):
        for oh in range(ho):
            for ow in range(wo):
                row = av[(nn * ho + oh) * wo + ow]
                for rr in range(r):
                    for ss in range(s):
                        for ci in range(c):
                            ih, iw = oh * st - p + rr, ow * st - p + ss
                            want = xv[nn][ih][iw][ci] if 0 <= ih < h and 0 <= iw < w else 0.0
                            assert row[(rr * s + ss) * c + ci] == want
                assert row[r * s * c:] == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("fcrs", [False, True])
@pytest.mark.parametrize("st,p", [(1, 1), (2, 1), (2, 2), (1, 0)])
def test_im2col_times_nk_is_conv(fcrs, st, p):
    # A (M x K) @ NK^T (K x C_out) is the convolution: the closed form the
    # fused method computes without writing A
    g = torch.Generator().manual_seed(31)
    x = (torch.rand(2, 7, 6, 4, generator=g) * 2 - 1).to(torch.float16)
    w = (torch.rand(*((5, 4, 3, 3) if fcrs else (3, 3, 4, 5)), generator=g) * 2 - 1).to(
        torch.float16)
    a = oracle.im2col(x, 3, 3, stride=st, padding=p).to(torch.float64).numpy()
    nk = oracle.filter_to_nk(w, fcrs).to(torch.float64).numpy()
    y = oracle.conv2d(x, w, filter_is_fcrs=fcrs, stride=st, padding=p)
    np.testing.assert_allclose(a @ nk.T, y.reshape(-1, 5), rtol=1e-12, atol=1e-12)


# ------------------------------------------------ transposed convolution pins
def _read_transposed():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "transposed_cases.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "case":
                cur = dict(name=vals[0], dims=[int(v) for v in vals[1:10]])
                cases.append(cur)
            else:
                cur[tag] = np.array([float(v) for v in vals])
    return cases


@pytest.mark.parametrize("case", _read_transposed(), ids=lambda c: c["name"])
def test_transposed_handworked(case):
    n, h, w, c, r, s, f, st, p = case["dims"]
    y = oracle.conv2d_transposed(case["x"].reshape(n, h, w, c), case["w"].reshape(r, s, f, c),
                                 stride=st, padding=p)
    np.testing.assert_array_equal(y.reshape(-1), case["y"])


@pytest.mark.parametrize("n,h,w,c,f,r,s,st,p,d", [
    (1, 3, 2, 2, 3, 3, 3, 1, 1, 1), (2, 2, 3, 1, 2, 2, 3, 2, 0, 1), (1, 3, 3, 2, 1, 3, 2, 2, 1, 1),
    (1, 2, 2, 1, 2, 3, 3, 1, 0, 2), (1, 3, 2, 2, 2, 4, 4, 2, 1, 1), (1, 2, 3, 3, 2, 1, 1, 3, 0, 1)])
def test_transposed_brute_force(n, h, w, c, f, r, s, st, p, d):
    g = np.random.default_rng(h * 31 + r)
    x = g.standard_normal((n, h, w, c))
    wt = g.standard_normal((r, s, f, c))
    y = oracle.conv2d_transposed(x, wt, stride=st, padding=p, dilation=d)
    ho, wo = (h - 1) * st - 2 * p + d * (r - 1) + 1, (w - 1) * st - 2 * p + d * (s - 1) + 1
    assert y.shape == (n, ho, wo, f)
    want = [[[[[] for _ in range(f)] for _ in range(wo)] for _ in range(ho)] for _ in range(n)]
    for b in range(n):
        for ih in range(h):
            for iw in range(w):
                for rr in range(r):
                    for ss in range(s):
                        oh, ow = ih * st - p + rr * d, iw * st - p + ss * d
                        if 0 <= oh < ho and 0 <= ow < wo:
                            for ff in range(f):
                                for cc in range(c):
                                    want[b][oh][ow][ff].append(x[b, ih, iw, cc] * wt[rr, ss, ff, cc])
    ref = np.array([[[[math.fsum(v) for v in px] for px in row] for row in img] for img in want])
    assert _rel(y, ref) < 1e-13


@pytest.mark.parametrize("h,w,r,st,p", [(6, 5, 3, 1, 1), (7, 7, 3, 2, 1), (5, 6, 5, 1, 2),
                                        (8, 8, 4, 2, 1), (5, 5, 1, 1, 0), (7, 5, 3, 2, 0)])
def test_transposed_is_adjoint_of_conv2d(h, w, r, st, p):
    # <conv2d(a, W), b> = <a, conv2d_transposed(b, W)>: the RSCF filter of the
    # forward convolution is the RSFC filter of its adjoint
    if (h + 2 * p - r) % st or (w + 2 * p - r) % st:
        pytest.skip("output extent must map back onto the input exactly")
    g = np.random.default_rng(h * 100 + w * 10 + r)
    cin, cout = 3, 4
    a = g.standard_normal((2, h, w, cin))
    wt = g.standard_normal((r, r, cin, cout))
    y = oracle.conv2d(a, wt, filter_is_fcrs=False, stride=st, padding=p)
    b = g.standard_normal(y.shape)
    at = oracle.conv2d_transposed(b, wt, stride=st, padding=p)
    assert at.shape == a.shape
    lhs, rhs = float(np.sum(y * b)), float(np.sum(a * at))
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0) * a.size


# ------------------------------------------------- general convolution
def _read_general():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "general_cases.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "case":
                cur = dict(name=vals[0], dims=[int(v) for v in vals[1:17]],
                           beta=float(vals[17]))
                cases.append(cur)
            elif vals == ["none"]:
                cur[tag] = None
            else:
                cur[tag] = np.array([float(v) for v in vals])
    return cases


@pytest.mark.parametrize("case", _read_general(), ids=lambda c: c["name"])
def test_general_handworked(case):
    n, h, w, c, r, s, f, sh, sw, dh, dw, pt, pl, pb, pr, g = case["dims"]
    x = case["x"].reshape(n, h, w, c)
    wt = case["w"].reshape(r, s, c // g, f)
    ho = oracle.out_size_general(h, r, sh, dh, pt, pb)
    wo = oracle.out_size_general(w, s, sw, dw, pl, pr)
    src = None if case["src"] is None else case["src"].reshape(n, ho, wo, f)
    kw = dict(stride=(sh, sw), dilation=(dh, dw), pad_begin=(pt, pl), pad_end=(pb, pr),
              groups=g, source=src, beta=case["beta"])
    y = oracle.conv2d_general(x, wt, filter_is_fcrs=False, **kw)
    np.testing.assert_array_equal(y.reshape(-1), case["y"])
    y2 = oracle.conv2d_general(x, wt.transpose(3, 2, 0, 1).copy(), filter_is_fcrs=True, **kw)
    np.testing.assert_array_equal(y2, y)


def _brute_general(x, w, st, dil, pb_, pe_, groups):
    """Pure-Python general convolution over an explicitly (asymmetrically)
    zero-padded copy, RSCF filter [R, S, Cg, F], each sum by math.fsum."""
    (sh, sw), (dh, dw), (pt, pl), (pb, pr) = st, dil, pb_, pe_
    n_, h, wd, c = x.shape
    r_, s_, cg, f = w.shape
    fg = f // groups
    xp = np.zeros((n_, h + pt + pb, wd + pl + pr, c))
    xp[:, pt:pt + h, pl:pl + wd, :] = x
    ho = (h + pt + pb - dh * (r_ - 1) - 1) // sh + 1
    wo = (wd + pl + pr - dw * (s_ - 1) - 1) // sw + 1
    y = np.zeros((n_, ho, wo, f))
    for n, oh, ow, co in itertools.product(range(n_), range(ho), range(wo), range(f)):
        g = co // fg
        y[n, oh, ow, co] = math.fsum(
            xp[n, oh * sh + rr * dh, ow * sw + ss * dw, g * cg + ci] * w[rr, ss, ci, co]
            for rr in range(r_) for ss in range(s_) for ci in range(cg))
    return y


GENERAL_CASES = [
    # N H W C F R S (sh, sw) (dh, dw) (pt, pl) (pb, pr) groups
    (1, 7, 8, 2, 2, 3, 3, (1, 1), (2, 2), (2, 2), (2, 2), 1),
    (2, 9, 7, 4, 6, 3, 2, (3, 2), (1, 3), (1, 0), (2, 3), 2),
    (1, 8, 8, 6, 3, 2, 2, (4, 4), (1, 1), (0, 0), (0, 0), 3),
    (1, 6, 9, 4, 4, 3, 3, (2, 1), (2, 1), (0, 3), (1, 0), 4),
    (2, 5, 5, 2, 4, 1, 3, (1, 2), (1, 2), (0, 2), (0, 2), 2),
    (1, 10, 6, 3, 3, 2, 3, (5, 3), (3, 1), (4, 1), (0, 1), 3),
]


@pytest.mark.parametrize("case", GENERAL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_general_brute_force(case):
    n, h, w, c, f, r, s, st, dil, pb_, pe_, g = case
    x = _rand((n, h, w, c))
    wt = _rand((r, s, c // g, f))
    y = oracle.conv2d_general(x, wt, filter_is_fcrs=False, stride=st, dilation=dil,
                              pad_begin=pb_, pad_end=pe_, groups=g)
    ref = _brute_general(x, wt, st, dil, pb_, pe_, g)
    assert y.shape == ref.shape
    assert _rel(y, ref) < 1e-12


@pytest.mark.parametrize("case", GENERAL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_general_matches_torch_f64(case):
    n, h, w, c, f, r, s, st, dil, pb_, pe_, g = case
    x = torch.from_numpy(_rand((n, h, w, c)))
    wf = torch.from_numpy(_rand((f, c // g, r, s)))      # FCRS is torch's layout
    y = oracle.conv2d_general(x, wf, filter_is_fcrs=True, stride=st, dilation=dil,
                              pad_begin=pb_, pad_end=pe_, groups=g)
    xp = torch.nn.functional.pad(x.permute(0, 3, 1, 2), (pb_[1], pe_[1], pb_[0], pe_[0]))
    ref = torch.nn.functional.conv2d(xp, wf, stride=st, dilation=dil, groups=g)
    np.testing.assert_allclose(y, ref.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("st,p", [(1, 0), (1, 1), (2, 2), (2, 1)])
def test_general_reduces_to_conv2d(st, p):
    x, wt = _rand((2, 9, 8, 3)), _rand((3, 3, 3, 4))
    a = oracle.conv2d_general(x, wt, filter_is_fcrs=False, stride=st, pad_begin=p, pad_end=p)
    b = oracle.conv2d(x, wt, filter_is_fcrs=False, stride=st, padding=p)
    np.testing.assert_array_equal(a, b)


def test_general_groups_are_independent_convolutions():
    g, cg, fg = 3, 2, 2
    x, wt = _rand((2, 7, 6, g * cg)), _rand((3, 2, cg, g * fg))
    y = oracle.conv2d_general(x, wt, filter_is_fcrs=False, stride=(1, 2), pad_begin=(1, 0),
                              pad_end=(1, 1), groups=g)
    for k in range(g):
        part = oracle.conv2d_general(x[..., k * cg:(k + 1) * cg], wt[..., k * fg:(k + 1) * fg],
                                     filter_is_fcrs=False, stride=(1, 2), pad_begin=(1, 0),
                                     pad_end=(1, 1))
        np.testing.assert_array_equal(y[..., k * fg:(k + 1) * fg], part)


def test_general_dilation_is_a_zero_inserted_filter():
    x, wt = _rand((1, 11, 10, 2)), _rand((3, 2, 2, 3))
    dh, dw = 3, 2
    wz = np.zeros((dh * 2 + 1, dw * 1 + 1, 2, 3))
    wz[::dh, ::dw] = wt
    a = oracle.conv2d_general(x, wt, filter_is_fcrs=False, dilation=(dh, dw), pad_begin=(1, 2),
                              pad_end=(0, 1))
    b = oracle.conv2d_general(x, wz, filter_is_fcrs=False, pad_begin=(1, 2), pad_end=(0, 1))
    assert a.shape == b.shape
    assert _rel(a, b) < 1e-12


def test_general_asymmetric_padding_is_a_padded_input():
    x, wt = _rand((2, 6, 7, 2)), _rand((3, 3, 2, 2))
    pt, pl, pb, pr = 2, 0, 1, 3
    xp = np.zeros((2, 6 + pt + pb, 7 + pl + pr, 2))
    xp[:, pt:pt + 6, pl:pl + 7] = x
    a = oracle.conv2d_general(x, wt, filter_is_fcrs=False, stride=(2, 1),
                              pad_begin=(pt, pl), pad_end=(pb, pr))
    b = oracle.conv2d_general(xp, wt, filter_is_fcrs=False, stride=(2, 1))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("sh,sw", [(3, 3), (4, 2), (5, 7)])
def test_general_stride_subsamples_stride1(sh, sw):
    x, wt = _rand((1, 16, 17, 2)), _rand((2, 3, 2, 2))
    a = oracle.conv2d_general(x, wt, filter_is_fcrs=False, stride=(sh, sw), dilation=(2, 1),
                              pad_begin=(1, 1), pad_end=(0, 2))
    b = oracle.conv2d_general(x, wt, filter_is_fcrs=False, dilation=(2, 1), pad_begin=(1, 1),
                              pad_end=(0, 2))
    np.testing.assert_array_equal(a, b[:, ::sh, ::sw][:, :a.shape[1], :a.shape[2]])


@pytest.mark.parametrize("case", GENERAL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_general_off_centre_delta(case):
    """A filter that is one 1 at an off-centre tap (r0, s0) and one input
    channel per output channel copies that channel of the input pixel the
    tap lands on, oh*sh - pt + r0*dh and ow*sw - pl + s0*dw (zero where it
    lands in the padding): the output is known exactly, element by element."""
    n, h, w, c, f, r, s, (sh, sw), (dh, dw), (pt, pl), (pb, pr), g = case
    cg, fg = c // g, f // g
    r0, s0 = r - 1, s // 2
    csel = [(co * 7 + 3) % cg for co in range(f)]
    wt = np.zeros((r, s, cg, f))
    for co in range(f):
        wt[r0, s0, csel[co], co] = 1.0
    x = _rand((n, h, w, c))
    y = oracle.conv2d_general(x, wt, filter_is_fcrs=False, stride=(sh, sw), dilation=(dh, dw),
                              pad_begin=(pt, pl), pad_end=(pb, pr), groups=g)
    ho = oracle.out_size_general(h, r, sh, dh, pt, pb)
    wo = oracle.out_size_general(w, s, sw, dw, pl, pr)
    want = np.zeros((n, ho, wo, f))
    for b, oh, ow, co in itertools.product(range(n), range(ho), range(wo), range(f)):
        ih, iw = oh * sh - pt + r0 * dh, ow * sw - pl + s0 * dw
        if 0 <= ih < h and 0 <= iw < w:
            want[b, oh, ow, co] = x[b, ih, iw, (co // fg) * cg + csel[co]]
    np.testing.assert_array_equal(y, want)

"""GPU parity of the fused per-channel epilogue
    D = act(scale[co] * conv + bias[co] + beta * source)
through conv2d_fwd_epilogue / conv2d_fwd_nk_epilogue, against the fp64
oracle (oracle.conv2d_epilogue), on one case per kernel variant the
dispatcher can pick.  Tolerances as for the plain convolution: the epilogue
adds a few fp32 operations before the single rounding to the output type.
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
from test_gpu_parity import PATH_CASES, TOL, _KERNEL, _assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def setup_module(_):
    if not os.path.exists(igc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _coefs(f, seed):
    g = torch.Generator().manual_seed(seed)
    scale = (torch.rand(f, generator=g) * 3.0 - 1.5).to(torch.float32)
    bias = torch.randn(f, generator=g).to(torch.float32)
    return scale, bias


def _out(x, f, ho, wo):
    return torch.empty((x.shape[0], ho, wo, f), dtype=datagen.OUT_DTYPES[str(x.dtype)[6:]],
                       device=DEV)


@pytest.mark.parametrize("act", ["relu", "silu"])
@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: c[0])
def test_epilogue_kernel_paths(case, act):
    cid, dt, n, h, w, c, f, r, s, st, p, resid, kern = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, s, st, p)
    _say(f"epilogue {act} {cid}: {dt} N{n} {h}x{w} C{c}->{f} {r}x{s} st{st} p{p} "
         f"residual={resid}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype=dt, fcrs=False,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(cid.encode()) % 1000)
    assert igc.conv2d_fwd_kernel_name(x.shape, wt.shape, (n, ho, wo, f), filter_is_fcrs=False,
                                      dtype=x.dtype, stride=st, padding=p) == _KERNEL[kern]
    scale, bias = _coefs(f, zlib.crc32((cid + act).encode()) % 1000)
    beta = 0.5 if resid else 0.0
    out = _out(x, f, ho, wo)
    rc = igc.conv2d_fwd_epilogue(x.to(DEV), wt.to(DEV), out, filter_is_fcrs=False, stride=st,
                                 padding=p, source=None if src is None else src.to(DEV),
                                 beta=beta, scale=scale.to(DEV), bias=bias.to(DEV),
                                 activation=act)
    assert rc == 1, rc
    torch.cuda.synchronize()
    kw = dict(filter_is_fcrs=False, stride=st, padding=p, source=src, beta=beta,
              scale=scale, bias=bias, act=act)
    ref = oracle.conv2d_epilogue(x, wt, **kw)
    _assert_close(out, ref, TOL[dt], cid)


@pytest.mark.parametrize("f", [3, 20, 64, 130])
def test_epilogue_partial_forms(f):
    # scale only, bias only, activation only, and the no-op epilogue (equal in
    # value to conv2d_fwd: fma(1, v, 0) may turn -0 into +0, so values, not bits)
    n, h, w, c = 2, 14, 13, 32
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=3, S=3, dtype="bfloat16",
                                   fcrs=True, x_dist=("normal", 1.0), w_dist=("normal", 0.2),
                                   src_dist=("normal", 1.0), out_hw=(h, w), seed=f)
    scale, bias = _coefs(f, 100 + f)
    xd, wd, sd = x.to(DEV), wt.to(DEV), src.to(DEV)
    plain = _out(x, f, h, w)
    assert igc.conv2d_fwd(xd, wd, plain, filter_is_fcrs=True, stride=1, padding=1,
                          source=sd, beta=-0.25) == 1
    forms = [dict(scale=scale), dict(bias=bias), dict(activation="relu"),
             dict(activation="silu", bias=bias),
             dict(scale=torch.ones(f), bias=torch.zeros(f), activation="none")]
    for kw in forms:
        _say(f"epilogue form C_out={f}: {sorted(kw)}")
        out = _out(x, f, h, w)
        dev_kw = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in kw.items()}
        assert igc.conv2d_fwd_epilogue(xd, wd, out, filter_is_fcrs=True, stride=1, padding=1,
                                       source=sd, beta=-0.25, **dev_kw) == 1
        torch.cuda.synchronize()
        ref = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=True, stride=1, padding=1,
                                     source=src, beta=-0.25, scale=kw.get("scale"),
                                     bias=kw.get("bias"), act=kw.get("activation", "none"))
        _assert_close(out, ref, TOL["bfloat16"], str(sorted(kw)))
        if "activation" in kw and kw["activation"] == "none":
            assert torch.equal(out.float(), plain.float())


def test_epilogue_nk_entry_matches_fwd():
    n, h, w, c, f = 2, 16, 16, 64, 96
    x, wt, _ = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=3, S=3, dtype="float16",
                                 fcrs=False, x_dist=("normal", 1.0), w_dist=("normal", 0.1),
                                 seed=21)
    scale, bias = _coefs(f, 22)
    xd, wd, scd, bid = x.to(DEV), wt.to(DEV), scale.to(DEV), bias.to(DEV)
    a = _out(x, f, h, w)
    assert igc.conv2d_fwd_epilogue(xd, wd, a, filter_is_fcrs=False, stride=1, padding=1,
                                   scale=scd, bias=bid, activation="silu") == 1
    nk = torch.empty(igc.conv2d_workspace_bytes(wt.shape, False, wt.dtype), dtype=torch.uint8,
                     device=DEV)
    assert igc.conv2d_filter_to_nk(wd, nk, filter_is_fcrs=False) == 1
    b = _out(x, f, h, w)
    assert igc.conv2d_fwd_nk_epilogue(xd, nk, wt.shape, b, filter_is_fcrs=False, stride=1,
                                      padding=1, scale=scd, bias=bid, activation="silu",
                                      dtype=1, in_shape=x.shape) == 1
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _epi_sweep():
    rng = np.random.default_rng(77)
    cases = []
    for i, (dt, fcrs, st, act) in enumerate(itertools.product(
            ["bfloat16", "float16", "float8_e4m3fn"], [False, True], [1, 2],
            ["relu", "silu"])):
        f = int(rng.choice([1, 3, 8, 17, 40, 64, 72, 130]))
        c = int(rng.choice([16, 32, 64] if dt != "float8_e4m3fn" else [16, 32, 64, 128]))
        r = int(rng.choice([1, 3, 5]))
        p = int(rng.integers(0, 3)) if r > 1 else 0
        h, w = int(rng.integers(max(r, 4), 20)), int(rng.integers(max(r, 4), 20))
        cases.append((dt, fcrs, st, act, bool(i % 2), int(rng.integers(1, 3)), h, w, c, f, r, p))
    return cases


@pytest.mark.parametrize("case", _epi_sweep(), ids=lambda c: "-".join(map(str, c)))
def test_epilogue_random_sweep(case):
    dt, fcrs, st, act, resid, n, h, w, c, f, r, p = case
    ho, wo = oracle.out_size(h, r, st, p), oracle.out_size(w, r, st, p)
    _say(f"epilogue sweep {case} -> out {n}x{ho}x{wo}x{f}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype=dt, fcrs=fcrs,
                                   x_dist=("normal", 1.0), w_dist=("uniform", 1.0),
                                   src_dist=("normal", 1.0) if resid else None,
                                   out_hw=(ho, wo), seed=zlib.crc32(repr(case).encode()) % 1000)
    scale, bias = _coefs(f, zlib.crc32(repr(case).encode()) % 997)
    beta = 0.75 if resid else 0.0
    out = igc.conv2d(x.to(DEV), wt.to(DEV), filter_is_fcrs=fcrs, stride=st, padding=p,
                     source=None if src is None else src.to(DEV), beta=beta,
                     scale=scale.to(DEV), bias=bias.to(DEV), activation=act)
    torch.cuda.synchronize()
    ref = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=fcrs, stride=st, padding=p, source=src,
                                 beta=beta, scale=scale, bias=bias, act=act)
    _assert_close(out, ref, TOL[dt], str(case))


@pytest.mark.parametrize("kern,dt,f", [("band", "bfloat16", 64), ("band", "float8_e4m3fn", 32),
                                       ("tapfold", "bfloat16", 3), ("tapfold", "float16", 3),
                                       ("tapfold", "float8_e4m3fn", 3),
                                       ("wide", "float16", 96), ("patch", "bfloat16", 128),
                                       ("resident", "bfloat16", 32),
                                       ("tiled", "bfloat16", 64)])
def test_epilogue_coefficients_at_4_byte_offsets(kern, dt, f):
    """scale and bias only 4-byte aligned (the gate's rule), on each kernel
    family, including the band kernel's 16-byte coefficient loads."""
    shapes = {"band": (2, 12, 12, 64 if dt != "float8_e4m3fn" else 128, 3),
              "tapfold": (2, 12, 12, 128, 3),
              "wide": (2, 12, 12, 64, 3), "patch": (16, 64, 64, 64, 3),
              "resident": (2, 12, 12, 48, 3),
              "tiled": (1, 12, 12, 96, 5)}
    n, h, w, c, r = shapes[kern]
    p = (r - 1) // 2
    _say(f"epilogue 4-byte offsets {kern} {dt} C{c}->{f} {r}x{r}")
    x, wt, src = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype=dt, fcrs=False,
                                   x_dist=("normal", 1.0), w_dist=("normal", 0.2),
                                   src_dist=("normal", 1.0), out_hw=(h, w), seed=f + r)
    assert igc.conv2d_fwd_kernel_name(x.shape, wt.shape, (n, h, w, f), filter_is_fcrs=False,
                                      dtype=x.dtype, stride=1, padding=p) == _KERNEL[kern]
    scale, bias = _coefs(f, 31 + f)
    for off in (1, 2, 3):   # element offsets of 4, 8 and 12 bytes
        buf_s = torch.zeros(f + 4, dtype=torch.float32, device=DEV)
        buf_b = torch.zeros(f + 4, dtype=torch.float32, device=DEV)
        buf_s[off:off + f] = scale.to(DEV)
        buf_b[off:off + f] = bias.to(DEV)
        sc, bi = buf_s[off:off + f], buf_b[off:off + f]
        assert sc.data_ptr() % 16 == 4 * off
        out = _out(x, f, h, w)
        assert igc.conv2d_fwd_epilogue(x.to(DEV), wt.to(DEV), out, filter_is_fcrs=False,
                                       stride=1, padding=p, source=src.to(DEV), beta=0.5,
                                       scale=sc, bias=bi, activation="silu") == 1
        torch.cuda.synchronize()
        ref = oracle.conv2d_epilogue(x, wt, filter_is_fcrs=False, stride=1, padding=p,
                                     source=src, beta=0.5, scale=scale, bias=bias, act="silu")
        _assert_close(out, ref, TOL[dt], f"{kern} offset {4 * off}")

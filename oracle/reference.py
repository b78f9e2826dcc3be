"""Oracle functions (TEST INFRASTRUCTURE ONLY; see the package docstring).

Inputs are torch tensors in their stored dtype (bfloat16, float16 or
float8_e4m3fn).  They are upcast to float64 by torch, which is exact for all
three formats (the fp8 decode is checked code by code against the OCP
definition in the tests), and handed to the C oracle in conv_oracle.c.
"""
import ctypes
import os

import numpy as np
import torch

from . import build as _build

_LIB = None

# Element types the MI355X dispatcher accepts, and the output type each one
# produces: page 1 ("dispatch_amd_4wave_conv2d"), Parameters section,
# input_type / filter_type / output_type.
DTYPES = {
    "bfloat16": "bfloat16",
    "float16": "float16",
    "float8_e4m3fn": "bfloat16",
}


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_int
        lib.oracle_conv2d_f64.argtypes = [
            dp, i64, i64, i64, i64, dp, ip, i64, i64, i64, i64, i64, i64, i64,
            dp, ctypes.c_double, dp, i64, i64]
        lib.oracle_conv2d_f64.restype = ctypes.c_int
        lib.oracle_conv2d_points_f64.argtypes = [
            dp, i64, i64, i64, i64, dp, ip, i64, i64, i64, i64, i64, i64, i64,
            dp, ctypes.c_double, ctypes.POINTER(ctypes.c_int64), i64, dp, i64, i64]
        lib.oracle_conv2d_points_f64.restype = ctypes.c_int
        lib.oracle_out_size.argtypes = [i64, i64, i64, i64]
        lib.oracle_out_size.restype = i64
        lib.oracle_out_size_general.argtypes = [i64, i64, i64, i64, i64, i64]
        lib.oracle_out_size_general.restype = i64
        lib.oracle_conv2d_general_f64.argtypes = [
            dp, i64, i64, i64, i64, dp, ip, i64, i64, i64, i64, i64, i64, i64, i64,
            i64, i64, i64, i64, i64, dp, ctypes.c_double, dp, i64, i64]
        lib.oracle_conv2d_general_f64.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_lib().oracle_num_threads())


def out_size(n_in: int, k: int, stride: int, pad: int) -> int:
    """Ho = floor((H + 2p - R) / stride) + 1, or 0 when the padded input is
    shorter than the filter.  Floor rounding is the standard reading; the
    pages state no formula (page 1, Args: stride and symmetric_padding)."""
    return int(_lib().oracle_out_size(n_in, k, stride, pad))


def filter_dims_rscf(w_shape, filter_is_fcrs: bool):
    """(R, S, C_in, C_out) of a filter stored as FCRS [C_out, C_in, R, S] or
    RSCF [R, S, C_in, C_out] (page 2, Parameters: filter_is_fcrs)."""
    if filter_is_fcrs:
        f, c, r, s = w_shape
    else:
        r, s, c, f = w_shape
    return int(r), int(s), int(c), int(f)


def _f64(t):
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t, dtype=np.float64)
    return np.ascontiguousarray(t.detach().cpu().to(torch.float64).numpy())


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(x, w, filter_is_fcrs, stride, padding, source):
    sh, sw = (stride, stride) if isinstance(stride, int) else stride
    ph, pw = (padding, padding) if isinstance(padding, int) else padding
    x64 = _f64(x)
    w64 = _f64(w)
    n, h, wd, c = x64.shape
    r, s, cw, f = filter_dims_rscf(w64.shape, filter_is_fcrs)
    if cw != c:
        raise ValueError(f"filter C_in {cw} != input C_in {c}")
    ho, wo = out_size(h, r, sh, ph), out_size(wd, s, sw, pw)
    src64 = None if source is None else _f64(source)
    if src64 is not None and src64.shape != (n, ho, wo, f):
        raise ValueError("source must have the output's NHWC shape")
    return x64, w64, (n, h, wd, c, r, s, f, sh, sw, ph, pw, ho, wo), src64


def conv2d(x, w, *, filter_is_fcrs: bool, stride=1, padding=0, source=None,
           beta: float = 0.0) -> np.ndarray:
    """Forward convolution of an NHWC input with an RSCF/FCRS filter, fp64.

    Follows page 1 ("dispatch_amd_4wave_conv2d"): summary (D = Conv + beta *
    source with an NHWC source of the output's shape) and Args (NHWC input and
    output, FCRS or RSCF filter, stride [sh, sw], symmetric padding [ph, pw]).
    Returns the unrounded float64 result, shape [N, Ho, Wo, C_out].
    """
    x64, w64, d, src64 = _prep(x, w, filter_is_fcrs, stride, padding, source)
    n, h, wd, c, r, s, f, sh, sw, ph, pw, ho, wo = d
    y = np.zeros((n, ho, wo, f), dtype=np.float64)
    rc = _lib().oracle_conv2d_f64(
        _ptr(x64), n, h, wd, c, _ptr(w64), int(bool(filter_is_fcrs)), r, s, f,
        sh, sw, ph, pw, None if src64 is None else _ptr(src64), float(beta),
        _ptr(y), ho, wo)
    if rc != 0:
        raise ValueError("oracle rejected the convolution arguments")
    return y


ACTIVATIONS = ("none", "relu", "silu")


def activation(v: np.ndarray, act: str) -> np.ndarray:
    """The epilogue activations, in float64: relu keeps v where v > 0 and
    gives +0 elsewhere; silu is v * sigmoid(v) = v / (1 + exp(-v))."""
    if act in (None, "none"):
        return v
    if act == "relu":
        return np.where(v > 0.0, v, 0.0)
    if act == "silu":
        with np.errstate(over="ignore"):
            return v / (1.0 + np.exp(-v))
    raise ValueError(f"unknown activation {act!r}")


def conv2d_epilogue(x, w, *, filter_is_fcrs: bool, stride=1, padding=0, source=None,
                    beta: float = 0.0, scale=None, bias=None, act: str = "none") -> np.ndarray:
    """The convolution with a fused per-channel elementwise epilogue, fp64.

    Page 1 ("dispatch_amd_4wave_conv2d", Parameters: elementwise_lambda_fn)
    and page 2 ("dispatch_fused_im2col_conv2d_apple", Parameters:
    maybe_epilogue_func) fuse an elementwise function of each output element
    and its coordinates into the convolution.  The pages leave the function
    to the caller; this oracle follows the fixed family the library offers:
        v = scale[co] * conv[n, oh, ow, co] + bias[co]
        v = v + beta * source[n, oh, ow, co]     (when a source is given)
        D = act(v)
    scale and bias are per-output-channel vectors (None = 1 and 0).
    Returns the unrounded float64 D, shape [N, Ho, Wo, C_out].
    """
    y = conv2d(x, w, filter_is_fcrs=filter_is_fcrs, stride=stride, padding=padding)
    return _epilogue(y, None if source is None else _f64(source), beta, scale, bias, act)


def _epilogue(y, src64, beta, scale, bias, act):
    f = y.shape[-1]
    sc = np.ones(f) if scale is None else _f64(scale).reshape(f)
    bi = np.zeros(f) if bias is None else _f64(bias).reshape(f)
    v = y * sc + bi
    if src64 is not None:
        v = v + beta * src64
    return activation(v, act)


def conv2d_epilogue_points(x, w, pix, *, filter_is_fcrs: bool, stride=1, padding=0,
                           source=None, beta: float = 0.0, scale=None, bias=None,
                           act: str = "none") -> np.ndarray:
    """conv2d_epilogue evaluated only at the flattened output pixels pix
    (as conv2d_points).  Returns [len(pix), C_out] float64."""
    y = conv2d_points(x, w, pix, filter_is_fcrs=filter_is_fcrs, stride=stride,
                      padding=padding)
    src64 = None
    if source is not None:
        s64 = _f64(source)
        src64 = s64.reshape(-1, s64.shape[-1])[np.asarray(pix, dtype=np.int64)]
    return _epilogue(y, src64, beta, scale, bias, act)


def conv2d_points(x, w, pix, *, filter_is_fcrs: bool, stride=1, padding=0,
                  source=None, beta: float = 0.0) -> np.ndarray:
    """The same definition as conv2d, evaluated only at the flattened output
    pixels pix[i] = (n*Ho + oh)*Wo + ow.  Returns [len(pix), C_out] float64."""
    x64, w64, d, src64 = _prep(x, w, filter_is_fcrs, stride, padding, source)
    n, h, wd, c, r, s, f, sh, sw, ph, pw, ho, wo = d
    pix = np.ascontiguousarray(np.asarray(pix, dtype=np.int64))
    y = np.zeros((pix.shape[0], f), dtype=np.float64)
    rc = _lib().oracle_conv2d_points_f64(
        _ptr(x64), n, h, wd, c, _ptr(w64), int(bool(filter_is_fcrs)), r, s, f,
        sh, sw, ph, pw, None if src64 is None else _ptr(src64), float(beta),
        pix.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), pix.shape[0],
        _ptr(y), ho, wo)
    if rc != 0:
        raise ValueError("oracle rejected the convolution arguments")
    return y


def filter_to_nk(w: torch.Tensor, filter_is_fcrs: bool, k_pad: int = None) -> torch.Tensor:
    """The filter as the (C_out, K = R*S*C_in) "NK" matrix of page 2
    ("dispatch_fused_im2col_conv2d_apple", summary), k ordered (r, s, ci)
    with ci fastest, i.e. NK[co, (r*S + s)*C_in + ci] = Wt(r, s, ci, co).

    A pure bit copy: the element bits are moved, never converted.  Columns
    K..k_pad-1 (when k_pad > K) are zero.  Returns a CPU tensor of w's dtype.
    """
    r, s, c, f = filter_dims_rscf(w.shape, filter_is_fcrs)
    k = r * s * c
    bits = w.detach().cpu().contiguous()
    bits = bits.view(torch.int16) if bits.element_size() == 2 else bits.view(torch.uint8)
    if filter_is_fcrs:   # [F, C, R, S] -> [F, R, S, C]
        nk = bits.permute(0, 2, 3, 1)
    else:                # [R, S, C, F] -> [F, R, S, C]
        nk = bits.permute(3, 0, 1, 2)
    nk = nk.reshape(f, k)
    if k_pad is not None and k_pad > k:
        nk = torch.cat([nk, torch.zeros(f, k_pad - k, dtype=nk.dtype)], dim=1)
    return nk.contiguous().view(w.dtype)


def conv2d_transposed(x, w_rsfc, *, stride=1, padding=0, dilation=1, source=None,
                      beta: float = 0.0, scale=None, bias=None, act: str = "none") -> np.ndarray:
    """Transposed convolution, fp64 (page 3, "conv_transposed_gpu": NHWC input,
    RSFC filter [R, S, F, C] with F output and C input channels, stride,
    dilation and padding per spatial axis; an optional elementwise epilogue
    after it).  Scatter form of the definition: every input pixel (ih, iw)
    adds in[n, ih, iw, :] . W[r, s, f, :] to output pixel
        (ih*sh - ph + r*dh,  iw*sw - pw + s*dw)
    when that lies inside the output of size
        Ho = (H - 1)*sh - 2*ph + dh*(R - 1) + 1  (and likewise Wo).
    Then the fused-epilogue family of conv2d_epilogue.  Returns the
    unrounded float64 result [N, Ho, Wo, F].
    """
    sh, sw = (stride, stride) if isinstance(stride, int) else stride
    ph, pw = (padding, padding) if isinstance(padding, int) else padding
    dh, dw = (dilation, dilation) if isinstance(dilation, int) else dilation
    x64, w64 = _f64(x), _f64(w_rsfc)
    n, h, wd, c = x64.shape
    r, s, f, cw = w64.shape
    if cw != c:
        raise ValueError(f"filter C {cw} != input C {c}")
    fh = (h - 1) * sh + dh * (r - 1) + 1     # output extent before the padding is cut
    fw = (wd - 1) * sw + dw * (s - 1) + 1
    ho, wo = fh - 2 * ph, fw - 2 * pw
    if ho < 1 or wo < 1:
        raise ValueError("empty transposed-convolution output")
    full = np.zeros((n, fh, fw, f))
    for rr in range(r):
        for ss in range(s):
            contrib = x64 @ w64[rr, ss].T                      # [N, H, W, F]
            full[:, rr * dh:rr * dh + (h - 1) * sh + 1:sh,
                 ss * dw:ss * dw + (wd - 1) * sw + 1:sw, :] += contrib
    y = np.ascontiguousarray(full[:, ph:ph + ho, pw:pw + wo, :])
    src64 = None if source is None else _f64(source)
    return _epilogue(y, src64, beta, scale, bias, act)


def im2col(x, r: int, s: int, *, stride=1, padding=0, k_pad: int = None) -> torch.Tensor:
    """The [M, K] patch matrix of page 2 ("dispatch_fused_im2col_conv2d_apple",
    summary: the matrix the fused kernel gathers on the fly instead of
    materialising), as a bit copy of the input's elements:
        A[(n*Ho + oh)*Wo + ow, (rr*S + ss)*C_in + ci]
            = x[n, oh*st - p + rr, ow*st - p + ss, ci],  0 outside the image
    k ordered (r, s, ci) with ci fastest, the order of filter_to_nk.
    Columns K..k_pad-1 (when k_pad > K) are zero.  Returns a CPU tensor
    [M, max(K, k_pad)] of x's dtype.
    """
    sh, sw = (stride, stride) if isinstance(stride, int) else stride
    ph, pw = (padding, padding) if isinstance(padding, int) else padding
    bits = x.detach().cpu().contiguous()
    bits = bits.view(torch.int16) if bits.element_size() == 2 else bits.view(torch.uint8)
    n, h, w, c = bits.shape
    ho, wo = out_size(h, r, sh, ph), out_size(w, s, sw, pw)
    padded = torch.zeros((n, h + 2 * ph, w + 2 * pw, c), dtype=bits.dtype)
    padded[:, ph:ph + h, pw:pw + w, :] = bits
    cols = []
    for rr in range(r):
        for ss in range(s):
            win = padded[:, rr:rr + sh * (ho - 1) + 1:sh, ss:ss + sw * (wo - 1) + 1:sw, :]
            cols.append(win.reshape(n * ho * wo, c))
    a = torch.cat(cols, dim=1) if cols else torch.zeros((n * ho * wo, 0), dtype=bits.dtype)
    k = r * s * c
    if k_pad is not None and k_pad > k:
        a = torch.cat([a, torch.zeros((a.shape[0], k_pad - k), dtype=a.dtype)], dim=1)
    return a.contiguous().view(x.dtype)


def gate_accepts(dtype: str, filter_dtype: str, out_dtype: str, in_nhwc,
                 filt_dims, filter_is_fcrs: bool, out_nhwc, stride, dilation,
                 padding, groups) -> bool:
    """Whether page 1's dispatcher would take the call.

    Rules, all from page 1 ("dispatch_amd_4wave_conv2d"):
      Parameters: input dtype is float8_e4m3fn, bfloat16 or float16; the
        filter dtype equals it; the output dtype is bfloat16 for fp8 inputs,
        otherwise the input dtype.
      Args: stride (1,1) or (2,2); dilation (1,1); symmetric padding (0,0),
        (1,1) or (2,2); groups 1; the filter's C_in equals the input's; the
        output is NHWC [N, Ho, Wo, C_out].
    Reading where the page is silent: a filter larger than the padded input
    (Ho or Wo < 1) or with R or S < 1 is not a convolution and is declined;
    an empty batch or C_out = 0 is accepted (nothing to compute).
    """
    if dtype not in DTYPES or filter_dtype != dtype or out_dtype != DTYPES[dtype]:
        return False
    if tuple(stride) not in ((1, 1), (2, 2)):
        return False
    if tuple(dilation) != (1, 1):
        return False
    if tuple(padding) not in ((0, 0), (1, 1), (2, 2)):
        return False
    if groups != 1:
        return False
    n, h, w, c = in_nhwc
    r, s, cf, f = filter_dims_rscf(filt_dims, filter_is_fcrs)
    if min(n, h, w, c, f) < 0 or r < 1 or s < 1:
        return False
    if cf != c:
        return False
    ho = out_size(h, r, stride[0], padding[0])
    wo = out_size(w, s, stride[1], padding[1])
    if ho < 1 or wo < 1:
        return False
    return tuple(out_nhwc) == (n, ho, wo, f)


def _pair2(v):
    return (int(v), int(v)) if isinstance(v, (int, np.integer)) else (int(v[0]), int(v[1]))


def out_size_general(n_in: int, k: int, stride: int, dilation: int, pad_before: int,
                     pad_after: int) -> int:
    """floor((n + pad_before + pad_after - dilation*(k - 1) - 1) / stride) + 1,
    or 0 when the padded input is shorter than the dilated filter."""
    return int(_lib().oracle_out_size_general(n_in, k, stride, dilation, pad_before,
                                              pad_after))


def conv2d_general(x, w, *, filter_is_fcrs: bool, stride=1, dilation=1, pad_begin=0,
                   pad_end=0, groups: int = 1, source=None, beta: float = 0.0, scale=None,
                   bias=None, act: str = "none") -> np.ndarray:
    """The forward convolution with the parameters page 1
    ("dispatch_amd_4wave_conv2d", Args: stride, dilation, symmetric_padding,
    num_groups) names and its dispatcher restricts, in their standard
    meaning: per-axis stride [sh, sw] and dilation [dh, dw], padding
    pad_begin = [top, left] and pad_end = [bottom, right], and `groups`
    channel groups (output channel co reads input channels
    g*Cg .. g*Cg + Cg - 1, g = co // (C_out / groups), Cg = C_in / groups,
    the filter's C_in being Cg).  Then the fused-epilogue family of
    conv2d_epilogue.  fp64; returns [N, Ho, Wo, C_out]."""
    sh, sw = _pair2(stride)
    dh, dw = _pair2(dilation)
    pt, pl = _pair2(pad_begin)
    pb, pr = _pair2(pad_end)
    x64, w64 = _f64(x), _f64(w)
    n, h, wd, c = x64.shape
    r, s, cg, f = filter_dims_rscf(w64.shape, filter_is_fcrs)
    if groups < 1 or cg * groups != c or f % groups:
        raise ValueError("channels do not split into the groups")
    ho = out_size_general(h, r, sh, dh, pt, pb)
    wo = out_size_general(wd, s, sw, dw, pl, pr)
    y = np.zeros((n, max(ho, 0), max(wo, 0), f), dtype=np.float64)
    rc = _lib().oracle_conv2d_general_f64(
        _ptr(x64), n, h, wd, c, _ptr(w64), int(bool(filter_is_fcrs)), r, s, cg, f,
        sh, sw, dh, dw, pt, pb, pl, pr, int(groups), None, 0.0, _ptr(y), ho, wo)
    if rc != 0:
        raise ValueError("oracle rejected the convolution arguments")
    src64 = None if source is None else _f64(source)
    return _epilogue(y, src64, beta, scale, bias, act)

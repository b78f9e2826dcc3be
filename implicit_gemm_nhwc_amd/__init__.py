"""Python binding of libigemmconv.so: forward NHWC convolution as an implicit
GEMM on MI355X (gfx950).

Argument marshalling only.  Every step of the computation (filter transpose,
gather, MFMA contraction, masks, residual epilogue) runs in the HIP kernels
behind the C ABI declared in include/igemm_conv.h; torch supplies device
memory and streams.  There is no fallback: if the library is not built, or a
call is declined, these functions say so instead of computing anything.
Tensor arguments of calls that enqueue work are checked first (contiguous,
on one GPU, of the types and sizes their shape arguments describe):
InvalidArgument is raised before anything is launched.

Names mirror the C entry points:
  conv2d_fwd, conv2d_fwd_check, conv2d_fwd_query, conv2d_fwd_noalloc, conv2d_fwd_nk,
  conv2d_filter_to_nk,
  conv2d_fwd_epilogue, conv2d_fwd_epilogue_check, conv2d_fwd_nk_epilogue,
  conv2d_epilogue_check,
  conv2d_im2col, conv2d_im2col_bytes,
  conv2d_transposed_fwd, conv2d_transposed_check, conv2d_transposed_workspace_bytes,
  conv2d_fwd_general, conv2d_fwd_general_check, conv2d_fwd_general_query,
  conv2d_fwd_general_kernel_name, conv2d_fwd_general_workspace_bytes,
  conv2d_fwd_kernel_name, conv2d_fwd_filter_in_kernel, conv2d_workspace_bytes,
  conv2d_nk_row_pitch, conv2d_build_flags, conv2d_reason_string, conv2d_abi_version
plus conv2d(), conv2d_general() and conv2d_transposed(), which allocate the
output and call conv2d_fwd_epilogue / conv2d_fwd_general /
conv2d_transposed_fwd, and
conv2d_materialized(), the write-then-GEMM route (conv2d_filter_to_nk,
conv2d_im2col, conv2d_fwd_nk on the 1x1 view) kept for measuring what the
fused gather saves.
"""
import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libigemmconv.so")
# debug build whose kernels fill their LDS with NaN bytes first (tests only)
POISON_LIB_PATH = os.path.join(_PKG, "libigemmconv_ldspoison.so")

DTYPE_CODES = {torch.bfloat16: 0, torch.float16: 1, torch.float8_e4m3fn: 2}
OUT_DTYPES = {torch.bfloat16: torch.bfloat16, torch.float16: torch.float16,
              torch.float8_e4m3fn: torch.bfloat16}

# decline reason codes (IGC_DECLINE_* in include/igemm_conv.h)
REASONS = {0: "ok", 1: "dtype", 2: "stride", 3: "dilation", 4: "padding", 5: "groups",
           6: "shape", 7: "output_shape", 8: "vector_width", 9: "alignment",
           10: "null_pointer", 11: "overlap", 12: "workspace", 13: "size_limit",
           14: "epilogue"}

# fused-epilogue activation codes (IGC_ACT_* in include/igemm_conv.h)
ACTIVATIONS = {None: 0, "none": 0, "relu": 1, "silu": 2}


class IgcEpilogue(ctypes.Structure):
    """struct igc_epilogue: per-channel scale and bias (device float
    arrays or NULL) and an activation code."""
    _fields_ = [("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("activation", ctypes.c_int32)]

class IgcConvParams(ctypes.Structure):
    """igc_conv_params of include/igemm_conv.h."""
    _fields_ = [("stride", ctypes.c_int32 * 2), ("dilation", ctypes.c_int32 * 2),
                ("pad_begin", ctypes.c_int32 * 2), ("pad_end", ctypes.c_int32 * 2),
                ("groups", ctypes.c_int32)]


_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


class Declined(RuntimeError):
    pass


_libs = {}


def lib():
    """The loaded C library with argument types set.  Raises if not built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Run the binding's calls inside the with-block on another build of the
    library (the LDS-poison debug build in the tests)."""
    global _lib
    prev = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def _load(path):
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python implicit_gemm_nhwc_amd/_build.py)")
    L = ctypes.CDLL(path)
    vp, i32, i64p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)
    i32p, f32, sz = ctypes.POINTER(ctypes.c_int32), ctypes.c_float, ctypes.c_size_t
    conv_head = [vp, i64p, vp, i32, i64p, vp, i64p, i32p, i32p, i32p, i32, i32, vp, f32]
    L.conv2d_abi_version.argtypes, L.conv2d_abi_version.restype = [], i32
    L.conv2d_build_flags.argtypes, L.conv2d_build_flags.restype = [], i32
    L.conv2d_reason_string.argtypes, L.conv2d_reason_string.restype = [i32], ctypes.c_char_p
    L.conv2d_fwd_check.argtypes = conv_head + [vp, sz]
    L.conv2d_fwd_check.restype = i32
    L.conv2d_fwd_query.argtypes = [i64p, i32, i64p, i64p, i32p, i32p, i32p, i32, i32]
    L.conv2d_fwd_query.restype = i32
    L.conv2d_fwd.argtypes = conv_head + [vp, sz, vp]
    L.conv2d_fwd.restype = i32
    L.conv2d_fwd_noalloc.argtypes = conv_head + [vp]
    L.conv2d_fwd_noalloc.restype = i32
    L.conv2d_fwd_nk.argtypes = conv_head + [vp]
    L.conv2d_fwd_nk.restype = i32
    L.conv2d_workspace_bytes.argtypes, L.conv2d_workspace_bytes.restype = [i64p, i32, i32], sz
    L.conv2d_nk_row_pitch.argtypes = [i64p, i32, i32]
    L.conv2d_nk_row_pitch.restype = ctypes.c_int64
    L.conv2d_fwd_kernel_name.argtypes = [i64p, i32, i64p, i64p, i32p, i32p, i32p, i32, i32]
    L.conv2d_fwd_kernel_name.restype = ctypes.c_char_p
    L.conv2d_fwd_filter_in_kernel.argtypes = [i64p, i32, i64p, i64p, i32p, i32p, i32p, i32,
                                              i32]
    L.conv2d_fwd_filter_in_kernel.restype = i32
    L.conv2d_filter_to_nk.argtypes = [vp, i32, i64p, i32, vp, sz, vp]
    L.conv2d_filter_to_nk.restype = i32
    epip = ctypes.POINTER(IgcEpilogue)
    L.conv2d_fwd_epilogue.argtypes = conv_head + [epip, vp, sz, vp]
    L.conv2d_fwd_epilogue.restype = i32
    L.conv2d_fwd_epilogue_check.argtypes = conv_head + [epip, vp, sz]
    L.conv2d_fwd_epilogue_check.restype = i32
    L.conv2d_fwd_nk_epilogue.argtypes = conv_head + [epip, vp]
    L.conv2d_fwd_nk_epilogue.restype = i32
    L.conv2d_epilogue_check.argtypes = [epip, vp, i64p]
    L.conv2d_epilogue_check.restype = i32
    i64p2 = ctypes.POINTER(ctypes.c_int64)
    L.conv2d_im2col.argtypes = [vp, i64p, i64p2, i32p, i32p, i32, vp, sz, vp]
    L.conv2d_im2col.restype = i32
    L.conv2d_im2col_bytes.argtypes = [i64p, i64p2, i32p, i32p, i32]
    L.conv2d_im2col_bytes.restype = sz
    tr_head = [vp, i64p, vp, i64p, vp, i64p, i32p, i32p, i32p, i32, vp, f32, epip]
    L.conv2d_transposed_fwd.argtypes = tr_head + [vp, sz, vp]
    L.conv2d_transposed_fwd.restype = i32
    L.conv2d_transposed_check.argtypes = tr_head + [vp, sz]
    L.conv2d_transposed_check.restype = i32
    L.conv2d_transposed_workspace_bytes.argtypes = [i64p, i64p, i32p, i32p, i32p, i32]
    L.conv2d_transposed_workspace_bytes.restype = sz
    prm = ctypes.POINTER(IgcConvParams)
    gen_head = [vp, i64p, vp, i32, i64p, vp, i64p, prm, i32, vp, f32, epip]
    L.conv2d_fwd_general.argtypes = gen_head + [vp, sz, vp]
    L.conv2d_fwd_general.restype = i32
    L.conv2d_fwd_general_check.argtypes = gen_head + [vp, sz]
    L.conv2d_fwd_general_check.restype = i32
    L.conv2d_fwd_general_query.argtypes = [i64p, i32, i64p, i64p, prm, i32]
    L.conv2d_fwd_general_query.restype = i32
    L.conv2d_fwd_general_kernel_name.argtypes = [i64p, i32, i64p, i64p, prm, i32]
    L.conv2d_fwd_general_kernel_name.restype = ctypes.c_char_p
    L.conv2d_fwd_general_workspace_bytes.argtypes = [i64p, i32, i64p, i64p, prm, i32]
    L.conv2d_fwd_general_workspace_bytes.restype = sz
    _libs[path] = L
    return L


class InvalidArgument(ValueError):
    """A tensor argument the C ABI cannot describe: not a contiguous tensor on
    the GPU, on another device than the others, or of the wrong type or
    shape.  Raised before anything is enqueued."""


def _check_tensors(named, device=None):
    """Every torch tensor among named (name -> tensor, raw int or None) must
    be a contiguous CUDA tensor, all on one device.  Returns that device."""
    for name, t in named.items():
        if not isinstance(t, torch.Tensor):
            continue
        if not t.is_cuda:
            raise InvalidArgument(f"{name} must be a GPU tensor (got device {t.device})")
        if not t.is_contiguous():
            raise InvalidArgument(f"{name} must be contiguous (densely packed, row-major)")
        if device is None:
            device = t.device
        elif t.device != device:
            raise InvalidArgument(f"{name} is on {t.device}, the other tensors on {device}")
    return device


def _nbytes(t):
    return t.numel() * t.element_size()


def _prod(shape):
    n = 1
    for v in shape:
        n *= int(v)
    return n


def _check_fwd(input, filter, output, source, dtype, in_shape, filt_shape, out_shape,
               filter_is_fcrs, *, scale=None, bias=None, workspace=None, workspace_bytes=0,
               nk=False):
    """The binding's own checks of a forward call's tensor arguments, before
    anything is enqueued (the C gate sees only pointers and shapes, so it
    cannot tell a host tensor, a strided view or a short buffer).  Every torch
    tensor must be a contiguous GPU tensor, all on one device, and hold at
    least the bytes its shape argument describes.  When the element type comes
    from the input tensor (dtype None), the filter must have the input's type,
    the output the type page 1 pairs with it, and a source the output's shape
    and type; an explicit dtype code marks the tensors as raw byte buffers.
    scale / bias must be float32 with at least C_out values.  Raw integer
    pointers pass unchecked."""
    _check_tensors(dict(input=input, filter=filter, output=output, source=source,
                        scale=scale, bias=bias, workspace=workspace))
    if dtype is None and isinstance(input, torch.Tensor):
        if input.dtype not in DTYPE_CODES:
            raise InvalidArgument(f"input dtype {input.dtype} is not bf16, fp16 or fp8 e4m3fn")
        if isinstance(filter, torch.Tensor) and not nk and filter.dtype != input.dtype:
            raise InvalidArgument(f"filter dtype {filter.dtype} differs from input {input.dtype}")
        if isinstance(output, torch.Tensor) and output.dtype != OUT_DTYPES[input.dtype]:
            raise InvalidArgument(f"output dtype must be {OUT_DTYPES[input.dtype]} for "
                                  f"{input.dtype} inputs (got {output.dtype})")
        if isinstance(source, torch.Tensor) and isinstance(output, torch.Tensor) and (
                source.shape != output.shape or source.dtype != output.dtype):
            raise InvalidArgument(f"source must have the output's shape and dtype "
                                  f"({tuple(output.shape)}, {output.dtype}); got "
                                  f"({tuple(source.shape)}, {source.dtype})")
    code = dtype if dtype is not None else (
        dtype_code(input.dtype) if isinstance(input, torch.Tensor) else None)
    if code not in (0, 1, 2):
        return   # the C gate declines the element type
    eb = 1 if code == 2 else 2
    if any(int(v) < 0 for v in (*in_shape, *filt_shape, *out_shape)):
        return   # the C gate declines negative dims
    if isinstance(input, torch.Tensor) and _nbytes(input) < _prod(in_shape) * eb:
        raise InvalidArgument(f"input holds {_nbytes(input)} bytes, the shape "
                              f"{tuple(in_shape)} needs {_prod(in_shape) * eb}")
    if isinstance(filter, torch.Tensor):
        need = (conv2d_workspace_bytes(filt_shape, filter_is_fcrs, code) if nk
                else _prod(filt_shape) * eb)
        if _nbytes(filter) < need:
            raise InvalidArgument(f"{'NK matrix' if nk else 'filter'} holds "
                                  f"{_nbytes(filter)} bytes, needs {need}")
    out_need = _prod(out_shape) * 2
    for name, t in (("output", output), ("source", source)):
        if isinstance(t, torch.Tensor) and _nbytes(t) < out_need:
            raise InvalidArgument(f"{name} holds {_nbytes(t)} bytes, the output shape "
                                  f"{tuple(out_shape)} needs {out_need}")
    c_out = int(out_shape[3]) if len(out_shape) == 4 else None
    for name, t in (("scale", scale), ("bias", bias)):
        if isinstance(t, torch.Tensor):
            if t.dtype != torch.float32:
                raise InvalidArgument(f"{name} must be float32 (got {t.dtype})")
            if c_out is not None and t.numel() < c_out:
                raise InvalidArgument(f"{name} holds {t.numel()} values, C_out is {c_out}")
    if isinstance(workspace, torch.Tensor) and _nbytes(workspace) < int(workspace_bytes):
        raise InvalidArgument(f"workspace holds {_nbytes(workspace)} bytes, "
                              f"workspace_bytes says {workspace_bytes}")


def _i64(vals):
    return (ctypes.c_int64 * 4)(*[int(v) for v in vals])


def _pair(v):
    if isinstance(v, int):
        v = (v, v)
    return (ctypes.c_int32 * 2)(int(v[0]), int(v[1]))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, ref):
    if stream is None:
        if isinstance(ref, torch.Tensor) and ref.is_cuda:
            return torch.cuda.current_stream(ref.device).cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dtype):
    if dtype not in DTYPE_CODES:
        return -1
    return DTYPE_CODES[dtype]


def _conv_head(input, filter, filter_is_fcrs, output, stride, dilation, padding, groups,
               dtype, source, beta, in_shape=None, filt_shape=None, out_shape=None, *,
               launch=False, nk=False, scale=None, bias=None, workspace=None,
               workspace_bytes=0):
    """The common leading arguments of the forward entry points; for a call
    that enqueues work (launch=True) the tensors are checked first
    (_check_fwd)."""
    in_shape = input.shape if in_shape is None else in_shape
    filt_shape = filter.shape if filt_shape is None else filt_shape
    out_shape = output.shape if out_shape is None else out_shape
    if launch:
        _check_fwd(input, filter, output, source, dtype, in_shape, filt_shape, out_shape,
                   filter_is_fcrs, scale=scale, bias=bias, workspace=workspace,
                   workspace_bytes=workspace_bytes, nk=nk)
    if dtype is None:
        dtype = dtype_code(input.dtype)
    return [_ptr(input), _i64(in_shape), _ptr(filter), int(bool(filter_is_fcrs)),
            _i64(filt_shape), _ptr(output), _i64(out_shape), _pair(stride), _pair(dilation),
            _pair(padding), int(groups), int(dtype), _ptr(source), float(beta)]


def conv2d_abi_version() -> int:
    return lib().conv2d_abi_version()


def conv2d_reason_string(code: int) -> str:
    return lib().conv2d_reason_string(int(code)).decode()


def conv2d_fwd_check(input, filter, output, *, filter_is_fcrs, stride=1, padding=0,
                     dilation=1, groups=1, source=None, beta=0.0, workspace=None,
                     workspace_bytes=0, dtype=None, in_shape=None, filt_shape=None,
                     out_shape=None) -> int:
    """Host-only gate: 0 or a decline reason code.  Tensors or raw ints."""
    head = _conv_head(input, filter, filter_is_fcrs, output, stride, dilation, padding,
                      groups, dtype, source, beta, in_shape, filt_shape, out_shape)
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return lib().conv2d_fwd_check(*head, _ptr(workspace), int(workspace_bytes))


def conv2d_fwd_kernel_name(in_shape, filt_shape, out_shape, *, filter_is_fcrs, dtype,
                           stride=1, padding=0, dilation=1, groups=1):
    """Name of the GEMM kernel the library would launch for these shapes
    ("none" when the output is empty), or None when the call would be
    declined.  Host-only; dtype is a torch dtype or a dtype code."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    name = lib().conv2d_fwd_kernel_name(_i64(in_shape), int(bool(filter_is_fcrs)),
                                        _i64(filt_shape), _i64(out_shape), _pair(stride),
                                        _pair(dilation), _pair(padding), int(groups),
                                        int(code))
    return None if name is None else name.decode()


def conv2d_fwd_filter_in_kernel(in_shape, filt_shape, out_shape, *, filter_is_fcrs, dtype,
                                stride=1, padding=0, dilation=1, groups=1) -> bool:
    """Whether conv2d_fwd runs these shapes as one kernel launch that
    transposes the stored filter itself (no NK matrix, workspace untouched).
    Host-only."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return bool(lib().conv2d_fwd_filter_in_kernel(_i64(in_shape), int(bool(filter_is_fcrs)),
                                                  _i64(filt_shape), _i64(out_shape),
                                                  _pair(stride), _pair(dilation),
                                                  _pair(padding), int(groups), int(code)))


def conv2d_fwd(input, filter, output, *, filter_is_fcrs, stride=1, padding=0, dilation=1,
               groups=1, source=None, beta=0.0, workspace=None, workspace_bytes=0,
               stream=None, dtype=None, in_shape=None, filt_shape=None,
               out_shape=None) -> int:
    """Enqueue the forward convolution.  1 handled, 0 declined, < 0 HIP error."""
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    head = _conv_head(input, filter, filter_is_fcrs, output, stride, dilation, padding,
                      groups, dtype, source, beta, in_shape, filt_shape, out_shape,
                      launch=True, workspace=workspace, workspace_bytes=workspace_bytes)
    return lib().conv2d_fwd(*head, _ptr(workspace), int(workspace_bytes),
                            _stream(stream, output))


NOALLOC_SCRATCH_BYTES = 8 << 20   # IGC_NOALLOC_SCRATCH_BYTES in include/igemm_conv.h


def conv2d_fwd_noalloc(input, filter, output, *, filter_is_fcrs, stride=1, padding=0,
                       dilation=1, groups=1, source=None, beta=0.0, stream=None, dtype=None,
                       in_shape=None, filt_shape=None, out_shape=None) -> int:
    """conv2d_fwd with the NK matrix in the library's static device scratch
    (no allocation).  1 handled, 0 declined, < 0 HIP error."""
    head = _conv_head(input, filter, filter_is_fcrs, output, stride, dilation, padding,
                      groups, dtype, source, beta, in_shape, filt_shape, out_shape,
                      launch=True)
    return lib().conv2d_fwd_noalloc(*head, _stream(stream, output))


def conv2d_fwd_nk(input, nk, filt_shape, output, *, filter_is_fcrs, stride=1, padding=0,
                  dilation=1, groups=1, source=None, beta=0.0, stream=None, dtype=None,
                  in_shape=None, out_shape=None) -> int:
    """Enqueue the implicit-GEMM kernel on an NK matrix from conv2d_filter_to_nk."""
    head = _conv_head(input, nk, filter_is_fcrs, output, stride, dilation, padding, groups,
                      dtype, source, beta, in_shape=in_shape, filt_shape=filt_shape,
                      out_shape=out_shape, launch=True, nk=True)
    return lib().conv2d_fwd_nk(*head, _stream(stream, output))


def make_epilogue(scale=None, bias=None, activation=None):
    """An IgcEpilogue from tensors / raw pointers and an activation name or
    code, or None when nothing is fused."""
    if scale is None and bias is None and activation in (None, "none", 0):
        return None
    act = activation if isinstance(activation, int) else ACTIVATIONS.get(activation, -1)
    return IgcEpilogue(_ptr(scale), _ptr(bias), int(act))


def _epi_ref(epi):
    return None if epi is None else ctypes.byref(epi)


def conv2d_epilogue_check(output, *, scale=None, bias=None, activation=None,
                          out_shape=None) -> int:
    """Host-only check of a fused epilogue against the output: 0 or a code."""
    out_shape = output.shape if out_shape is None else out_shape
    return lib().conv2d_epilogue_check(_epi_ref(make_epilogue(scale, bias, activation)),
                                       _ptr(output), _i64(out_shape))


def conv2d_fwd_epilogue_check(input, filter, output, *, filter_is_fcrs, stride=1, padding=0,
                              dilation=1, groups=1, source=None, beta=0.0, scale=None,
                              bias=None, activation=None, workspace=None, workspace_bytes=0,
                              dtype=None, in_shape=None, filt_shape=None,
                              out_shape=None) -> int:
    """Host-only gate of conv2d_fwd_epilogue: 0 or a decline reason code."""
    head = _conv_head(input, filter, filter_is_fcrs, output, stride, dilation, padding,
                      groups, dtype, source, beta, in_shape, filt_shape, out_shape)
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    epi = make_epilogue(scale, bias, activation)
    return lib().conv2d_fwd_epilogue_check(*head, _epi_ref(epi), _ptr(workspace),
                                           int(workspace_bytes))


def conv2d_fwd_query(in_shape, filt_shape, out_shape, *, filter_is_fcrs, dtype, stride=1,
                     padding=0, dilation=1, groups=1) -> int:
    """Pointer-free gate of the problem's shapes and parameters: 0 or a
    decline reason code.  dtype is a torch dtype or a dtype code."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return lib().conv2d_fwd_query(_i64(in_shape), int(bool(filter_is_fcrs)), _i64(filt_shape),
                                  _i64(out_shape), _pair(stride), _pair(dilation),
                                  _pair(padding), int(groups), int(code))


def conv2d_fwd_epilogue(input, filter, output, *, filter_is_fcrs, stride=1, padding=0,
                        dilation=1, groups=1, source=None, beta=0.0, scale=None, bias=None,
                        activation=None, workspace=None, workspace_bytes=0, stream=None,
                        dtype=None, in_shape=None, filt_shape=None, out_shape=None) -> int:
    """conv2d_fwd with the fused per-channel epilogue
    act(scale[co] * conv + bias[co] + beta * source)."""
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    head = _conv_head(input, filter, filter_is_fcrs, output, stride, dilation, padding,
                      groups, dtype, source, beta, in_shape, filt_shape, out_shape,
                      launch=True, scale=scale, bias=bias, workspace=workspace,
                      workspace_bytes=workspace_bytes)
    epi = make_epilogue(scale, bias, activation)
    return lib().conv2d_fwd_epilogue(*head, _epi_ref(epi), _ptr(workspace),
                                     int(workspace_bytes), _stream(stream, output))


def conv2d_fwd_nk_epilogue(input, nk, filt_shape, output, *, filter_is_fcrs, stride=1,
                           padding=0, dilation=1, groups=1, source=None, beta=0.0,
                           scale=None, bias=None, activation=None, stream=None, dtype=None,
                           in_shape=None, out_shape=None) -> int:
    """conv2d_fwd_nk with the fused per-channel epilogue."""
    head = _conv_head(input, nk, filter_is_fcrs, output, stride, dilation, padding, groups,
                      dtype, source, beta, in_shape=in_shape, filt_shape=filt_shape,
                      out_shape=out_shape, launch=True, nk=True, scale=scale, bias=bias)
    epi = make_epilogue(scale, bias, activation)
    return lib().conv2d_fwd_nk_epilogue(*head, _epi_ref(epi), _stream(stream, output))


def conv2d_workspace_bytes(filt_shape, filter_is_fcrs, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib().conv2d_workspace_bytes(_i64(filt_shape), int(bool(filter_is_fcrs)), code))


def conv2d_nk_row_pitch(filt_shape, filter_is_fcrs, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib().conv2d_nk_row_pitch(_i64(filt_shape), int(bool(filter_is_fcrs)), code))


def conv2d_filter_to_nk(filter, nk, *, filter_is_fcrs, stream=None, dtype=None,
                        filt_shape=None, nk_bytes=None) -> int:
    """Enqueue the filter transpose into nk.  1 enqueued, 0 declined, < 0 error.
    Tensors must be contiguous GPU tensors on one device, nk holding at least
    nk_bytes."""
    _check_tensors(dict(filter=filter, nk=nk))
    filt_shape = filter.shape if filt_shape is None else filt_shape
    code = dtype_code(filter.dtype) if dtype is None else dtype
    if nk_bytes is None:
        nk_bytes = nk.numel() * nk.element_size()
    elif isinstance(nk, torch.Tensor) and _nbytes(nk) < int(nk_bytes):
        raise InvalidArgument(f"nk holds {_nbytes(nk)} bytes, nk_bytes says {nk_bytes}")
    if (isinstance(filter, torch.Tensor) and code in (0, 1, 2)
            and min(int(v) for v in filt_shape) >= 0
            and _nbytes(filter) < _prod(filt_shape) * (1 if code == 2 else 2)):
        raise InvalidArgument(f"filter holds {_nbytes(filter)} bytes, the shape "
                              f"{tuple(filt_shape)} needs more")
    return lib().conv2d_filter_to_nk(_ptr(filter), int(bool(filter_is_fcrs)),
                                     _i64(filt_shape), int(code), _ptr(nk), int(nk_bytes),
                                     _stream(stream, nk))


def _rs(r, s):
    return (ctypes.c_int64 * 2)(int(r), int(s))


def conv2d_im2col_bytes(in_shape, r, s, *, stride=1, padding=0, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib().conv2d_im2col_bytes(_i64(in_shape), _rs(r, s), _pair(stride),
                                         _pair(padding), int(code)))


def conv2d_im2col(input, r, s, a_out, *, stride=1, padding=0, stream=None, dtype=None,
                  in_shape=None, a_bytes=None) -> int:
    """Enqueue the materialised im2col of input into a_out (rows of Kp
    elements).  1 enqueued, 0 declined, < 0 HIP error.  Tensors must be
    contiguous GPU tensors on one device, a_out holding at least a_bytes."""
    _check_tensors(dict(input=input, a_out=a_out))
    in_shape = input.shape if in_shape is None else in_shape
    code = dtype_code(input.dtype) if dtype is None else dtype
    if a_bytes is None:
        a_bytes = a_out.numel() * a_out.element_size()
    elif isinstance(a_out, torch.Tensor) and _nbytes(a_out) < int(a_bytes):
        raise InvalidArgument(f"a_out holds {_nbytes(a_out)} bytes, a_bytes says {a_bytes}")
    if (isinstance(input, torch.Tensor) and code in (0, 1, 2)
            and min(int(v) for v in in_shape) >= 0
            and _nbytes(input) < _prod(in_shape) * (1 if code == 2 else 2)):
        raise InvalidArgument(f"input holds {_nbytes(input)} bytes, the shape "
                              f"{tuple(in_shape)} needs more")
    return lib().conv2d_im2col(_ptr(input), _i64(in_shape), _rs(r, s), _pair(stride),
                               _pair(padding), int(code), _ptr(a_out), int(a_bytes),
                               _stream(stream, a_out))


def im2col_row_elems(r, s, c, dtype) -> int:
    """Kp: K = R*S*C_in rounded up to a multiple of 128 bytes."""
    per = 128 // (1 if dtype == torch.float8_e4m3fn else 2)
    k = r * s * c
    return (k + per - 1) // per * per


def conv2d_materialized(input, filter, output, nk, a_buf, *, filter_is_fcrs, stride=1,
                        padding=0, source=None, beta=0.0, stream=None, transpose=True):
    """The write-then-GEMM route: filter -> NK (unless transpose=False and nk
    already holds it), input -> im2col matrix a_buf, then the 1x1 stride-1
    convolution of a_buf viewed as [N, Ho, Wo, Kp] with the same NK matrix.
    Returns the first nonzero-but-not-1 code, or 1."""
    if filter_is_fcrs:
        f, c, r, s = filter.shape
    else:
        r, s, c, f = filter.shape
    n, ho, wo, _ = output.shape
    kp = im2col_row_elems(r, s, c, input.dtype)
    if transpose:
        rc = conv2d_filter_to_nk(filter, nk, filter_is_fcrs=filter_is_fcrs, stream=stream)
        if rc != 1:
            return rc
    rc = conv2d_im2col(input, r, s, a_buf, stride=stride, padding=padding, stream=stream)
    if rc != 1:
        return rc
    return conv2d_fwd_nk(a_buf, nk, (f, kp, 1, 1), output, filter_is_fcrs=True, stride=1,
                         padding=0, source=source, beta=beta, stream=stream,
                         dtype=dtype_code(input.dtype), in_shape=(n, ho, wo, kp))


def conv2d_transposed_workspace_bytes(in_shape, filt_rsfc, *, stride=1, padding=0, dilation=1,
                                      dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib().conv2d_transposed_workspace_bytes(_i64(in_shape), _i64(filt_rsfc),
                                                       _pair(stride), _pair(dilation),
                                                       _pair(padding), code))


def _tr_head(input, filter, output, stride, dilation, padding, dtype, source, beta, scale,
             bias, activation, in_shape, filt_shape, out_shape, *, launch=False,
             workspace=None, workspace_bytes=0):
    in_shape = input.shape if in_shape is None else in_shape
    filt_shape = filter.shape if filt_shape is None else filt_shape
    out_shape = output.shape if out_shape is None else out_shape
    if launch:
        # the RSFC filter [R, S, F, C] holds as many elements as an RSCF one
        _check_fwd(input, filter, output, source, dtype, in_shape, filt_shape, out_shape,
                   False, scale=scale, bias=bias, workspace=workspace,
                   workspace_bytes=workspace_bytes)
    if dtype is None:
        dtype = dtype_code(input.dtype)
    return [_ptr(input), _i64(in_shape), _ptr(filter), _i64(filt_shape), _ptr(output),
            _i64(out_shape), _pair(stride), _pair(dilation), _pair(padding), int(dtype),
            _ptr(source), float(beta), _epi_ref(make_epilogue(scale, bias, activation))]


def conv2d_transposed_check(input, filter, output, *, stride=1, padding=0, dilation=1,
                            source=None, beta=0.0, scale=None, bias=None, activation=None,
                            workspace=None, workspace_bytes=0, dtype=None, in_shape=None,
                            filt_shape=None, out_shape=None) -> int:
    """Host-only gate of the transposed convolution: 0 or a decline code."""
    head = _tr_head(input, filter, output, stride, dilation, padding, dtype, source, beta,
                    scale, bias, activation, in_shape, filt_shape, out_shape)
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return lib().conv2d_transposed_check(*head, _ptr(workspace), int(workspace_bytes))


def conv2d_transposed_fwd(input, filter, output, *, stride=1, padding=0, dilation=1,
                          source=None, beta=0.0, scale=None, bias=None, activation=None,
                          workspace=None, workspace_bytes=0, stream=None, dtype=None,
                          in_shape=None, filt_shape=None, out_shape=None) -> int:
    """Enqueue the transposed convolution (RSFC filter).  1 handled, 0
    declined, < 0 HIP error."""
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    head = _tr_head(input, filter, output, stride, dilation, padding, dtype, source, beta,
                    scale, bias, activation, in_shape, filt_shape, out_shape, launch=True,
                    workspace=workspace, workspace_bytes=workspace_bytes)
    return lib().conv2d_transposed_fwd(*head, _ptr(workspace), int(workspace_bytes),
                                       _stream(stream, output))


def transposed_out_hw(h, w, r, s, *, stride=1, padding=0, dilation=1):
    """Ho, Wo of the transposed convolution: (H-1)*st - 2p + d*(R-1) + 1."""
    st, p, d = (_two(v) for v in (stride, padding, dilation))
    return ((h - 1) * st[0] - 2 * p[0] + d[0] * (r - 1) + 1,
            (w - 1) * st[1] - 2 * p[1] + d[1] * (s - 1) + 1)


def _two(v):
    return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))


def conv2d_transposed(input, filter, *, stride=1, padding=0, dilation=1, source=None,
                      beta=0.0, scale=None, bias=None, activation=None, stream=None):
    """Allocate the NHWC output and run conv2d_transposed_fwd into it
    (filter RSFC [R, S, F, C])."""
    r, s, f, _ = filter.shape
    n, h, w, _ = input.shape
    ho, wo = transposed_out_hw(h, w, r, s, stride=stride, padding=padding, dilation=dilation)
    out = torch.empty((n, ho, wo, f), dtype=OUT_DTYPES.get(input.dtype, input.dtype),
                      device=input.device)
    ws = torch.empty(max(conv2d_transposed_workspace_bytes(
        input.shape, filter.shape, stride=stride, padding=padding, dilation=dilation,
        dtype=input.dtype), 16), dtype=torch.uint8, device=input.device)
    kw = dict(stride=stride, padding=padding, dilation=dilation, source=source, beta=beta,
              scale=scale, bias=bias, activation=activation, workspace=ws)
    rc = conv2d_transposed_fwd(input, filter, out, stream=stream, **kw)
    if rc == 0:
        reason = conv2d_transposed_check(input, filter, out, **kw)
        raise Declined(f"conv2d_transposed_fwd declined: {REASONS.get(reason, reason)}")
    if rc < 0:
        raise RuntimeError(f"conv2d_transposed_fwd failed with HIP error {-rc}")
    return out


def out_hw(h, w, r, s, stride, padding):
    """Output size of the convolution (floor rounding)."""
    return (h + 2 * padding - r) // stride + 1, (w + 2 * padding - s) // stride + 1


def conv2d(input, filter, *, filter_is_fcrs, stride=1, padding=0, source=None, beta=0.0,
           scale=None, bias=None, activation=None, stream=None):
    """Allocate the NHWC output (torch memory) and run conv2d_fwd_epilogue
    into it (with no scale, bias or activation this is conv2d_fwd)."""
    if filter_is_fcrs:
        f, _, r, s = filter.shape
    else:
        r, s, _, f = filter.shape
    n, h, w, _ = input.shape
    ho, wo = out_hw(h, w, r, s, stride, padding)
    out = torch.empty((n, ho, wo, f), dtype=OUT_DTYPES.get(input.dtype, input.dtype),
                      device=input.device)
    ws_bytes = conv2d_workspace_bytes(filter.shape, filter_is_fcrs, input.dtype)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=input.device)
    rc = conv2d_fwd_epilogue(input, filter, out, filter_is_fcrs=filter_is_fcrs,
                             stride=stride, padding=padding, source=source, beta=beta,
                             scale=scale, bias=bias, activation=activation, workspace=ws,
                             stream=stream)
    if rc == 0:
        reason = conv2d_fwd_epilogue_check(input, filter, out, filter_is_fcrs=filter_is_fcrs,
                                           stride=stride, padding=padding, source=source,
                                           beta=beta, scale=scale, bias=bias,
                                           activation=activation, workspace=ws)
        raise Declined(f"conv2d_fwd declined: {REASONS.get(reason, reason)}")
    if rc < 0:
        raise RuntimeError(f"conv2d_fwd failed with HIP error {-rc}")
    return out


# ------------------------------------------------ general convolution
def conv_params(*, stride=1, dilation=1, pad_begin=0, pad_end=None, groups=1):
    """An IgcConvParams; each of stride, dilation, pad_begin (top, left) and
    pad_end (bottom, right; None = pad_begin) is an int or a pair."""
    def two(v):
        return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))
    pe = pad_begin if pad_end is None else pad_end
    return IgcConvParams((ctypes.c_int32 * 2)(*two(stride)), (ctypes.c_int32 * 2)(*two(dilation)),
                         (ctypes.c_int32 * 2)(*two(pad_begin)), (ctypes.c_int32 * 2)(*two(pe)),
                         int(groups))


def out_hw_general(h, w, r, s, params):
    """Ho, Wo of the general convolution (floor rounding; 0 when empty)."""
    def one(n, k, st, d, a, b):
        span = n + a + b - d * (k - 1) - 1
        return 0 if span < 0 else span // st + 1
    return (one(h, r, params.stride[0], params.dilation[0], params.pad_begin[0],
                params.pad_end[0]),
            one(w, s, params.stride[1], params.dilation[1], params.pad_begin[1],
                params.pad_end[1]))


def _gen_head(input, filter, filter_is_fcrs, output, params, dtype, source, beta, scale, bias,
              activation, in_shape, filt_shape, out_shape, *, launch=False, workspace=None,
              workspace_bytes=0):
    in_shape = input.shape if in_shape is None else in_shape
    filt_shape = filter.shape if filt_shape is None else filt_shape
    out_shape = output.shape if out_shape is None else out_shape
    if launch:
        _check_fwd(input, filter, output, source, dtype, in_shape, filt_shape, out_shape,
                   filter_is_fcrs, scale=scale, bias=bias, workspace=workspace,
                   workspace_bytes=workspace_bytes)
    if dtype is None:
        dtype = dtype_code(input.dtype)
    return [_ptr(input), _i64(in_shape), _ptr(filter), int(bool(filter_is_fcrs)),
            _i64(filt_shape), _ptr(output), _i64(out_shape), ctypes.byref(params), int(dtype),
            _ptr(source), float(beta), _epi_ref(make_epilogue(scale, bias, activation))]


def conv2d_fwd_general_query(in_shape, filt_shape, out_shape, params, *, filter_is_fcrs,
                             dtype) -> int:
    """Pointer-free gate of the general convolution: 0 or a decline code."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return lib().conv2d_fwd_general_query(_i64(in_shape), int(bool(filter_is_fcrs)),
                                          _i64(filt_shape), _i64(out_shape),
                                          ctypes.byref(params), int(code))


def conv2d_fwd_general_kernel_name(in_shape, filt_shape, out_shape, params, *, filter_is_fcrs,
                                   dtype):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    name = lib().conv2d_fwd_general_kernel_name(_i64(in_shape), int(bool(filter_is_fcrs)),
                                                _i64(filt_shape), _i64(out_shape),
                                                ctypes.byref(params), int(code))
    return None if name is None else name.decode()


def conv2d_fwd_general_workspace_bytes(in_shape, filt_shape, out_shape, params, *,
                                       filter_is_fcrs, dtype) -> int:
    """Workspace bytes conv2d_fwd_general needs for this problem (0 when
    declined)."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib().conv2d_fwd_general_workspace_bytes(
        _i64(in_shape), int(bool(filter_is_fcrs)), _i64(filt_shape), _i64(out_shape),
        ctypes.byref(params), int(code)))


def conv2d_fwd_general_check(input, filter, output, params, *, filter_is_fcrs, source=None,
                             beta=0.0, scale=None, bias=None, activation=None, workspace=None,
                             workspace_bytes=0, dtype=None, in_shape=None, filt_shape=None,
                             out_shape=None) -> int:
    """Host-only gate of conv2d_fwd_general: 0 or a decline code."""
    head = _gen_head(input, filter, filter_is_fcrs, output, params, dtype, source, beta, scale,
                     bias, activation, in_shape, filt_shape, out_shape)
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return lib().conv2d_fwd_general_check(*head, _ptr(workspace), int(workspace_bytes))


def conv2d_fwd_general(input, filter, output, params, *, filter_is_fcrs, source=None, beta=0.0,
                       scale=None, bias=None, activation=None, workspace=None,
                       workspace_bytes=0, stream=None, dtype=None, in_shape=None,
                       filt_shape=None, out_shape=None) -> int:
    """Enqueue the general forward convolution.  1 handled, 0 declined, < 0
    HIP error."""
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    head = _gen_head(input, filter, filter_is_fcrs, output, params, dtype, source, beta, scale,
                     bias, activation, in_shape, filt_shape, out_shape, launch=True,
                     workspace=workspace, workspace_bytes=workspace_bytes)
    return lib().conv2d_fwd_general(*head, _ptr(workspace), int(workspace_bytes),
                                    _stream(stream, output))


def conv2d_general(input, filter, *, filter_is_fcrs, stride=1, dilation=1, pad_begin=0,
                   pad_end=None, groups=1, source=None, beta=0.0, scale=None, bias=None,
                   activation=None, stream=None):
    """Allocate the NHWC output and run conv2d_fwd_general into it."""
    params = conv_params(stride=stride, dilation=dilation, pad_begin=pad_begin,
                         pad_end=pad_end, groups=groups)
    if filter_is_fcrs:
        f, _, r, s = filter.shape
    else:
        r, s, _, f = filter.shape
    n, h, w, _ = input.shape
    ho, wo = out_hw_general(h, w, r, s, params)
    out = torch.empty((n, ho, wo, f), dtype=OUT_DTYPES.get(input.dtype, input.dtype),
                      device=input.device)
    wsb = conv2d_fwd_general_workspace_bytes(input.shape, filter.shape, out.shape, params,
                                             filter_is_fcrs=filter_is_fcrs, dtype=input.dtype)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=input.device)
    kw = dict(filter_is_fcrs=filter_is_fcrs, source=source, beta=beta, scale=scale, bias=bias,
              activation=activation, workspace=ws)
    rc = conv2d_fwd_general(input, filter, out, params, stream=stream, **kw)
    if rc == 0:
        reason = conv2d_fwd_general_check(input, filter, out, params, **kw)
        raise Declined(f"conv2d_fwd_general declined: {REASONS.get(reason, reason)}")
    if rc < 0:
        raise RuntimeError(f"conv2d_fwd_general failed with HIP error {-rc}")
    return out

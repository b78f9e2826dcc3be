"""Seeded synthetic inputs for the forward NHWC convolution.

Shared by the tests, the benchmark and the smoke check.  This module holds no
convolution arithmetic: it only draws tensors of given shapes, dtypes and
distributions.  Output sizes (needed for the residual source) are given by
the caller or written into the workload table, never computed here.

Recipe (for every workload):
  * one CPU torch.Generator seeded with the seed (0 for the named workloads);
  * draws in the order input, filter, source, each as one float32 tensor in
    that tensor's stored layout (NHWC input, RSCF [R,S,C_in,C_out] or FCRS
    [C_out,C_in,R,S] filter, NHWC source);
  * uniform(a) is U[-a, a] (torch.rand * 2a - a); normal(sd) is N(0, sd^2)
    (torch.randn * sd);
  * float8_e4m3fn values are first clamped to [-448, 448] (torch's fp8 cast
    does not saturate: 464 rounds to 448 but 500 becomes NaN), then every
    tensor is rounded to its stored dtype by torch's round-to-nearest-even cast.
"""
import math

import torch

TORCH_DTYPES = {
    "bfloat16": torch.bfloat16,
    "float16": torch.float16,
    "float8_e4m3fn": torch.float8_e4m3fn,
}
# Output element type per input type (bf16 for fp8 inputs, else the input type).
OUT_DTYPES = {
    "bfloat16": torch.bfloat16,
    "float16": torch.float16,
    "float8_e4m3fn": torch.bfloat16,
}
FP8_MAX = 448.0

# The five named workloads.  Sizes, layouts and distributions as specified;
# "normal" takes the standard deviation.  out_hw is the stated output size.
WORKLOADS = {
    "tiny_3x3_16c": dict(
        N=1, H=16, W=16, C=16, F=16, R=3, S=3, stride=1, pad=1, out_hw=(16, 16),
        dtype="bfloat16", fcrs=False, x=("uniform", 1.0), w=("uniform", 1.0),
        src=None, beta=0.0),
    "resnet_3x3_64c_n32": dict(
        N=32, H=56, W=56, C=64, F=64, R=3, S=3, stride=1, pad=1, out_hw=(56, 56),
        dtype="bfloat16", fcrs=True, x=("normal", 1.0),
        w=("normal", 1.0 / math.sqrt(576.0)), src=None, beta=0.0),
    "strided_3x3_s2_128to256_n32": dict(
        N=32, H=56, W=56, C=128, F=256, R=3, S=3, stride=2, pad=1, out_hw=(28, 28),
        dtype="float16", fcrs=False, x=("uniform", 1.0), w=("uniform", 1.0),
        src=None, beta=0.0),
    "fp8_5x5_256c_residual_n16": dict(
        N=16, H=64, W=64, C=256, F=256, R=5, S=5, stride=1, pad=2, out_hw=(64, 64),
        dtype="float8_e4m3fn", fcrs=False, x=("normal", 1.0), w=("normal", 1.0),
        src=("normal", 1.0), beta=0.5),
    "rgb_3x3_128to3_512px": dict(
        N=1, H=512, W=512, C=128, F=3, R=3, S=3, stride=1, pad=1, out_hw=(512, 512),
        dtype="bfloat16", fcrs=False, x=("normal", 1.0),
        w=("normal", 1.0 / math.sqrt(1152.0)), src=None, beta=0.0),
}
WORKLOAD_ORDER = list(WORKLOADS)


def _draw(gen, shape, dist):
    kind, a = dist
    if kind == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * (2.0 * a) - a
    if kind == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * a
    raise ValueError(f"unknown distribution {kind}")


def _round(t32, dtype_name, out=False):
    table = OUT_DTYPES if out else TORCH_DTYPES
    if table[dtype_name] == torch.float8_e4m3fn:
        t32 = t32.clamp(-FP8_MAX, FP8_MAX)
    return t32.to(table[dtype_name])


def filter_shape(R, S, C, F, fcrs):
    return (F, C, R, S) if fcrs else (R, S, C, F)


def make_case(*, N, H, W, C, F, R, S, dtype, fcrs, x_dist, w_dist,
              src_dist=None, out_hw=None, seed=0, filt_c=None):
    """Draws (x, w, src) as CPU tensors in their stored dtypes.  src is None
    unless src_dist is given, in which case out_hw = (Ho, Wo) is required.
    filt_c: the filter's input channels when they differ from the input's
    (a grouped convolution's per-group count)."""
    gen = torch.Generator().manual_seed(seed)
    x = _round(_draw(gen, (N, H, W, C), x_dist), dtype)
    w = _round(_draw(gen, filter_shape(R, S, C if filt_c is None else filt_c, F, fcrs), w_dist),
               dtype)
    src = None
    if src_dist is not None:
        ho, wo = out_hw
        src = _round(_draw(gen, (N, ho, wo, F), src_dist), dtype, out=True)
    return x, w, src


def make_workload(name, *, seed=0, fcrs=None):
    """(spec, x, w, src) for a named workload.  fcrs overrides the filter
    layout (the same seed then draws the filter in the other layout)."""
    spec = dict(WORKLOADS[name])
    if fcrs is not None:
        spec["fcrs"] = bool(fcrs)
    x, w, src = make_case(
        N=spec["N"], H=spec["H"], W=spec["W"], C=spec["C"], F=spec["F"],
        R=spec["R"], S=spec["S"], dtype=spec["dtype"], fcrs=spec["fcrs"],
        x_dist=spec["x"], w_dist=spec["w"], src_dist=spec["src"],
        out_hw=spec["out_hw"], seed=seed)
    return spec, x, w, src

"""Oracle for the forward NHWC convolution (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library and never
imports it.  Every function cites the page passage it follows; the pages are
three API documentation pages of Modular's kernel library:

  page 1  "dispatch_amd_4wave_conv2d"          (MI355X dispatcher)
  page 2  "dispatch_fused_im2col_conv2d_apple" (Apple fused online-im2col conv)
  page 3  "conv_transposed_gpu"                (cuDNN transposed conv)

Parity status of each function (what pins it is in tests/test_oracle_pins.py):
  conv2d, conv2d_points  pinned: brute force, hand-worked example, 1x1 matmul
                          closed form, delta filters, border counts,
                          stride subsampling, layout and bilinearity
                          invariants, residual identities.
  conv2d_epilogue(_points) pinned: hand-worked golden values
  activation              (tests/golden/epilogue_cases.txt), reduction to
                          conv2d with no epilogue, bias as an extra
                          constant-one input channel, scale folded into the
                          filter, textbook sigmoid values, relu's sign split.
  conv2d_general         pinned: hand-worked golden values
                          (tests/golden/general_cases.txt), pure-Python
                          brute force with dilation, groups, per-axis
                          strides and asymmetric padding, torch conv2d in
                          fp64, reduction to conv2d, groups as the
                          concatenation of per-group convolutions,
                          dilation as a zero-inserted filter, asymmetric
                          padding as an explicitly padded input, stride as
                          subsampling of stride 1.
  filter_to_nk           pinned: element-wise brute force from the index
                          formula on small filters.
  conv2d_transposed      pinned: hand-worked golden values
                          (tests/golden/transposed_cases.txt), pure-Python
                          brute force with strides, dilations and padding,
                          the adjoint identity <conv2d(a, W), b> =
                          <a, conv2d_transposed(b, W)> against conv2d.
  im2col                 pinned: pure-Python brute force on tiny shapes,
                          im2col(x) @ filter_to_nk(w)^T equals conv2d,
                          zero columns past K.
  gate_accepts           pinned: hand-written case table from page 1's
                          Parameters/Args rules (tests/golden/gate_cases.txt).
"""
from .reference import (  # noqa: F401
    ACTIVATIONS,
    DTYPES,
    activation,
    conv2d,
    conv2d_epilogue,
    conv2d_epilogue_points,
    conv2d_general,
    conv2d_points,
    conv2d_transposed,
    filter_dims_rscf,
    filter_to_nk,
    gate_accepts,
    im2col,
    num_threads,
    out_size,
    out_size_general,
)

"""The seeded input generators are deterministic and draw the stated
distributions (CPU only)."""
import math

import torch

import datagen


def test_same_seed_same_bytes():
    a = datagen.make_workload("tiny_3x3_16c")
    b = datagen.make_workload("tiny_3x3_16c")
    for t1, t2 in zip(a[1:3], b[1:3]):
        assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))
    c = datagen.make_workload("tiny_3x3_16c", seed=1)
    assert not torch.equal(a[1].view(torch.int16), c[1].view(torch.int16))


def test_workload_shapes_and_dtypes():
    spec, x, w, src = datagen.make_workload("tiny_3x3_16c")
    assert x.shape == (1, 16, 16, 16) and x.dtype == torch.bfloat16
    assert w.shape == (3, 3, 16, 16) and src is None
    assert float(x.float().abs().max()) <= 1.0
    spec = datagen.WORKLOADS["fp8_5x5_256c_residual_n16"]
    x, w, src = datagen.make_case(N=2, H=8, W=8, C=32, F=16, R=5, S=5,
                                  dtype=spec["dtype"], fcrs=False, x_dist=spec["x"],
                                  w_dist=spec["w"], src_dist=spec["src"], out_hw=(8, 8))
    assert x.dtype == torch.float8_e4m3fn and src.dtype == torch.bfloat16
    assert src.shape == (2, 8, 8, 16)


def test_fp8_clamp_keeps_values_finite():
    x, w, _ = datagen.make_case(N=1, H=4, W=4, C=16, F=16, R=1, S=1,
                                dtype="float8_e4m3fn", fcrs=False,
                                x_dist=("normal", 1000.0), w_dist=("normal", 1.0))
    xf = x.to(torch.float32)
    assert torch.isfinite(xf).all() and float(xf.abs().max()) == 448.0


def test_distribution_moments():
    x, w, _ = datagen.make_case(N=4, H=32, W=32, C=64, F=64, R=3, S=3,
                                dtype="bfloat16", fcrs=True, x_dist=("normal", 1.0),
                                w_dist=("normal", 1 / 24))
    assert abs(float(x.float().std()) - 1.0) < 0.02
    assert abs(float(w.float().std()) * 24 - 1.0) < 0.05
    x, _, _ = datagen.make_case(N=4, H=32, W=32, C=64, F=8, R=1, S=1, dtype="float16",
                                fcrs=False, x_dist=("uniform", 1.0), w_dist=("uniform", 1.0))
    assert abs(float(x.float().std()) - 1 / math.sqrt(3)) < 0.01

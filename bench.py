"""Benchmark: forward NHWC convolution as an implicit GEMM on one MI355X.

One step = the whole path on one batch: one conv2d_fwd call, i.e. the filter
transpose to NK and the implicit-GEMM kernel with its fused epilogue, or, on
the band kernel, the one kernel that transposes the stored filter into its
LDS itself (conv2d_fwd_filter_in_kernel tells which).  Each buffer set's step
is captured in HIP graphs of up to 25 steps (replays checked bit for bit
against the eager steps), and the timed loop replays them, so host-side
launch overhead does not pace the GPU.

Headline workload: the ResNet-style 3x3 body conv (N=32, 56x56, 64->64,
stride 1, padding 1, bf16, FCRS filter).  value = 2*N*Ho*Wo*C_out*R*S*C_in /
step time, in TFLOP/s.  Inputs are resident in HBM: each step uses the next
of several identical buffer sets whose total size (>= 640 MB, at most 64
sets) exceeds the 256 MB Infinity Cache and the L2s, so no step finds its
operands in cache.

Also reported on the same line:
  roofline      the GEMM kernel's (on the band kernel: the whole call's one
                kernel's) algorithmic bytes (or FLOPs) per launch over
                its mean duration from HIP events around back-to-back launches
                (queued behind a spin kernel), against the MI355X peak;
  cpu_baseline  the fp64 oracle timed on this host's cores on the same
                workload (the full batch);
  shapes        the same measurement for each of the five named workloads;
  launch_floor_us  an empty kernel's time per launch, back to back (the
                floor under the tiny layer's kernel time);
  next          the fused per-channel epilogue's cost on the headline layer,
                the materialised im2col + GEMM route against the fused
                kernel on the two memory-bound layers, transposed
                convolutions (whole calls), and layers outside page 1's gate
                through conv2d_fwd_general (whole calls).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HEADLINE = "resnet_3x3_64c_n32"
PEAK = {"bf16_tflops": 2516.6, "fp16_tflops": 2516.6, "fp8_tflops": 5033.2,
        "hbm_gbs": 8000.0}
RIDGE_BF16 = PEAK["bf16_tflops"] * 1e12 / (PEAK["hbm_gbs"] * 1e9)
ROTATE_BYTES = 640 << 20   # default; --rotate-mib 0 = one set (warm caches, labelled)
MAX_SETS = 64
MAX_STEPS_PER_GRAPH = 25   # steps captured in one HIP graph at most


def steps_per_graph(steps):
    """The largest divisor of `steps` up to MAX_STEPS_PER_GRAPH: the timed
    steps split into whole graphs.  Each graph replay costs a few us of host
    and queue work of its own (measured on the ResNet layer: 21.2 us per step
    one step per graph, 17.0 at five, 15.7 at ten, 15.6 at fifty, against a
    15.3 us kernel), so longer graphs keep it off the per-step figure."""
    for d in range(min(MAX_STEPS_PER_GRAPH, max(steps, 1)), 0, -1):
        if steps % d == 0:
            return d
    return 1
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "igemm_fwd_resnet_3x3_64c_n32_traffic.txt")


def _source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "implicit_gemm_nhwc_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()


def _algorithmic(spec):
    """FLOPs and bytes (input + filter + source + output, each once)."""
    n, h, w, c, f, r, s = (spec[k] for k in ("N", "H", "W", "C", "F", "R", "S"))
    ho, wo = spec["out_hw"]
    eb = 1 if spec["dtype"] == "float8_e4m3fn" else 2
    flops = 2 * n * ho * wo * f * r * s * c
    nbytes = n * h * w * c * eb + r * s * c * f * eb + n * ho * wo * f * 2
    if spec["src"] is not None:
        nbytes += n * ho * wo * f * 2
    return flops, nbytes


def _bound(spec, flops, nbytes):
    peak_t = PEAK["fp8_tflops"] if spec["dtype"] == "float8_e4m3fn" else PEAK["bf16_tflops"]
    ridge = peak_t * 1e12 / (PEAK["hbm_gbs"] * 1e9)
    return ("mfma" if flops / nbytes >= ridge else "hbm"), peak_t


class Bufsets:
    """Identical copies of one workload's tensors, rotated across steps."""

    def __init__(self, torch, igc, spec, x, w, src, rotate_bytes=ROTATE_BYTES):
        dev = torch.device("cuda:0")
        self.spec = spec
        self.fcrs = spec["fcrs"]
        n, f = spec["N"], spec["F"]
        ho, wo = spec["out_hw"]
        out_dt = {"bfloat16": torch.bfloat16, "float16": torch.float16,
                  "float8_e4m3fn": torch.bfloat16}[spec["dtype"]]
        nk_bytes = igc.conv2d_workspace_bytes(w.shape, self.fcrs, w.dtype)
        per_set = (x.numel() * x.element_size() + w.numel() * w.element_size() +
                   nk_bytes + n * ho * wo * f * 2 * (2 if src is not None else 1))
        # enough sets to cover rotate_bytes, at most MAX_SETS (tiny layers
        # fit in the caches whatever the count)
        self.nsets = min(MAX_SETS, max(1, -(-rotate_bytes // per_set)))
        xd, wd = x.to(dev), w.to(dev)
        sd = None if src is None else src.to(dev)
        self.sets = []
        for _ in range(self.nsets):
            self.sets.append(dict(
                x=xd.clone(), w=wd.clone(),
                nk=torch.empty(max(nk_bytes, 16), dtype=torch.uint8, device=dev),
                y=torch.empty((n, ho, wo, f), dtype=out_dt, device=dev),
                src=None if sd is None else sd.clone()))
        # whether conv2d_fwd is one kernel that transposes the filter itself
        # (the band kernel) or a transpose launch followed by the GEMM kernel
        self.fused = igc.conv2d_fwd_filter_in_kernel(
            x.shape, w.shape, (n, ho, wo, f), filter_is_fcrs=self.fcrs, dtype=w.dtype,
            stride=spec["stride"], padding=spec["pad"])
        # every set's NK matrix, made once, for the rows that run on a given
        # NK matrix (conv2d_fwd_nk; the fused path leaves it untouched)
        for i in range(self.nsets):
            self.transpose(igc, i)
        torch.cuda.synchronize()

    def step(self, igc, i):
        """One step on set i: the whole conv2d_fwd call (the filter transpose
        into the set's workspace and the GEMM kernel, or the one kernel that
        transposes the filter itself)."""
        b = self.sets[i % self.nsets]
        sp = self.spec
        rc = igc.conv2d_fwd(b["x"], b["w"], b["y"], filter_is_fcrs=self.fcrs,
                            stride=sp["stride"], padding=sp["pad"], source=b["src"],
                            beta=sp["beta"], workspace=b["nk"])
        if rc != 1:
            raise RuntimeError(f"conv2d_fwd returned {rc}")

    def transpose(self, igc, i):
        """The filter transpose of set i into its NK matrix."""
        b = self.sets[i % self.nsets]
        rc = igc.conv2d_filter_to_nk(b["w"], b["nk"], filter_is_fcrs=self.fcrs)
        if rc != 1:
            raise RuntimeError(f"conv2d_filter_to_nk returned {rc}")

    def fwd_only(self, igc, i):
        """The GEMM kernel alone on set i: conv2d_fwd when that is one kernel,
        else conv2d_fwd_nk on the set's NK matrix."""
        if self.fused:
            self.step(igc, i)
            return
        b = self.sets[i % self.nsets]
        sp = self.spec
        rc = igc.conv2d_fwd_nk(b["x"], b["nk"], b["w"].shape, b["y"], filter_is_fcrs=self.fcrs,
                               stride=sp["stride"], padding=sp["pad"], source=b["src"],
                               beta=sp["beta"])
        if rc != 1:
            raise RuntimeError(f"conv2d_fwd_nk returned {rc}")

    def capture(self, torch, igc, per_graph):
        """HIP graphs of `per_graph` consecutive steps each (graph g runs the
        steps on sets g*per_graph + u, u < per_graph, modulo the set count),
        so the timed loop is not paced by host-side launch overhead.  Every
        replay is checked bit for bit against the eager steps' outputs, with
        eager work and synchronizations between the replays."""
        self.per_graph = per_graph
        ngraphs = -(-self.nsets // per_graph)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(self.nsets):
                self.step(igc, i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = []
        for i in range(self.nsets):
            self.step(igc, i)
            torch.cuda.synchronize()
            ref.append(self.sets[i]["y"].clone())
        self.graphs = []
        for g in range(ngraphs):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for u in range(per_graph):
                    self.step(igc, g * per_graph + u)
            self.graphs.append(graph)
        torch.cuda.synchronize()
        for rep in range(2):
            for g in range(ngraphs):
                sets = sorted({(g * per_graph + u) % self.nsets for u in range(per_graph)})
                for i in sets:
                    self.sets[i]["y"].zero_()
                torch.cuda.synchronize()
                self.graphs[g].replay()
                torch.cuda.synchronize()
                for i in sets:
                    if not torch.equal(self.sets[i]["y"].view(torch.int16),
                                       ref[i].view(torch.int16)):
                        raise RuntimeError(f"graph {g} replay {rep}: set {i} differs from "
                                           "the eager step")
                self.step(igc, g)   # eager work between replays
                torch.cuda.synchronize()

    def replay(self, r):
        """Replay r runs steps r*per_graph .. r*per_graph + per_graph - 1."""
        self.graphs[r % len(self.graphs)].replay()


def kernel_times(torch, igc, bufs, launches):
    """Mean duration of the GEMM kernel (Bufsets.fwd_only: conv2d_fwd_nk, or
    conv2d_fwd when that is the one kernel) from HIP events on the launch
    stream around `launches` back-to-back launches (rotating sets).  A spin kernel
    holds the stream while the host enqueues them, so the GPU never waits on
    the host inside the bracket (host-side launch latency would otherwise
    count as kernel time); no event sits between the launches."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * (0.002 + 60e-6 * launches)))   # ~2 ms + 60 us per launch
    e0.record(stream)
    for i in range(launches):
        bufs.fwd_only(igc, i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / launches


def event_time(torch, fn, launches):
    """Mean duration of fn(i) (launches on the current stream) from HIP events
    around `launches` back-to-back calls, queued behind a spin kernel as in
    kernel_times."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * (0.002 + 80e-6 * launches)))
    e0.record(stream)
    for i in range(launches):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / launches * 1e3   # us


def _ok(rc, what):
    if rc != 1:
        raise RuntimeError(f"{what} returned {rc}")


def measure_next(torch, igc, launches, rotate_bytes=ROTATE_BYTES):
    """The rows past the core path, on cold rotating buffer sets:
      epilogue  the headline layer's GEMM kernel with the fused per-channel
                scale, bias and ReLU, against the same kernel without them;
      im2col    the write-then-GEMM route on the two memory-bound layers: the
                im2col kernel, the GEMM on the materialised matrix (a 1x1
                convolution), and both back to back, against the fused kernel.
    Times in us from HIP events around back-to-back launches."""
    import datagen

    out = {}
    spec, x, w, src = datagen.make_workload(HEADLINE)
    bufs = Bufsets(torch, igc, spec, x, w, src, rotate_bytes)
    for i in range(bufs.nsets):
        bufs.step(igc, i)
    f = spec["F"]
    g = torch.Generator().manual_seed(0)
    scale = (torch.rand(f, generator=g) + 0.5).to("cuda:0")
    bias = torch.randn(f, generator=g).to("cuda:0")

    def epi(i):
        b = bufs.sets[i % bufs.nsets]
        if bufs.fused:   # the same one kernel as the plain call, with the epilogue
            _ok(igc.conv2d_fwd_epilogue(b["x"], b["w"], b["y"], filter_is_fcrs=bufs.fcrs,
                                        stride=spec["stride"], padding=spec["pad"],
                                        scale=scale, bias=bias, activation="relu",
                                        workspace=b["nk"]), "conv2d_fwd_epilogue")
            return
        _ok(igc.conv2d_fwd_nk_epilogue(b["x"], b["nk"], b["w"].shape, b["y"],
                                       filter_is_fcrs=bufs.fcrs, stride=spec["stride"],
                                       padding=spec["pad"], scale=scale, bias=bias,
                                       activation="relu"), "conv2d_fwd_nk_epilogue")
    for i in range(3):
        epi(i)
    plain = kernel_times(torch, igc, bufs, launches) * 1e3
    fused = event_time(torch, epi, launches)
    out["epilogue"] = {"workload": HEADLINE, "fused": "scale, bias, relu",
                       "kernel_us": round(fused, 3), "plain_kernel_us": round(plain, 3),
                       "extra_us": round(fused - plain, 3)}
    del bufs
    torch.cuda.empty_cache()

    abl = {}
    for name in ("resnet_3x3_64c_n32", "rgb_3x3_128to3_512px"):
        spec, x, w, src = datagen.make_workload(name)
        bufs = Bufsets(torch, igc, spec, x, w, src, rotate_bytes)
        for i in range(bufs.nsets):
            bufs.step(igc, i)
        r, s_, c = spec["R"], spec["S"], spec["C"]
        kp = igc.im2col_row_elems(r, s_, c, x.dtype)
        nbytes = igc.conv2d_im2col_bytes(x.shape, r, s_, stride=spec["stride"],
                                         padding=spec["pad"], dtype=x.dtype)
        a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        n, (ho, wo) = spec["N"], spec["out_hw"]

        def im2col(i):
            b = bufs.sets[i % bufs.nsets]
            _ok(igc.conv2d_im2col(b["x"], r, s_, a, stride=spec["stride"],
                                  padding=spec["pad"]), "conv2d_im2col")

        def gemm(i):
            b = bufs.sets[i % bufs.nsets]
            _ok(igc.conv2d_fwd_nk(a, b["nk"], (spec["F"], kp, 1, 1), b["y"],
                                  filter_is_fcrs=True, stride=1, padding=0, source=b["src"],
                                  beta=spec["beta"], dtype=igc.dtype_code(x.dtype),
                                  in_shape=(n, ho, wo, kp)), "conv2d_fwd_nk (1x1 view)")

        def route(i):
            im2col(i)
            gemm(i)
        route(0)
        torch.cuda.synchronize()
        fused = kernel_times(torch, igc, bufs, launches) * 1e3
        t_i = event_time(torch, im2col, launches)
        t_g = event_time(torch, gemm, launches)
        t_r = event_time(torch, route, launches)
        in_bytes = x.numel() * x.element_size()
        abl[name] = {"fused_kernel_us": round(fused, 3), "im2col_us": round(t_i, 3),
                     "gemm_on_matrix_us": round(t_g, 3), "route_us": round(t_r, 3),
                     "route_over_fused": round(t_r / fused, 3),
                     "matrix_bytes": nbytes,
                     "im2col_gbs": round((nbytes + in_bytes) / (t_i * 1e-6) / 1e9, 1),
                     "gemm_kernel": igc.conv2d_fwd_kernel_name(
                         (n, ho, wo, kp), (spec["F"], kp, 1, 1), (n, ho, wo, spec["F"]),
                         filter_is_fcrs=True, dtype=x.dtype, stride=1, padding=0)}
        del bufs, a
        torch.cuda.empty_cache()
    out["im2col_ablation"] = abl

    # transposed convolutions: a decoder-style 3x3 stride-1 layer and the 4x4
    # stride-2 2x upsampler, each call timed whole (the phases' filter flips
    # and GEMMs) over rotating buffer sets
    out["transposed"] = {}
    for tag, (n, h, w, c, f, r, st, p) in {
            "3x3_s1": (8, 64, 64, 256, 128, 3, 1, 1),
            "4x4_s2_upsample": (8, 32, 32, 256, 128, 4, 2, 1)}.items():
        x, wf, _ = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=r, dtype="bfloat16",
                                     fcrs=False, x_dist=("normal", 1.0),
                                     w_dist=("normal", 1.0 / (r * r * c) ** 0.5), seed=0)
        wt = wf.permute(0, 1, 3, 2).contiguous()          # RSFC [R, S, F, C]
        ho, wo = (h - 1) * st - 2 * p + r, (w - 1) * st - 2 * p + r
        per = x.numel() * 2 + n * ho * wo * f * 2
        nsets = min(MAX_SETS, max(1, -(-rotate_bytes // per)))
        wsb = igc.conv2d_transposed_workspace_bytes(x.shape, wt.shape, stride=st, padding=p,
                                                    dtype=wt.dtype)
        sets = [dict(x=x.to("cuda:0"), w=wt.to("cuda:0"),
                     y=torch.empty((n, ho, wo, f), dtype=torch.bfloat16, device="cuda:0"),
                     ws=torch.empty(wsb, dtype=torch.uint8, device="cuda:0"))
                for _ in range(nsets)]

        def tconv(i):
            b = sets[i % nsets]
            _ok(igc.conv2d_transposed_fwd(b["x"], b["w"], b["y"], stride=st, padding=p,
                                          workspace=b["ws"]), "conv2d_transposed_fwd")
        for i in range(nsets):
            tconv(i)
        t = event_time(torch, tconv, launches)
        # useful FLOPs: every input pixel meets every tap once
        flops = 2 * n * h * w * f * r * r * c
        out["transposed"][tag] = {
            "shape": f"N={n} {h}x{w} C={c} -> F={f}, {r}x{r}, stride {st}, pad {p} -> "
                     f"{ho}x{wo}, bf16",
            "call_us": round(t, 3), "tflops": round(flops / (t * 1e-6) / 1e12, 1),
            "frac_mfma": round(flops / (t * 1e-6) / 1e12 / PEAK["bf16_tflops"], 4)}
        del sets
        torch.cuda.empty_cache()
    out["general"] = measure_general(torch, igc, launches, rotate_bytes)
    return out


# Layers outside page 1's gate, run through conv2d_fwd_general (the tiled
# kernel with its general gather): a dilated 3x3 on the headline layer's
# shape, a ResNeXt-style grouped 3x3 (32 groups of 8 channels) and a 4x4
# stride-4 patchify stem (8 input channels).
GENERAL_LAYERS = {
    "dilated2_3x3_64c_n32": dict(N=32, H=56, W=56, C=64, F=64, R=3, S=3, stride=1,
                                 dilation=2, pad=2, groups=1),
    "grouped32_3x3_256c_n32": dict(N=32, H=28, W=28, C=256, F=256, R=3, S=3, stride=1,
                                   dilation=1, pad=1, groups=32),
    "patchify_4x4_s4_8to96_n32": dict(N=32, H=224, W=224, C=8, F=96, R=4, S=4, stride=4,
                                      dilation=1, pad=0, groups=1),
}


def measure_general(torch, igc, launches, rotate_bytes=ROTATE_BYTES):
    """Each general layer's whole conv2d_fwd_general call (filter transpose
    and GEMM), bf16, on rotating buffer sets; TFLOP/s from the useful FLOPs
    (2 * N * Ho * Wo * C_out * R * S * C_in / groups)."""
    import datagen

    res = {}
    for tag, L in GENERAL_LAYERS.items():
        n, h, w, c, f, r, s = (L[k] for k in ("N", "H", "W", "C", "F", "R", "S"))
        g = L["groups"]
        p = igc.conv_params(stride=L["stride"], dilation=L["dilation"], pad_begin=L["pad"],
                            groups=g)
        ho, wo = igc.out_hw_general(h, w, r, s, p)
        x, wt, _ = datagen.make_case(N=n, H=h, W=w, C=c, F=f, R=r, S=s, dtype="bfloat16",
                                     fcrs=False, x_dist=("normal", 1.0),
                                     w_dist=("normal", 1.0 / (r * s * c / g) ** 0.5), seed=0,
                                     filt_c=c // g)
        per = x.numel() * 2 + n * ho * wo * f * 2
        nsets = min(MAX_SETS, max(1, -(-rotate_bytes // per)))
        wsb = max(igc.conv2d_fwd_general_workspace_bytes(x.shape, wt.shape, (n, ho, wo, f), p,
                                                         filter_is_fcrs=False, dtype=wt.dtype),
                  16)
        sets = [dict(x=x.to("cuda:0"), w=wt.to("cuda:0"),
                     y=torch.empty((n, ho, wo, f), dtype=torch.bfloat16, device="cuda:0"),
                     ws=torch.empty(wsb, dtype=torch.uint8, device="cuda:0"))
                for _ in range(nsets)]

        def call(i):
            b = sets[i % nsets]
            _ok(igc.conv2d_fwd_general(b["x"], b["w"], b["y"], p, filter_is_fcrs=False,
                                       workspace=b["ws"]), "conv2d_fwd_general")
        for i in range(nsets):
            call(i)
        t = event_time(torch, call, launches)
        flops = 2 * n * ho * wo * f * r * s * (c // g)
        nbytes = x.numel() * 2 + wt.numel() * 2 + n * ho * wo * f * 2
        res[tag] = {
            "shape": f"N={n} {h}x{w} C={c} -> F={f}, {r}x{s}, stride {L['stride']}, "
                     f"dilation {L['dilation']}, pad {L['pad']}, groups {g} -> {ho}x{wo}, bf16",
            "kernel": igc.conv2d_fwd_general_kernel_name(x.shape, wt.shape, (n, ho, wo, f), p,
                                                         filter_is_fcrs=False, dtype=x.dtype),
            "call_us": round(t, 3), "tflops": round(flops / (t * 1e-6) / 1e12, 1),
            "frac_mfma": round(flops / (t * 1e-6) / 1e12 / PEAK["bf16_tflops"], 4),
            "gbs": round(nbytes / (t * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (t * 1e-6) / 1e9 / PEAK["hbm_gbs"], 4)}
        del sets
        torch.cuda.empty_cache()
    return res


def launch_floor(torch, launches=200):
    """Mean time per launch of an empty kernel (torch's spin kernel with a
    zero count) back to back behind a spin kernel: the per-launch floor under
    every kernel time above."""
    return event_time(torch, lambda i: torch.cuda._sleep(0), launches)


def measure(torch, igc, name, steps, warmup, rotate_bytes=ROTATE_BYTES, graphs=True):
    """Timed loop: `steps` steps as replays of the captured step graphs
    (eager steps with graphs=False), bracketed by synchronizations, after
    `warmup` eager steps and one untimed round of replays; then the GEMM
    kernel's own duration from events around `steps` back-to-back launches."""
    import datagen

    spec, x, w, src = datagen.make_workload(name)
    bufs = Bufsets(torch, igc, spec, x, w, src, rotate_bytes)
    for i in range(warmup):
        bufs.step(igc, i)
    torch.cuda.synchronize()
    per_graph = steps_per_graph(steps)
    if graphs:
        bufs.capture(torch, igc, per_graph)
        for r in range(len(bufs.graphs)):
            bufs.replay(r)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for r in range(steps // per_graph):
            bufs.replay(r)
    else:
        for i in range(steps):
            bufs.step(igc, warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = kernel_times(torch, igc, bufs, steps)
    # the transpose launch a step makes (none when the kernel transposes the
    # filter itself)
    transpose_us = 0.0 if bufs.fused else event_time(torch, lambda i: bufs.transpose(igc, i),
                                                     steps)
    flops, nbytes = _algorithmic(spec)
    ms_step = (t1 - t0) * 1e3 / steps
    bound, peak_t = _bound(spec, flops, nbytes)
    res = dict(workload=name, dtype=spec["dtype"], ms_per_step=ms_step,
               step_tflops=flops / (ms_step * 1e-3) / 1e12,
               kernel_us_mean=kern_ms * 1e3, transpose_us_mean=transpose_us,
               kernel_tflops=flops / (kern_ms * 1e-3) / 1e12,
               kernel_gbs=nbytes / (kern_ms * 1e-3) / 1e9, flops=flops, alg_bytes=nbytes,
               bound=bound, rotating_sets=bufs.nsets, filter_in_kernel=bufs.fused,
               steps_per_graph=per_graph if graphs else 0)
    res["frac_mfma"] = res["kernel_tflops"] / peak_t
    res["frac_hbm"] = res["kernel_gbs"] / PEAK["hbm_gbs"]
    del bufs
    torch.cuda.empty_cache()
    return res, spec, x, w


def cpu_baseline(spec, x, w, budget_s=10.0):
    """The fp64 oracle, as it stands, on the full batch of the workload."""
    import oracle

    flops = _algorithmic(spec)[0]
    runs, t_total = 0, 0.0
    while runs < 1 or (t_total < budget_s and runs < 200):
        t0 = time.perf_counter()
        oracle.conv2d(x, w, filter_is_fcrs=spec["fcrs"], stride=spec["stride"],
                      padding=spec["pad"])
        t_total += time.perf_counter() - t0
        runs += 1
    per = t_total / runs
    return {"value": flops / per / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"full batch of {spec['N']} images, {runs} run(s), "
                      f"{per:.2f} s per run (fp64 direct convolution, OpenMP)"}


def _traffic(res):
    """HBM bytes per launch from committed FETCH_SIZE/WRITE_SIZE counters, if
    they were taken on the current kernel source; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.loads(fh.read().split("---json---", 1)[1])
    except (IndexError, ValueError):
        return None
    if rec.get("source_sha256") != _source_digest():
        return None
    return int(rec["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-workload table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the fused-epilogue and im2col-ablation measurements")
    ap.add_argument("--only", default=None,
                    help="run only this workload's timed loop (for profiling); prints one line")
    ap.add_argument("--rotate-mib", type=int, default=ROTATE_BYTES >> 20,
                    help="total size of the rotated buffer sets; 0 keeps one set, so "
                         "operands stay in cache (warm figures, labelled as such)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="time eager steps instead of graph replays (host-paced; used for "
                         "counter runs, where every launch then works on cold buffers)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 3 times "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the path shards by batch with no exchange step; see the design "
              "notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import implicit_gemm_nhwc_amd as igc

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(igc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    igc.lib()

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return

    if args.only:
        res, _, _, _ = measure(torch, igc, args.only, args.steps, args.warmup,
                               args.rotate_mib << 20, graphs=not args.no_graphs)
        res["caches"] = "cold" if args.rotate_mib else "warm"
        print(json.dumps(res), flush=True)
        return

    rotate = args.rotate_mib << 20
    head, spec, x, w = measure(torch, igc, args.workload, args.steps, args.warmup, rotate)
    flops, nbytes = head["flops"], head["alg_bytes"]
    if head["bound"] == "hbm":
        achieved, peak, unit = head["kernel_gbs"], PEAK["hbm_gbs"], "GB/s"
    else:
        achieved, peak, unit = head["kernel_tflops"], _bound(spec, flops, nbytes)[1], "TFLOP/s"
    roofline = {"bound": head["bound"], "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "traffic": _traffic(head),
                "kernel": igc.conv2d_fwd_kernel_name(
                    (spec["N"], spec["H"], spec["W"], spec["C"]), w.shape,
                    (spec["N"],) + tuple(spec["out_hw"]) + (spec["F"],),
                    filter_is_fcrs=spec["fcrs"], dtype=w.dtype, stride=spec["stride"],
                    padding=spec["pad"]),
                "kernel_us_mean": round(head["kernel_us_mean"], 3),
                "alg_bytes_per_launch": nbytes, "flops_per_launch": flops}

    shapes = {}
    if not args.no_shapes:
        import datagen
        for name in datagen.WORKLOAD_ORDER:
            r, _, _, _ = measure(torch, igc, name, max(10, args.steps // 2 // 5 * 5), args.warmup,
                                 rotate)
            shapes[name] = {k: (round(v, 4) if isinstance(v, float) else v)
                            for k, v in r.items() if k not in ("flops", "alg_bytes")}
            print(f"# {name}: step {r['ms_per_step'] * 1e3:.1f} us, transpose "
                  f"{r['transpose_us_mean']:.1f} us, kernel "
                  f"{r['kernel_us_mean']:.1f} us = {r['kernel_tflops']:.1f} TFLOP/s "
                  f"({100 * r['frac_mfma']:.1f}% MFMA peak), {r['kernel_gbs']:.0f} GB/s "
                  f"({100 * r['frac_hbm']:.1f}% HBM), bound {r['bound']}",
                  file=sys.stderr, flush=True)

    floor_us = launch_floor(torch)
    print(f"# empty-kernel launch floor: {floor_us:.2f} us per launch", file=sys.stderr,
          flush=True)
    nxt = None
    if not args.no_next:
        nxt = measure_next(torch, igc, max(10, args.steps // 2), rotate)
        print(f"# next rows: {json.dumps(nxt)}", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(spec, x, w)
    line = {
        "metric": "conv2d fwd TFLOP/s per shape + % of MFMA peak (or % HBM BW if memory-bound)",
        "value": round(head["step_tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["dtype"].replace("bfloat16", "bf16").replace("float16", "fp16")
                                .replace("float8_e4m3fn", "fp8_e4m3fn"),
        "data": "synthetic",
        "config": {"workload": args.workload, "N": spec["N"], "H": spec["H"], "W": spec["W"],
                   "C_in": spec["C"], "C_out": spec["F"], "R": spec["R"], "S": spec["S"],
                   "stride": spec["stride"], "pad": spec["pad"],
                   "filter_layout": "FCRS" if spec["fcrs"] else "RSCF",
                   "residual": spec["src"] is not None, "parallelism": "single_gpu"},
        "roofline": roofline,
        "launch_floor_us": round(floor_us, 3),
        "cpu_baseline": cpu,
        "shapes": shapes,
        "next": nxt,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

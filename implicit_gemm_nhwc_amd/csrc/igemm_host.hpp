// Host-side pieces shared by the library's translation units: the planning
// constants of gfx950, the per-device dynamic-LDS attribute, the band-kernel
// plan, and the per-family launchers (each family is compiled in its own
// translation unit so the library builds in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "igemm_kernels.hpp"

namespace igc {

constexpr int kLdsBytes = 160 * 1024;            // LDS per CU on gfx950
constexpr int kNumCUs = 256;                     // compute units of one MI355X
constexpr size_t kResidentLdsMax = 80 * 1024;    // resident kernel: two workgroups per CU
constexpr int kResidentTN = 4;                   // resident kernel: 64 pixels per wave

// hipFuncSetAttribute acts on the current device, so the dynamic-LDS limit
// of each kernel is raised once per device (the first launch there).
constexpr int kMaxDevices = 64;
struct LdsAttr {
    std::mutex mu;
    bool done[kMaxDevices] = {};
    hipError_t err[kMaxDevices] = {};
};

inline hipError_t ensure_lds(LdsAttr& at, const void* kern, size_t lds) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(at.mu);
    if (!at.done[dev]) {
        at.err[dev] = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        at.done[dev] = true;
    }
    return at.err[dev];
}

inline int log2_exact(int64_t v) {
    int l = 0;
    while (((int64_t)1 << l) < v) ++l;
    return ((int64_t)1 << l) == v ? l : -1;
}

// Planning figures of the device a launch runs on: compute units and LDS
// bytes per CU, looked up once per device (hipDeviceGetAttribute); MI355X's
// (kNumCUs, kLdsBytes) when the lookup fails, and for host-only queries
// that make no HIP call (kernel names).
struct DevInfo {
    int cus = kNumCUs;
    int lds = kLdsBytes;
};
DevInfo device_info();

struct BandPlan {
    int TH, TW, PH, PW, TN, fpitch, ppitch, prow, spitch, lds, tiles_h, tiles_w;
    int64_t tiles;
    int groups;   // tap-fold kernel: input rows in the LDS ring
};

// Plan of the patch-resident kernel (patch_plan): output tile TH x TW, patch
// PH x PW pixels at prow bytes per row, TM 32-channel blocks per wave (BCO =
// 64*TM output channels per workgroup), TN 32-pixel blocks per wave (64*TN
// pixel slots per workgroup), nstage filter stages, tiles = N * tiles_h *
// tiles_w * channel tiles workgroups of lds bytes.
struct PatchPlan {
    int TH, TW, PH, PW, prow, lds, tiles_h, tiles_w, TM, TN, nstage;
    int64_t tiles;
};

// Launchers of each kernel family, per element type DT (DT_BF16, DT_FP16 or
// DT_FP8; resid: a residual source is read).  They fill the family's own fields of a and
// enqueue one launch on the stream.
template <int DT>
hipError_t launch_band_any(bool resid, const ConvArgs& a, const BandPlan& bp, hipStream_t stream);
template <int DT>
hipError_t launch_tapfold_any(bool resid, const ConvArgs& a, const BandPlan& bp,
                              hipStream_t stream);
template <int DT>
hipError_t launch_wide_any(bool resid, const ConvArgs& a, hipStream_t stream);
template <int DT>
hipError_t launch_patch_any(bool resid, const ConvArgs& a, const PatchPlan& pp,
                            hipStream_t stream);
template <int DT>
hipError_t launch_resident_any(bool resid, const ConvArgs& a, hipStream_t stream);
template <int DT>
hipError_t launch_tiled_any(bool resid, const ConvArgs& a, hipStream_t stream);

}  // namespace igc

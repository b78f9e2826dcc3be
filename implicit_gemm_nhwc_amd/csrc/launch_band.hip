// Launchers of the band kernel (narrow layers: the NK filter and one tile's
// input patch in LDS); the plan comes from band_plan in igemm_conv.hip.  One
// element type per translation unit: IGC_DT selects it (the build compiles
// this file once per type).
#include "igemm_host.hpp"

#ifndef IGC_DT
#error "IGC_DT must name the element type of this translation unit"
#endif

namespace igc {
namespace {

template <int DT, int TM, int TN, int U, bool RESID, bool RAW>
hipError_t launch_band(ConvArgs a, const BandPlan& bp, hipStream_t stream) {
    auto kern = igemm_fwd_band_kernel<DT, TM, TN, U, RESID, RAW>;
    static LdsAttr attr;
    const hipError_t attr_err = ensure_lds(attr, (const void*)kern, (size_t)device_info().lds);
    if (attr_err != hipSuccess) return attr_err;
    a.TH = bp.TH; a.TW = bp.TW; a.PH = bp.PH; a.PW = bp.PW;
    a.tiles_h = bp.tiles_h; a.tiles_w = bp.tiles_w;
    a.fpitch = bp.fpitch; a.ppitch = bp.ppitch; a.prow = bp.prow; a.spitch = bp.spitch;
    a.frows = a.F + 1 < TM * 32 ? a.F + 1 : TM * 32;
    a.patch_off = (a.frows * bp.fpitch + 1023) / 1024 * 1024;
    {
        const int E = DtTraits<DT>::E;
        a.cpp_log2 = log2_exact(a.C * E / 16);
    }
    if (bp.tiles == 0) return hipSuccess;
    a.lds_bytes = bp.lds;
    hipLaunchKernelGGL(kern, dim3((unsigned)(bp.tiles * (a.groups > 1 ? a.groups : 1))),
                       dim3(band_waves(DT) * 64), (size_t)bp.lds,
                       stream, a);
    return hipGetLastError();
}

// k-steps per unrolled block: the largest of 4, 2, 1 dividing the steps per tap
template <int DT, int TM, int TN, bool RESID>
hipError_t launch_band_u(const ConvArgs& a, const BandPlan& bp, hipStream_t stream) {
    constexpr int KSB = DT == DT_FP8 ? 64 : 32;
    const int steps = a.C * DtTraits<DT>::E / KSB;
    // the stored filter transposed in the kernel: bf16 / fp16 only
    if constexpr (DT != DT_FP8) {
        if (a.wraw) {
            if (steps % 4 == 0) return launch_band<DT, TM, TN, 4, RESID, true>(a, bp, stream);
            if (steps % 2 == 0) return launch_band<DT, TM, TN, 2, RESID, true>(a, bp, stream);
            return launch_band<DT, TM, TN, 1, RESID, true>(a, bp, stream);
        }
    }
    if (a.wraw) return hipErrorInvalidValue;
    if (steps % 4 == 0) return launch_band<DT, TM, TN, 4, RESID, false>(a, bp, stream);
    if (steps % 2 == 0) return launch_band<DT, TM, TN, 2, RESID, false>(a, bp, stream);
    return launch_band<DT, TM, TN, 1, RESID, false>(a, bp, stream);
}

template <int DT, int TM, bool RESID>
hipError_t launch_band_tm(const ConvArgs& a, const BandPlan& bp, hipStream_t stream) {
    switch (bp.TN) {
        case 1: return launch_band_u<DT, TM, 1, RESID>(a, bp, stream);
        case 2: return launch_band_u<DT, TM, 2, RESID>(a, bp, stream);
        case 3: return launch_band_u<DT, TM, 3, RESID>(a, bp, stream);
        default: return launch_band_u<DT, TM, 4, RESID>(a, bp, stream);
    }
}

template <int DT, bool RESID>
hipError_t launch_band_dt(const ConvArgs& a, const BandPlan& bp, hipStream_t stream) {
    if (a.F <= 32) return launch_band_tm<DT, 1, RESID>(a, bp, stream);
    return launch_band_tm<DT, 2, RESID>(a, bp, stream);
}

}  // namespace

template <int DT>
hipError_t launch_band_any(bool resid, const ConvArgs& a, const BandPlan& bp, hipStream_t stream) {
    return resid ? launch_band_dt<DT, true>(a, bp, stream) : launch_band_dt<DT, false>(a, bp, stream);
}

template hipError_t launch_band_any<IGC_DT>(bool, const ConvArgs&, const BandPlan&, hipStream_t);

}  // namespace igc

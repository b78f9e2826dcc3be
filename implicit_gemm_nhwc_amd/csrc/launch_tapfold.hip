// Launchers of the tap-fold kernel (few output channels: the (channel, tap)
// pairs are the MFMA rows); the plan comes from tapfold_plan in
// igemm_conv.hip.  One element type per translation unit: IGC_DT selects it
// (the build compiles this file once per type).
#include "igemm_host.hpp"
#include "igemm_tapfold.hpp"

#ifndef IGC_DT
#error "IGC_DT must name the element type of this translation unit"
#endif

namespace igc {
namespace {

template <int DT, int KS, bool T3, bool RESID, bool RPF>
hipError_t launch_tf_kern(ConvArgs a, const BandPlan& bp, hipStream_t stream) {
    auto kern = igemm_fwd_tapfold_kernel<DT, KS, T3, RESID, RPF>;
    static LdsAttr attr;
    const hipError_t attr_err = ensure_lds(attr, (const void*)kern, (size_t)device_info().lds);
    if (attr_err != hipSuccess) return attr_err;
    a.TH = bp.TH; a.TW = bp.TW; a.PH = bp.PH; a.PW = bp.PW;
    a.tiles_h = bp.tiles_h; a.tiles_w = bp.tiles_w;
    a.ppitch = bp.ppitch; a.prow = bp.prow; a.spitch = bp.spitch;
    a.patch_off = bp.fpitch;   // the ring starts past the coefficients and NK rows
    a.nslot = bp.groups;
    if (bp.tiles == 0) return hipSuccess;
    a.lds_bytes = bp.lds;
    hipLaunchKernelGGL(kern, dim3((unsigned)(bp.tiles * (a.groups > 1 ? a.groups : 1))),
                       dim3(TF_WAVES * 64), (size_t)bp.lds, stream, a);
    return hipGetLastError();
}

// Rows of at most TF_RPF_BLOCKS 1 KB blocks in a two-slot ring go through the
// loader waves' registers (two rows in flight); others through the
// load-to-LDS ring.  The register path is built where its A fragments fit
// the four-waves-per-SIMD bound without spilling: up to 32 registers of
// them (KS <= 8 for 16-bit types); fp8, whose fragments are twice as wide,
// spills from KS = 4 and takes it up to KS = 2.
template <int DT, int KS, bool T3, bool RESID>
hipError_t launch_tf(const ConvArgs& a, const BandPlan& bp, hipStream_t stream) {
    if constexpr (DT == DT_FP8 ? KS <= 2 : KS <= 8) {
        if (bp.groups == 2 && (bp.prow >> 10) <= TF_RPF_BLOCKS)
            return launch_tf_kern<DT, KS, T3, RESID, true>(a, bp, stream);
    }
    return launch_tf_kern<DT, KS, T3, RESID, false>(a, bp, stream);
}

template <int DT, bool T3, bool RESID>
hipError_t launch_tf_ks(const ConvArgs& a, const BandPlan& bp, hipStream_t stream) {
    constexpr int KSB = DT == DT_FP8 ? 64 : 32;
    switch (a.C * DtTraits<DT>::E / KSB) {
        case 1: return launch_tf<DT, 1, T3, RESID>(a, bp, stream);
        case 2: return launch_tf<DT, 2, T3, RESID>(a, bp, stream);
        case 4: return launch_tf<DT, 4, T3, RESID>(a, bp, stream);
        case 8: return launch_tf<DT, 8, T3, RESID>(a, bp, stream);
        case 16: return launch_tf<DT, 16, T3, RESID>(a, bp, stream);
        default: return hipErrorInvalidValue;   // the planner only picks these
    }
}

}  // namespace

template <int DT>
hipError_t launch_tapfold_any(bool resid, const ConvArgs& a, const BandPlan& bp,
                              hipStream_t stream) {
    const bool t3 = a.R == 3 && a.S == 3;
    if (resid)
        return t3 ? launch_tf_ks<DT, true, true>(a, bp, stream)
                  : launch_tf_ks<DT, false, true>(a, bp, stream);
    return t3 ? launch_tf_ks<DT, true, false>(a, bp, stream)
              : launch_tf_ks<DT, false, false>(a, bp, stream);
}

template hipError_t launch_tapfold_any<IGC_DT>(bool, const ConvArgs&, const BandPlan&,
                                               hipStream_t);

}  // namespace igc

// Launchers of the patch-resident kernel (wide layers with a spatial filter:
// the tile's input patch in LDS, the filter streamed per tap); the plan
// comes from patch_plan in igemm_conv.hip.  One element type per
// translation unit: IGC_DT selects it (the build compiles this file once per
// type).
#include "igemm_host.hpp"
#include "igemm_patch.hpp"

#ifndef IGC_DT
#error "IGC_DT must name the element type of this translation unit"
#endif

namespace igc {
namespace {

template <int DT, int TM, int TN, int NSTAGE, bool RESID>
hipError_t launch_patch(ConvArgs a, const PatchPlan& pp, hipStream_t stream) {
    constexpr int WCO = 2, WPX = 2;
    constexpr int BCO = WCO * TM * 32;
    auto kern = igemm_fwd_patch_kernel<DT, TM, TN, WCO, WPX, NSTAGE, RESID>;
    static LdsAttr attr;
    const hipError_t attr_err = ensure_lds(attr, (const void*)kern, (size_t)device_info().lds);
    if (attr_err != hipSuccess) return attr_err;
    a.TH = pp.TH; a.TW = pp.TW; a.PH = pp.PH; a.PW = pp.PW;
    a.tiles_h = pp.tiles_h; a.tiles_w = pp.tiles_w;
    a.ppitch = PATCH_PP;
    a.prow = pp.prow;
    a.patch_off = NSTAGE * BCO * 128;
    a.co_tiles = (a.F + BCO - 1) / BCO;
    a.px_tiles = (int)(pp.tiles / a.co_tiles);
    if (pp.tiles == 0) return hipSuccess;
    a.lds_bytes = pp.lds;
    hipLaunchKernelGGL(kern, dim3((unsigned)(pp.tiles * (a.groups > 1 ? a.groups : 1))),
                       dim3(WCO * WPX * 64), (size_t)pp.lds, stream, a);
    return hipGetLastError();
}

template <int DT, int TM, int TN, bool RESID>
hipError_t launch_patch_tn(const ConvArgs& a, const PatchPlan& pp, hipStream_t stream) {
    if (pp.nstage == 3) return launch_patch<DT, TM, TN, 3, RESID>(a, pp, stream);
    return launch_patch<DT, TM, TN, 2, RESID>(a, pp, stream);
}

template <int DT, int TM, bool RESID>
hipError_t launch_patch_tm(const ConvArgs& a, const PatchPlan& pp, hipStream_t stream) {
    if (pp.TN == 4) return launch_patch_tn<DT, TM, 4, RESID>(a, pp, stream);
    return launch_patch_tn<DT, TM, 2, RESID>(a, pp, stream);
}

template <int DT, bool RESID>
hipError_t launch_patch_dt(const ConvArgs& a, const PatchPlan& pp, hipStream_t stream) {
    if (pp.TM == 4) return launch_patch_tm<DT, 4, RESID>(a, pp, stream);
    return launch_patch_tm<DT, 2, RESID>(a, pp, stream);
}

}  // namespace

template <int DT>
hipError_t launch_patch_any(bool resid, const ConvArgs& a, const PatchPlan& pp,
                            hipStream_t stream) {
    return resid ? launch_patch_dt<DT, true>(a, pp, stream) : launch_patch_dt<DT, false>(a, pp, stream);
}

template hipError_t launch_patch_any<IGC_DT>(bool, const ConvArgs&, const PatchPlan&, hipStream_t);

}  // namespace igc

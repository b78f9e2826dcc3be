// Launchers of the filter-resident kernel (C_out <= 64 when the band plan
// does not fit) and of the plain tiled fallback kernel.  One family
// (IGC_FAMILY 0 = resident, 1 = tiled) and one element type (IGC_DT) per
// translation unit; the build compiles this file once per pair.
#include "igemm_host.hpp"

#if !defined(IGC_DT) || !defined(IGC_FAMILY)
#error "IGC_DT and IGC_FAMILY must select this translation unit's launchers"
#endif

namespace igc {
namespace {

template <int DT, int BCO, int BPX, int WCO, int WPX, bool RESID, bool EG>
hipError_t launch_tile(ConvArgs a, hipStream_t stream) {
    constexpr size_t lds = 2 * (size_t)(BCO + BPX) * KT_BYTES;
    auto kern = igemm_fwd_kernel<DT, BCO, BPX, WCO, WPX, RESID, EG>;
    static LdsAttr attr;
    const hipError_t attr_err = ensure_lds(attr, (const void*)kern, (size_t)(lds));
    if (attr_err != hipSuccess) return attr_err;
    a.px_tiles = (a.M + BPX - 1) / BPX;
    a.co_tiles = (a.F + BCO - 1) / BCO;
    const int64_t blocks = (int64_t)a.px_tiles * a.co_tiles;
    if (blocks == 0) return hipSuccess;
    a.lds_bytes = (int)lds;
    hipLaunchKernelGGL(kern, dim3((unsigned)(blocks * (a.groups > 1 ? a.groups : 1))),
                       dim3(NTHREADS), lds, stream, a);
    return hipGetLastError();
}

template <int DT, int TM, bool RESID, bool ALIGNED>
hipError_t launch_resident(ConvArgs a, hipStream_t stream) {
    constexpr int E = DtTraits<DT>::E;
    auto kern = igemm_fwd_resident_kernel<DT, TM, kResidentTN, RESID, ALIGNED>;
    static LdsAttr attr;
    const hipError_t attr_err = ensure_lds(attr, (const void*)kern, kResidentLdsMax);
    if (attr_err != hipSuccess) return attr_err;
    // the filter is staged in whole 1 KB blocks: round the allocation up
    const size_t lds = ((size_t)TM * 16 * ((size_t)a.kpitch * E) + 1023) / 1024 * 1024;
    const int64_t wtiles = ((int64_t)a.M + kResidentTN * 16 - 1) / (kResidentTN * 16);
    const int64_t blocks = (wtiles + RES_WAVES - 1) / RES_WAVES;
    if (blocks == 0) return hipSuccess;
    a.lds_bytes = (int)lds;
    hipLaunchKernelGGL(kern, dim3((unsigned)(blocks * (a.groups > 1 ? a.groups : 1))),
                       dim3(RES_WAVES * 64), lds, stream, a);
    return hipGetLastError();
}

template <int DT, bool RESID, bool ALIGNED>
hipError_t launch_resident_tm(const ConvArgs& a, hipStream_t stream) {
    if (a.F <= 16) return launch_resident<DT, 1, RESID, ALIGNED>(a, stream);
    if (a.F <= 32) return launch_resident<DT, 2, RESID, ALIGNED>(a, stream);
    if (a.F <= 48) return launch_resident<DT, 3, RESID, ALIGNED>(a, stream);
    return launch_resident<DT, 4, RESID, ALIGNED>(a, stream);
}

// C_in a multiple of the 128-byte k-tile: each k-tile sits inside one tap.
template <int DT, bool RESID>
hipError_t launch_resident_dt(const ConvArgs& a, hipStream_t stream) {
    constexpr int KT = KT_BYTES / DtTraits<DT>::E;
    if (a.C > 0 && a.C % KT == 0) return launch_resident_tm<DT, RESID, true>(a, stream);
    return launch_resident_tm<DT, RESID, false>(a, stream);
}

template <int DT, bool RESID, bool EG>
hipError_t launch_dt_eg(const ConvArgs& a, hipStream_t stream) {
    // Tile by C_out: one 16x16 MFMA row block per wave for tiny C_out, up to
    // 128 x 128 workgroup tiles (64 x 64 per wave) for wide layers.
    if (a.F <= 16) return launch_tile<DT, 16, 256, 1, 4, RESID, EG>(a, stream);
    if (a.F <= 32) return launch_tile<DT, 32, 256, 1, 4, RESID, EG>(a, stream);
    if (a.F <= 64) return launch_tile<DT, 64, 256, 1, 4, RESID, EG>(a, stream);
    return launch_tile<DT, 128, 128, 2, 2, RESID, EG>(a, stream);
}

// C_in (per group) * E not a multiple of 16: the element gather.
template <int DT, bool RESID>
hipError_t launch_dt(const ConvArgs& a, hipStream_t stream) {
    if ((a.C * DtTraits<DT>::E) % 16 != 0) return launch_dt_eg<DT, RESID, true>(a, stream);
    return launch_dt_eg<DT, RESID, false>(a, stream);
}

}  // namespace

template <int DT>
hipError_t launch_resident_any(bool resid, const ConvArgs& a, hipStream_t stream) {
    return resid ? launch_resident_dt<DT, true>(a, stream) : launch_resident_dt<DT, false>(a, stream);
}

template <int DT>
hipError_t launch_tiled_any(bool resid, const ConvArgs& a, hipStream_t stream) {
    return resid ? launch_dt<DT, true>(a, stream) : launch_dt<DT, false>(a, stream);
}

#if IGC_FAMILY == 0
template hipError_t launch_resident_any<IGC_DT>(bool, const ConvArgs&, hipStream_t);
#else
template hipError_t launch_tiled_any<IGC_DT>(bool, const ConvArgs&, hipStream_t);
#endif

}  // namespace igc

// Launchers of the wide-layer kernel (C_out > 64), one element type per
// translation unit: IGC_DT selects it (the build compiles this file once
// per type).
#include "igemm_host.hpp"

#ifndef IGC_DT
#error "IGC_DT must name the element type of this translation unit"
#endif

namespace igc {
namespace {

// ---- wide-layer kernel with direct-to-LDS staging ---------------------------
template <int DT, int TM, int TN, int WCO, int WPX, int KTB, int NSTAGE, bool RESID, bool TAPK,
          bool GROUPED = false>
hipError_t launch_wide(ConvArgs a, hipStream_t stream) {
    constexpr int BCO = WCO * TM * 32, BPX = WPX * TN * 32;
    constexpr size_t lds = (size_t)NSTAGE * (BCO + BPX) * KTB;
    static_assert(lds <= (size_t)kLdsBytes, "stages fit in LDS");
    auto kern = igemm_fwd_wide_kernel<DT, TM, TN, WCO, WPX, KTB, NSTAGE, RESID, TAPK, GROUPED>;
    static LdsAttr attr;
    const hipError_t attr_err = ensure_lds(attr, (const void*)kern, (size_t)(lds));
    if (attr_err != hipSuccess) return attr_err;
    a.ktiles = a.ktiles * (KT_BYTES / KTB);   // NK rows hold whole 128-byte k-tiles
    a.px_tiles = (a.M + BPX - 1) / BPX;
    a.co_tiles = (a.F + BCO - 1) / BCO;
    const int64_t blocks = (int64_t)a.px_tiles * a.co_tiles;
    if (blocks == 0) return hipSuccess;
    a.lds_bytes = (int)lds;
    hipLaunchKernelGGL(kern, dim3((unsigned)(blocks * (a.groups > 1 ? a.groups : 1))),
                       dim3(WCO * WPX * 64), lds, stream, a);
    return hipGetLastError();
}

// Tile choice for C_out > 64, four waves, 128-byte k-tiles (whole cache
// lines per request).  256 x 256 tiles (128 x 128 per wave, 256 accumulator
// registers) in two stages (128 KB of LDS, one workgroup per CU) whenever
// that still gives a tile per CU; otherwise 128 x 128 tiles (64 x 64 per
// wave) in two stages, 64 KB, so two workgroups share a CU and one's
// prologue, epilogue and waits overlap the other's MFMAs.  Measured on the
// strided 3x3 128->256 layer (N=32, 56x56, fp16; kernel time, cold operands):
// 128x128 in 2 stages 27.9 us, 256x128 in 3 stages 30.4 us, 256x128 in 2
// stages 31.0 us, 128x256 in 3 stages 30.7 us, 128x128 in 4 stages (one
// workgroup per CU) 35.1 us, 256x256 in 2 stages (98 tiles) 42.7 us.  On the
// fp8 5x5 256->256 layer (256 tiles of 256x256): 256x256 in 2 stages 105 us,
// 128x128 in 2 stages 115 us, 256x128 in 3 stages 125 us (these four-wave
// figures predate the eight-wave 256 x 128 tile below).  TAPK when C_in is
// a whole number of k-tiles.  With at most one 128 x 128 tile per CU,
// 128 x 64 tiles in three stages.
template <int DT, bool RESID>
hipError_t launch_wide_dt(const ConvArgs& a, hipStream_t stream) {
    constexpr int E = DtTraits<DT>::E;
    const bool tap128 = a.C > 0 && (a.C * E) % 128 == 0;
    const int64_t co_tiles256 = (a.F + 255) / 256;
    const int64_t px_tiles256 = ((int64_t)a.M + 255) / 256;
    // grouped or mapped launches (the phases of a transposed convolution):
    // three stages (measured on the 4x4 stride-2 upsampler, N=8 32x32
    // 256->128 bf16, whole call: 22.0 us in two stages, 20.7 us in three);
    // 128 x 64 tiles when 128 x 128 ones would not give every CU two
    // workgroups (upsampler: 256 tiles of 128 x 128, 20.9 us; 512 of
    // 128 x 64, 20.0 us; 64 x 128, 21.5 us)
    if (a.groups > 1 || a.ymap) {
        const int64_t tiles128 = (((int64_t)a.M + 127) / 128) * ((a.F + 127) / 128) *
                                 (a.groups > 1 ? a.groups : 1);
        if (tiles128 < 2 * (int64_t)device_info().cus)
            return tap128 ? launch_wide<DT, 2, 1, 2, 2, 128, 3, RESID, true, true>(a, stream)
                          : launch_wide<DT, 2, 1, 2, 2, 128, 3, RESID, false, true>(a, stream);
        return tap128 ? launch_wide<DT, 2, 2, 2, 2, 128, 3, RESID, true, true>(a, stream)
                      : launch_wide<DT, 2, 2, 2, 2, 128, 3, RESID, false, true>(a, stream);
    }
    if (a.F > 128 && px_tiles256 * co_tiles256 >= device_info().cus)
        return tap128 ? launch_wide<DT, 4, 4, 2, 2, 128, 2, RESID, true>(a, stream)
                      : launch_wide<DT, 4, 4, 2, 2, 128, 2, RESID, false>(a, stream);
    // 128 x 128 tiles that would fill between 1.25 and 2 workgroups per CU
    // (the second slot of many CUs empty) but 256 x 128 tiles that fit one
    // round: 256 x 128 tiles, 8 waves of 64 x 64 (two per SIMD) in three
    // stages (144 KB), which read 1.5 rather than 2 staged rows per 128
    // outputs (strided 3x3 128->256 layer, N=32 56x56 fp16, alternating
    // medians: 26.1 -> 24.0 us; in two stages 26.4 us)
    {
        const int64_t t128 = (((int64_t)a.M + 127) / 128) * ((a.F + 127) / 128);
        const int64_t t256x128 = (((int64_t)a.M + 127) / 128) * ((a.F + 255) / 256);
        const int64_t cus = device_info().cus;
        if (a.F % 256 == 0 && 4 * t128 > 5 * cus && t128 < 2 * cus && t256x128 <= cus)
            return tap128 ? launch_wide<DT, 2, 2, 4, 2, 128, 3, RESID, true>(a, stream)
                          : launch_wide<DT, 2, 2, 4, 2, 128, 3, RESID, false>(a, stream);
    }
    // at most one 128 x 128 tile per CU: 128 x 64 tiles in three stages
    // (72 KB, two workgroups per CU) fill the second workgroup slot
    // (transposed 3x3 stride-1 layer, N=8 64x64 256->128 bf16, whole call:
    // 33.9 -> 30.5 us; two stages 31.7 us)
    const int64_t tiles128 = (((int64_t)a.M + 127) / 128) * ((a.F + 127) / 128);
    if (tiles128 <= device_info().cus)
        return tap128 ? launch_wide<DT, 2, 1, 2, 2, 128, 3, RESID, true>(a, stream)
                      : launch_wide<DT, 2, 1, 2, 2, 128, 3, RESID, false>(a, stream);
    return tap128 ? launch_wide<DT, 2, 2, 2, 2, 128, 2, RESID, true>(a, stream)
                  : launch_wide<DT, 2, 2, 2, 2, 128, 2, RESID, false>(a, stream);
}

}  // namespace

template <int DT>
hipError_t launch_wide_any(bool resid, const ConvArgs& a, hipStream_t stream) {
    return resid ? launch_wide_dt<DT, true>(a, stream) : launch_wide_dt<DT, false>(a, stream);
}

template hipError_t launch_wide_any<IGC_DT>(bool, const ConvArgs&, hipStream_t);

}  // namespace igc

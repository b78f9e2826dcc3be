// C-ABI entry points of the forward NHWC implicit-GEMM convolution
// (declarations and contracts in include/igemm_conv.h).
//
// Host side: the acceptance gate of the page "dispatch_amd_4wave_conv2d"
// (Parameters and Args sections) plus this library's own limits, the NK
// workspace, tile-shape selection by C_out, and the launches.  Every step of
// the computation runs in the kernels of igemm_kernels.hpp.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>
#include <vector>

#include "igemm_conv.h"
#include "igemm_host.hpp"
#include "igemm_aux_kernels.hpp"

namespace igc {

DevInfo device_info() {
    static std::mutex mu;
    static bool done[kMaxDevices] = {};
    static DevInfo info[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DevInfo{};
    std::lock_guard<std::mutex> g(mu);
    if (!done[dev]) {
        int cus = 0, lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus > 0)
            info[dev].cus = cus;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
                hipSuccess &&
            lds > 0)
            info[dev].lds = lds < kLdsBytes ? lds : kLdsBytes;
        done[dev] = true;
    }
    return info[dev];
}

}  // namespace igc

namespace {

using namespace igc;

constexpr int32_t kAbiVersion = 5;

int elem_bytes(int32_t dtype) { return dtype == IGC_DTYPE_FP8_E4M3FN ? 1 : 2; }

struct Shape {
    int64_t N, H, W, C, R, S, F, Ho, Wo, M, K;
    int64_t kpad;    // K rounded up to whole 128-byte k-tiles (elements)
    int64_t kpitch;  // NK row stride (elements), see nk_pitch
    int32_t st, pad;
    int32_t pt, pl;  // padding before each axis (pad, or the general or phase problem's own)
};

void filter_rscf(const int64_t* fd, int32_t fcrs, int64_t* R, int64_t* S, int64_t* C, int64_t* F) {
    if (fcrs) { *F = fd[0]; *C = fd[1]; *R = fd[2]; *S = fd[3]; }
    else { *R = fd[0]; *S = fd[1]; *C = fd[2]; *F = fd[3]; }
}

int64_t out_size(int64_t in, int64_t k, int64_t st, int64_t pad) {
    const int64_t span = in + 2 * pad - k;
    return span < 0 ? 0 : span / st + 1;
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// NK row stride in elements: K rounded up to whole 128-byte k-tiles; for
// C_out <= 64 plus a 16-byte zero pad, since those kernels copy the rows
// straight into LDS and read fragments across them (a pitch of 16 mod 128
// bytes spreads the rows over the banks), while the wide-layer kernel
// requests whole 128-byte row segments and wants them line aligned.
int64_t nk_pitch(int64_t K, int64_t F, int64_t eb) {
    return round_up(K, KT_BYTES / eb) + (F <= 64 ? 16 / eb : 0);
}

// Shape-only part of the gate: page rules, shape consistency, limits.
int32_t check_shapes(const int64_t in_nhwc[4], int32_t fcrs, const int64_t filt_dims[4],
                     const int64_t out_nhwc[4], const int32_t stride[2],
                     const int32_t dilation[2], const int32_t padding[2], int32_t groups,
                     int32_t dtype, Shape* sh) {
    if (!in_nhwc || !filt_dims || !out_nhwc || !stride || !dilation || !padding)
        return IGC_DECLINE_NULL_POINTER;
    if (dtype != IGC_DTYPE_BF16 && dtype != IGC_DTYPE_FP16 && dtype != IGC_DTYPE_FP8_E4M3FN)
        return IGC_DECLINE_DTYPE;
    if (!((stride[0] == 1 && stride[1] == 1) || (stride[0] == 2 && stride[1] == 2)))
        return IGC_DECLINE_STRIDE;
    if (dilation[0] != 1 || dilation[1] != 1) return IGC_DECLINE_DILATION;
    if (padding[0] != padding[1] || padding[0] < 0 || padding[0] > 2) return IGC_DECLINE_PADDING;
    if (groups != 1) return IGC_DECLINE_GROUPS;

    Shape s{};
    s.N = in_nhwc[0]; s.H = in_nhwc[1]; s.W = in_nhwc[2]; s.C = in_nhwc[3];
    filter_rscf(filt_dims, fcrs, &s.R, &s.S, &s.C, &s.F);
    const int64_t cin = in_nhwc[3];
    if (s.N < 0 || s.H < 0 || s.W < 0 || cin < 0 || s.F < 0 || s.C < 0 || s.R < 1 || s.S < 1)
        return IGC_DECLINE_SHAPE;
    if (s.C != cin) return IGC_DECLINE_SHAPE;
    s.st = stride[0];
    s.pad = padding[0];
    s.pt = s.pl = s.pad;
    s.Ho = out_size(s.H, s.R, s.st, s.pad);
    s.Wo = out_size(s.W, s.S, s.st, s.pad);
    if (s.Ho < 1 || s.Wo < 1) return IGC_DECLINE_OUTPUT_SHAPE;
    if (out_nhwc[0] != s.N || out_nhwc[1] != s.Ho || out_nhwc[2] != s.Wo || out_nhwc[3] != s.F)
        return IGC_DECLINE_OUTPUT_SHAPE;
    const int64_t eb = elem_bytes(dtype);

    const int64_t lim = (int64_t)1 << 31;
    if (s.H >= lim || s.W >= lim || s.R >= lim || s.S >= lim || s.C >= lim || s.F >= lim)
        return IGC_DECLINE_SIZE_LIMIT;
    s.M = s.N * s.Ho * s.Wo;
    s.K = s.R * s.S * s.C;
    if (s.Ho > lim / (s.Wo > 0 ? s.Wo : 1) || s.M >= lim || s.K >= lim ||
        (s.R * s.W + s.S) * s.C >= lim)
        return IGC_DECLINE_SIZE_LIMIT;
    s.kpad = round_up(s.K, KT_BYTES / eb);
    s.kpitch = nk_pitch(s.K, s.F, eb);
    if (s.kpitch >= lim || s.F * s.kpitch * eb >= lim) return IGC_DECLINE_SIZE_LIMIT;
    if (sh) *sh = s;
    return IGC_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Pointer rules of a forward call, given the byte sizes of its tensors
// (nk_bytes: what the filter transpose writes into the workspace).
int32_t check_pointers(const void* input, size_t in_bytes, const void* filter, size_t f_bytes,
                       const void* output, size_t out_bytes, const void* source,
                       const void* workspace, size_t nk_bytes, size_t workspace_bytes) {
    if ((in_bytes && !input) || (f_bytes && !filter) || (out_bytes && !output))
        return IGC_DECLINE_NULL_POINTER;
    if (!aligned16(input) || !aligned16(filter) || !aligned16(output) || !aligned16(source) ||
        !aligned16(workspace))
        return IGC_DECLINE_ALIGNMENT;
    if (overlaps(output, out_bytes, input, in_bytes) || overlaps(output, out_bytes, filter, f_bytes))
        return IGC_DECLINE_OVERLAP;
    if (workspace && overlaps(output, out_bytes, workspace, nk_bytes)) return IGC_DECLINE_OVERLAP;
    // the NK transpose writes the workspace before the GEMM reads the
    // input, the filter and the residual source
    if (workspace && (overlaps(workspace, nk_bytes, input, in_bytes) ||
                      overlaps(workspace, nk_bytes, filter, f_bytes) ||
                      (source && overlaps(workspace, nk_bytes, source, out_bytes))))
        return IGC_DECLINE_OVERLAP;
    if (source && source != output && overlaps(source, out_bytes, output, out_bytes))
        return IGC_DECLINE_OVERLAP;
    if (workspace && workspace_bytes < nk_bytes) return IGC_DECLINE_WORKSPACE;
    return IGC_OK;
}

// Full gate: shapes plus pointers.  filter may be the NK matrix (nk_bytes
// then gives its size); workspace is NULL for conv2d_fwd_nk.
int32_t check_all(const void* input, const int64_t in_nhwc[4], const void* filter,
                  size_t filter_bytes_override, int32_t fcrs, const int64_t filt_dims[4],
                  const void* output, const int64_t out_nhwc[4], const int32_t stride[2],
                  const int32_t dilation[2], const int32_t padding[2], int32_t groups,
                  int32_t dtype, const void* source, const void* workspace,
                  size_t workspace_bytes, Shape* out_shape) {
    Shape s;
    int32_t rc = check_shapes(in_nhwc, fcrs, filt_dims, out_nhwc, stride, dilation, padding,
                              groups, dtype, &s);
    if (rc != IGC_OK) return rc;
    const size_t eb = (size_t)elem_bytes(dtype);
    const size_t in_bytes = (size_t)(s.N * s.H * s.W * s.C) * eb;
    const size_t f_bytes = filter_bytes_override ? filter_bytes_override
                                                 : (size_t)(s.R * s.S * s.C * s.F) * eb;
    const size_t out_bytes = (size_t)(s.M * s.F) * 2;
    const size_t nk_bytes = (size_t)(s.F * s.kpitch) * eb;
    rc = check_pointers(input, in_bytes, filter, f_bytes, output, out_bytes, source, workspace,
                        nk_bytes, workspace_bytes);
    if (rc != IGC_OK) return rc;
    if (out_shape) *out_shape = s;
    return IGC_OK;
}

int32_t hip_fail(hipError_t e) { return e == hipSuccess ? 1 : -(int32_t)e; }


// The fused epilogue's own gate: a known activation, 4-byte aligned
// coefficient arrays, and none of them overlapping the output (every
// workgroup reads them while others write the output) or the workspace
// (written by the filter transpose before the GEMM reads them).
int32_t check_epilogue(const igc_epilogue* epi, const void* output, const Shape& s,
                       const void* workspace = nullptr, size_t workspace_used = 0) {
    if (!epi) return IGC_OK;
    if (epi->activation != IGC_ACT_NONE && epi->activation != IGC_ACT_RELU &&
        epi->activation != IGC_ACT_SILU)
        return IGC_DECLINE_EPILOGUE;
    const size_t out_bytes = (size_t)(s.M * s.F) * 2;
    const size_t coef_bytes = (size_t)s.F * sizeof(float);
    for (const float* c : {epi->scale, epi->bias}) {
        if (!c) continue;
        if (((uintptr_t)c & 3u) != 0) return IGC_DECLINE_EPILOGUE;
        if (overlaps(c, coef_bytes, output, out_bytes)) return IGC_DECLINE_EPILOGUE;
        if (workspace && overlaps(c, coef_bytes, workspace, workspace_used))
            return IGC_DECLINE_EPILOGUE;
    }
    return IGC_OK;
}

// ---- launches -----------------------------------------------------------

hipError_t launch_transpose(const void* filter, int32_t fcrs, const Shape& s, int32_t dtype,
                            void* nk, hipStream_t stream) {
    const int eb = elem_bytes(dtype);
    const int64_t row_chunks = s.kpitch / (16 / eb);
    if (s.F == 0 || row_chunks == 0) return hipSuccess;
    // 64-thread workgroups along the stored layout's contiguous direction
    // (FCRS: a row's chunks; RSCF: C_out), one grid row per NK row (FCRS)
    // or chunk (RSCF), rows past 65535 looping; many small workgroups keep
    // many CUs' loads in flight
    const int64_t gx = fcrs ? row_chunks : s.F, gy = fcrs ? s.F : row_chunks;
    const dim3 grid((unsigned)((gx + 63) / 64), (unsigned)(gy < 65535 ? gy : 65535));
    if (eb == 2)
        hipLaunchKernelGGL(filter_to_nk_kernel<2>, grid, dim3(64), 0, stream,
                           (const uint8_t*)filter, (uint8_t*)nk, fcrs, (int)s.R, (int)s.S,
                           (int)s.C, (int)s.F, (int)s.K, (int)s.kpitch);
    else
        hipLaunchKernelGGL(filter_to_nk_kernel<1>, grid, dim3(64), 0, stream,
                           (const uint8_t*)filter, (uint8_t*)nk, fcrs, (int)s.R, (int)s.S,
                           (int)s.C, (int)s.F, (int)s.K, (int)s.kpitch);
    return hipGetLastError();
}

// The filter-resident kernel applies when the padded NK matrix fits its LDS
// budget and every wave's gather window (the images its 64 pixels touch)
// stays below the 2^31-byte buffer range.
bool resident_ok(const Shape& s, int32_t dtype) {
    if (s.F > 64) return false;
    const int64_t eb = elem_bytes(dtype);
    const int64_t rows = (s.F + 15) / 16 * 16;
    if ((rows * s.kpitch * eb + 1023) / 1024 * 1024 > (int64_t)kResidentLdsMax) return false;
    const int64_t howo = s.Ho * s.Wo;
    int64_t imgs = (kResidentTN * 16 - 1) / howo + 2;
    if (imgs > s.N) imgs = s.N;
    return imgs * s.H * s.W * s.C * eb < ((int64_t)1 << 31);
}


// ---- band kernel planning ------------------------------------------------

// 32-pixel blocks per wave the band kernel is built for.
int band_tn(int64_t blocks_per_wave) {
    for (int tn : {1, 2, 3, 4})
        if (blocks_per_wave <= tn) return tn;
    return 0;
}

// Pick the output tile (TH x TW) for the band kernel, or return false when
// the layer does not fit it (C_out > 64, filter + smallest patch > LDS, or
// C_in not a power-of-two number of MFMA k-steps).  The estimate charges
// each round of resident workgroups its load time (filter + patch at
// ~48 B/clk/CU plus a fixed latency) and its MFMA time (32 clk per 32x32
// block step, band_waves / 4 waves per SIMD with TN blocks each, padding
// included).
bool band_plan(const Shape& s, int32_t dtype, BandPlan* out, const DevInfo& dev,
               double* cost_out = nullptr) {
    const int64_t E = elem_bytes(dtype);
    const int64_t ksb = dtype == IGC_DTYPE_FP8_E4M3FN ? 64 : 32;
    if (s.F > 64 || s.F < 1 || s.C < 1 || (s.C * E) % ksb != 0) return false;
    if (log2_exact(s.C * E / 16) < 0) return false;
    if (s.H * s.W * s.C * E >= ((int64_t)1 << 31)) return false;
    const int64_t tm = s.F <= 32 ? 1 : 2;
    const int64_t waves = band_waves(dtype == IGC_DTYPE_FP8_E4M3FN ? DT_FP8 : DT_BF16);
    const int64_t fpitch = s.kpitch * E;
    // filter rows kept in LDS: C_out real rows plus one zero row that the
    // fragment reads of rows >= C_out all point at (up to the TM*32 rows the
    // MFMAs span)
    const int64_t frows = s.F + 1 < tm * 32 ? s.F + 1 : tm * 32;
    const int64_t fbytes = frows * fpitch;
    const int64_t ppitch = s.C * E + 16;
    const int64_t spitch = tm * 32 + 4;
    const int64_t ksteps = s.R * s.S * (s.C * E / ksb);
    if (fbytes >= dev.lds) return false;
    int tws[6], ntw = 0;
    if (s.Wo <= 128) tws[ntw++] = (int)s.Wo;
    for (int c : {128, 64, 32})
        if (c < s.Wo) tws[ntw++] = c;
    double best = 1e300;
    bool found = false;
    for (int k = 0; k < ntw; ++k) {
        const int64_t tw = tws[k];
        for (int64_t th = 1; th <= s.Ho && th * tw <= 32 * BAND_MAX_TN * waves; ++th) {
            const int64_t P = th * tw, NB = (P + 31) / 32;
            const int tn = band_tn((NB + waves - 1) / waves);
            if (tn == 0) continue;
            const int64_t ph = (th - 1) * s.st + s.R, pw = (tw - 1) * s.st + s.S;
            // row pad: (prow - tw * ppitch) % 256 == 0, so the 16 lanes of a
            // fragment read served together (64 banks, 256 bytes) keep hitting
            // distinct 16-byte bank groups when their pixels wrap to the next
            // tile row
            const int64_t prow = pw * ppitch + (((tw - pw) * ppitch) % 256 + 256) % 256;
            // filter and patch are each staged in whole 1 KB blocks
            const int64_t patch = (ph * prow + 1023) / 1024 * 1024;
            int64_t lds = (fbytes + 1023) / 1024 * 1024 + patch;
            const int64_t stage = P * spitch * 4;
            if (stage > lds) lds = stage;
            if (lds > dev.lds) continue;
            const int64_t th_tiles = (s.Ho + th - 1) / th, tw_tiles = (s.Wo + tw - 1) / tw;
            const int64_t tiles = s.N * th_tiles * tw_tiles;
            const int64_t per_cu = dev.lds / lds;
            const int64_t rounds = (tiles + dev.cus * per_cu - 1) / (dev.cus * per_cu);
            const int64_t conc = tiles < dev.cus * per_cu ? (tiles + dev.cus - 1) / dev.cus : per_cu;
            const double load = (double)(fbytes + patch) / 48.0 + 2500.0;
            const double mfma = (double)tn * (waves / 4) * tm * ksteps * 32.0;
            const double cost = rounds * (load + mfma * (double)conc);
            if (cost < best) {
                best = cost;
                found = true;
                if (cost_out) *cost_out = cost;
                *out = BandPlan{(int)th, (int)tw, (int)ph, (int)pw, tn, (int)fpitch, (int)ppitch,
                                (int)prow, (int)spitch, (int)lds, (int)th_tiles, (int)tw_tiles,
                                tiles, 0};
            }
        }
    }
    return found;
}


// The wide kernel bases each tile's pixel buffer at its first image; the
// images one tile's 256 pixels can touch must fit the 2^31-byte range.
bool wide_ok(const Shape& s, int32_t dtype) {
    if (s.F <= 64) return false;
    const int64_t howo = s.Ho * s.Wo;
    int64_t imgs = 255 / howo + 2;
    if (imgs > s.N) imgs = s.N;
    return imgs * s.H * s.W * s.C * elem_bytes(dtype) < ((int64_t)1 << 31);
}


// Plan of the tap-fold kernel (igemm_tapfold.hpp), or false when the layer
// does not fit it: C_out * R * S <= 32 (the (channel, tap) pairs of one
// 32-row MFMA block) with R * S >= 2, C_in a whole number of 1, 2, 4, 8 or
// 16 MFMA k-steps, and an image below 2^31 bytes.  The workgroup streams a
// strip of output columns whose input row (PW = (TW - 1)*st + S pixels) is
// one to four 32-pixel blocks, over TH output rows; strips times row
// segments are chosen near one round of resident workgroups (as many per CU
// as their LDS allows), the estimate charging each
// workgroup its input bytes (at ~16 B/clk), a fixed start and ~400 clocks
// per input row (more with fewer than four ring slots).  LDS: coefficients,
// the NK rows, a ring of up to four input rows and R + 1 rows of fp32 partial
// products.  The plan fields carry the kernel's geometry: TW/TH, PW/PH,
// ppitch (bytes per staged pixel), prow (bytes per ring slot), spitch
// (floats per partial-product pixel), fpitch (LDS offset of the ring),
// groups (ring slots).
bool tapfold_plan(const Shape& s, int32_t dtype, BandPlan* out, const DevInfo& dev) {
    const int64_t E = elem_bytes(dtype);
    const int64_t ksb = dtype == IGC_DTYPE_FP8_E4M3FN ? 64 : 32;
    const int64_t rs = s.R * s.S;
    if (s.F < 1 || rs < 2 || s.F * rs > 32 || s.C < 1 || (s.C * E) % ksb != 0) return false;
    const int64_t ks = s.C * E / ksb;
    if (ks != 1 && ks != 2 && ks != 4 && ks != 8 && ks != 16) return false;
    if (s.H * s.W * s.C * E >= ((int64_t)1 << 31)) return false;
    const int64_t ppitch = s.C * E;   // unpadded, swizzled staging
    const int64_t spitch = 33;
    const int64_t nk_bytes = s.F * s.kpitch * E;
    const int64_t ring_off = 256;   // past the coefficients; the NK rows are staged in the ring
    double best = 1e300;
    bool found = false;
    for (int64_t blocks = 1; blocks <= 4; ++blocks) {
        int64_t tw = (32 * blocks - s.S) / s.st + 1;
        if (tw < 1) continue;
        if (tw > s.Wo) tw = s.Wo;
        const int64_t pw = (tw - 1) * s.st + s.S;
        const int64_t prow = (pw * ppitch + 1023) / 1024 * 1024;
        const int64_t pslot = (pw * spitch * 4 + 15) / 16 * 16;
        const int64_t fixed = ring_off + (s.R + 1) * pslot;
        // two slots (one row in flight per workgroup): small workgroups, so
        // several share a CU and one's row work overlaps another's waits
        // (measured on the RGB layer: 29.0 us at two per CU with four slots,
        // 24.4 us at three per CU with three slots)
        int64_t nslot = 2;
        if (fixed + nslot * prow > dev.lds || nk_bytes > nslot * prow) continue;
        const int64_t strips = (s.Wo + tw - 1) / tw;
        const int64_t per = s.N * strips;
        const int64_t per_cu = dev.lds / (fixed + nslot * prow);   // workgroups per CU
        for (int64_t want : {(int64_t)dev.cus * per_cu, (int64_t)dev.cus * per_cu * 2}) {
            int64_t segs = want / per;
            if (segs < 1) segs = 1;
            if (segs > s.Ho) segs = s.Ho;
            const int64_t th = (s.Ho + segs - 1) / segs;
            const int64_t tiles_h = (s.Ho + th - 1) / th;
            const int64_t ph = (th - 1) * s.st + s.R;
            const int64_t tiles = per * tiles_h;
            const int64_t rounds = (tiles + dev.cus * per_cu - 1) / (dev.cus * per_cu);
            // fewer than four ring slots leave too few rows in flight
            const double cost =
                rounds * ((double)(ph * prow) / 16.0 + 2500.0 + (nslot < 4 ? 1000.0 : 400.0) * ph);
            if (cost < best) {
                best = cost;
                found = true;
                *out = BandPlan{(int)th, (int)tw, (int)ph, (int)pw, 0, (int)ring_off, (int)ppitch,
                                (int)prow, (int)spitch, (int)(fixed + nslot * prow),
                                (int)tiles_h, (int)strips, tiles, (int)nslot};
            }
        }
    }
    return found;
}

// An output map (ConvArgs::ymap): GEMM pixel (n, oh, ow) to output pixel
// (n, oh*ysh, ow*ysw) of images of Hy x Wy pixels.
struct OutMap {
    int Hy, Wy, ysh, ysw;
};

// Plan of the patch-resident kernel (igemm_patch.hpp), or false when the
// layer does not fit it: C_out > 64 and a multiple of 4, stride 1, R*S >= 2,
// C_in a whole number of 128-byte chunks, an image's input and output each
// below 2^31 bytes (an output row below 2^24).  Workgroups of 64*TM output
// channels (TM = 4, or 2 when C_out <= 128) and 256 pixel slots; the tile
// TH x TW of one image (TW = W_out or a power of two from 8 to 256 below
// it, at least 8; TH = 256 / TW or H_out) must fill at least 3/4 of the
// slots, and the tiles at least one round of one workgroup per CU, three
// quarters of the last round busy.  Among those: the fewest rounds, then
// three filter stages over two, then the smallest patch (the input bytes
// each tile stages).  When no 256-slot tile qualifies, the same with 128
// pixel slots (two 32-pixel blocks per wave), which gives mid-size layers
// enough tiles.  A grouped launch of `groups` problems counts all their
// tiles; an output map (map) sets the output image and row the limits
// above apply to.
bool patch_plan(const Shape& s, int32_t dtype, PatchPlan* out, const DevInfo& dev,
                int groups = 1, const OutMap* map = nullptr) {
    const int64_t E = elem_bytes(dtype);
    if (s.F <= 64 || s.F % 4 != 0 || s.st != 1 || s.R * s.S < 2 || (s.C * E) % 128 != 0)
        return false;
    const int64_t hy = map ? map->Hy : s.Ho, wy = map ? map->Wy : s.Wo;
    const int64_t row_px = map ? (int64_t)map->ysh * map->Wy : s.Wo;   // pixels per tile row
    if (s.H * s.W * s.C * E >= ((int64_t)1 << 31) || hy * wy * s.F * 2 >= ((int64_t)1 << 31))
        return false;
    // the epilogue's 24-bit offset arithmetic: an output row below 2^24 bytes
    if (row_px * s.F * 2 >= ((int64_t)1 << 24)) return false;
    const int64_t ng = groups > 1 ? groups : 1;
    const int tm = s.F > 128 ? 4 : 2;
    const int64_t bco = 64 * tm;
    const int64_t co_tiles = (s.F + bco - 1) / bco;
    const int64_t epi = 4 * 32 * (tm * 32 * 4 + 16);   // the epilogue's per-wave regions
    for (int64_t bpx : {256, 128}) {
        int64_t tws[7];
        int ntw = 0;
        if (s.Wo <= bpx) tws[ntw++] = s.Wo;
        for (int64_t c : {8, 16, 32, 64, 128, 256})
            if (c < s.Wo && c <= bpx) tws[ntw++] = c;
        bool found = false;
        int64_t best_rounds = 0, best_patch = 0;
        int best_ns = 0;
        for (int k = 0; k < ntw; ++k) {
            const int64_t tw = tws[k];
            const int64_t th = s.Ho < bpx / tw ? s.Ho : bpx / tw;
            // (tiles at least 8 pixels wide: the epilogue walks a lane's
            // pixels 2 or 4 columns at a time with at most one wrap per step)
            if (tw < 8 || th < 1 || 4 * th * tw < 3 * bpx) continue;
            const int64_t ph = th - 1 + s.R, pw = tw - 1 + s.S;
            const int64_t prow = pw * PATCH_PP + (((tw - pw) * PATCH_PP) % 256 + 256) % 256;
            const int64_t patch = (ph * prow + 1023) / 1024 * 1024;   // whole 1 KB request blocks
            int ns = 0;
            int64_t lds = 0;
            for (int c : {3, 2}) {
                lds = c * bco * 128 + patch;
                if (lds < epi) lds = epi;
                if (lds <= dev.lds) {
                    ns = c;
                    break;
                }
            }
            if (ns == 0) continue;
            const int64_t tiles_h = (s.Ho + th - 1) / th, tiles_w = (s.Wo + tw - 1) / tw;
            const int64_t tiles = s.N * tiles_h * tiles_w * co_tiles;   // per problem
            const int64_t all = tiles * ng;
            if (all < dev.cus) continue;
            const int64_t rounds = (all + dev.cus - 1) / dev.cus;
            if (4 * (all - (rounds - 1) * dev.cus) < 3 * dev.cus) continue;
            const bool better = !found || rounds < best_rounds ||
                                (rounds == best_rounds &&
                                 (ns > best_ns || (ns == best_ns && patch < best_patch)));
            if (better) {
                found = true;
                best_rounds = rounds;
                best_ns = ns;
                best_patch = patch;
                *out = PatchPlan{(int)th, (int)tw, (int)ph, (int)pw, (int)prow, (int)lds,
                                 (int)tiles_h, (int)tiles_w, tm, (int)(bpx / 64), ns, tiles};
            }
        }
        if (found) return true;
    }
    return false;
}

// The kernel a problem goes to, in order of preference.
enum KernelKind { K_NONE, K_TAPFOLD, K_BAND, K_PATCH, K_WIDE, K_RESIDENT, K_TILED };

// tapfold_ok: the tap-fold kernel may be chosen (it has no output map and
// is only exercised on the page's symmetric paddings); groups, map: a
// grouped launch of that many problems, an output map (the patch kernel's
// plan counts the tiles of all the problems).
KernelKind select_kernel(const Shape& s, int32_t dtype, BandPlan* bp, bool tapfold_ok = true,
                         const DevInfo& dev = DevInfo{}, PatchPlan* pp = nullptr,
                         int groups = 1, const OutMap* map = nullptr) {
    if (s.M == 0 || s.F == 0) return K_NONE;
    // C_in not a whole number of 16-byte vectors: only the tiled kernel's
    // element gather takes it
    if ((s.C * elem_bytes(dtype)) % 16 != 0) return K_TILED;
    if (tapfold_ok && tapfold_plan(s, dtype, bp, dev)) return K_TAPFOLD;
    if (band_plan(s, dtype, bp, dev)) return K_BAND;
    PatchPlan tmp;
    if (patch_plan(s, dtype, pp ? pp : &tmp, dev, groups, map)) return K_PATCH;
    if (wide_ok(s, dtype)) return K_WIDE;
    if (resident_ok(s, dtype)) return K_RESIDENT;
    return K_TILED;
}

// Several problems of one shape in one launch (the phases of a strided
// transposed convolution): NK matrices a fixed byte stride apart; problem
// gi = gh*split + gw (split = 0: gh = 0, gw = gi) writes its output at
// gw*y + gh*y2 bytes and reads its source at gw*src + gh*src2 bytes past
// the first's, and has its padding lowered by gh*dpt (top), gw*dpl (left).
struct Group {
    int n;
    int64_t nk, y, src;
    int split = 0;
    int64_t y2 = 0, src2 = 0;
    int dpt = 0, dpl = 0;
};

template <int DT>
hipError_t launch_kind(KernelKind kind, bool resid, const ConvArgs& a, const BandPlan& bp,
                       const PatchPlan& pp, hipStream_t stream) {
    switch (kind) {
        case K_PATCH: return launch_patch_any<DT>(resid, a, pp, stream);
        case K_TAPFOLD: return launch_tapfold_any<DT>(resid, a, bp, stream);
        case K_BAND: return launch_band_any<DT>(resid, a, bp, stream);
        case K_WIDE: return launch_wide_any<DT>(resid, a, stream);
        case K_RESIDENT: return launch_resident_any<DT>(resid, a, stream);
        default: return launch_tiled_any<DT>(resid, a, stream);
    }
}

// The kernel arguments every family reads, for problem s (one group's
// shape); the tiled kernel's general geometry is set to the page form
// (square stride, symmetric padding, unit dilation, dense pixels).
ConvArgs base_args(const void* input, const void* nk, void* output, const void* source,
                   float beta, const igc_epilogue* epi, const Shape& s, int32_t dtype) {
    ConvArgs a{};
    a.x = (const uint8_t*)input;
    a.nk = (const uint8_t*)nk;
    a.y = (uint16_t*)output;
    a.src = (const uint16_t*)source;
    a.beta = beta;
    if (epi) {
        a.scale = epi->scale;
        a.bias = epi->bias;
        a.act = epi->activation;
        a.epi = (a.scale || a.bias || a.act != IGC_ACT_NONE) ? 1 : 0;
    }
    a.H = (int)s.H; a.W = (int)s.W; a.C = (int)s.C;
    a.Ho = (int)s.Ho; a.Wo = (int)s.Wo; a.F = (int)s.F;
    a.R = (int)s.R; a.S = (int)s.S; a.stride = s.st;
    a.K = (int)s.K; a.kpitch = (int)s.kpitch; a.M = (int)s.M;
    a.ktiles = (int)(s.kpad / (KT_BYTES / elem_bytes(dtype)));
    a.pt = s.pt;
    a.pl = s.pl;
    a.sh = a.sw = s.st;
    a.dh = a.dw = 1;
    a.xpitch = (int)s.C;
    a.ypitch = (int)s.F;
    a.ymap = 0;
    a.Hy = (int)s.Ho;
    a.Wy = (int)s.Wo;
    a.ysh = a.ysw = 1;
    return a;
}

// wraw: the stored filter (RSCF, or FCRS when wfcrs), passed instead of an
// NK matrix to a problem for which filter_in_kernel holds.
hipError_t launch_igemm(const void* input, const void* nk, void* output, const void* source,
                        float beta, const igc_epilogue* epi, const Shape& s, int32_t dtype,
                        hipStream_t stream, const Group* grp = nullptr, bool tapfold_ok = true,
                        const OutMap* map = nullptr, const void* wraw = nullptr,
                        int32_t wfcrs = 0) {
    ConvArgs a = base_args(input, nk, output, source, beta, epi, s, dtype);
    a.wraw = (const uint8_t*)wraw;
    a.wrs = wfcrs ? (int)(s.R * s.S) : 0;
    if (grp && grp->n > 1) {
        a.groups = grp->n;
        a.g_nk = grp->nk;
        a.g_y = grp->y;
        a.g_src = grp->src;
        a.gsplit = grp->split;
        a.g_y2 = grp->y2;
        a.g_src2 = grp->src2;
        a.g_pt = grp->dpt;
        a.g_pl = grp->dpl;
    }
    if (map) {
        a.ymap = 1;
        a.Hy = map->Hy;
        a.Wy = map->Wy;
        a.ysh = map->ysh;
        a.ysw = map->ysw;
        tapfold_ok = false;
    }
    const bool resid = source != nullptr;
    BandPlan bp;
    PatchPlan pp;
    const KernelKind kind = select_kernel(s, dtype, &bp, tapfold_ok, device_info(), &pp,
                                          grp ? grp->n : 1, map);
    if (kind == K_NONE) return hipSuccess;
    if (wraw && kind != K_BAND) return hipErrorInvalidValue;
    switch (dtype) {
        case IGC_DTYPE_BF16: return launch_kind<DT_BF16>(kind, resid, a, bp, pp, stream);
        case IGC_DTYPE_FP16: return launch_kind<DT_FP16>(kind, resid, a, bp, pp, stream);
        default: return launch_kind<DT_FP8>(kind, resid, a, bp, pp, stream);
    }
}

// One launch instead of two: the band kernel transposes the stored filter
// into its LDS itself, so no NK matrix and no transpose launch are needed.
// Its register transposes take whole 16-byte loads of 2-byte elements
// (bf16, fp16): an RSCF filter needs C_out a multiple of 8, an FCRS filter
// R*S of 1 or 9 (the register transposes are built for those tap counts:
// 1x1 and 3x3 filters; a 25-tap block needed 100 registers).  (The tap-fold kernel keeps its NK
// matrix: with its many small workgroups, making the rows in each one cost
// more than the transpose launch saved, measured on the RGB layer: 22.0 ->
// 23.9 us kernel.)
bool raw_filter_ok(const Shape& s, int32_t dtype, int32_t fcrs) {
    if (s.M == 0 || s.F == 0 || dtype == IGC_DTYPE_FP8_E4M3FN) return false;
    return fcrs ? (s.R * s.S == 1 || s.R * s.S == 9) : s.F % 8 == 0;
}

bool filter_in_kernel(const Shape& s, int32_t dtype, int32_t fcrs, bool tapfold_ok = true) {
    if (!raw_filter_ok(s, dtype, fcrs)) return false;
    BandPlan bp;
    return select_kernel(s, dtype, &bp, tapfold_ok, device_info()) == K_BAND;
}

FastDiv make_fastdiv(uint32_t d) {
    uint32_t sh = 0;
    while (sh < 31 && ((uint64_t)1 << sh) < d) ++sh;
    const uint64_t m = (((uint64_t)1 << (32 + sh)) + d - 1) / d;
    return FastDiv{(uint32_t)(m - ((uint64_t)1 << 32)), sh};
}

// Shapes of the materialised im2col: the convolution gate applied to a
// filter of R x S taps (C_out plays no part), plus the 16-byte vector count
// below 2^31.  Row pitch Kp: K rounded up to whole 128-byte k-tiles.
int32_t im2col_shape(const int64_t in_nhwc[4], const int64_t filt_rs[2],
                     const int32_t stride[2], const int32_t padding[2], int32_t dtype,
                     Shape* sh, int64_t* kp) {
    if (!in_nhwc || !filt_rs) return IGC_DECLINE_NULL_POINTER;
    const int64_t fd[4] = {filt_rs[0], filt_rs[1], in_nhwc[3], 1};
    const int32_t dil[2] = {1, 1};
    const int64_t eb = elem_bytes(dtype);
    // Ho, Wo as the gate computes them (a first pass fills the shape)
    Shape s{};
    int64_t od[4] = {in_nhwc[0], 1, 1, 1};
    if (stride && padding && filt_rs[0] >= 1 && filt_rs[1] >= 1 && stride[0] >= 1 &&
        stride[1] >= 1) {
        od[1] = out_size(in_nhwc[1], filt_rs[0], stride[0], padding[0]);
        od[2] = out_size(in_nhwc[2], filt_rs[1], stride[1], padding[1]);
    }
    const int32_t rc = check_shapes(in_nhwc, 0, fd, od, stride, dil, padding, 1, dtype, &s);
    if (rc != IGC_OK) return rc;
    // the im2col kernel moves 16-byte vectors of one tap
    if ((s.C * eb) % 16 != 0) return IGC_DECLINE_VECTOR_WIDTH;
    if ((s.M * s.kpad * eb) / 16 >= ((int64_t)1 << 31)) return IGC_DECLINE_SIZE_LIMIT;
    *sh = s;
    *kp = s.kpad;
    return IGC_OK;
}

// ---- transposed convolution (page "conv_transposed_gpu") -----------------
// Definition (cross-correlation form; per axis stride st, dilation d and
// padding p cut from both ends):
//   out[n, oh, ow, f] = sum over oh = ih*st - p + r*d, ow = iw*st - p + s*d
//                       of in[n, ih, iw, c] * W[r][s][f][c]
// Along one axis, the output rows of phase a (oh = st*q + a, 0 <= a < st)
// take the taps r with r*d = a + p (mod st).  With g = gcd(st, d) these are
// r = B + L*j, j < J (L = st/g, B the smallest such tap, J = 0 when there is
// none below R), at input row ih = q + c - j*e with e = d/g and
// c = (a + p - B*d)/st.  Read with the taps in increasing input order
// (j' = J - 1 - j) that is a stride-1 forward correlation with J taps at
// dilation e and padding P = (J - 1)*e - c before the axis (negative P: the
// window starts inside the image), whose output row q is output row
// st*q + a.  Each (row phase, column phase) pair is thus one forward
// implicit GEMM over the whole input, with its tap subset flipped and the
// channel roles swapped as NK matrix, that stores through an output map
// straight into every st-th row and column of the output from (a_h, a_w),
// reading the residual source at the same places: no phase buffers, and the
// fused epilogue with its single rounding stays in the GEMMs.  A phase with
// no tap gets the epilogue alone (a GEMM with K = 0).
struct TAxis {
    int J = 0, B = 0, L = 1, e = 1, P = 0;
    int64_t Q = 0;   // output rows (columns) of the phase
};

struct TPhase {
    int ah = 0, aw = 0;
    Shape s{};        // the phase's forward problem (R = JH, S = JW, Ho = QH, Wo = QW)
    TAxis h, w;
    size_t nk_off = 0;
};

struct TPlan {
    int64_t N = 0, H = 0, W = 0, C = 0, R = 0, S = 0, F = 0, Ho = 0, Wo = 0;
    int32_t sh = 1, sw = 1;
    std::vector<TPhase> ph;
    size_t ws_bytes = 0;
    bool grouped = false;   // every phase one shape: one grouped launch
    int dpt = 0, dpl = 0;   // padding step between phase rows / columns (grouped)
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

TAxis axis_phase(int64_t a, int64_t st, int64_t d, int64_t p, int64_t R, int64_t out) {
    TAxis x;
    const int64_t g = gcd64(st, d);
    x.L = (int)(st / g);
    x.e = (int)(d / g);
    x.Q = a < out ? (out - a + st - 1) / st : 0;
    for (int64_t r = 0; r < x.L && r < R; ++r) {
        if (((a + p - r * d) % st + st) % st == 0) {
            x.B = (int)r;
            x.J = (int)((R - 1 - r) / x.L + 1);
            const int64_t c = (a + p - r * d) / st;   // exact
            x.P = (int)((x.J - 1) * (int64_t)x.e - c);
            break;
        }
    }
    return x;
}

// The phase's forward problem within the forward kernels' limits (those of
// check_shapes), or false.
bool phase_shape(const TPlan& t, const TAxis& h, const TAxis& w, int64_t eb, Shape* out) {
    Shape s{};
    s.N = t.N; s.H = t.H; s.W = t.W; s.C = t.C; s.F = t.F;
    s.R = h.J; s.S = w.J;
    s.Ho = h.Q; s.Wo = w.Q;
    s.st = 1;
    s.pad = 0;
    s.pt = h.P;
    s.pl = w.P;
    const int64_t lim = (int64_t)1 << 31;
    s.M = s.N * s.Ho * s.Wo;
    s.K = s.R * s.S * s.C;
    if (s.M >= lim || s.K >= lim || (s.R * s.W + s.S) * s.C >= lim) return false;
    s.kpad = round_up(s.K, KT_BYTES / eb);
    s.kpitch = nk_pitch(s.K, s.F, eb);
    if (s.kpitch >= lim || s.F * s.kpitch * eb >= lim) return false;
    *out = s;
    return true;
}

int32_t transposed_plan(const int64_t in_nhwc[4], const int64_t filt_rsfc[4],
                        const int64_t out_nhwc[4], const int32_t stride[2],
                        const int32_t dilation[2], const int32_t padding[2], int32_t dtype,
                        TPlan* tp) {
    if (!in_nhwc || !filt_rsfc || !out_nhwc || !stride || !dilation || !padding)
        return IGC_DECLINE_NULL_POINTER;
    if (dtype != IGC_DTYPE_BF16 && dtype != IGC_DTYPE_FP16 && dtype != IGC_DTYPE_FP8_E4M3FN)
        return IGC_DECLINE_DTYPE;
    if (stride[0] < 1 || stride[1] < 1) return IGC_DECLINE_STRIDE;
    if (dilation[0] < 1 || dilation[1] < 1) return IGC_DECLINE_DILATION;
    if (padding[0] < 0 || padding[1] < 0) return IGC_DECLINE_PADDING;
    TPlan t;
    t.sh = stride[0];
    t.sw = stride[1];
    t.N = in_nhwc[0]; t.H = in_nhwc[1]; t.W = in_nhwc[2]; t.C = in_nhwc[3];
    t.R = filt_rsfc[0]; t.S = filt_rsfc[1]; t.F = filt_rsfc[2];
    if (t.R < 1 || t.S < 1 || t.F < 0 || t.C < 0 || filt_rsfc[3] != t.C || t.N < 0 || t.H < 1 ||
        t.W < 1)
        return IGC_DECLINE_SHAPE;
    const int64_t lim = (int64_t)1 << 31, l30 = (int64_t)1 << 30;
    if (t.N >= lim || t.H >= lim || t.W >= lim || t.C >= lim || t.F >= lim || t.R >= lim ||
        t.S >= lim)
        return IGC_DECLINE_SIZE_LIMIT;
    // output extents before the padding is cut, and the padding, below 2^30:
    // every phase coordinate then fits the kernels' 32-bit arithmetic
    const int64_t fh = (t.H - 1) * t.sh + (int64_t)dilation[0] * (t.R - 1) + 1;
    const int64_t fw = (t.W - 1) * t.sw + (int64_t)dilation[1] * (t.S - 1) + 1;
    if (fh >= l30 || fw >= l30 || padding[0] >= l30 || padding[1] >= l30)
        return IGC_DECLINE_SIZE_LIMIT;
    t.Ho = fh - 2 * (int64_t)padding[0];
    t.Wo = fw - 2 * (int64_t)padding[1];
    if (t.Ho < 1 || t.Wo < 1 || out_nhwc[0] != t.N || out_nhwc[1] != t.Ho ||
        out_nhwc[2] != t.Wo || out_nhwc[3] != t.F)
        return IGC_DECLINE_OUTPUT_SHAPE;
    const int64_t eb = elem_bytes(dtype);
    // the wide kernel places a 32-pixel block's mapped pixels at 32-bit byte
    // offsets from its first one
    if ((33 * t.sh * t.Wo + 32 * (int64_t)t.sw) * t.F * 2 >= lim) return IGC_DECLINE_SIZE_LIMIT;
    if (t.sh * (int64_t)t.sw > 4096) return IGC_DECLINE_SIZE_LIMIT;
    size_t off = 0;
    for (int ah = 0; ah < t.sh; ++ah) {
        const TAxis h = axis_phase(ah, t.sh, dilation[0], padding[0], t.R, t.Ho);
        for (int aw = 0; aw < t.sw; ++aw) {
            const TAxis w = axis_phase(aw, t.sw, dilation[1], padding[1], t.S, t.Wo);
            TPhase p;
            p.ah = ah;
            p.aw = aw;
            p.h = h;
            p.w = w;
            if (h.Q == 0 || w.Q == 0) continue;   // no output pixel of this phase
            if (!phase_shape(t, h, w, eb, &p.s)) return IGC_DECLINE_SIZE_LIMIT;
            p.nk_off = off;
            off += align256((size_t)(p.s.F * p.s.kpitch * eb));
            t.ph.push_back(p);
        }
    }
    t.ws_bytes = off;
    // one grouped launch when every phase has one shape and the paddings step
    // evenly from phase to phase (always so for strides of 1 and 2)
    const size_t nph = t.ph.size();
    t.grouped = nph == (size_t)t.sh * t.sw && nph > 1;
    if (t.grouped) {
        const TPhase& p0 = t.ph[0];
        const TPhase& p1 = t.ph[nph - 1];
        t.dpt = t.sh > 1 ? (p0.h.P - p1.h.P) / (t.sh - 1) : 0;
        t.dpl = t.sw > 1 ? (p0.w.P - p1.w.P) / (t.sw - 1) : 0;
        for (const TPhase& p : t.ph) {
            if (p.h.J != p0.h.J || p.w.J != p0.w.J || p.h.Q != p0.h.Q || p.w.Q != p0.w.Q ||
                p.h.e != p0.h.e || p.w.e != p0.w.e || p.h.P != p0.h.P - p.ah * t.dpt ||
                p.w.P != p0.w.P - p.aw * t.dpl)
                t.grouped = false;
        }
    }
    *tp = t;
    return IGC_OK;
}

// Pointer rules of the transposed convolution (as conv2d_fwd's, plus the
// coefficient arrays of the epilogue against the workspace).
int32_t transposed_pointers(const TPlan& t, int32_t dtype, const void* input, const void* filter,
                            const void* output, const void* source, const igc_epilogue* epi,
                            const void* workspace, size_t workspace_bytes) {
    const size_t eb = (size_t)elem_bytes(dtype);
    const size_t in_bytes = (size_t)(t.N * t.H * t.W * t.C) * eb;
    const size_t f_bytes = (size_t)(t.R * t.S * t.F * t.C) * eb;
    const size_t out_bytes = (size_t)(t.N * t.Ho * t.Wo * t.F) * 2;
    if ((in_bytes && !input) || (f_bytes && !filter) || (out_bytes && !output))
        return IGC_DECLINE_NULL_POINTER;
    if (!aligned16(input) || !aligned16(filter) || !aligned16(output) || !aligned16(source) ||
        !aligned16(workspace))
        return IGC_DECLINE_ALIGNMENT;
    if (overlaps(output, out_bytes, input, in_bytes) || overlaps(output, out_bytes, filter, f_bytes))
        return IGC_DECLINE_OVERLAP;
    if (source && source != output && overlaps(source, out_bytes, output, out_bytes))
        return IGC_DECLINE_OVERLAP;
    if (workspace) {
        const size_t w = t.ws_bytes;
        if (overlaps(workspace, w, output, out_bytes) || overlaps(workspace, w, input, in_bytes) ||
            overlaps(workspace, w, filter, f_bytes) ||
            (source && overlaps(workspace, w, source, out_bytes)))
            return IGC_DECLINE_OVERLAP;
        if (workspace_bytes < w) return IGC_DECLINE_WORKSPACE;
        if (epi) {
            for (const float* c : {epi->scale, epi->bias})
                if (c && overlaps(c, (size_t)t.F * sizeof(float), workspace, w))
                    return IGC_DECLINE_EPILOGUE;
        }
    }
    Shape so{};
    so.M = t.N * t.Ho * t.Wo;
    so.F = t.F;
    return check_epilogue(epi, output, so);
}

// The flipped NK matrices of every phase, four phases per launch (grid rows
// = phases); ws + nk_off receives each phase's.
hipError_t launch_transpose_flipped(const void* filter, const TPlan& t, int32_t dtype, uint8_t* ws,
                                    hipStream_t stream) {
    const int eb = elem_bytes(dtype);
    for (size_t b = 0; b < t.ph.size(); b += 4) {
        TapSels ts{};
        int64_t most = 0;
        const int cnt = (int)(t.ph.size() - b < 4 ? t.ph.size() - b : 4);
        for (int i = 0; i < cnt; ++i) {
            const TPhase& p = t.ph[b + i];
            TapSel& sel = ts.t[i];
            sel.R = (int)t.R; sel.S = (int)t.S; sel.F = (int)t.F; sel.C = (int)t.C;
            sel.BH = p.h.B; sel.BW = p.w.B;
            sel.JH = p.h.J; sel.JW = p.w.J;
            sel.LH = p.h.L; sel.LW = p.w.L;
            sel.K = (int)p.s.K;
            sel.kpitch = (int)p.s.kpitch;
            ts.nk[i] = ws + p.nk_off;
            const int64_t chunks = p.s.F * (p.s.kpitch / (16 / eb));
            if (chunks > most) most = chunks;
        }
        if (most == 0) continue;
        const dim3 grid((unsigned)((most + 255) / 256 < 4096 ? (most + 255) / 256 : 4096),
                        (unsigned)cnt);
        if (eb == 2)
            hipLaunchKernelGGL(filter_rsfc_to_nk_flipped_kernel<2>, grid, dim3(256), 0, stream,
                               (const uint8_t*)filter, ts);
        else
            hipLaunchKernelGGL(filter_rsfc_to_nk_flipped_kernel<1>, grid, dim3(256), 0, stream,
                               (const uint8_t*)filter, ts);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// One phase GEMM (or all of them, grouped): the forward kernels when the
// phase has unit dilation and at least one tap, else the tiled kernel with
// the phase's dilation (and K = 0 for a phase without taps).
hipError_t launch_phase(const TPlan& t, const TPhase& p, const void* input, const uint8_t* nk,
                        void* out, const void* src, float beta, const igc_epilogue* epi,
                        int32_t dtype, hipStream_t stream, const Group* grp) {
    const OutMap map{(int)t.Ho, (int)t.Wo, t.sh, t.sw};
    const bool ident = t.sh == 1 && t.sw == 1;
    if (p.h.e == 1 && p.w.e == 1 && p.s.K > 0)
        return launch_igemm(input, nk, out, src, beta, epi, p.s, dtype, stream, grp, false,
                            ident ? nullptr : &map);
    ConvArgs a = base_args(input, nk, out, src, beta, epi, p.s, dtype);
    a.dh = p.h.e;
    a.dw = p.w.e;
    if (!ident) {
        a.ymap = 1;
        a.Hy = map.Hy; a.Wy = map.Wy; a.ysh = map.ysh; a.ysw = map.ysw;
    }
    if (grp && grp->n > 1) {
        a.groups = grp->n;
        a.g_nk = grp->nk; a.g_y = grp->y; a.g_src = grp->src;
        a.gsplit = grp->split; a.g_y2 = grp->y2; a.g_src2 = grp->src2;
        a.g_pt = grp->dpt; a.g_pl = grp->dpl;
    }
    const bool resid = src != nullptr;
    switch (dtype) {
        case IGC_DTYPE_BF16: return launch_tiled_any<DT_BF16>(resid, a, stream);
        case IGC_DTYPE_FP16: return launch_tiled_any<DT_FP16>(resid, a, stream);
        default: return launch_tiled_any<DT_FP8>(resid, a, stream);
    }
}

hipError_t run_transposed(const TPlan& t, const void* input, const void* filter, void* output,
                          const void* source, float beta, const igc_epilogue* epi, int32_t dtype,
                          uint8_t* ws, hipStream_t stream) {
    hipError_t e = launch_transpose_flipped(filter, t, dtype, ws, stream);
    const int64_t px = t.F * 2;   // bytes per output pixel
    if (t.grouped) {
        // phase gi = ah*sw + aw starts at output pixel (ah, aw)
        Group g{(int)t.ph.size(), (int64_t)(t.ph[1].nk_off - t.ph[0].nk_off), px,
                source ? px : 0};
        g.split = t.sw;
        g.y2 = t.Wo * px;
        g.src2 = source ? t.Wo * px : 0;
        g.dpt = t.dpt;
        g.dpl = t.dpl;
        if (e == hipSuccess)
            e = launch_phase(t, t.ph[0], input, ws + t.ph[0].nk_off, output, source, beta, epi,
                             dtype, stream, &g);
        return e;
    }
    for (const TPhase& p : t.ph) {
        if (e != hipSuccess) break;
        const int64_t o = (p.ah * t.Wo + p.aw) * px;
        e = launch_phase(t, p, input, ws + p.nk_off, (uint8_t*)output + o,
                         source ? (const void*)((const uint8_t*)source + o) : nullptr, beta, epi,
                         dtype, stream, nullptr);
    }
    return e;
}

// ---- general forward convolution -----------------------------------------
// The parameters page "dispatch_amd_4wave_conv2d" (Args) lists and its
// dispatcher restricts, widened: per-axis stride, dilation, padding before
// and after each axis, and channel groups.  A problem inside the page's gate
// runs exactly as conv2d_fwd.  One group at unit dilation and equal strides
// with any other padding or stride runs on the same forward kernels (each
// takes the padding before each axis and any stride; the tap-fold kernel is
// left to the page's problems).  Several groups at unit dilation and stride (1,1) or
// (2,2) run as super-groups on the band kernel when its gate admits them
// (see supergroup_plan); one group at stride 1 with dilation as dilation
// phases on the band kernel (see dilation_plan).  Any other problem runs on
// the tiled kernel with its general geometry, the groups as one grouped
// launch (group g reads input channels g*Cg.., NK rows, output channels,
// source channels and scale / bias entries g*Fg..).
struct GShape {
    Shape s;          // C = C_in per group (Cg), F = all output channels
    int64_t cin;      // input channels, groups * Cg
    int32_t sh, sw, dh, dw, pt, pl, pb, pr, groups;
    bool page;        // inside the page's gate: conv2d_fwd's kernels run it
    bool fast;        // one group, unit dilation, equal strides, any
                      // padding: the forward kernels (but the tap-fold one) run it
    int32_t q;        // > 0: groups run as super-groups of q (sg below)
    Shape sg;         // one super-group's problem (C = q*Cg, F = q*Fg, its K,
                      // kpad and kpitch); N, H, W, Ho, Wo, R, S as s
    int64_t nk_bytes; // the NK matrix's bytes (all output channels' rows)
    bool dil;         // dilation phases (sd below)
    Shape sd;         // one dilation phase's problem: the input view H/dh x
                      // W/dw, output Ho/dh x Wo/dw, padding pt/dh, pl/dw,
                      // stride 1 and no dilation; C, F, R, S, K as s
};

int64_t out_size_general(int64_t in, int64_t k, int64_t st, int64_t dil, int64_t pb, int64_t pe) {
    const int64_t span = in + pb + pe - dil * (k - 1) - 1;
    return span < 0 ? 0 : span / st + 1;
}

// Super-groups: q consecutive channel groups form one problem of q*Cg input
// and q*Fg output channels whose NK matrix is block diagonal (zero where an
// input channel's group differs from the output channel's), and the G/q
// problems run as one grouped launch of the band kernel: each reads its
// input channels at pixel pitch C_in and writes its output channels at
// pixel pitch C_out.  The zero blocks cost MFMA work (q times the useful
// products) but the gathers become whole 16-byte chunks of q*Cg channels,
// where the tiled kernel's grouped launch gathers Cg channels per pixel.
// The band kernel's gate applies to the super-group: q*Fg <= 64, q*Cg
// elements a power-of-two multiple of the MFMA k-step, one image below
// 2^31 bytes.  q is the divisor of G with the lowest band-kernel cost
// estimate over the whole grouped launch.
void supergroup_plan(GShape& t, int32_t dtype, const DevInfo& dev) {
    const Shape& s = t.s;
    if (t.groups < 2 || t.dh != 1 || t.dw != 1 || t.sh != t.sw || t.sh > 2) return;
    const int64_t eb = elem_bytes(dtype);
    const int64_t lim = (int64_t)1 << 31;
    const int64_t fg = s.F / t.groups;
    if (fg < 1 || s.M == 0 || s.C < 1) return;
    if (s.H * s.W * t.cin * eb >= lim) return;
    double best = 1e300;
    for (int64_t q = 1; q <= t.groups && q * fg <= 64; ++q) {
        if (t.groups % q) continue;
        Shape u = s;
        u.C = q * s.C;
        u.F = q * fg;
        u.K = s.R * s.S * u.C;
        if (u.K >= lim) continue;
        u.kpad = round_up(u.K, KT_BYTES / eb);
        u.kpitch = nk_pitch(u.K, u.F, eb);
        if (u.kpitch >= lim || s.F * u.kpitch * eb >= lim) continue;
        // plan over the whole grouped launch: G/q times the images
        Shape pl = u;
        pl.N = s.N * (t.groups / q);
        BandPlan bp;
        double cost = 0;
        if (!band_plan(pl, dtype, &bp, dev, &cost)) continue;
        if (bp.tiles >= lim) continue;
        if (cost < best) {
            best = cost;
            t.q = (int32_t)q;
            t.sg = u;
        }
    }
    if (t.q > 0) t.nk_bytes = s.F * t.sg.kpitch * eb;
}

// Dilation phases: at stride 1, output row oh = a + dh*i (phase a < dh)
// reads input rows oh - pt + dh*r = a + dh*(i + r - pt/dh) when dh divides
// pt: only rows a, a + dh, ..., an undilated convolution with padding
// pt/dh over every dh-th input row, and likewise along the width.  When dh
// and dw divide the padding before each axis and the input and output
// extents, the dh*dw phases have one shape and run as one grouped launch of
// the band kernel: phase (a_h, a_w) reads the input view of every dh-th row
// and dw-th column from pixel (a_h, a_w) and stores through an output map
// (view pixel (i, j) -> output pixel (a_h + dh*i, a_w + dw*j)), with the
// plain NK matrix.  The same products as the definition, only grouped by
// phase.
void dilation_plan(GShape& t, int32_t dtype, const DevInfo& dev) {
    const Shape& s = t.s;
    if (t.groups != 1 || t.sh != 1 || t.sw != 1 || (t.dh == 1 && t.dw == 1)) return;
    if (t.pt % t.dh || t.pl % t.dw || s.H % t.dh || s.W % t.dw || s.Ho % t.dh || s.Wo % t.dw)
        return;
    if (s.M == 0 || s.F == 0 || s.H * s.W * s.C * elem_bytes(dtype) >= ((int64_t)1 << 31)) return;
    Shape u = s;
    u.H = s.H / t.dh; u.W = s.W / t.dw;
    u.Ho = s.Ho / t.dh; u.Wo = s.Wo / t.dw;
    u.st = 1;
    u.pt = t.pt / t.dh; u.pl = t.pl / t.dw;
    u.M = u.N * u.Ho * u.Wo;
    Shape pl = u;
    pl.N = u.N * t.dh * t.dw;
    BandPlan bp;
    if (!band_plan(pl, dtype, &bp, dev)) return;
    if (bp.tiles >= ((int64_t)1 << 31)) return;
    t.dil = true;
    t.sd = u;
}

int32_t check_general_shapes(const int64_t in_nhwc[4], int32_t fcrs, const int64_t filt_dims[4],
                             const int64_t out_nhwc[4], const igc_conv_params* p, int32_t dtype,
                             GShape* g) {
    if (!in_nhwc || !filt_dims || !out_nhwc || !p) return IGC_DECLINE_NULL_POINTER;
    if (dtype != IGC_DTYPE_BF16 && dtype != IGC_DTYPE_FP16 && dtype != IGC_DTYPE_FP8_E4M3FN)
        return IGC_DECLINE_DTYPE;
    if (p->stride[0] < 1 || p->stride[1] < 1) return IGC_DECLINE_STRIDE;
    if (p->dilation[0] < 1 || p->dilation[1] < 1) return IGC_DECLINE_DILATION;
    if (p->pad_begin[0] < 0 || p->pad_begin[1] < 0 || p->pad_end[0] < 0 || p->pad_end[1] < 0)
        return IGC_DECLINE_PADDING;
    if (p->groups < 1) return IGC_DECLINE_GROUPS;
    GShape t{};
    Shape& s = t.s;
    s.N = in_nhwc[0]; s.H = in_nhwc[1]; s.W = in_nhwc[2];
    t.cin = in_nhwc[3];
    filter_rscf(filt_dims, fcrs, &s.R, &s.S, &s.C, &s.F);
    if (s.N < 0 || s.H < 0 || s.W < 0 || t.cin < 0 || s.F < 0 || s.C < 0 || s.R < 1 || s.S < 1)
        return IGC_DECLINE_SHAPE;
    const int64_t lim = (int64_t)1 << 31;
    if (s.H >= lim || s.W >= lim || s.R >= lim || s.S >= lim || s.C >= lim || s.F >= lim ||
        t.cin >= lim)
        return IGC_DECLINE_SIZE_LIMIT;
    t.groups = p->groups;
    if (s.C * t.groups != t.cin) return IGC_DECLINE_SHAPE;
    if (s.F % t.groups != 0) return IGC_DECLINE_GROUPS;
    t.sh = p->stride[0]; t.sw = p->stride[1];
    t.dh = p->dilation[0]; t.dw = p->dilation[1];
    t.pt = p->pad_begin[0]; t.pl = p->pad_begin[1];
    t.pb = p->pad_end[0]; t.pr = p->pad_end[1];
    s.Ho = out_size_general(s.H, s.R, t.sh, t.dh, t.pt, t.pb);
    s.Wo = out_size_general(s.W, s.S, t.sw, t.dw, t.pl, t.pr);
    if (s.Ho < 1 || s.Wo < 1) return IGC_DECLINE_OUTPUT_SHAPE;
    if (out_nhwc[0] != s.N || out_nhwc[1] != s.Ho || out_nhwc[2] != s.Wo || out_nhwc[3] != s.F)
        return IGC_DECLINE_OUTPUT_SHAPE;
    const int64_t eb = elem_bytes(dtype);
    // the tiled kernel's 32-bit coordinates: padded extents and dilated
    // filter spans below 2^30 keep every tap's row and column in range
    const int64_t l30 = (int64_t)1 << 30;
    if (s.H + t.pt + t.pb >= l30 || s.W + t.pl + t.pr >= l30 || (int64_t)t.dh * (s.R - 1) >= l30 ||
        (int64_t)t.dw * (s.S - 1) >= l30)
        return IGC_DECLINE_SIZE_LIMIT;
    if (s.Ho > lim / s.Wo) return IGC_DECLINE_SIZE_LIMIT;
    s.M = s.N * s.Ho * s.Wo;
    s.K = s.R * s.S * s.C;
    if (s.M >= lim || s.K >= lim || (s.R * s.W + s.S) * s.C >= lim) return IGC_DECLINE_SIZE_LIMIT;
    s.kpad = round_up(s.K, KT_BYTES / eb);
    s.kpitch = nk_pitch(s.K, s.F, eb);
    if (s.kpitch >= lim || s.F * s.kpitch * eb >= lim) return IGC_DECLINE_SIZE_LIMIT;
    // the grouped launch's grid: at most (M / 128) x (C_out per group / 16)
    // tiles per group
    if ((s.M + 127) / 128 * ((s.F / t.groups + 15) / 16) * t.groups >= lim)
        return IGC_DECLINE_SIZE_LIMIT;
    // one group at unit dilation and equal strides: the forward kernels
    // (their gathers take any stride; the page restricts it to 1 or 2)
    t.fast = t.groups == 1 && t.dh == 1 && t.dw == 1 && t.sh == t.sw;
    t.page = t.fast && t.sh <= 2 && t.pt == t.pb && t.pt == t.pl && t.pt == t.pr && t.pt <= 2;
    s.st = t.sh;
    s.pad = 0;
    s.pt = t.pt;
    s.pl = t.pl;
    if (t.page) {
        // the page form: conv2d_fwd's own gate, limits included
        const int32_t st[2] = {t.sh, t.sw}, dil[2] = {1, 1}, pad[2] = {t.pt, t.pl};
        const int32_t rc = check_shapes(in_nhwc, fcrs, filt_dims, out_nhwc, st, dil, pad, 1,
                                        dtype, &t.s);
        if (rc != IGC_OK) return rc;
    }
    t.q = 0;
    t.dil = false;
    t.nk_bytes = s.F * s.kpitch * eb;
    if (!t.fast) supergroup_plan(t, dtype, device_info());
    if (!t.fast && t.q == 0) dilation_plan(t, dtype, device_info());
    if (g) *g = t;
    return IGC_OK;
}

int32_t check_general(const void* input, const int64_t in_nhwc[4], const void* filter,
                      int32_t fcrs, const int64_t filt_dims[4], const void* output,
                      const int64_t out_nhwc[4], const igc_conv_params* p, int32_t dtype,
                      const void* source, const igc_epilogue* epi, const void* workspace,
                      size_t workspace_bytes, GShape* out) {
    GShape g;
    int32_t rc = check_general_shapes(in_nhwc, fcrs, filt_dims, out_nhwc, p, dtype, &g);
    if (rc != IGC_OK) return rc;
    const Shape& s = g.s;
    const size_t eb = (size_t)elem_bytes(dtype);
    const size_t in_bytes = (size_t)(s.N * s.H * s.W * g.cin) * eb;
    const size_t f_bytes = (size_t)(s.R * s.S * s.C * s.F) * eb;
    const size_t out_bytes = (size_t)(s.M * s.F) * 2;
    const size_t nk_bytes = (size_t)g.nk_bytes;
    rc = check_pointers(input, in_bytes, filter, f_bytes, output, out_bytes, source, workspace,
                        nk_bytes, workspace_bytes);
    if (rc != IGC_OK) return rc;
    rc = check_epilogue(epi, output, s, workspace, nk_bytes);
    if (rc != IGC_OK) return rc;
    if (out) *out = g;
    return IGC_OK;
}

// The NK matrix of a general problem: the plain transpose (group g's Fg rows
// from row g*Fg), or the super-groups' block-diagonal one.
hipError_t launch_general_nk(const void* filter, int32_t fcrs, const GShape& g, int32_t dtype,
                             void* nk, hipStream_t stream) {
    if (g.q == 0) return launch_transpose(filter, fcrs, g.s, dtype, nk, stream);
    const Shape& u = g.sg;
    const int eb = elem_bytes(dtype);
    const int64_t row_chunks = u.kpitch / (16 / eb);
    const int64_t F = g.s.F;
    if (F == 0 || row_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((row_chunks + 63) / 64), (unsigned)(F < 65535 ? F : 65535));
    const int fg = (int)(F / g.groups);
    if (eb == 2)
        hipLaunchKernelGGL(filter_to_nk_blockdiag_kernel<2>, grid, dim3(64), 0, stream,
                           (const uint8_t*)filter, (uint8_t*)nk, fcrs, (int)u.R, (int)u.S,
                           (int)g.s.C, (int)F, fg, (int)g.q, (int)u.kpitch);
    else
        hipLaunchKernelGGL(filter_to_nk_blockdiag_kernel<1>, grid, dim3(64), 0, stream,
                           (const uint8_t*)filter, (uint8_t*)nk, fcrs, (int)u.R, (int)u.S,
                           (int)g.s.C, (int)F, fg, (int)g.q, (int)u.kpitch);
    return hipGetLastError();
}

// The super-groups' grouped launch of the band kernel.
hipError_t launch_supergroups(const void* input, const void* nk, void* output,
                              const void* source, float beta, const igc_epilogue* epi,
                              const GShape& g, int32_t dtype, hipStream_t stream) {
    const Shape& u = g.sg;
    const int64_t eb = elem_bytes(dtype);
    const int64_t ng = g.groups / g.q;
    Shape pl = u;
    pl.N = u.N * ng;
    BandPlan bp;
    if (!band_plan(pl, dtype, &bp, device_info())) return hipErrorInvalidValue;
    bp.tiles = u.N * bp.tiles_h * bp.tiles_w;   // per super-group
    ConvArgs a = base_args(input, nk, output, source, beta, epi, u, dtype);
    a.xpitch = (int)g.cin;
    a.ypitch = (int)g.s.F;
    if (ng > 1) {
        a.groups = (int)ng;
        a.g_x = u.C * eb;
        a.g_nk = u.F * u.kpitch * eb;
        a.g_y = u.F * 2;
        a.g_src = source ? u.F * 2 : 0;
        a.g_c = (int)u.F;
    }
    const bool resid = source != nullptr;
    switch (dtype) {
        case IGC_DTYPE_BF16: return launch_band_any<DT_BF16>(resid, a, bp, stream);
        case IGC_DTYPE_FP16: return launch_band_any<DT_FP16>(resid, a, bp, stream);
        default: return launch_band_any<DT_FP8>(resid, a, bp, stream);
    }
}

// The dilation phases' grouped launch of the band kernel: nk is the plain
// NK matrix, or nullptr with wraw the stored filter (filter_in_kernel's
// layout rules; the kernel transposes it itself).
hipError_t launch_dilation_phases(const void* input, const void* nk, void* output,
                                  const void* source, float beta, const igc_epilogue* epi,
                                  const GShape& g, int32_t dtype, hipStream_t stream,
                                  const void* wraw = nullptr, int32_t wfcrs = 0) {
    const Shape& u = g.sd;
    const Shape& s = g.s;
    const int64_t eb = elem_bytes(dtype);
    const int64_t np = (int64_t)g.dh * g.dw;
    Shape pl = u;
    pl.N = u.N * np;
    BandPlan bp;
    if (!band_plan(pl, dtype, &bp, device_info())) return hipErrorInvalidValue;
    bp.tiles = u.N * bp.tiles_h * bp.tiles_w;   // per phase
    ConvArgs a = base_args(input, nk, output, source, beta, epi, u, dtype);
    a.wraw = (const uint8_t*)wraw;
    a.wrs = wfcrs ? (int)(s.R * s.S) : 0;
    a.vrow = (int)(g.dh * s.W);
    a.vcol = g.dw;
    a.vimg = (int)(s.H * s.W);
    a.ymap = 1;
    a.Hy = (int)s.Ho;
    a.Wy = (int)s.Wo;
    a.ysh = g.dh;
    a.ysw = g.dw;
    if (np > 1) {
        // phase (a_h, a_w) = (gh, gw) of a grid of dw columns; with one
        // column (dw = 1) the launch is one-dimensional over the row phases
        a.groups = (int)np;
        const int64_t xr = s.W * s.C * eb, yr = s.Wo * s.F * 2;
        if (g.dw > 1) {
            a.gsplit = g.dw;
            a.g_x = s.C * eb;
            a.g_x2 = xr;
            a.g_y = s.F * 2;
            a.g_y2 = yr;
            a.g_src = source ? s.F * 2 : 0;
            a.g_src2 = source ? yr : 0;
        } else {
            a.g_x = xr;
            a.g_y = yr;
            a.g_src = source ? yr : 0;
        }
    }
    const bool resid = source != nullptr;
    switch (dtype) {
        case IGC_DTYPE_BF16: return launch_band_any<DT_BF16>(resid, a, bp, stream);
        case IGC_DTYPE_FP16: return launch_band_any<DT_FP16>(resid, a, bp, stream);
        default: return launch_band_any<DT_FP8>(resid, a, bp, stream);
    }
}

// The GEMM of a general problem whose NK matrix is in nk (all groups' rows,
// group g's Fg rows starting at row g*Fg; super-group j's q*Fg rows starting
// at row j*q*Fg).
hipError_t launch_general(const void* input, const void* nk, void* output, const void* source,
                          float beta, const igc_epilogue* epi, const GShape& g, int32_t dtype,
                          hipStream_t stream) {
    if (g.fast)
        return launch_igemm(input, nk, output, source, beta, epi, g.s, dtype, stream, nullptr,
                             g.page);
    const Shape& s = g.s;
    const int64_t eb = elem_bytes(dtype);
    const int64_t fg = s.F / g.groups;
    if (s.M == 0 || fg == 0) return hipSuccess;
    if (g.q > 0) return launch_supergroups(input, nk, output, source, beta, epi, g, dtype, stream);
    if (g.dil)
        return launch_dilation_phases(input, nk, output, source, beta, epi, g, dtype, stream);
    ConvArgs a = base_args(input, nk, output, source, beta, epi, s, dtype);
    a.F = (int)fg;
    a.sh = g.sh; a.sw = g.sw;
    a.pt = g.pt; a.pl = g.pl;
    a.dh = g.dh; a.dw = g.dw;
    a.xpitch = (int)g.cin;
    a.ypitch = (int)s.F;
    if (g.groups > 1) {
        a.groups = g.groups;
        a.g_x = s.C * eb;
        a.g_nk = fg * s.kpitch * eb;
        a.g_y = fg * 2;
        a.g_src = source ? fg * 2 : 0;
        a.g_c = (int)fg;
    }
    const bool resid = source != nullptr;
    switch (dtype) {
        case IGC_DTYPE_BF16: return launch_tiled_any<DT_BF16>(resid, a, stream);
        case IGC_DTYPE_FP16: return launch_tiled_any<DT_FP16>(resid, a, stream);
        default: return launch_tiled_any<DT_FP8>(resid, a, stream);
    }
}

// ---- the allocation-free entry point's scratch ----------------------------
// The NK matrix of conv2d_fwd_noalloc lives in this file-scope device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in, not a device
// address): on the first call on each device, with that device current, the
// device address is looked up once and kept per device.
constexpr size_t kScratchBytes = IGC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchPtrs {
    std::mutex mu;
    bool done[kMaxDevices] = {};
    hipError_t err[kMaxDevices] = {};
    void* ptr[kMaxDevices] = {};
};
ScratchPtrs g_scratch;

hipError_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_scratch.mu);
    if (!g_scratch.done[dev]) {
        void* p = nullptr;
        g_scratch.err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch.ptr[dev] = p;
        g_scratch.done[dev] = true;
    }
    *out = g_scratch.ptr[dev];
    return g_scratch.err[dev];
}

}  // namespace

extern "C" {

int32_t conv2d_fwd_noalloc(const void* input, const int64_t in_nhwc[4], const void* filter,
                           int32_t filter_is_fcrs, const int64_t filt_dims[4], void* output,
                           const int64_t out_nhwc[4], const int32_t stride[2],
                           const int32_t dilation[2], const int32_t padding[2], int32_t groups,
                           int32_t dtype, const void* source, float beta, void* stream) {
    Shape s;
    // the gate of conv2d_fwd with no caller workspace (the scratch is the
    // library's own, so no caller buffer can overlap it)
    const int32_t rc = check_all(input, in_nhwc, filter, 0, filter_is_fcrs, filt_dims, output,
                                 out_nhwc, stride, dilation, padding, groups, dtype, source,
                                 nullptr, 0, &s);
    if (rc != IGC_OK) return 0;
    const size_t nk_bytes = (size_t)(s.F * s.kpitch) * (size_t)elem_bytes(dtype);
    if (nk_bytes > kScratchBytes) return 0;   // beyond the static scratch: declined
    if (s.M == 0 || s.F == 0) return 1;       // empty output: nothing to compute
    void* nk = nullptr;
    hipError_t e = scratch_ptr(&nk);
    if (e != hipSuccess) return -(int32_t)e;
    hipStream_t st = (hipStream_t)stream;
    e = launch_transpose(filter, filter_is_fcrs, s, dtype, nk, st);
    if (e == hipSuccess) e = launch_igemm(input, nk, output, source, beta, nullptr, s, dtype, st);
    return hip_fail(e);
}

size_t conv2d_transposed_workspace_bytes(const int64_t in_nhwc[4], const int64_t filt_rsfc[4],
                                         const int32_t stride[2], const int32_t dilation[2],
                                         const int32_t padding[2], int32_t dtype) {
    if (!in_nhwc || !filt_rsfc || !stride || !dilation || !padding) return 0;
    int64_t od[4] = {in_nhwc[0], 0, 0, filt_rsfc[2]};
    for (int i = 0; i < 2; ++i)
        od[1 + i] = (in_nhwc[1 + i] - 1) * stride[i] - 2 * (int64_t)padding[i] +
                    (int64_t)dilation[i] * (filt_rsfc[i] - 1) + 1;
    TPlan t;
    if (transposed_plan(in_nhwc, filt_rsfc, od, stride, dilation, padding, dtype, &t) != IGC_OK)
        return 0;
    return t.ws_bytes;
}

int32_t conv2d_transposed_check(const void* input, const int64_t in_nhwc[4], const void* filter,
                                const int64_t filt_rsfc[4], const void* output,
                                const int64_t out_nhwc[4], const int32_t stride[2],
                                const int32_t dilation[2], const int32_t padding[2],
                                int32_t dtype, const void* source, float beta,
                                const igc_epilogue* epilogue, const void* workspace,
                                size_t workspace_bytes) {
    (void)beta;
    TPlan t;
    const int32_t rc = transposed_plan(in_nhwc, filt_rsfc, out_nhwc, stride, dilation, padding,
                                       dtype, &t);
    if (rc != IGC_OK) return rc;
    return transposed_pointers(t, dtype, input, filter, output, source, epilogue, workspace,
                               workspace_bytes);
}

int32_t conv2d_transposed_fwd(const void* input, const int64_t in_nhwc[4], const void* filter,
                              const int64_t filt_rsfc[4], void* output,
                              const int64_t out_nhwc[4], const int32_t stride[2],
                              const int32_t dilation[2], const int32_t padding[2],
                              int32_t dtype, const void* source, float beta,
                              const igc_epilogue* epilogue, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (conv2d_transposed_check(input, in_nhwc, filter, filt_rsfc, output, out_nhwc, stride,
                                dilation, padding, dtype, source, beta, epilogue, workspace,
                                workspace_bytes) != IGC_OK)
        return 0;
    TPlan t;
    transposed_plan(in_nhwc, filt_rsfc, out_nhwc, stride, dilation, padding, dtype, &t);
    if (t.N == 0 || t.F == 0) return 1;  // empty output: nothing to compute
    hipStream_t st = (hipStream_t)stream;
    void* ws = workspace;
    bool owned = false;
    if (!ws && t.ws_bytes) {
        hipError_t e = hipMallocAsync(&ws, t.ws_bytes, st);
        if (e != hipSuccess) return -(int32_t)e;
        owned = true;
    }
    hipError_t e = run_transposed(t, input, filter, output, source, beta, epilogue, dtype,
                                  (uint8_t*)ws, st);
    if (owned) {
        hipError_t f = hipFreeAsync(ws, st);
        if (e == hipSuccess) e = f;
    }
    return hip_fail(e);
}

size_t conv2d_im2col_bytes(const int64_t in_nhwc[4], const int64_t filt_rs[2],
                           const int32_t stride[2], const int32_t padding[2], int32_t dtype) {
    Shape s;
    int64_t kp;
    if (im2col_shape(in_nhwc, filt_rs, stride, padding, dtype, &s, &kp) != IGC_OK) return 0;
    return (size_t)(s.M * kp * elem_bytes(dtype));
}

int32_t conv2d_im2col(const void* input, const int64_t in_nhwc[4], const int64_t filt_rs[2],
                      const int32_t stride[2], const int32_t padding[2], int32_t dtype,
                      void* a_out, size_t a_bytes, void* stream) {
    Shape s;
    int64_t kp;
    if (im2col_shape(in_nhwc, filt_rs, stride, padding, dtype, &s, &kp) != IGC_OK) return 0;
    const int64_t eb = elem_bytes(dtype);
    const size_t need = (size_t)(s.M * kp * eb);
    const size_t in_bytes = (size_t)(s.N * s.H * s.W * s.C * eb);
    if (a_bytes < need) return 0;
    if ((need && !a_out) || (in_bytes && !input)) return 0;
    if (!aligned16(input) || !aligned16(a_out)) return 0;
    if (overlaps(a_out, need, input, in_bytes)) return 0;
    if (need == 0) return 1;
    Im2colArgs a{};
    a.x = (const uint8_t*)input;
    a.a = (uint8_t*)a_out;
    a.H = (int)s.H; a.W = (int)s.W; a.Ho = (int)s.Ho; a.Wo = (int)s.Wo;
    a.S = (int)s.S; a.stride = s.st; a.pad = s.pad;
    a.RS = (int)(s.R * s.S);
    a.CB = (int)(s.C * eb);
    a.VPR = (uint32_t)(kp * eb / 16);
    a.CV = (uint32_t)(s.C * eb / 16);
    a.total = (uint32_t)(s.M * a.VPR);
    a.HoWo = (uint32_t)(s.Ho * s.Wo);
    // need > 0, so M, C_in and hence VPR and CV are at least 1
    a.d_vpr = make_fastdiv(a.VPR);
    a.d_cv = make_fastdiv(a.CV);
    a.d_s = make_fastdiv((uint32_t)s.S);
    a.d_howo = make_fastdiv(a.HoWo);
    a.d_wo = make_fastdiv((uint32_t)s.Wo);
    const uint32_t blocks = (a.total + 255) / 256 < 4096u ? (a.total + 255) / 256 : 4096u;
    hipLaunchKernelGGL(im2col_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, a);
    return hip_fail(hipGetLastError());
}


int32_t conv2d_abi_version(void) { return kAbiVersion; }

int32_t conv2d_build_flags(void) {
#ifdef IGC_LDS_POISON
    return 1;
#else
    return 0;
#endif
}

const char* conv2d_reason_string(int32_t reason) {
    switch (reason) {
        case IGC_OK: return "ok";
        case IGC_DECLINE_DTYPE: return "dtype";
        case IGC_DECLINE_STRIDE: return "stride";
        case IGC_DECLINE_DILATION: return "dilation";
        case IGC_DECLINE_PADDING: return "padding";
        case IGC_DECLINE_GROUPS: return "groups";
        case IGC_DECLINE_SHAPE: return "shape";
        case IGC_DECLINE_OUTPUT_SHAPE: return "output_shape";
        case IGC_DECLINE_VECTOR_WIDTH: return "vector_width";
        case IGC_DECLINE_ALIGNMENT: return "alignment";
        case IGC_DECLINE_NULL_POINTER: return "null_pointer";
        case IGC_DECLINE_OVERLAP: return "overlap";
        case IGC_DECLINE_WORKSPACE: return "workspace";
        case IGC_DECLINE_SIZE_LIMIT: return "size_limit";
        case IGC_DECLINE_EPILOGUE: return "epilogue";
        default: return "unknown";
    }
}

int32_t conv2d_fwd_query(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                         const int64_t filt_dims[4], const int64_t out_nhwc[4],
                         const int32_t stride[2], const int32_t dilation[2],
                         const int32_t padding[2], int32_t groups, int32_t dtype) {
    return check_shapes(in_nhwc, filter_is_fcrs, filt_dims, out_nhwc, stride, dilation, padding,
                        groups, dtype, nullptr);
}

int32_t conv2d_fwd_epilogue_check(const void* input, const int64_t in_nhwc[4],
                                  const void* filter, int32_t filter_is_fcrs,
                                  const int64_t filt_dims[4], const void* output,
                                  const int64_t out_nhwc[4], const int32_t stride[2],
                                  const int32_t dilation[2], const int32_t padding[2],
                                  int32_t groups, int32_t dtype, const void* source, float beta,
                                  const igc_epilogue* epilogue, const void* workspace,
                                  size_t workspace_bytes) {
    (void)beta;
    Shape s;
    const int32_t rc = check_all(input, in_nhwc, filter, 0, filter_is_fcrs, filt_dims, output,
                                 out_nhwc, stride, dilation, padding, groups, dtype, source,
                                 workspace, workspace_bytes, &s);
    if (rc != IGC_OK) return rc;
    return check_epilogue(epilogue, output, s, workspace,
                          (size_t)(s.F * s.kpitch) * (size_t)elem_bytes(dtype));
}

int32_t conv2d_fwd_check(const void* input, const int64_t in_nhwc[4], const void* filter,
                         int32_t filter_is_fcrs, const int64_t filt_dims[4], const void* output,
                         const int64_t out_nhwc[4], const int32_t stride[2],
                         const int32_t dilation[2], const int32_t padding[2], int32_t groups,
                         int32_t dtype, const void* source, float beta, const void* workspace,
                         size_t workspace_bytes) {
    (void)beta;
    return check_all(input, in_nhwc, filter, 0, filter_is_fcrs, filt_dims, output, out_nhwc,
                     stride, dilation, padding, groups, dtype, source, workspace,
                     workspace_bytes, nullptr);
}

const char* conv2d_fwd_kernel_name(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                   const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                   const int32_t stride[2], const int32_t dilation[2],
                                   const int32_t padding[2], int32_t groups, int32_t dtype) {
    Shape s;
    if (check_shapes(in_nhwc, filter_is_fcrs, filt_dims, out_nhwc, stride, dilation, padding,
                     groups, dtype, &s) != IGC_OK)
        return nullptr;
    BandPlan bp;
    switch (select_kernel(s, dtype, &bp)) {
        case K_NONE: return "none";
        case K_TAPFOLD: return "igemm_fwd_tapfold_kernel";
        case K_BAND: return "igemm_fwd_band_kernel";
        case K_PATCH: return "igemm_fwd_patch_kernel";
        case K_WIDE: return "igemm_fwd_wide_kernel";
        case K_RESIDENT: return "igemm_fwd_resident_kernel";
        default: return "igemm_fwd_kernel";
    }
}

size_t conv2d_workspace_bytes(const int64_t filt_dims[4], int32_t filter_is_fcrs, int32_t dtype) {
    const int64_t p = conv2d_nk_row_pitch(filt_dims, filter_is_fcrs, dtype);
    if (p < 0) return 0;
    int64_t R, S, C, F;
    filter_rscf(filt_dims, filter_is_fcrs, &R, &S, &C, &F);
    return (size_t)(F * p) * (size_t)elem_bytes(dtype);
}

int64_t conv2d_nk_row_pitch(const int64_t filt_dims[4], int32_t filter_is_fcrs, int32_t dtype) {
    if (!filt_dims) return -1;
    if (dtype != IGC_DTYPE_BF16 && dtype != IGC_DTYPE_FP16 && dtype != IGC_DTYPE_FP8_E4M3FN)
        return -1;
    int64_t R, S, C, F;
    filter_rscf(filt_dims, filter_is_fcrs, &R, &S, &C, &F);
    if (R < 0 || S < 0 || C < 0 || F < 0) return -1;
    return nk_pitch(R * S * C, F, elem_bytes(dtype));
}

int32_t conv2d_filter_to_nk(const void* filter, int32_t filter_is_fcrs, const int64_t filt_dims[4],
                            int32_t dtype, void* nk, size_t nk_bytes, void* stream) {
    if (!filt_dims) return 0;
    if (dtype != IGC_DTYPE_BF16 && dtype != IGC_DTYPE_FP16 && dtype != IGC_DTYPE_FP8_E4M3FN)
        return 0;
    Shape s{};
    filter_rscf(filt_dims, filter_is_fcrs, &s.R, &s.S, &s.C, &s.F);
    const int64_t eb = elem_bytes(dtype);
    const int64_t lim = (int64_t)1 << 31;
    if (s.R < 1 || s.S < 1 || s.C < 0 || s.F < 0) return 0;
    if (s.R >= lim || s.S >= lim || s.C >= lim || s.F >= lim) return 0;
    s.K = s.R * s.S * s.C;
    if (s.K >= lim) return 0;
    s.kpad = round_up(s.K, KT_BYTES / eb);
    s.kpitch = nk_pitch(s.K, s.F, eb);
    // the transpose kernel indexes both matrices with 32-bit integers
    if (s.kpitch >= lim || s.F * s.kpitch * eb >= lim) return 0;
    const size_t need = (size_t)(s.F * s.kpitch) * (size_t)eb;
    const size_t fbytes = (size_t)(s.K * s.F) * (size_t)eb;
    if (nk_bytes < need) return 0;
    if ((fbytes && !filter) || (need && !nk)) return 0;
    if (!aligned16(nk) || !aligned16(filter)) return 0;
    if (overlaps(nk, need, filter, fbytes)) return 0;
    return hip_fail(launch_transpose(filter, filter_is_fcrs, s, dtype, nk, (hipStream_t)stream));
}

int32_t conv2d_fwd_nk_epilogue(const void* input, const int64_t in_nhwc[4], const void* nk,
                               int32_t filter_is_fcrs, const int64_t filt_dims[4], void* output,
                               const int64_t out_nhwc[4], const int32_t stride[2],
                               const int32_t dilation[2], const int32_t padding[2],
                               int32_t groups, int32_t dtype, const void* source, float beta,
                               const igc_epilogue* epilogue, void* stream) {
    Shape s;
    size_t nk_bytes = conv2d_workspace_bytes(filt_dims, filter_is_fcrs, dtype);
    const int32_t rc = check_all(input, in_nhwc, nk, nk_bytes ? nk_bytes : 1, filter_is_fcrs,
                                 filt_dims, output, out_nhwc, stride, dilation, padding, groups,
                                 dtype, source, nullptr, 0, &s);
    if (rc != IGC_OK) return 0;
    if (check_epilogue(epilogue, output, s) != IGC_OK) return 0;
    return hip_fail(launch_igemm(input, nk, output, source, beta, epilogue, s, dtype,
                                 (hipStream_t)stream));
}

int32_t conv2d_fwd_nk(const void* input, const int64_t in_nhwc[4], const void* nk,
                      int32_t filter_is_fcrs, const int64_t filt_dims[4], void* output,
                      const int64_t out_nhwc[4], const int32_t stride[2],
                      const int32_t dilation[2], const int32_t padding[2], int32_t groups,
                      int32_t dtype, const void* source, float beta, void* stream) {
    return conv2d_fwd_nk_epilogue(input, in_nhwc, nk, filter_is_fcrs, filt_dims, output,
                                  out_nhwc, stride, dilation, padding, groups, dtype, source,
                                  beta, nullptr, stream);
}

int32_t conv2d_fwd_epilogue(const void* input, const int64_t in_nhwc[4], const void* filter,
                            int32_t filter_is_fcrs, const int64_t filt_dims[4], void* output,
                            const int64_t out_nhwc[4], const int32_t stride[2],
                            const int32_t dilation[2], const int32_t padding[2], int32_t groups,
                            int32_t dtype, const void* source, float beta,
                            const igc_epilogue* epilogue, void* workspace,
                            size_t workspace_bytes, void* stream) {
    Shape s;
    const int32_t rc = check_all(input, in_nhwc, filter, 0, filter_is_fcrs, filt_dims, output,
                                 out_nhwc, stride, dilation, padding, groups, dtype, source,
                                 workspace, workspace_bytes, &s);
    if (rc != IGC_OK) return 0;
    const size_t nk_bytes = (size_t)(s.F * s.kpitch) * (size_t)elem_bytes(dtype);
    if (check_epilogue(epilogue, output, s, workspace, nk_bytes) != IGC_OK) return 0;
    if (s.M == 0 || s.F == 0) return 1;  // empty output: nothing to compute
    hipStream_t st = (hipStream_t)stream;
    if (filter_in_kernel(s, dtype, filter_is_fcrs))
        return hip_fail(launch_igemm(input, nullptr, output, source, beta, epilogue, s, dtype, st,
                                     nullptr, true, nullptr, filter, filter_is_fcrs));
    void* nk = workspace;
    bool owned = false;
    if (!nk && nk_bytes) {
        hipError_t e = hipMallocAsync(&nk, nk_bytes, st);
        if (e != hipSuccess) return -(int32_t)e;
        owned = true;
    }
    hipError_t e = launch_transpose(filter, filter_is_fcrs, s, dtype, nk, st);
    if (e == hipSuccess) e = launch_igemm(input, nk, output, source, beta, epilogue, s, dtype, st);
    if (owned) {
        hipError_t f = hipFreeAsync(nk, st);
        if (e == hipSuccess) e = f;
    }
    return hip_fail(e);
}

int32_t conv2d_fwd(const void* input, const int64_t in_nhwc[4], const void* filter,
                   int32_t filter_is_fcrs, const int64_t filt_dims[4], void* output,
                   const int64_t out_nhwc[4], const int32_t stride[2], const int32_t dilation[2],
                   const int32_t padding[2], int32_t groups, int32_t dtype, const void* source,
                   float beta, void* workspace, size_t workspace_bytes, void* stream) {
    return conv2d_fwd_epilogue(input, in_nhwc, filter, filter_is_fcrs, filt_dims, output,
                               out_nhwc, stride, dilation, padding, groups, dtype, source, beta,
                               nullptr, workspace, workspace_bytes, stream);
}

int32_t conv2d_epilogue_check(const igc_epilogue* epilogue, const void* output,
                              const int64_t out_nhwc[4]) {
    if (!out_nhwc) return IGC_DECLINE_NULL_POINTER;
    for (int i = 0; i < 4; ++i)
        if (out_nhwc[i] < 0) return IGC_DECLINE_SHAPE;
    Shape s{};
    s.M = out_nhwc[0] * out_nhwc[1] * out_nhwc[2];
    s.F = out_nhwc[3];
    return check_epilogue(epilogue, output, s);
}

const char* conv2d_fwd_general_kernel_name(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                           const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                           const igc_conv_params* params, int32_t dtype) {
    GShape g;
    if (check_general_shapes(in_nhwc, filter_is_fcrs, filt_dims, out_nhwc, params, dtype, &g) !=
        IGC_OK)
        return nullptr;
    if (g.fast) {
        BandPlan bp;
        switch (select_kernel(g.s, dtype, &bp, g.page)) {
            case K_NONE: return "none";
            case K_TAPFOLD: return "igemm_fwd_tapfold_kernel";
            case K_BAND: return "igemm_fwd_band_kernel";
            case K_PATCH: return "igemm_fwd_patch_kernel";
            case K_WIDE: return "igemm_fwd_wide_kernel";
            case K_RESIDENT: return "igemm_fwd_resident_kernel";
            default: return "igemm_fwd_kernel";
        }
    }
    if (g.s.M == 0 || g.s.F == 0) return "none";
    return (g.q > 0 || g.dil) ? "igemm_fwd_band_kernel" : "igemm_fwd_kernel";
}

int32_t conv2d_fwd_filter_in_kernel(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                    const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                    const int32_t stride[2], const int32_t dilation[2],
                                    const int32_t padding[2], int32_t groups, int32_t dtype) {
    Shape s;
    if (check_shapes(in_nhwc, filter_is_fcrs, filt_dims, out_nhwc, stride, dilation, padding,
                     groups, dtype, &s) != IGC_OK)
        return 0;
    return filter_in_kernel(s, dtype, filter_is_fcrs) ? 1 : 0;
}

size_t conv2d_fwd_general_workspace_bytes(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                          const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                          const igc_conv_params* params, int32_t dtype) {
    GShape g;
    if (check_general_shapes(in_nhwc, filter_is_fcrs, filt_dims, out_nhwc, params, dtype, &g) !=
        IGC_OK)
        return 0;
    return (size_t)g.nk_bytes;
}

int32_t conv2d_fwd_general_query(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                 const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                 const igc_conv_params* params, int32_t dtype) {
    return check_general_shapes(in_nhwc, filter_is_fcrs, filt_dims, out_nhwc, params, dtype,
                                nullptr);
}

int32_t conv2d_fwd_general_check(const void* input, const int64_t in_nhwc[4],
                                 const void* filter, int32_t filter_is_fcrs,
                                 const int64_t filt_dims[4], const void* output,
                                 const int64_t out_nhwc[4], const igc_conv_params* params,
                                 int32_t dtype, const void* source, float beta,
                                 const igc_epilogue* epilogue, const void* workspace,
                                 size_t workspace_bytes) {
    (void)beta;
    return check_general(input, in_nhwc, filter, filter_is_fcrs, filt_dims, output, out_nhwc,
                         params, dtype, source, epilogue, workspace, workspace_bytes, nullptr);
}

int32_t conv2d_fwd_general(const void* input, const int64_t in_nhwc[4], const void* filter,
                           int32_t filter_is_fcrs, const int64_t filt_dims[4], void* output,
                           const int64_t out_nhwc[4], const igc_conv_params* params,
                           int32_t dtype, const void* source, float beta,
                           const igc_epilogue* epilogue, void* workspace,
                           size_t workspace_bytes, void* stream) {
    GShape g;
    if (check_general(input, in_nhwc, filter, filter_is_fcrs, filt_dims, output, out_nhwc,
                      params, dtype, source, epilogue, workspace, workspace_bytes,
                      &g) != IGC_OK)
        return 0;
    const Shape& s = g.s;
    if (s.M == 0 || s.F == 0) return 1;  // empty output: nothing to compute
    const size_t nk_bytes = (size_t)g.nk_bytes;
    hipStream_t st = (hipStream_t)stream;
    if (g.fast && filter_in_kernel(s, dtype, filter_is_fcrs, g.page))
        return hip_fail(launch_igemm(input, nullptr, output, source, beta, epilogue, s, dtype, st,
                                     nullptr, g.page, nullptr, filter, filter_is_fcrs));
    if (g.dil && raw_filter_ok(s, dtype, filter_is_fcrs))
        return hip_fail(launch_dilation_phases(input, nullptr, output, source, beta, epilogue, g,
                                               dtype, st, filter, filter_is_fcrs));
    void* nk = workspace;
    bool owned = false;
    if (!nk && nk_bytes) {
        hipError_t e = hipMallocAsync(&nk, nk_bytes, st);
        if (e != hipSuccess) return -(int32_t)e;
        owned = true;
    }
    hipError_t e = launch_general_nk(filter, filter_is_fcrs, g, dtype, nk, st);
    if (e == hipSuccess)
        e = launch_general(input, nk, output, source, beta, epilogue, g, dtype, st);
    if (owned) {
        hipError_t f = hipFreeAsync(nk, st);
        if (e == hipSuccess) e = f;
    }
    return hip_fail(e);
}

}  // extern "C"

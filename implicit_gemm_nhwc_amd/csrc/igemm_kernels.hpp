// Device kernels for the forward NHWC convolution as an implicit GEMM on
// gfx950 (CDNA4, 64-lane wavefronts, MFMA).
//
// GEMM view (page "dispatch_fused_im2col_conv2d_apple", summary: filter
// transposed to the (C_out, K = R*S*C_in) NK matrix, A operand gathered from
// the NHWC input on the fly):
//   rows    co in [0, C_out)                  -- read from NK[co][k]
//   columns m = (n*Ho + oh)*Wo + ow in [0, M)  -- gathered from x
//   k       (r*S + s)*C_in + ci, ci fastest   -- contiguous in both
//   acc[co][m] = sum_k NK[co][k] * x[n, oh*st - p + r, ow*st - p + s, ci]
// Because NHWC output flattened over (n, oh, ow) is the row-major [M][C_out]
// result, the epilogue's (m, co) coordinates address the output directly.
//
// The filter is the MFMA "A" operand and the gathered pixels the "B"
// operand, so in the 16x16 result each lane owns one pixel and four
// consecutive output channels: stores and residual loads are 8-byte vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace igc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

enum { DT_BF16 = 0, DT_FP16 = 1, DT_FP8 = 2 };

// Every k-tile is 128 bytes of K: 64 bf16/fp16 or 128 fp8 elements, as eight
// 16-byte chunks.  A chunk is 8 (or 16) channels of a single filter tap,
// which the C_in * element_bytes % 16 == 0 rule guarantees.
constexpr int KT_BYTES = 128;
constexpr int CHUNKS = KT_BYTES / 16;
constexpr int NTHREADS = 256;

template <int DT> struct DtTraits;
template <> struct DtTraits<DT_BF16> { static constexpr int E = 2; };
template <> struct DtTraits<DT_FP16> { static constexpr int E = 2; };
template <> struct DtTraits<DT_FP8> { static constexpr int E = 1; };

struct ConvArgs {
    const uint8_t* x;   // NHWC input
    const uint8_t* nk;  // [C_out][kpitch] transposed filter, zero past K
    // band kernel only: when set, the stored filter that the kernel
    // transposes into its LDS itself (nk is then unused): RSCF [R][S][C][F]
    // when wrs == 0, else FCRS [F][C][R][S] with R*S == wrs (1 or 9)
    const uint8_t* wraw;
    int wrs;
    uint16_t* y;        // NHWC output (bf16 or fp16 bits)
    const uint16_t* src;  // residual source, same layout and type as y
    float beta;
    // fused per-channel epilogue (all unused when epi == 0)
    const float* scale;   // [C_out] multiplier of the convolution, or null (1)
    const float* bias;    // [C_out] addend, or null (0)
    int act;              // ACT_NONE, ACT_RELU or ACT_SILU
    int epi;              // nonzero when scale, bias or act is present
    // grouped launch: `groups` problems of the same shape whose NK matrix,
    // output and source lie g_nk, g_y and g_src bytes apart (0 or 1 = one)
    int groups;
    int64_t g_nk, g_y, g_src;
    int H, W, C;        // input (N only enters through M)
    int Ho, Wo, F;      // output spatial size and C_out
    int S, stride;      // filter width; stride of both axes (all kernels but the tiled one)
    int R;              // filter height
    int K;              // R*S*C elements
    int kpitch;         // elements per NK row (stride; a 16-byte zero pad when C_out <= 64)
    int M;              // N*Ho*Wo
    int ktiles;         // 128-byte k-tiles covering K
    int px_tiles;       // ceil(M / BPX)
    int co_tiles;       // ceil(F / BCO)
    // band kernel: output tile TH x TW, input patch PH x PW (LDS)
    int TH, TW, PH, PW;
    int tiles_h, tiles_w;  // tiles per image along Ho / Wo
    int fpitch;            // LDS bytes per filter row
    int frows;             // filter rows in LDS: min(C_out + 1, TM*32), the last zero
    int ppitch;            // LDS bytes per patch pixel (all C_in channels + 16)
    int prow;              // LDS bytes per patch row (PW pixels + row pad)
    int patch_off;         // LDS byte offset of the patch
    int spitch;            // LDS floats per staged output pixel (epilogue)
    int cpp_log2;          // log2(16-byte chunks per input pixel)
    int nslot;             // tap-fold kernel: input rows in the LDS ring
    // padding before each axis (top, left), read by every kernel; it may be
    // negative (the output window then starts inside the image)
    int pt, pl;
    // general geometry, read by the tiled kernel only: per-axis stride and
    // dilation
    int sh, sw, dh, dw;
    // elements per input / output pixel (the whole tensors' C_in / C_out
    // when a grouped launch runs the channel groups of one convolution; C
    // and F above are one group's), read by the tiled and band kernels
    int xpitch, ypitch;
    // output map (every kernel but the tap-fold one): GEMM pixel (n, oh, ow)
    // is output pixel (n, oh*ysh, ow*ysw) of an image of Hy x Wy pixels, the
    // residual source read at the same place (identity: ysh = ysw = 1,
    // Hy = Ho, Wy = Wo; ymap = 0 then).  A constant pixel offset rides in
    // the y and src pointers.
    int ymap, Hy, Wy, ysh, ysw;
    // grouped launch: input bytes and scale / bias entries between problems
    int64_t g_x;
    int g_c;
    // grouped launch on a grid of gsplit columns (gsplit > 1): problem
    // gi = gh*gsplit + gw moves the input by gw*g_x + gh*g_x2 bytes, the
    // output by gw*g_y + gh*g_y2, the source by gw*g_src + gh*g_src2, and
    // its padding by -gh*g_pt, -gw*g_pl
    int gsplit;
    int64_t g_x2, g_y2, g_src2;
    int g_pt, g_pl;
    // band kernel: the input as a view of every vrow-th / vcol-th pixel
    // (input pixel (ih, iw) of the view at pixel ih*vrow + iw*vcol of its
    // image, images vimg pixels apart); 0 for the plain tensor (W, 1, H*W)
    int vrow, vcol, vimg;
    int lds_bytes;      // dynamic LDS of the launch (the poison fill below)
};

// Workgroup b is placed on XCD b % 8 by the hardware's round-robin
// dispatch.  Renumber so each XCD gets one contiguous run of tiles: tiles
// that share input halo rows and filter rows then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    constexpr int X = 8;
    const int q = n / X, rem = n % X;
    const int x = b % X, j = b / X;
    return x * q + (x < rem ? x : rem) + j;
}

// The block index within this workgroup's problem of a grouped launch
// (gridDim.x = groups * per), after moving the input, NK, output, source
// and scale / bias pointers to that problem.  A launch of one problem
// returns blockIdx.x.
__device__ __forceinline__ int group_block(ConvArgs& a, int per) {
    int b = blockIdx.x;
    if (a.groups > 1) {
        const int gi = b / per;
        b -= gi * per;
        if (a.scale) a.scale += (int64_t)gi * a.g_c;
        if (a.bias) a.bias += (int64_t)gi * a.g_c;
        a.nk += gi * a.g_nk;
        const int gh = a.gsplit > 1 ? gi / a.gsplit : 0;
        const int gw = gi - gh * (a.gsplit > 1 ? a.gsplit : 0);
        a.x += gw * a.g_x + gh * a.g_x2;
        a.y = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(a.y) + gw * a.g_y +
                                          gh * a.g_y2);
        if (a.src)
            a.src = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.src) +
                                                      gw * a.g_src + gh * a.g_src2);
        a.pt -= gh * a.g_pt;
        a.pl -= gw * a.g_pl;
    }
    return b;
}

// Debug build (IGC_LDS_POISON): every workgroup first fills its dynamic LDS
// with 0xFF bytes, a NaN in every element type it holds (bf16, fp16, fp8
// e4m3fn, fp32), so a read that runs ahead of its data (a missing wait or
// barrier) shows up as NaN outputs instead of plausible stale values.  The
// normal build compiles this to nothing.
template <int NT>
__device__ __forceinline__ void lds_poison(uint8_t* lds, int bytes) {
#ifdef IGC_LDS_POISON
    for (int i = (int)threadIdx.x * 16; i < bytes; i += NT * 16)
        *reinterpret_cast<i32x4*>(lds + i) = i32x4{-1, -1, -1, -1};
    __syncthreads();
#else
    (void)lds;
    (void)bytes;
#endif
}

// Output pixel index of GEMM pixel (n, oh, ow) under the output map.
__device__ __forceinline__ int64_t out_pixel3(const ConvArgs& a, int n, int oh, int ow) {
    return ((int64_t)n * a.Hy + (int64_t)oh * a.ysh) * a.Wy + (int64_t)ow * a.ysw;
}

// Output pixel index of GEMM pixel m = (n*Ho + oh)*Wo + ow: m itself
// without a map.
__device__ __forceinline__ int64_t out_pixel(const ConvArgs& a, int m) {
    if (!a.ymap) return m;
    const int howo = a.Ho * a.Wo;
    const int n = m / howo;
    const int rem = m - n * howo;
    const int oh = rem / a.Wo;
    return out_pixel3(a, n, oh, rem - oh * a.Wo);
}

// LDS tiles: rows of 128 bytes, chunk c of row r stored at c ^ ((r >> 1) & 7)
// so that 16 consecutive rows read at one logical chunk (the 16 lanes a
// 16-byte LDS read serves per clock from 64 banks) hit 16 different 16-byte
// bank groups of a 256-byte window.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * KT_BYTES + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ uint16_t f32_to_out(float v, int dt) {
    if (dt == DT_FP16) {
        _Float16 h = (_Float16)v;
        return __builtin_bit_cast(uint16_t, h);
    }
    __bf16 b = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

// Two outputs rounded and packed into one 32-bit word (lo in the low half)
// by one packed conversion (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32), the same
// round-to-nearest-even as f32_to_out.
__device__ __forceinline__ uint32_t pack_out2(float lo, float hi, int dt) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 f = {lo, hi};
    if (dt == DT_FP16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h2));
    }
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2));
}

__device__ __forceinline__ float out_to_f32(uint16_t bits, int dt) {
    if (dt == DT_FP16) return (float)__builtin_bit_cast(_Float16, bits);
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// Fused elementwise epilogue (page "dispatch_amd_4wave_conv2d", Parameters:
// an optional elementwise function fused on each output element; page
// "dispatch_fused_im2col_conv2d_apple", Parameters: the same in 4-D NHWC
// coordinates).  A C ABI cannot carry a device closure, so the library
// offers a fixed one, per output channel co:
//   v = scale[co] * acc + bias[co];  v += beta * src;  v = act(v)
// then the single rounding to the output type.  scale / bias may be null
// (1 / 0).
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_SILU = 2 };

// The coefficients are read through buffer descriptors: a null array gets
// an empty range and channels co >= C_out fall outside it, and such loads
// return 0 without touching memory, so no load needs a branch.
__device__ __forceinline__ float epi_pre(const ConvArgs& a, int co, float v) {
    const int nb = a.F * 4;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.scale), (short)0, a.scale ? nb : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.bias), (short)0, a.bias ? nb : 0, 0x00020000);
    const float sc = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(srs, (unsigned)co * 4u, 0, 0));
    const float bi = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(brs, (unsigned)co * 4u, 0, 0));
    return __builtin_fmaf(a.scale ? sc : 1.0f, v, bi);
}

// The scale and bias of channel co (1 and 0 when absent), for hoisting out
// of unrolled loops; v = fma(sc, acc, bi) is then epi_pre's value.
__device__ __forceinline__ void epi_coef(const ConvArgs& a, int co, float* sc, float* bi) {
    const int nb = a.F * 4;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.scale), (short)0, a.scale ? nb : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.bias), (short)0, a.bias ? nb : 0, 0x00020000);
    const float s = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(srs, (unsigned)co * 4u, 0, 0));
    *sc = a.scale ? s : 1.0f;
    *bi = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(brs, (unsigned)co * 4u, 0, 0));
}

// ReLU keeps v when v > 0, else +0; SiLU is v * sigmoid(v) = v / (1 + e^-v),
// here v times the hardware reciprocal (about 1 ulp) of 1 + e^-v: a few
// instructions instead of an IEEE division, far below the output rounding.
// The activation is uniform, so the branches are scalar, and the two
// quarter-rate transcendentals run only for SiLU.
template <int NV>
__device__ __forceinline__ void epi_act_n(const ConvArgs& a, float* v) {
    if (a.act == ACT_SILU) {
#pragma unroll
        for (int e = 0; e < NV; ++e) v[e] = v[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-v[e]));
    } else if (a.act == ACT_RELU) {
#pragma unroll
        for (int e = 0; e < NV; ++e) v[e] = v[e] > 0.0f ? v[e] : 0.0f;
    }
}

__device__ __forceinline__ float epi_act(const ConvArgs& a, float v) {
    epi_act_n<1>(a, &v);
    return v;
}

// Wait states between the last scaled fp8 MFMA and an epilogue that may read
// its accumulators at once.  For the scaled fp8 MFMAs the wait states the
// compiler inserts before such a read were measured (in a kernel whose
// epilogue read the final MFMA's result first) to be too few: the
// last-written result rows read stale.  Every fp8 kernel therefore puts 24
// extra independent wait states between its last MFMA and its epilogue; the
// scheduling fences keep the compiler from moving either across them.
template <int DT>
__device__ __forceinline__ void fp8_accumulator_margin() {
    if constexpr (DT == DT_FP8) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_step(const i32x4* a, const i32x4* b, f32x4 acc);

// bf16 / fp16: v_mfma_f32_16x16x32_{bf16,f16}; lane l supplies row (l & 15)
// and 8 consecutive k at offset 8 * (l >> 4) of the 32-wide k step.
template <>
__device__ __forceinline__ f32x4 mfma_step<DT_BF16>(const i32x4* a, const i32x4* b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_step<DT_FP16>(const i32x4* a, const i32x4* b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[0]),
                                                  __builtin_bit_cast(f16x8, b[0]), acc, 0, 0, 0);
}
// fp8 e4m3fn: v_mfma_scale_f32_16x16x128_f8f6f4 with both operand formats
// FP8 E4M3 (code 0) and unit E8M0 scales (127 = 2^0).  Lane l supplies 32
// consecutive bytes of row (l & 15); A and B use the same k assignment, so
// the sum covers each k exactly once.
template <>
__device__ __forceinline__ f32x4 mfma_step<DT_FP8>(const i32x4* a, const i32x4* b, f32x4 acc) {
    i32x8 av = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
    i32x8 bv = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// Implicit-GEMM forward convolution.
//   BCO x BPX  workgroup tile (output channels x output pixels)
//   WCO x WPX  arrangement of the 4 waves; each wave owns a
//              (BCO/WCO) x (BPX/WPX) sub-tile of 16x16 MFMA blocks.
// K loop: one 128-byte k-tile per iteration, double-buffered in LDS; the
// next tile's global loads are issued before the current tile's MFMAs.
// Masks (in registers): gathered pixels outside the input (padding), pixel
// rows m >= M and k >= K load zero; filter rows co >= C_out load zero;
// the epilogue stores only m < M, co < C_out.
// Geometry is general: tap (r, s) of output pixel (oh, ow) reads input pixel
// (oh*sh - pt + r*dh, ow*sw - pl + s*dw), input pixels lie xpitch elements
// apart and output pixels ypitch apart, so one launch per channel group (or
// one grouped launch) covers a grouped convolution.
// EG (element gather): C_in * E is not a multiple of 16, so a 16-byte chunk
// of k can span taps; each of its VEC elements is then gathered on its own.
template <int DT, int BCO, int BPX, int WCO, int WPX, bool RESID, bool EG = false>
__global__ __launch_bounds__(NTHREADS) void igemm_fwd_kernel(ConvArgs a) {
    constexpr int E = DtTraits<DT>::E;
    constexpr int VEC = 16 / E;            // elements per 16-byte chunk
    constexpr int KT = KT_BYTES / E;       // elements per k-tile
    constexpr int WTCO = BCO / WCO;        // wave tile
    constexpr int WTPX = BPX / WPX;
    constexpr int TM = WTCO / 16;          // 16x16 blocks per wave
    constexpr int TN = WTPX / 16;
    constexpr int PX_ROWS = BPX / 32;      // gathered rows per thread
    constexpr int CO_ROWS = (BCO + 31) / 32;
    static_assert(WCO * WPX == NTHREADS / 64, "four waves");
    static_assert(WTCO % 16 == 0 && WTPX % 16 == 0, "16x16 MFMA blocks");
    static_assert(BPX % 32 == 0, "pixel rows per load pass");
    constexpr int STAGE = (BCO + BPX) * KT_BYTES;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    lds_poison<NTHREADS>(lds, a.lds_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wco = wave / WPX, wpx = wave % WPX;

    const int tile = xcd_remap(group_block(a, a.px_tiles * a.co_tiles), a.px_tiles * a.co_tiles);
    const int co_tile = tile % a.co_tiles;
    const int px_tile = tile / a.co_tiles;
    const int co0 = co_tile * BCO;
    const int m0 = px_tile * BPX;

    // ---- per-thread load assignment: chunk column c, rows lrow + 32*i
    const int c = tid & (CHUNKS - 1);
    const int lrow = tid >> 3;

    // k decomposition of this thread's chunk, advanced one k-tile at a time
    const int Cdiv = a.C > 0 ? a.C : 1;    // C == 0 means K == 0: no k-tiles
    int kk = c * VEC;                      // element index into K
    int tap = kk / Cdiv;
    int ci = kk - tap * Cdiv;
    int fr = tap / a.S;
    int fs = tap - fr * a.S;

    // pixel rows: 64-bit base offset (elements) and the top-left input
    // coordinate of each row's window; rows past M never pass the check
    int64_t pbase[PX_ROWS];
    int pih[PX_ROWS], piw[PX_ROWS];
    const int howo = a.Ho * a.Wo;
#pragma unroll
    for (int i = 0; i < PX_ROWS; ++i) {
        const int m = m0 + lrow + 32 * i;
        if (m < a.M) {
            const int n = m / howo;
            const int rem = m - n * howo;
            const int oh = rem / a.Wo;
            const int ow = rem - oh * a.Wo;
            pih[i] = oh * a.sh - a.pt;
            piw[i] = ow * a.sw - a.pl;
            pbase[i] = (((int64_t)n * a.H + pih[i]) * a.W + piw[i]) * a.xpitch;
        } else {
            pih[i] = -(1 << 30);
            piw[i] = 0;
            pbase[i] = 0;
        }
    }
    const uint8_t* frow[CO_ROWS];
    bool fvalid[CO_ROWS];
#pragma unroll
    for (int i = 0; i < CO_ROWS; ++i) {
        const int row = lrow + 32 * i;
        const int co = co0 + row;
        fvalid[i] = (row < BCO) && (co < a.F);
        frow[i] = a.nk + ((int64_t)(fvalid[i] ? co : 0) * a.kpitch + c * VEC) * E;
    }

    i32x4 px_reg[PX_ROWS];
    i32x4 co_reg[CO_ROWS];

    auto load_tile = [&](int kt) {
        if constexpr (EG) {
            // each element k = kk + e of the chunk: its own tap and channel
            int64_t eoff[VEC];
            int etr[VEC], ets[VEC];
            bool ekin[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int k = kk + e;
                ekin[e] = k < a.K;
                const int tap = ekin[e] ? k / Cdiv : 0;
                const int c = ekin[e] ? k - tap * Cdiv : 0;
                const int r = tap / a.S, sx = tap - r * a.S;
                etr[e] = r * a.dh;
                ets[e] = sx * a.dw;
                eoff[e] = ((int64_t)etr[e] * a.W + ets[e]) * a.xpitch + c;
            }
#pragma unroll
            for (int i = 0; i < PX_ROWS; ++i) {
                union { i32x4 v; uint16_t h[8]; uint8_t b[16]; } u;
                u.v = i32x4{0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const bool ok = ekin[e] && (unsigned)(pih[i] + etr[e]) < (unsigned)a.H &&
                                    (unsigned)(piw[i] + ets[e]) < (unsigned)a.W;
                    if (ok) {
                        if constexpr (E == 2)
                            u.h[e] = reinterpret_cast<const uint16_t*>(a.x)[pbase[i] + eoff[e]];
                        else
                            u.b[e] = a.x[pbase[i] + eoff[e]];
                    }
                }
                px_reg[i] = u.v;
            }
        } else {
            const bool kin = kk < a.K;
            const int tr = fr * a.dh, ts = fs * a.dw;
            const int64_t koff = ((int64_t)tr * a.W + ts) * a.xpitch + ci;
#pragma unroll
            for (int i = 0; i < PX_ROWS; ++i) {
                const bool ok = kin && (unsigned)(pih[i] + tr) < (unsigned)a.H &&
                                (unsigned)(piw[i] + ts) < (unsigned)a.W;
                i32x4 v = {0, 0, 0, 0};
                if (ok) v = *reinterpret_cast<const i32x4*>(a.x + (pbase[i] + koff) * E);
                px_reg[i] = v;
            }
        }
#pragma unroll
        for (int i = 0; i < CO_ROWS; ++i) {
            i32x4 v = {0, 0, 0, 0};
            if (fvalid[i]) v = *reinterpret_cast<const i32x4*>(frow[i] + (int64_t)kt * KT_BYTES);
            co_reg[i] = v;
        }
        // advance this thread's k decomposition to the next k-tile
        kk += KT;
        if constexpr (!EG) {
            ci += KT;
            while (ci >= a.C && a.C > 0) {
                ci -= a.C;
                if (++fs == a.S) { fs = 0; ++fr; }
            }
        }
    };
    auto store_tile = [&](int stage) {
        uint8_t* base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < CO_ROWS; ++i) {
            const int row = lrow + 32 * i;
            if (row < BCO) *reinterpret_cast<i32x4*>(base + lds_off(row, c)) = co_reg[i];
        }
#pragma unroll
        for (int i = 0; i < PX_ROWS; ++i) {
            const int row = lrow + 32 * i;
            *reinterpret_cast<i32x4*>(base + BCO * KT_BYTES + lds_off(row, c)) = px_reg[i];
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frag_row = lane & 15;
    const int frag_grp = lane >> 4;       // 0..3
    const int wrow_co = wco * WTCO;
    const int wrow_px = wpx * WTPX;

    if (a.ktiles > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }
    for (int kt = 0; kt < a.ktiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < a.ktiles;
        if (more) load_tile(kt + 1);
        const uint8_t* As = lds + cur * STAGE;
        const uint8_t* Bs = As + BCO * KT_BYTES;
        if constexpr (DT == DT_FP8) {
            // one 16x16x128 step covers the whole 128-byte k-tile
            i32x4 af[TM][2], bfr[TN][2];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wrow_co + i * 16 + frag_row;
                af[i][0] = *reinterpret_cast<const i32x4*>(As + lds_off(row, 2 * frag_grp));
                af[i][1] = *reinterpret_cast<const i32x4*>(As + lds_off(row, 2 * frag_grp + 1));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wrow_px + j * 16 + frag_row;
                bfr[j][0] = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, 2 * frag_grp));
                bfr[j][1] = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, 2 * frag_grp + 1));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma_step<DT>(af[i], bfr[j], acc[i][j]);
        } else {
            // two 16x16x32 steps: chunks 0-3 then 4-7
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                i32x4 af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int row = wrow_co + i * 16 + frag_row;
                    af[i] = *reinterpret_cast<const i32x4*>(As + lds_off(row, 4 * h + frag_grp));
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int row = wrow_px + j * 16 + frag_row;
                    bfr[j] = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, 4 * h + frag_grp));
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma_step<DT>(&af[i], &bfr[j], acc[i][j]);
            }
        }
        if (more) store_tile(cur ^ 1);
        __syncthreads();
    }

    fp8_accumulator_margin<DT>();
    // ---- epilogue: lane owns pixel (lane & 15) and channels 4*(lane>>4)+0..3
    // of each 16x16 block.  D = acc (+ beta * src), one rounding, NHWC store.
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    const bool vec_ok = (a.F & 3) == 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int m = m0 + wrow_px + j * 16 + frag_row;
        if (m >= a.M) continue;
        const int64_t obase = out_pixel(a, m) * a.ypitch;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int co = co0 + wrow_co + i * 16 + frag_grp * 4;
            if (co >= a.F) continue;
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            if (vec_ok) {
                if (a.epi) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = epi_pre(a, co + q, v[q]);
                }
                if constexpr (RESID) {
                    const u16x4 s = *reinterpret_cast<const u16x4*>(a.src + obase + co);
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(a.beta, out_to_f32(s[q], ODT), v[q]);
                }
                if (a.epi) epi_act_n<4>(a, v);
                u16x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = f32_to_out(v[q], ODT);
                *reinterpret_cast<u16x4*>(a.y + obase + co) = o;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (co + q < a.F) {
                        float d = v[q];
                        if (a.epi) d = epi_pre(a, co + q, d);
                        if constexpr (RESID) d = __builtin_fmaf(a.beta, out_to_f32(a.src[obase + co + q], ODT), d);
                        if (a.epi) d = epi_act(a, d);
                        a.y[obase + co + q] = f32_to_out(d, ODT);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Filter-resident implicit GEMM for narrow layers (C_out <= 64).
//
// The whole NK matrix (TM*16 rows, zero past C_out) is copied into LDS once
// per workgroup; after one barrier every wave runs on its own: it owns
// TN*16 consecutive output pixels and all TM*16 output channels, gathers its
// pixel operand straight from global memory into MFMA-layout registers with
// 16-byte buffer loads, and reads the filter fragments from LDS.  There are
// no barriers in the K loop, and the gather runs PREFETCH k-tiles ahead.
//
// Gather masking is done by the buffer unit: a lane whose tap falls in the
// padding (or past M or K) gets an offset beyond the buffer's num_records
// and the load returns zero without touching memory.  Every load is
// therefore issued unconditionally and the memory-count waits stay exact.
// The buffer is based at the first image the wave touches; the host gate
// guarantees every valid offset of the wave fits below 2^31 bytes.
constexpr uint32_t OOB_OFFSET = 0x80000000u;
constexpr int RES_WAVES = 4;
constexpr int PREFETCH = 3;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // raw buffer: stride 0, num_records = bytes, default data format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int DT, int TM, int TN, bool RESID, bool TAP_ALIGNED>
__global__ __launch_bounds__(RES_WAVES * 64) void igemm_fwd_resident_kernel(ConvArgs a) {
    constexpr int E = DtTraits<DT>::E;
    constexpr int VEC = 16 / E;
    constexpr int KT = KT_BYTES / E;
    constexpr int ROWS = TM * 16;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    lds_poison<RES_WAVES * 64>(lds, a.lds_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep the
    // buffer descriptors derived from it in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lpitch = a.kpitch * E;  // includes the 16-byte pad: conflict-free fragment reads
    // this workgroup's problem of a grouped launch (before any pointer use)
    const int per = a.groups > 1 ? (int)gridDim.x / a.groups : (int)gridDim.x;
    const int gblock = group_block(a, per);

    // ---- stage the filter (all of K) in LDS, rows >= C_out as zeros.
    // NK rows already carry their 16-byte zero pad, so the LDS image is the
    // first ROWS rows copied byte for byte.  Direct-to-LDS buffer loads: each
    // wave instruction fills one contiguous 1 KB block; bytes past C_out's
    // rows are out of range and zero-filled.  All loads are issued back to
    // back, then waited for once.
    {
        const int slots = ROWS * a.kpitch * E / 16;
        const uint32_t valid = (uint32_t)(a.F * a.kpitch * E);
        const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.nk, valid);
        for (int s0 = wave * 64; s0 < slots; s0 += RES_WAVES * 64) {
            const uint32_t off = (uint32_t)(s0 + lane) * 16u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(frs, (__attribute__((address_space(3))) void*)(lds + s0 * 16),
                                                     16, off < valid ? off : OOB_OFFSET, 0, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();

    const int n_wtiles = (a.M + TN * 16 - 1) / (TN * 16);
    const int wtile = xcd_remap(gblock, per) * RES_WAVES + wave;
    if (wtile >= n_wtiles) return;  // no barrier follows
    const int m0 = wtile * TN * 16;

    const int frag_row = lane & 15;
    const int grp = lane >> 4;
    const int howo = a.Ho * a.Wo;
    const int64_t img = (int64_t)a.H * a.W * a.C;   // elements per image
    const int n0 = m0 / howo;
    const int64_t base_el = (int64_t)n0 * img;
    const int64_t total_el = (int64_t)(a.M / howo) * img;
    int64_t span = (total_el - base_el) * E;
    const uint32_t nrec = span > (int64_t)OOB_OFFSET ? OOB_OFFSET : (uint32_t)span;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.x + base_el * E, nrec);

    // pixel rows of this lane: one per 16-wide block
    int prel[TN], pih[TN], piw[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int m = m0 + j * 16 + frag_row;
        if (m < a.M) {
            const int n = m / howo;
            const int rem = m - n * howo;
            const int oh = rem / a.Wo;
            const int ow = rem - oh * a.Wo;
            pih[j] = oh * a.stride - a.pt;
            piw[j] = ow * a.stride - a.pl;
            prel[j] = (int)((int64_t)(n - n0) * img + ((int64_t)pih[j] * a.W + piw[j]) * a.C);
        } else {
            pih[j] = -(1 << 30);
            piw[j] = 0;
            prel[j] = 0;
        }
    }
    // The two 16-byte chunks of each k-tile this lane supplies to the MFMA.
    // Offsets are computed branch-free: a masked lane (padding, m >= M,
    // k >= K) gets bit 31 set, which is past num_records, so the load
    // returns zero; every load is issued and the wait counts stay exact.
    const int chunk0 = (DT == DT_FP8) ? 2 * grp : grp;
    const int chunk1 = (DT == DT_FP8) ? 2 * grp + 1 : 4 + grp;
    i32x4 vb[PREFETCH][TN][2];

    // TAP_ALIGNED (C_in is a multiple of the k-tile): a k-tile lies inside
    // one filter tap, shared by both chunks; the tap advances by at most one
    // per k-tile, with selects only.
    int t_ci = 0, t_r = 0, t_s = 0, t_kt = 0;
    // general case: each chunk tracks its own (k, tap, channel)
    int kk[2], ci[2], fr[2], fs[2];
    if constexpr (!TAP_ALIGNED) {
        const int Cdiv = a.C > 0 ? a.C : 1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            kk[t] = (t == 0 ? chunk0 : chunk1) * VEC;
            const int tap = kk[t] / Cdiv;
            ci[t] = kk[t] - tap * Cdiv;
            fr[t] = tap / a.S;
            fs[t] = tap - fr[t] * a.S;
        }
    }

    auto gather = [&](i32x4 (&v)[TN][2]) {
        if constexpr (TAP_ALIGNED) {
            const bool kin = t_kt < a.ktiles;
            const int koff = (t_r * a.W + t_s) * a.C + t_ci;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const bool ok = kin & ((unsigned)(pih[j] + t_r) < (unsigned)a.H) &
                                ((unsigned)(piw[j] + t_s) < (unsigned)a.W);
                const uint32_t bad = (uint32_t)(!ok) << 31;
                const uint32_t o = (uint32_t)(prel[j] + koff) * E;
                v[j][0] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (o + chunk0 * 16) | bad, 0, 0);
                v[j][1] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (o + chunk1 * 16) | bad, 0, 0);
            }
            ++t_kt;
            t_ci += KT;
            const bool wrap = t_ci >= a.C;
            t_ci = wrap ? 0 : t_ci;
            t_s += wrap ? 1 : 0;
            const bool wrap2 = t_s >= a.S;
            t_s = wrap2 ? 0 : t_s;
            t_r += wrap2 ? 1 : 0;
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bool kin = kk[t] < a.K;
                const int koff = (fr[t] * a.W + fs[t]) * a.C + ci[t];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const bool ok = kin & ((unsigned)(pih[j] + fr[t]) < (unsigned)a.H) &
                                    ((unsigned)(piw[j] + fs[t]) < (unsigned)a.W);
                    const uint32_t bad = (uint32_t)(!ok) << 31;
                    v[j][t] = __builtin_amdgcn_raw_buffer_load_b128(
                        rsrc, ((uint32_t)(prel[j] + koff) * E) | bad, 0, 0);
                }
                kk[t] += KT;
                ci[t] += KT;
                while (ci[t] >= a.C && a.C > 0) {
                    ci[t] -= a.C;
                    if (++fs[t] == a.S) { fs[t] = 0; ++fr[t]; }
                }
            }
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int kt, const i32x4 (&v)[TN][2]) {
        const uint8_t* arow = lds + frag_row * lpitch + kt * KT_BYTES;
        if constexpr (DT == DT_FP8) {
            i32x4 af[TM][2];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                af[i][0] = *reinterpret_cast<const i32x4*>(arow + i * 16 * lpitch + (2 * grp) * 16);
                af[i][1] = *reinterpret_cast<const i32x4*>(arow + i * 16 * lpitch + (2 * grp + 1) * 16);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i) acc[i][j] = mfma_step<DT>(af[i], v[j], acc[i][j]);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                i32x4 af[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = *reinterpret_cast<const i32x4*>(arow + i * 16 * lpitch + (4 * h + grp) * 16);
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        acc[i][j] = mfma_step<DT>(&af[i], &v[j][h], acc[i][j]);
            }
        }
    };

    const int nkt = a.ktiles;
#pragma unroll
    for (int p = 0; p < PREFETCH - 1; ++p) gather(vb[p]);
    for (int kt = 0; kt < nkt; kt += PREFETCH) {
#pragma unroll
        for (int u = 0; u < PREFETCH; ++u) {
            // always gather (past the last k-tile every lane is masked, so the
            // loads return zeros and only keep the wait counts uniform)
            gather(vb[(u + PREFETCH - 1) % PREFETCH]);
            // keep the loads ahead of this k-tile's MFMAs (the scheduler would
            // otherwise sink them and shrink the prefetch distance)
            __builtin_amdgcn_sched_barrier(0);
            if (kt + u < nkt) compute(kt + u, vb[u]);
        }
    }

    fp8_accumulator_margin<DT>();
    // ---- epilogue: lane owns pixel (lane & 15) of each 16-pixel block
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    const bool vec_ok = (a.F & 3) == 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int m = m0 + j * 16 + frag_row;
        if (m >= a.M) continue;
        const int64_t obase = out_pixel(a, m) * a.F;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int co = i * 16 + grp * 4;
            if (co >= a.F) continue;
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            if (vec_ok) {
                if (a.epi) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = epi_pre(a, co + q, v[q]);
                }
                if constexpr (RESID) {
                    const u16x4 s = *reinterpret_cast<const u16x4*>(a.src + obase + co);
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(a.beta, out_to_f32(s[q], ODT), v[q]);
                }
                if (a.epi) epi_act_n<4>(a, v);
                u16x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = f32_to_out(v[q], ODT);
                *reinterpret_cast<u16x4*>(a.y + obase + co) = o;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (co + q < a.F) {
                        float d = v[q];
                        if (a.epi) d = epi_pre(a, co + q, d);
                        if constexpr (RESID) d = __builtin_fmaf(a.beta, out_to_f32(a.src[obase + co + q], ODT), d);
                        if (a.epi) d = epi_act(a, d);
                        a.y[obase + co + q] = f32_to_out(d, ODT);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Exact n / d for 0 <= n < 2^22 and d >= 1 via a float reciprocal and one
// correction step (|n * (1/d) - n/d| < 1 there); a handful of full-rate
// VALU ops instead of a ~30-instruction integer division.
__device__ __forceinline__ int small_div(int n, int d, float inv_d) {
    int q = (int)((float)n * inv_d);
    const int r = n - __mul24(q, d);
    q += (r >= d) ? 1 : 0;
    q -= (r < 0) ? 1 : 0;
    return q;
}

#define IGC_VMCNT_CASE(n) \
    case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time: a scalar
// jump over the counter's 64 immediate forms.  n is clamped to [0, 63]; at
// most 63 requests are ever counted, so a larger n means no wait.
__device__ __forceinline__ void wait_vmcnt_le(int n) {
    switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
        IGC_VMCNT_CASE(0) IGC_VMCNT_CASE(1) IGC_VMCNT_CASE(2) IGC_VMCNT_CASE(3)
        IGC_VMCNT_CASE(4) IGC_VMCNT_CASE(5) IGC_VMCNT_CASE(6) IGC_VMCNT_CASE(7)
        IGC_VMCNT_CASE(8) IGC_VMCNT_CASE(9) IGC_VMCNT_CASE(10) IGC_VMCNT_CASE(11)
        IGC_VMCNT_CASE(12) IGC_VMCNT_CASE(13) IGC_VMCNT_CASE(14) IGC_VMCNT_CASE(15)
        IGC_VMCNT_CASE(16) IGC_VMCNT_CASE(17) IGC_VMCNT_CASE(18) IGC_VMCNT_CASE(19)
        IGC_VMCNT_CASE(20) IGC_VMCNT_CASE(21) IGC_VMCNT_CASE(22) IGC_VMCNT_CASE(23)
        IGC_VMCNT_CASE(24) IGC_VMCNT_CASE(25) IGC_VMCNT_CASE(26) IGC_VMCNT_CASE(27)
        IGC_VMCNT_CASE(28) IGC_VMCNT_CASE(29) IGC_VMCNT_CASE(30) IGC_VMCNT_CASE(31)
        IGC_VMCNT_CASE(32) IGC_VMCNT_CASE(33) IGC_VMCNT_CASE(34) IGC_VMCNT_CASE(35)
        IGC_VMCNT_CASE(36) IGC_VMCNT_CASE(37) IGC_VMCNT_CASE(38) IGC_VMCNT_CASE(39)
        IGC_VMCNT_CASE(40) IGC_VMCNT_CASE(41) IGC_VMCNT_CASE(42) IGC_VMCNT_CASE(43)
        IGC_VMCNT_CASE(44) IGC_VMCNT_CASE(45) IGC_VMCNT_CASE(46) IGC_VMCNT_CASE(47)
        IGC_VMCNT_CASE(48) IGC_VMCNT_CASE(49) IGC_VMCNT_CASE(50) IGC_VMCNT_CASE(51)
        IGC_VMCNT_CASE(52) IGC_VMCNT_CASE(53) IGC_VMCNT_CASE(54) IGC_VMCNT_CASE(55)
        IGC_VMCNT_CASE(56) IGC_VMCNT_CASE(57) IGC_VMCNT_CASE(58) IGC_VMCNT_CASE(59)
        IGC_VMCNT_CASE(60) IGC_VMCNT_CASE(61) IGC_VMCNT_CASE(62)
        default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
    }
}
#undef IGC_VMCNT_CASE

template <int V>
struct IntC { static constexpr int value = V; };

// Band kernel waves: eight for bf16 / fp16, two per SIMD, so while one
// waits on its LDS fragment reads the other multiplies (measured on the
// ResNet 3x3 layer: 16.3 -> 14.9 us against four waves with the same
// tiles, identical bits); four for fp8, whose twice-as-wide fragments need
// more than the 256 registers a wave has at two waves per SIMD.
constexpr int band_waves(int dt) { return dt == DT_FP8 ? 4 : 8; }
constexpr int BAND_MAX_TN = 4;   // 32-pixel blocks per wave at most
// Patch-resident kernel (igemm_patch.hpp): LDS bytes per staged patch pixel,
// one 128-byte chunk of its channels plus a 16-byte pad.
constexpr int PATCH_PP = 144;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32 MFMA steps (one wave per SIMD keeps these near full rate):
//   bf16/fp16  v_mfma_f32_32x32x16_{bf16,f16}: lane l supplies row (l & 31)
//              and 8 consecutive k at offset 8 * (l >> 5) of the 16-wide step;
//   fp8        v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, unit E8M0 scales):
//              lane l supplies 32 consecutive bytes of row (l & 31).
// Result: lane l holds column (l & 31), rows 8*(v>>2) + 4*(l>>5) + (v&3).
template <int DT>
__device__ __forceinline__ f32x16 mfma32(const i32x4* a, const i32x4* b, f32x16 acc);
template <>
__device__ __forceinline__ f32x16 mfma32<DT_BF16>(const i32x4* a, const i32x4* b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<DT_FP16>(const i32x4* a, const i32x4* b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]),
                                                  __builtin_bit_cast(f16x8, b[0]), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<DT_FP8>(const i32x4* a, const i32x4* b, f32x16 acc) {
    i32x8 av = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
    i32x8 bv = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
}

// The band kernel's filter rows made from the stored filter in the kernel,
// instead of by a separate transpose launch: NK row co at LDS byte
// co*fpitch, k = (r*S + s)*C_in + c at byte k*E (VEC = 16 / E elements per
// 16-byte chunk).  The stored filter is read in whole 16-byte loads and
// transposed in registers:
//  * RSCF [K][F] (RS == 0): block (kb, cb) = VEC x VEC elements, rows
//    k = kb*VEC.. of VEC output channels cb*VEC..; its VEC loads (one per
//    k) become the VEC output channels' chunks at k = kb*VEC (needs C_out a
//    multiple of VEC);
//  * FCRS [F][C][R][S] with R*S == RS (1 or 9): block (co, cb) = the RS
//    taps of VEC input channels cb*VEC.. of output channel co, RS
//    contiguous loads in (c, tap) order; tap t's chunk holds elements
//    j*RS + t, j < VEC.
// K is a whole number of VEC (the band kernel's C_in * E is a multiple of
// 32).  Consecutive threads take consecutive blocks (adjacent addresses).
// load issues one round's loads (NB blocks per thread); store writes them
// once they have arrived.  The pad k >= K of each row is left as it is (the
// MFMA loop never reads it).
template <int E, int NT, int RS>
struct FilterGather {
    static constexpr int VEC = 16 / E;
    static constexpr int NL = RS == 0 ? VEC : RS;              // loads per block
    static constexpr int NB = 1;                                 // blocks per thread per round
    union Block {
        i32x4 w[NL];
        uint16_t h[NL * 8];
        uint8_t b[NL * 16];
    };
    int nblk, ncb;
    float inv_ncb;
    __amdgpu_buffer_rsrc_t rs;
    Block v[NB];

    __device__ __forceinline__ void init(const ConvArgs& a) {
        ncb = (RS == 0 ? a.F : a.C) / VEC;
        nblk = RS == 0 ? (a.K / VEC) * ncb : a.F * ncb;
        inv_ncb = 1.0f / (float)ncb;
        rs = make_rsrc(a.wraw, (uint32_t)(a.F * a.K * E));
    }
    __device__ __forceinline__ void load(const ConvArgs& a, int b0) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int b = b0 + n * NT;
            if (b < nblk) {
                const int hi = small_div(b, ncb, inv_ncb), lo = b - hi * ncb;
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const unsigned off = RS == 0
                        ? (unsigned)(((hi * VEC + i) * a.F + lo * VEC) * E)
                        : (unsigned)((hi * a.C + lo * VEC) * RS * E + i * 16);
                    v[n].w[i] = __builtin_bit_cast(
                        i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                }
            }
        }
    }
    __device__ __forceinline__ void store(const ConvArgs& a, uint8_t* lds, int b0) const {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int b = b0 + n * NT;
            if (b >= nblk) continue;
            const int hi = small_div(b, ncb, inv_ncb), lo = b - hi * ncb;
            constexpr int NOUT = RS == 0 ? VEC : RS;     // chunks per block
#pragma unroll
            for (int t = 0; t < NOUT; ++t) {
                Block c;   // only c.w[0] used
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    // RSCF: chunk of channel lo*VEC + t holds k = hi*VEC + j
                    // (load j, element t); FCRS: chunk of tap t holds input
                    // channel lo*VEC + j (block element j*RS + t)
                    const int src = RS == 0 ? j * VEC + t : j * RS + t;
                    if constexpr (E == 2) c.h[j] = v[n].h[src];
                    else c.b[j] = v[n].b[src];
                }
                const int off = RS == 0 ? (lo * VEC + t) * a.fpitch + hi * VEC * E
                                        : hi * a.fpitch + (t * a.C + lo * VEC) * E;
                *reinterpret_cast<i32x4*>(lds + off) = c.w[0];
            }
        }
    }
};

// Phase A's filter rows from the stored filter (FilterGather), after the
// patch DMA (issue_patch): the patch's requests, mostly to HBM, go out
// first, the filter's L2 reads behind them, as on the NK path (measured on
// the ResNet 3x3 layer: 16.3 -> 15.5 us against the filter loads first).
template <int E, int NT, int RS, class PatchFn>
__device__ __forceinline__ void gather_filter(const ConvArgs& a, uint8_t* lds, int tid,
                                              PatchFn issue_patch) {
    FilterGather<E, NT, RS> g;
    g.init(a);
    issue_patch();
    g.load(a, tid);
    g.store(a, lds, tid);
    constexpr int STEP = NT * FilterGather<E, NT, RS>::NB;
    for (int b0 = tid + STEP; b0 < g.nblk; b0 += STEP) {
        g.load(a, b0);
        g.store(a, lds, b0);
    }
}

// Band kernel: narrow layers (C_out <= 64) whose whole NK filter and one
// tile's input patch fit in LDS together.
//
// A workgroup owns a TH x TW rectangle of output pixels of one image and all
// output channels.  Phase A copies the padded filter and the tile's input
// patch (the (TH-1)*st + R rows and (TW-1)*st + S columns it reads, padding
// as zeros) into LDS with coalesced 16-byte loads, so every input line is
// fetched once per tile instead of once per filter tap.  After one barrier
// each wave runs its MFMAs from LDS alone: for every tap (r, s) the B operand
// of output pixel (th, tw) is patch pixel (th*st + r, tw*st + s).  The
// epilogue (fused coefficients, residual, one rounding) stores 16 bytes per
// lane straight from the accumulators when C_out and the output pixel pitch
// are multiples of 8, else through an fp32 LDS stage.
//
// TM: 32-row blocks of output channels; TN: 32-pixel blocks per wave; U:
// MFMA k-steps per unrolled block (1, 2 or 4, dividing the steps per tap);
// RAW: the filter comes as the stored filter (a.wraw) and is transposed
// here (bf16 / fp16 only), a separate instantiation because the transpose's
// registers would otherwise set every variant's register floor (and halve
// the occupancy of the small ones).
// The input pixel size C_in * elem bytes is a power-of-two multiple of the
// MFMA k-step (cpp_log2 = log2 of its 16-byte chunks).
template <int DT, int TM, int TN, int U, bool RESID, bool RAW = false>
__global__ __launch_bounds__(band_waves(DT) * 64) void igemm_fwd_band_kernel(ConvArgs a) {
    constexpr int BAND_WAVES = band_waves(DT);
    constexpr int E = DtTraits<DT>::E;
    constexpr int KSB = (DT == DT_FP8) ? 64 : 32;   // K bytes per 32x32 MFMA
    constexpr int FR = (DT == DT_FP8) ? 2 : 1;      // 16-byte chunks per fragment
    constexpr int NT = BAND_WAVES * 64;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    lds_poison<BAND_WAVES * 64>(lds, a.lds_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frag_row = lane & 31;
    const int half = lane >> 5;

    const int per_img = a.tiles_h * a.tiles_w;
    const int per = a.groups > 1 ? (int)gridDim.x / a.groups : (int)gridDim.x;
    const int tile = xcd_remap(group_block(a, per), per);
    const int n = tile / per_img;
    const int trem = tile - n * per_img;
    const int oh0 = (trem / a.tiles_w) * a.TH;
    const int ow0 = (trem % a.tiles_w) * a.TW;
    const int ih0 = oh0 * a.stride - a.pt;
    const int iw0 = ow0 * a.stride - a.pl;
    const int cbytes = a.C * E;       // bytes of one input pixel's channels (one group's)
    const int xbytes = a.xpitch * E;  // bytes between input pixels (all groups)
    const int lg = a.cpp_log2;        // log2(chunks per input pixel)

    // ---- phase A: filter rows [frows][fpitch] and the input patch
    // [PH][prow bytes: PW pixels of ppitch bytes, then a row pad] into LDS
    // with direct-to-LDS buffer loads: no register round trip and no
    // LDS-write instructions.  Each wave instruction fills one contiguous
    // 1 KB block (lane t -> 16-byte slot t), so every lane picks the source
    // chunk that belongs at its slot:
    //  * filter: NK rows already carry their 16-byte zero pad, so slot s is
    //    NK byte 16 s (row C_out, when staged, is past the range: zero);
    //  * patch: slot s is in patch row s / rs (rs = prow / 16 slots); within
    //    the row, chunk r % (cpp+1) of pixel r / (cpp+1) for r = s % rs; the
    //    last slot of each pixel, the row pad and padding pixels read out of
    //    range (zero).  The row pad keeps a fragment read whose 32 pixels
    //    wrap to the next tile row free of bank conflicts.
    // All loads go out back to back (patch first), then one wait.
    {
        const int cpp = 1 << lg;                      // data chunks per input pixel
        const int spp = cpp + 1;                      // LDS slots per patch pixel
        const float inv_spp = 1.0f / (float)spp;
        const int rs = a.prow >> 4;                   // LDS slots per patch row
        const int pblocks = (a.PH * rs + 63) >> 6;
        // the input view's strides in pixels (plain tensor: W, 1, H*W)
        const int vrow = a.vrow ? a.vrow : a.W;
        const int vcol = a.vcol ? a.vcol : 1;
        const int64_t img = (int64_t)(a.vimg ? a.vimg : a.H * a.W) * xbytes;
        const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (int64_t)n * img, (uint32_t)img);
        uint8_t* patch = lds + a.patch_off;
        auto issue_patch = [&]() {
            // slot of this lane in block `wave` as (row, slot in row),
            // advanced by one block per wave per instruction with
            // add-and-carry
            const int sl = wave * 64 + lane;
            int ph = sl / rs, rem = sl - (sl / rs) * rs;
            const int dph = (BAND_WAVES * 64) / rs, drem = (BAND_WAVES * 64) % rs;
            for (int b = wave; b < pblocks; b += BAND_WAVES) {
                const int pw = small_div(rem, spp, inv_spp), pos = rem - pw * spp;
                const int ih = ih0 + ph, iw = iw0 + pw;
                const bool ok = (pos < cpp) & (pw < a.PW) & (ph < a.PH) &
                                ((unsigned)ih < (unsigned)a.H) &
                                ((unsigned)iw < (unsigned)a.W);
                const uint32_t off = (uint32_t)((ih * vrow + iw * vcol) * xbytes + pos * 16);
                // non-temporal: each input line is wanted by this tile and
                // at most its neighbours, which run at the same time, so the
                // patch should not push the filter (read by every workgroup)
                // out of L2 (measured: ResNet 3x3 layer 17.0 -> 15.9 us, RGB
                // layer 32.1 -> 30.6 us)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xrs, (__attribute__((address_space(3))) void*)(patch + b * 1024), 16,
                    off | ((uint32_t)!ok << 31), 0, 0, 2);
                rem += drem;
                const int car = rem >= rs ? 1 : 0;
                rem -= car ? rs : 0;
                ph += dph + car;
            }
        };
        if constexpr (RAW && E == 2) {   // (fp8 filters always come as NK matrices)
            // the stored filter, transposed here, then the zero row (row
            // C_out) cleared when it is staged
            switch (a.wrs) {
                case 0: gather_filter<E, NT, 0>(a, lds, tid, issue_patch); break;
                case 1: gather_filter<E, NT, 1>(a, lds, tid, issue_patch); break;
                default: gather_filter<E, NT, 9>(a, lds, tid, issue_patch); break;
            }
            if (a.frows > a.F)
                for (int i = tid; i < a.fpitch / 16; i += NT)
                    *reinterpret_cast<i32x4*>(lds + a.F * a.fpitch + i * 16) = i32x4{0, 0, 0, 0};
        } else {
            issue_patch();
            // the filter after the patch: its rows come from L2, the patch's
            // mostly from HBM, so the longer requests go out first
            const uint32_t fvalid = (uint32_t)(a.F * a.fpitch);
            const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.nk, fvalid);
            const int fblocks = (a.frows * a.fpitch + 1023) >> 10;
            for (int b = wave; b < fblocks; b += BAND_WAVES) {
                const uint32_t off = (uint32_t)(b * 1024 + lane * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    frs, (__attribute__((address_space(3))) void*)(lds + b * 1024), 16,
                    off < fvalid ? off : OOB_OFFSET, 0, 0, 0);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();

    // ---- phase B: MFMAs from LDS.  Wave w owns pixel blocks w,
    // w + BAND_WAVES, ..., always TN of them; blocks past the tile read
    // patch pixel 0 and are never stored.  The k-steps run in blocks of U
    // inside one filter tap:
    // per block one scalar base per operand, the U steps at immediate LDS
    // offsets, and the fragments of step g + LA read while step g multiplies
    // (LA = 2 steps ahead when U >= 2, else 1), into NSET = 2 LA register
    // sets fixed at compile time: step g uses set g % NSET.
    const int P = a.TH * a.TW;
    int pb[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int p = (wave + BAND_WAVES * t) * 32 + frag_row;
        const int tp = p / a.TW, tq = p - tp * a.TW;
        pb[t] = a.patch_off + half * 16 * FR +
                ((p < P) ? tp * a.stride * a.prow + tq * a.stride * a.ppitch : 0);
    }
    int fr_off[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)   // rows >= C_out read the zero row (a broadcast)
        fr_off[i] = min(i * 32 + frag_row, a.frows - 1) * a.fpitch + half * 16 * FR;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = f32x16{};

    const int bpt = cbytes / (KSB * U);   // blocks per tap
    const int NB = a.R * a.S * bpt;
    // uniform walk over blocks: (r, s, b) -> patch and filter byte bases; past
    // the last block it wraps to block 0, so the spare prefetch of the final
    // block still reads valid LDS
    int w_r = 0, w_s = 0, w_b = 0;
    auto next_bases = [&](int& pbase, int& fbase) {
        if (++w_b == bpt) {
            w_b = 0;
            if (++w_s == a.S) { w_s = 0; if (++w_r == a.R) w_r = 0; }
        }
        pbase = w_r * a.prow + w_s * a.ppitch + w_b * U * KSB;
        fbase = (w_r * a.S + w_s) * cbytes + w_b * U * KSB;
    };
    constexpr int LA = U >= 2 ? 2 : 1;   // fragment lookahead in k-steps
    constexpr int NSET = 2 * LA;
    i32x4 fa[NSET][TM][FR], fb[NSET][TN][FR];
    auto rd = [&](int set, int pbase, int fbase, int j) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int h = 0; h < FR; ++h)
                fa[set][i][h] = *reinterpret_cast<const i32x4*>(lds + fr_off[i] + fbase + j * KSB + h * 16);
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int h = 0; h < FR; ++h)
                fb[set][t][h] = *reinterpret_cast<const i32x4*>(lds + pb[t] + pbase + j * KSB + h * 16);
    };
    auto mma = [&](int set) {
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i][t] = mfma32<DT>(fa[set][i], fb[set][t], acc[i][t]);
    };
    // Interleave the next step's fragment reads with this step's MFMAs so
    // the LDS latency hides behind matrix work.
    constexpr int MPG = (TM * TN + TM + TN - 1) / (TM + TN);
    auto interleave = [&]() {
#pragma unroll
        for (int g = 0; g < TM + TN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);   // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, MPG, 0);  // MFMAs
        }
    };
    // one block at bases (pb0, fb0) whose step 0 is in set S0; step j + LA
    // comes from this block or (past its end) from the next one
    int pb0 = 0, fb0 = 0;
    auto block = [&](auto s0c) {
        constexpr int S0 = decltype(s0c)::value;
        int pbn, fbn;
        next_bases(pbn, fbn);
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if (j + LA < U) rd((S0 + j + LA) % NSET, pb0, fb0, j + LA);
            else rd((S0 + j + LA) % NSET, pbn, fbn, j + LA - U);
            mma((S0 + j) % NSET);
            interleave();
            // fence: the scheduler must not pull the next step's MFMAs up
            // next to their own reads
            __builtin_amdgcn_sched_barrier(0);
        }
        pb0 = pbn;
        fb0 = fbn;
    };
    if (NB > 0) {
#pragma unroll
        for (int g = 0; g < LA; ++g) rd(g, 0, 0, g);   // LA <= U: all in block 0
    }
    if constexpr (U % NSET == 0) {
        for (int q = 0; q < NB; ++q) block(IntC<0>{});
    } else {
        // sets rotate by U per block (U = NSET / 2): two blocks per iteration
        // with no early exit, so every accumulator stays in place; an odd
        // last block after
        static_assert(2 * U == NSET, "two blocks cover the set rotation");
        int q = 0;
        for (; q + 2 <= NB; q += 2) {
            block(IntC<0>{});
            block(IntC<U>{});
        }
        if (q < NB) block(IntC<0>{});
    }
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    fp8_accumulator_margin<DT>();   // the epilogue may read the last MFMA first
    const int th_n = min(a.TH, a.Ho - oh0);
    const int tw_n = min(a.TW, a.Wo - ow0);
    if (((a.F | a.ypitch) & 7) == 0) {
        // the fused epilogue's coefficients of this lane's channels
        // i*32 + 8*(2k + half) + 0..7, loaded once (16-byte buffer loads; the
        // whole 8-channel group is inside C_out or outside it)
        f32x4 esc[TM][2][2], ebi[TM][2][2];
        if (a.epi) {
            const int nb = a.F * 4;
            const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.scale), (short)0, a.scale ? nb : 0, 0x00020000);
            const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.bias), (short)0, a.bias ? nb : 0, 0x00020000);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const unsigned off = (unsigned)(i * 32 + 8 * (2 * k + half) + 4 * h) * 4u;
                        const f32x4 sv = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, 0));
                        esc[i][k][h] = a.scale ? sv : f32x4{1.0f, 1.0f, 1.0f, 1.0f};
                        ebi[i][k][h] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, 0));
                    }
        }
        // ---- epilogue straight from the accumulators.  Lane l holds pixel
        // (l & 31) and channels 8g + 4h + 0..3 (h = l >> 5) of each 32-channel
        // block; swapping groups 2k and 2k+1 across the wave halves
        // (v_permlane32_swap) leaves the lower half with all 8 channels of
        // group 2k and the upper half with group 2k+1, so every lane stores
        // 16 contiguous bytes and a store instruction writes 32 pixels x 32
        // contiguous bytes.  No LDS, no barrier.  EPI: the scale / bias /
        // activation path, chosen once (a per-element select would cost its
        // VALU work on every element).
        auto run = [&](auto epic) {
            constexpr bool EPI = decltype(epic)::value;
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int p = (wave + BAND_WAVES * t) * 32 + frag_row;
                const int th = p / a.TW, tw = p - (p / a.TW) * a.TW;
                const bool pix_ok = (p < P) & (th < th_n) & (tw < tw_n);
                const int64_t obase = out_pixel3(a, n, oh0 + th, ow0 + tw) * a.ypitch;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        float v[8];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            // copy the elements out first: a bit cast applied
                            // to a vector subscript reads element 0
                            const float lo = acc[i][t][8 * k + j];
                            const float hi = acc[i][t][8 * k + 4 + j];
                            const auto r = __builtin_amdgcn_permlane32_swap(
                                __builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi),
                                false, false);
                            const unsigned r0 = r[0], r1 = r[1];
                            v[j] = __builtin_bit_cast(float, r0);
                            v[4 + j] = __builtin_bit_cast(float, r1);
                        }
                        const int co = i * 32 + 8 * (2 * k + half);
                        if (pix_ok & (co < a.F)) {
                            if constexpr (EPI) {
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const float sc = esc[i][k][e >> 2][e & 3];
                                    const float bi = ebi[i][k][e >> 2][e & 3];
                                    v[e] = __builtin_fmaf(sc, v[e], bi);
                                }
                            }
                            if constexpr (RESID) {
                                const i32x4 sv = *reinterpret_cast<const i32x4*>(a.src + obase + co);
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const uint16_t hb =
                                        (uint16_t)((unsigned)sv[e >> 1] >> (16 * (e & 1)));
                                    v[e] = __builtin_fmaf(a.beta, out_to_f32(hb, ODT), v[e]);
                                }
                            }
                            if constexpr (EPI) epi_act_n<8>(a, v);
                            i32x4 ov;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                ov[e] = (int)pack_out2(v[2 * e], v[2 * e + 1], ODT);
                            *reinterpret_cast<i32x4*>(a.y + obase + co) = ov;
                        }
                    }
            }
        };
        if (a.epi) run(IntC<1>{});
        else run(IntC<0>{});
        return;
    }
    __syncthreads();  // patch and filter no longer read

    // ---- epilogue for C_out not a multiple of 8: fp32 tile -> LDS
    // [P][spitch floats] -> coalesced stores
    float* stage = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int p = (wave + BAND_WAVES * t) * 32 + frag_row;
        if (p < P) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 v4 = {acc[i][t][4 * g], acc[i][t][4 * g + 1], acc[i][t][4 * g + 2],
                                      acc[i][t][4 * g + 3]};
                    *reinterpret_cast<f32x4*>(stage + p * a.spitch + i * 32 + g * 8 + half * 4) = v4;
                }
        }
    }
    __syncthreads();
    const float inv_twn = 1.0f / (float)tw_n;
    {
        const int items = th_n * tw_n * a.F;
        const float inv_f = 1.0f / (float)a.F;
        for (int it = tid; it < items; it += NT) {
            const int q = small_div(it, a.F, inv_f), co = it - q * a.F;
            const int th = small_div(q, tw_n, inv_twn), tw = q - th * tw_n;
            float v = stage[(th * a.TW + tw) * a.spitch + co];
            const int64_t o = out_pixel3(a, n, oh0 + th, ow0 + tw) * a.ypitch + co;
            if (a.epi) v = epi_pre(a, co, v);
            if constexpr (RESID) v = __builtin_fmaf(a.beta, out_to_f32(a.src[o], ODT), v);
            if (a.epi) v = epi_act(a, v);
            a.y[o] = f32_to_out(v, ODT);
        }
    }
}

// ---------------------------------------------------------------------------
// Wide-layer implicit GEMM (C_out > 64) with direct-to-LDS staging: BCO x BPX
// workgroup tiles (BCO = WCO*TM*32 output channels, BPX = WPX*TN*32 output
// pixels), WCO x WPX waves, each computing TM x TN blocks of 32x32 with 32x32
// MFMAs.  K streams through LDS in k-tiles that reach it by buffer-load-to-LDS:
// no staging registers and no LDS-write instructions in the loop, which
// matters because LDS writes run at about half the LDS read rate.  Gather
// masks are buffer range checks: padding, m >= M, k >= K and co >= C_out lanes
// load zero.  When C_in is a whole number of k-tiles (TAPK) every k-tile lies
// inside one filter tap, so the tap walk is uniform scalar work.
//
// Stage layout: BCO filter rows then BPX pixel rows of KTB bytes (64 or 128),
// unpadded.  Chunk d (16 bytes) of row r sits at position d ^ swz(r), with
// swz(r) = (r >> 1) & 7 for 128-byte rows and (r >> 2) & 3 for 64-byte rows
// (r's 256-byte window), so the 16 lanes of a fragment read served together
// land in 16 different 16-byte bank groups.  One wave DMA instruction fills 1 KB = 1024 / KTB
// whole rows (lane t -> position t % CPR of row t / CPR), so each lane
// fetches the chunk that belongs at its position.
//
// NSTAGE stages rotate.  A k-tile runs its MFMA steps with the next step's
// fragments read in between; before its last step it waits for k-tile
// kt + 1 and meets the other waves at a barrier, after which its own stage
// is free: it requests k-tile kt + NSTAGE there (a fully masked request past
// the end keeps the wait counts uniform) and reads the first fragments of
// k-tile kt + 1 while the last step multiplies.  A request thus has
// NSTAGE - 1 whole k-tiles to arrive.
//
// The epilogue goes through LDS per 32-pixel block: each wave writes its
// fp32 block in [pixel][channel] order into a private region and reads it
// back with consecutive lanes on consecutive channels of one pixel.  The
// residual of block j + 1 is requested while block j is finished; stores
// are 8 bytes per lane, contiguous over the wave's channels, and buffer
// range checks drop pixels past the end.
template <int DT>
struct WideStep;
template <>
struct WideStep<DT_BF16> { static constexpr int KSB = 32; };
template <>
struct WideStep<DT_FP16> { static constexpr int KSB = 32; };
template <>
struct WideStep<DT_FP8> { static constexpr int KSB = 64; };


// GROUPED: a grouped launch (group_block) or an output map (ymap); a
// compile-time choice here, since the runtime pointer selection costs the
// single-problem 256x256 fp8 kernel twelve VGPRs and a quarter of its speed,
// and the map's per-pixel placement as much again (measured: 91 -> 122 us).
template <int DT, int TM, int TN, int WCO, int WPX, int KTB, int NSTAGE, bool RESID, bool TAPK,
          bool GROUPED = false>
__global__ __launch_bounds__(WCO * WPX * 64) void igemm_fwd_wide_kernel(ConvArgs a) {
    constexpr int E = DtTraits<DT>::E;
    constexpr int VEC = 16 / E;
    constexpr int KTE = KTB / E;                      // k elements per k-tile
    constexpr int CPR = KTB / 16;                     // chunks per staged row
    constexpr int RPI = 64 / CPR;                     // rows per DMA instruction
    constexpr int NW = WCO * WPX;
    constexpr int BCO = WCO * TM * 32;
    constexpr int BPX = WPX * TN * 32;
    constexpr int AI = BCO / (RPI * NW), BI = BPX / (RPI * NW);   // DMA instrs per wave
    constexpr int KSB = WideStep<DT>::KSB;            // k bytes per MFMA step
    constexpr int FR = KSB / 32;                      // 16-byte chunks per fragment
    constexpr int KS = KTB / KSB;                     // MFMA steps per k-tile
    constexpr int STAGE = (BCO + BPX) * KTB;
    constexpr int WAITN = (NSTAGE - 2) * (AI + BI);   // requests left in flight
    static_assert(KTB == 64 || KTB == 128, "64- or 128-byte k-tiles");
    static_assert(AI * RPI * NW == BCO && BI * RPI * NW == BPX, "whole DMA rows per wave");
    static_assert(NSTAGE >= 2 && (NSTAGE - 1) * (AI + BI) < 64, "stage count within the wait counter");
    static_assert(CPR == 4 || (AI % 2 == 0 && BI % 2 == 0), "request parity fixed per instruction index");
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    lds_poison<WCO * WPX * 64>(lds, a.lds_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wco = wave / WPX, wpx = wave % WPX;

    const int ntile = a.px_tiles * a.co_tiles;
    const int tile = xcd_remap(GROUPED ? group_block(a, ntile) : (int)blockIdx.x, ntile);
    const int co_tile = tile % a.co_tiles;
    const int px_tile = tile / a.co_tiles;
    const int co0 = co_tile * BCO;
    const int m0 = px_tile * BPX;

    // Bank groups: a 64-lane 16-byte read is served 16 lanes per clock from 64
    // banks (256 bytes), so the 16 rows a fragment read touches at one chunk
    // index must land on 16 different 16-byte groups of a 256-byte window:
    // the position is XORed with the row's index among 256-byte windows.
    auto swz = [](int r) { return CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
    // this lane's DMA slot: row `sub` of each RPI-row group; the data chunk
    // it fetches for request i is dch(i) (for 128-byte rows the row group's
    // parity, which is i's parity since AI and BI are even, flips bit 2)
    const int sub = lane / CPR;
    const int dch0 = (lane % CPR) ^ swz(sub);
    auto dch = [&](int i) { return CPR == 8 ? dch0 ^ ((i & 1) << 2) : dch0; };

    // filter rows: the NK matrix (below 2^31 bytes), rows >= C_out out of range
    const uint32_t nk_bytes = (uint32_t)a.F * (uint32_t)a.kpitch * (uint32_t)E;
    const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.nk, nk_bytes);
    uint32_t aoff[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int co = co0 + (wave * AI + i) * RPI + sub;
        aoff[i] = co < a.F ? (uint32_t)co * (uint32_t)(a.kpitch * E) + dch(i) * 16 : OOB_OFFSET;
    }
    // pixel rows: the buffer starts at the tile's first image
    const int howo = a.Ho * a.Wo;
    const int n0 = m0 / howo;
    const int64_t img = (int64_t)a.H * a.W * a.C * E;   // bytes per image
    const int64_t base = (int64_t)n0 * img;
    const int64_t span = (int64_t)(a.M / howo) * img - base;
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(a.x + base, span > (int64_t)OOB_OFFSET ? OOB_OFFSET : (uint32_t)span);
    int prel[BI], pih[BI], piw[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int m = m0 + (wave * BI + i) * RPI + sub;
        if (m < a.M) {
            const int n = m / howo;
            const int rem = m - n * howo;
            const int oh = rem / a.Wo;
            const int ow = rem - oh * a.Wo;
            pih[i] = oh * a.stride - a.pt;
            piw[i] = ow * a.stride - a.pl;
            // TAPK: the lane's chunk offset rides here; otherwise the per-lane
            // k walks below already start at chunk dch(i)
            prel[i] = (int)((int64_t)(n - n0) * img + (int64_t)(pih[i] * a.W + piw[i]) * a.C * E) +
                      (TAPK ? dch(i) * 16 : 0);
        } else {
            pih[i] = -(1 << 28);
            piw[i] = 0;
            prel[i] = 0;
        }
    }
    // k walk: uniform (TAPK) or per lane, one per distinct chunk (walk w
    // follows chunk dch(w))
    constexpr int NWALK = CPR == 8 ? 2 : 1;
    int t_ci = 0, t_r = 0, t_s = 0;
    int kk[NWALK], ci[NWALK], fr[NWALK], fs[NWALK];
#pragma unroll
    for (int w = 0; w < NWALK; ++w) {
        kk[w] = dch(w) * VEC;
        ci[w] = fr[w] = fs[w] = 0;
        if constexpr (!TAPK) {
            const int Cdiv = a.C > 0 ? a.C : 1;
            const int tap = kk[w] / Cdiv;
            ci[w] = kk[w] - tap * Cdiv;
            fr[w] = tap / a.S;
            fs[w] = tap - fr[w] * a.S;
        }
    }
    auto dma = [](__amdgpu_buffer_rsrc_t rs, uint8_t* dst, uint32_t off) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
    };
    const int nkt = a.ktiles;
    // request the next k-tile into stage `st` (fully masked past the end)
    int kt_next = 0;
    auto issue = [&](int st) {
        const int kt = kt_next++;
        const uint32_t past = kt < nkt ? 0u : OOB_OFFSET;
        uint8_t* sb = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            dma(frs, sb + (wave * AI + i) * 1024, (aoff[i] + (uint32_t)(kt * KTB)) | past);
        uint8_t* pb = sb + BCO * KTB;
        if constexpr (TAPK) {
            const int koff = ((t_r * a.W + t_s) * a.C + t_ci) * E;
#pragma unroll
            for (int i = 0; i < BI; ++i) {
                const bool ok = ((unsigned)(pih[i] + t_r) < (unsigned)a.H) &
                                ((unsigned)(piw[i] + t_s) < (unsigned)a.W);
                dma(xrs, pb + (wave * BI + i) * 1024,
                    (uint32_t)(prel[i] + koff) | ((uint32_t)!ok << 31) | past);
            }
            t_ci += KTE;
            const bool wrap = t_ci >= a.C;
            t_ci = wrap ? 0 : t_ci;
            t_s += wrap ? 1 : 0;
            const bool wrap2 = t_s >= a.S;
            t_s = wrap2 ? 0 : t_s;
            t_r += wrap2 ? 1 : 0;
        } else {
            bool kin[NWALK];
            int koff[NWALK];
#pragma unroll
            for (int w = 0; w < NWALK; ++w) {
                kin[w] = kk[w] < a.K;
                koff[w] = ((fr[w] * a.W + fs[w]) * a.C + ci[w]) * E;
            }
#pragma unroll
            for (int i = 0; i < BI; ++i) {
                const int w = i % NWALK;
                const bool ok = kin[w] & ((unsigned)(pih[i] + fr[w]) < (unsigned)a.H) &
                                ((unsigned)(piw[i] + fs[w]) < (unsigned)a.W);
                dma(xrs, pb + (wave * BI + i) * 1024,
                    (uint32_t)(prel[i] + koff[w]) | ((uint32_t)!ok << 31) | past);
            }
#pragma unroll
            for (int w = 0; w < NWALK; ++w) {
                kk[w] += KTE;
                ci[w] += KTE;
                while (ci[w] >= a.C && a.C > 0) {
                    ci[w] -= a.C;
                    if (++fs[w] == a.S) { fs[w] = 0; ++fr[w]; }
                }
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // fragment addresses: row (lane & 31) of each 32-row block, chunk
    // ks*2*FR + half*FR + h at its swizzled position
    const int frow = lane & 31, half = lane >> 5;
    int xa[KS][FR], xb[KS][FR];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int h = 0; h < FR; ++h) {
            const int x = frow * KTB + (((ks * 2 * FR + half * FR + h) ^ swz(frow)) << 4);
            xa[ks][h] = x + wco * TM * 32 * KTB;
            xb[ks][h] = x + (BCO + wpx * TN * 32) * KTB;
        }
    i32x4 af[2][TM][FR], bfr[2][TN][FR];
    auto read_frags = [&](int st, int ks, int fb) {
        const uint8_t* sb = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int h = 0; h < FR; ++h)
                af[fb][i][h] = *reinterpret_cast<const i32x4*>(sb + xa[ks][h] + i * 32 * KTB);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int h = 0; h < FR; ++h)
                bfr[fb][j][h] = *reinterpret_cast<const i32x4*>(sb + xb[ks][h] + j * 32 * KTB);
    };
    auto mma = [&](int fb) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i][j] = mfma32<DT>(af[fb][i], bfr[fb][j], acc[i][j]);
    };
    constexpr int MPG = (TM * TN + TM + TN - 1) / (TM + TN);
    // last step of a k-tile: the first DMAM MFMAs carry the requests, the
    // rest the next k-tile's first fragment reads
    constexpr int DMAM = TM * TN / 2;
    constexpr int DMAG = (AI + BI + DMAM - 1) / DMAM;                  // requests per MFMA
    constexpr int VALUG = 6 * DMAG;                                    // their address math
    constexpr int RDG = ((TM + TN) * FR + TM * TN - DMAM - 1) / (TM * TN - DMAM);   // reads per MFMA
    auto interleave = [&]() {
#pragma unroll
        for (int g = 0; g < TM + TN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);   // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, MPG, 0);  // MFMAs
        }
    };

    int cur = 0;   // stage of the k-tile being multiplied
    // one k-tile whose step-0 fragments are in buffer FB0
    auto ktile = [&](auto fb0c) {
        constexpr int FB0 = decltype(fb0c)::value;
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            read_frags(cur, ks + 1, (FB0 + ks + 1) & 1);
            mma((FB0 + ks) & 1);
            interleave();
        }
        // k-tile kt + 1 complete in this wave's part and this wave's reads of
        // stage `cur` finished; then a bare barrier (__syncthreads would
        // also drain the requests still in flight)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(WAITN) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int freed = cur;   // free in every wave now: receives k-tile kt + NSTAGE
        cur = cur + 1 == NSTAGE ? 0 : cur + 1;
        issue(freed);
        read_frags(cur, 0, (FB0 + KS) & 1);   // past the last k-tile: a harmless read
        mma((FB0 + KS - 1) & 1);
        // Spread the requests, then the fragment reads, between this step's
        // MFMAs so the matrix pipe is not idle while the wave issues them (the
        // requests write LDS, so they stay ahead of the reads in program order).
#pragma unroll
        for (int g = 0; g < DMAM; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x010, DMAG, 0);       // buffer loads to LDS
            __builtin_amdgcn_sched_group_barrier(0x002, VALUG, 0);      // their address math
        }
#pragma unroll
        for (int g = DMAM; g < TM * TN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, RDG, 0);        // DS reads
        }
    };

    if (nkt > 0) {
#pragma unroll
        for (int st = 0; st < NSTAGE; ++st) issue(st);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSTAGE - 1) * (AI + BI)) : "memory");
        __syncthreads();
        read_frags(0, 0, 0);
        if constexpr (KS % 2 == 0) {
            for (int kt = 0; kt < nkt; ++kt) ktile(IntC<0>{});
        } else {
            // buffers alternate between k-tiles: two per iteration.  KS is
            // odd only for 64-byte k-tiles, and NK rows hold whole 128-byte
            // k-tiles, so nkt is even.
            static_assert(KTB == 64, "odd step counts only with 64-byte k-tiles");
            for (int kt = 0; kt < nkt; kt += 2) {
                ktile(IntC<0>{});
                ktile(IntC<1>{});
            }
        }
    }
    fp8_accumulator_margin<DT>();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // masked tail requests
    __syncthreads();   // stages no longer read or written

    // ---- epilogue through a private LDS region per wave
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    constexpr int WCH = TM * 32;                 // channels per wave
    constexpr int EP = WCH * 4 + 16;             // bytes per pixel row (padded)
    constexpr int LPP = WCH / 4;                 // lanes per pixel on read-back
    constexpr int PPI = 64 / LPP;                // pixels per read-back instruction
    constexpr int NI = 32 / PPI;                 // read-back instructions per block
    static_assert(NW * 32 * EP <= NSTAGE * STAGE, "epilogue region fits the stages");
    uint8_t* ereg = lds + wave * 32 * EP;
    const int c4 = lane % LPP, pl = lane / LPP;
    const int co = co0 + wco * WCH + c4 * 4;     // this lane's first channel
    // the fused epilogue's coefficients of this lane's four channels
    float esc[4], ebi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) epi_coef(a, co + e, &esc[e], &ebi[e]);
    auto stage_block = [&](int j) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v4 = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                  acc[i][j][4 * g + 3]};
                *reinterpret_cast<f32x4*>(ereg + frow * EP + (i * 32 + g * 8 + half * 4) * 4) = v4;
            }
    };
    if ((a.F & 3) == 0) {
        // Block j's pixels [mb, mb + 32) go through buffers based at the
        // block's first output pixel bpx(mb), reaching to one past the last
        // output pixel: without an output map that is pixel mb and [mb, M)
        // (pixels past M fall outside); with one, each lane's pixel is placed
        // by the map and pixels past M are masked.
        const bool mapped = GROUPED && a.ymap;
        const int64_t last_px = mapped ? out_pixel(a, a.M - 1) + 1 : (int64_t)a.M;
        auto bpx = [&](int mb) -> int64_t {
            return mapped ? (mb < a.M ? out_pixel(a, mb) : last_px) : (int64_t)mb;
        };
        auto blk = [&](const uint16_t* p, int64_t b0) {
            const int64_t bytes = b0 < last_px ? (last_px - b0) * a.F * 2 : 0;
            return make_rsrc(p + b0 * a.F,
                             bytes > (int64_t)OOB_OFFSET ? OOB_OFFSET : (uint32_t)bytes);
        };
        // pixel offsets of this lane's NI pixels from the block's base
        auto rel_px = [&](int mb, int64_t b0, uint32_t (&rel)[NI]) {
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const int m = mb + q * PPI + pl;
                rel[q] = !mapped ? (uint32_t)(q * PPI + pl)
                                 : (m < a.M ? (uint32_t)(out_pixel(a, m) - b0) : OOB_OFFSET);
            }
        };
        const uint32_t cmask = co < a.F ? 0u : OOB_OFFSET;
        const int mw = m0 + wpx * TN * 32;      // this wave's first pixel
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        u32x2 sv[2][NI];
        auto load_src = [&](int j) {
            const int mb = mw + j * 32;
            const int64_t b0 = bpx(mb);
            uint32_t rel[NI];
            rel_px(mb, b0, rel);
            const __amdgpu_buffer_rsrc_t srs = blk(a.src, b0);
#pragma unroll
            for (int q = 0; q < NI; ++q)
                // non-temporal: the source is read exactly once (measured
                // on the fp8 5x5 layer: 101.5 -> 97 us)
                sv[j & 1][q] = __builtin_amdgcn_raw_buffer_load_b64(
                    srs, ((rel[q] * (uint32_t)a.F + co) * 2) | (rel[q] & OOB_OFFSET) | cmask, 0,
                    2);
        };
        // EPI: the scale / bias / activation path, chosen once (a
        // per-element select would cost its VALU work on every element)
        auto run = [&](auto epic) {
        constexpr bool EPI = decltype(epic)::value;
        if constexpr (RESID) load_src(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (RESID) {
                if (j + 1 < TN) load_src(j + 1);
            }
            stage_block(j);
            const int mb = mw + j * 32;
            const int64_t b0 = bpx(mb);
            uint32_t rel[NI];
            rel_px(mb, b0, rel);
            const __amdgpu_buffer_rsrc_t yrs = blk(a.y, b0);
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(ereg + (q * PPI + pl) * EP + c4 * 16);
                float v[4] = {v4[0], v4[1], v4[2], v4[3]};
                if constexpr (EPI) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(esc[e], v[e], ebi[e]);
                }
                if constexpr (RESID) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint16_t h = (uint16_t)(sv[j & 1][q][e >> 1] >> (16 * (e & 1)));
                        v[e] = __builtin_fmaf(a.beta, out_to_f32(h, ODT), v[e]);
                    }
                }
                if constexpr (EPI) epi_act_n<4>(a, v);
                u32x2 ov;
                ov[0] = pack_out2(v[0], v[1], ODT);
                ov[1] = pack_out2(v[2], v[3], ODT);
                // non-temporal (cache policy NT): the output is written once
                // and not read again by this kernel; each instruction writes
                // 128 or 256 contiguous bytes per pixel (measured with C_out
                // = 256: fp8 5x5 layer 105.6 -> 103.3 us, strided 3x3 layer
                // 28.1 -> 26.8 us)
                __builtin_amdgcn_raw_buffer_store_b64(
                    ov, yrs, ((rel[q] * (uint32_t)a.F + co) * 2) | (rel[q] & OOB_OFFSET) | cmask,
                    0, 2);
            }
        }
        };
        if (a.epi) run(IntC<1>{});
        else run(IntC<0>{});
    } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            stage_block(j);
            const int mb = m0 + wpx * TN * 32 + j * 32;
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const int m = mb + q * PPI + pl;
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(ereg + (q * PPI + pl) * EP + c4 * 16);
                if (m >= a.M) continue;
                const int64_t o = (GROUPED ? out_pixel(a, m) : (int64_t)m) * a.F + co;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (co + e < a.F) {
                        float d = v4[e];
                        if (a.epi) d = __builtin_fmaf(esc[e], d, ebi[e]);
                        if constexpr (RESID) d = __builtin_fmaf(a.beta, out_to_f32(a.src[o + e], ODT), d);
                        if (a.epi) d = epi_act(a, d);
                        a.y[o + e] = f32_to_out(d, ODT);
                    }
                }
            }
        }
    }
}

}  // namespace igc

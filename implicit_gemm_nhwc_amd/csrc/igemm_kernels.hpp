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
    uint16_t* y;        // NHWC output (bf16 or fp16 bits)
    const uint16_t* src;  // residual source, same layout and type as y
    float beta;
    int H, W, C;        // input (N only enters through M)
    int Ho, Wo, F;      // output spatial size and C_out
    int S, stride, pad;
    int K;              // R*S*C elements
    int kpitch;         // elements per NK row
    int M;              // N*Ho*Wo
    int ktiles;         // kpitch / (KT_BYTES / E)
    int px_tiles;       // ceil(M / BPX)
    int co_tiles;       // ceil(F / BCO)
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

// LDS tiles: rows of 128 bytes, chunk c of row r stored at c ^ (r & 7) so
// that eight consecutive rows read at one logical chunk hit eight
// different 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * KT_BYTES + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ uint16_t f32_to_out(float v, int dt) {
    if (dt == DT_FP16) {
        _Float16 h = (_Float16)v;
        return __builtin_bit_cast(uint16_t, h);
    }
    __bf16 b = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float out_to_f32(uint16_t bits, int dt) {
    if (dt == DT_FP16) return (float)__builtin_bit_cast(_Float16, bits);
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
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
// Filter transpose to NK (page "dispatch_fused_im2col_conv2d_apple", summary).
// One thread writes one 16-byte chunk of an NK row; the chunk's elements are
// VEC channels of one tap (C % VEC == 0), gathered from the stored layout:
//   RSCF [R,S,C,F]: W(k, co) = w[k*F + co]              (k = (r*S+s)*C + ci)
//   FCRS [F,C,R,S]: W(k, co) = w[((co*C + ci)*R + r)*S + s]
// Chunks at or past K are zero.
template <int E>
__global__ __launch_bounds__(256) void filter_to_nk_kernel(
    const uint8_t* __restrict__ w, uint8_t* __restrict__ nk, int fcrs, int R, int S,
    int C, int F, int K, int kpitch) {
    constexpr int VEC = 16 / E;
    const int chunks_per_row = kpitch / VEC;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)chunks_per_row * F) return;
    const int co = (int)(gid / chunks_per_row);
    const int k0 = (int)(gid % chunks_per_row) * VEC;
    union { i32x4 v; uint8_t b[16]; uint16_t h[8]; } u;
    u.v = i32x4{0, 0, 0, 0};
    if (k0 < K) {
        const int tap = k0 / C, ci0 = k0 - tap * C;
        const int r = tap / S, s = tap - r * S;
        for (int j = 0; j < VEC; ++j) {
            int64_t idx;
            if (fcrs) idx = ((int64_t)(co * C + ci0 + j) * R + r) * S + s;
            else idx = (int64_t)(k0 + j) * F + co;
            if (E == 2) u.h[j] = reinterpret_cast<const uint16_t*>(w)[idx];
            else u.b[j] = w[idx];
        }
    }
    *reinterpret_cast<i32x4*>(nk + ((int64_t)co * kpitch + k0) * E) = u.v;
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
template <int DT, int BCO, int BPX, int WCO, int WPX, bool RESID>
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

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wco = wave / WPX, wpx = wave % WPX;

    const int tile = xcd_remap(blockIdx.x, a.px_tiles * a.co_tiles);
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
            pih[i] = oh * a.stride - a.pad;
            piw[i] = ow * a.stride - a.pad;
            pbase[i] = (((int64_t)n * a.H + pih[i]) * a.W + piw[i]) * a.C;
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
        const bool kin = kk < a.K;
        const int64_t koff = ((int64_t)fr * a.W + fs) * a.C + ci;
#pragma unroll
        for (int i = 0; i < PX_ROWS; ++i) {
            const bool ok = kin && (unsigned)(pih[i] + fr) < (unsigned)a.H &&
                            (unsigned)(piw[i] + fs) < (unsigned)a.W;
            i32x4 v = {0, 0, 0, 0};
            if (ok) v = *reinterpret_cast<const i32x4*>(a.x + (pbase[i] + koff) * E);
            px_reg[i] = v;
        }
#pragma unroll
        for (int i = 0; i < CO_ROWS; ++i) {
            i32x4 v = {0, 0, 0, 0};
            if (fvalid[i]) v = *reinterpret_cast<const i32x4*>(frow[i] + (int64_t)kt * KT_BYTES);
            co_reg[i] = v;
        }
        // advance this thread's k decomposition to the next k-tile
        kk += KT;
        ci += KT;
        while (ci >= a.C && a.C > 0) {
            ci -= a.C;
            if (++fs == a.S) { fs = 0; ++fr; }
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

    // ---- epilogue: lane owns pixel (lane & 15) and channels 4*(lane>>4)+0..3
    // of each 16x16 block.  D = acc (+ beta * src), one rounding, NHWC store.
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    const bool vec_ok = (a.F & 3) == 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int m = m0 + wrow_px + j * 16 + frag_row;
        if (m >= a.M) continue;
        const int64_t obase = (int64_t)m * a.F;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int co = co0 + wrow_co + i * 16 + frag_grp * 4;
            if (co >= a.F) continue;
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            if (vec_ok) {
                if constexpr (RESID) {
                    const u16x4 s = *reinterpret_cast<const u16x4*>(a.src + obase + co);
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(a.beta, out_to_f32(s[q], ODT), v[q]);
                }
                u16x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = f32_to_out(v[q], ODT);
                *reinterpret_cast<u16x4*>(a.y + obase + co) = o;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (co + q < a.F) {
                        float d = v[q];
                        if constexpr (RESID) d = __builtin_fmaf(a.beta, out_to_f32(a.src[obase + co + q], ODT), d);
                        a.y[obase + co + q] = f32_to_out(d, ODT);
                    }
                }
            }
        }
    }
}

}  // namespace igc

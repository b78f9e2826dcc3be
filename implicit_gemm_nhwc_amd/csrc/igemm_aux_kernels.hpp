// Kernels besides the implicit GEMMs: the filter transposes into NK
// matrices and the materialised im2col.  Included only by the translation unit of the C
// entry points.
#pragma once

#include "igemm_kernels.hpp"

namespace igc {

// ---------------------------------------------------------------------------
// Filter transpose to NK (page "dispatch_fused_im2col_conv2d_apple", summary).
// One thread writes one 16-byte chunk of an NK row, gathered element by
// element from the stored layout:
//   RSCF [R,S,C,F]: W(k, co) = w[k*F + co]              (k = (r*S+s)*C + ci)
//   FCRS [F,C,R,S]: W(k, co) = w[((co*C + ci)*R + r)*S + s]
// When C % VEC == 0 a chunk's VEC elements are channels of one tap, at a
// fixed stride in the source; otherwise each element finds its own tap.
// Elements at or past K are zero.  Consecutive lanes take the stored
// layout's contiguous direction, so each of a wave's VEC loads touches few
// lines:
//   RSCF: lanes along co (x), chunks along y;
//   FCRS: lanes along the chunks of one row (x), rows along y.
// Grid rows past 65535 loop.  Indices are 32-bit: the NK matrix is below
// 2^31 bytes.
template <int E>
__global__ __launch_bounds__(64) void filter_to_nk_kernel(
    const uint8_t* __restrict__ w, uint8_t* __restrict__ nk, int fcrs, int R, int S,
    int C, int F, int K, int kpitch) {
    constexpr int VEC = 16 / E;
    const int row_chunks = kpitch / VEC;
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    auto chunk_out = [&](int co, int chunk) {
        const int k0 = chunk * VEC;
        union { i32x4 v; uint8_t b[16]; uint16_t h[8]; } u;
        u.v = i32x4{0, 0, 0, 0};
        if (k0 < K && C % VEC == 0) {
            const int tap = k0 / C, ci0 = k0 - tap * C;
            const int r = tap / S, s = tap - r * S;
            // VEC independent element loads at a fixed stride, all in flight
            const int base = fcrs ? ((co * C + ci0) * R + r) * S + s : k0 * F + co;
            const int step = fcrs ? R * S : F;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                if (E == 2) u.h[j] = reinterpret_cast<const uint16_t*>(w)[base + j * step];
                else u.b[j] = w[base + j * step];
            }
        } else if (k0 < K) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int k = k0 + j;
                const int tap = k / C, ci = k - tap * C;
                const int r = tap / S, s = tap - r * S;
                const int idx = k < K ? (fcrs ? ((co * C + ci) * R + r) * S + s : k * F + co) : 0;
                if (E == 2) u.h[j] = k < K ? reinterpret_cast<const uint16_t*>(w)[idx] : 0;
                else u.b[j] = k < K ? w[idx] : 0;
            }
        }
        *reinterpret_cast<i32x4*>(nk + ((int64_t)co * kpitch + k0) * E) = u.v;
    };
    if (fcrs) {
        if (x >= row_chunks) return;
        for (int co = blockIdx.y; co < F; co += gridDim.y) chunk_out(co, x);
    } else {
        if (x >= F) return;
        for (int chunk = blockIdx.y; chunk < row_chunks; chunk += gridDim.y) chunk_out(x, chunk);
    }
}

// ---------------------------------------------------------------------------
// NK matrix of a grouped convolution run as super-groups: q consecutive
// channel groups (Cg input, Fg output channels each) form one problem of
// q*Cg input and q*Fg output channels whose filter is block diagonal:
//   NK'[co][tap*qCg + c'] = W(tap, c' - j*Cg, co)  if c' / Cg == j,
//                           0                       otherwise,
// j = (co % qFg) / Fg the group of co inside its super-group, W the stored
// filter (RSCF [R][S][Cg][F] or FCRS [F][Cg][R][S]); zero at or past
// K' = R*S*qCg.  One thread per 16-byte chunk, element by element; grid
// rows past 65535 loop; 32-bit indices (below 2^31 bytes).
template <int E>
__global__ __launch_bounds__(64) void filter_to_nk_blockdiag_kernel(
    const uint8_t* __restrict__ w, uint8_t* __restrict__ nk, int fcrs, int R, int S, int Cg,
    int F, int Fg, int q, int kpitch) {
    constexpr int VEC = 16 / E;
    const int row_chunks = kpitch / VEC;
    const int qcg = q * Cg, qfg = q * Fg;
    const int Kp = R * S * qcg;
    const int chunk = blockIdx.x * blockDim.x + threadIdx.x;
    if (chunk >= row_chunks) return;
    for (int co = blockIdx.y; co < F; co += gridDim.y) {
        const int j = (co % qfg) / Fg;
        union { i32x4 v; uint16_t h[8]; uint8_t b[16]; } u;
        u.v = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int k = chunk * VEC + e;
            const int tap = k / qcg, cp = k - tap * qcg;
            const int c = cp - j * Cg;
            if (k < Kp && c >= 0 && c < Cg) {
                const int r = tap / S, sx = tap - r * S;
                const int idx = fcrs ? ((co * Cg + c) * R + r) * S + sx : (tap * Cg + c) * F + co;
                if constexpr (E == 2) u.h[e] = reinterpret_cast<const uint16_t*>(w)[idx];
                else u.b[e] = w[idx];
            }
        }
        *reinterpret_cast<i32x4*>(nk + ((int64_t)co * kpitch + chunk * VEC) * E) = u.v;
    }
}

// ---------------------------------------------------------------------------
// NK matrices of a transposed convolution's phases (page "conv_transposed_gpu":
// RSFC filter [R][S][F][C], F output and C input channels).  A phase takes the
// taps BH + LH*j (j < JH) along the height and BW + LW*j (j < JW) along the
// width and reads them in reverse order (see the phase decomposition in the
// host code), so its NK matrix is
//   NK'[f][(t_h*JW + t_w)*C + c] = W[BH + LH*(JH-1-t_h)][BW + LW*(JW-1-t_w)][f][c]
// for each (f, t_h, t_w) a contiguous run of C elements of W.  One thread
// writes one 16-byte chunk: a single 16-byte copy when C * E % 16 == 0,
// else element by element (each finding its own tap); elements at or past K
// are zero.
struct TapSel {
    int R, S, F, C;    // stored filter
    int BH, BW;        // first tap of the phase along each axis
    int JH, JW;        // taps of the phase along each axis
    int LH, LW;        // tap step along each axis
    int K, kpitch;     // K = JH*JW*C; NK row pitch (elements)
};

// Up to four phases in one launch: blockIdx.y selects the phase.
struct TapSels {
    TapSel t[4];
    uint8_t* nk[4];
};

template <int E>
__global__ __launch_bounds__(256) void filter_rsfc_to_nk_flipped_kernel(
    const uint8_t* __restrict__ w, TapSels ts) {
    constexpr int VEC = 16 / E;
    const TapSel& t = ts.t[blockIdx.y];
    uint8_t* __restrict__ nk = ts.nk[blockIdx.y];
    const int row_chunks = t.kpitch / VEC;
    const int64_t total = (int64_t)t.F * row_chunks;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * 256) {
        const int f = (int)(g / row_chunks), chunk = (int)(g - (int64_t)f * row_chunks);
        const int k0 = chunk * VEC;
        auto src_of = [&](int k) {
            const int tap = k / t.C, c = k - tap * t.C;
            const int th = tap / t.JW, tw = tap - th * t.JW;
            const int r = t.BH + t.LH * (t.JH - 1 - th), sx = t.BW + t.LW * (t.JW - 1 - tw);
            return (((int64_t)r * t.S + sx) * t.F + f) * t.C + c;   // element index
        };
        union { i32x4 v; uint16_t h[8]; uint8_t b[16]; } u;
        u.v = i32x4{0, 0, 0, 0};
        if (k0 < t.K && (t.C * E) % 16 == 0) {
            u.v = *reinterpret_cast<const i32x4*>(w + src_of(k0) * E);
        } else if (k0 < t.K) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                if (k0 + j < t.K) {
                    if constexpr (E == 2)
                        u.h[j] = reinterpret_cast<const uint16_t*>(w)[src_of(k0 + j)];
                    else
                        u.b[j] = w[src_of(k0 + j)];
                }
            }
        }
        *reinterpret_cast<i32x4*>(nk + ((int64_t)f * t.kpitch + k0) * E) = u.v;
    }
}

// ---------------------------------------------------------------------------
// Materialised im2col (page "dispatch_fused_im2col_conv2d_apple", summary:
// the [M, K] patch matrix the fused path never writes), for comparing the
// fused gather against the write-then-GEMM route on the same MFMA kernels:
//   A[m][k] = x[n, oh*st - p + r, ow*st - p + s, ci]   (0 in the padding)
//   m = (n*Ho + oh)*Wo + ow,  k = (r*S + s)*C_in + ci,  rows of Kp elements
// (K rounded up to whole 128-byte k-tiles, zero past K).  Read as an NHWC
// tensor [N, Ho, Wo, Kp], A is the input of a 1x1, stride-1 convolution
// whose NK matrix is the original filter's.
//
// One thread per 16-byte vector of A, grid-stride; a vector is VEC channels
// of one tap (C_in * E % 16 == 0).  Stores are fully coalesced; loads are
// contiguous within a tap's channels.  Divisions by runtime constants use
// multiply-high magic numbers made on the host.
struct FastDiv {
    uint32_t mul;    // ceil(2^(32+shift) / d) - 2^32
    uint32_t shift;  // ceil(log2(d))
};

// floor(n / d) for 0 <= n < 2^31: with m = ceil(2^(32+s) / d), s = ceil(log2 d),
// n * m / 2^(32+s) exceeds n / d by less than n / 2^(32+s) < 1/d, which never
// reaches the next integer.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv d) {
    return (__umulhi(n, d.mul) + n) >> d.shift;
}

struct Im2colArgs {
    const uint8_t* x;
    uint8_t* a;
    int H, W, Ho, Wo, S, stride, pad;
    int RS;             // taps
    int CB;             // bytes per input pixel (C_in * E)
    uint32_t total;     // 16-byte vectors of A: M * VPR
    uint32_t VPR, CV;   // vectors per A row; per tap
    uint32_t HoWo;
    FastDiv d_vpr, d_cv, d_s, d_howo, d_wo;
};

__global__ __launch_bounds__(256) void im2col_kernel(Im2colArgs a) {
    const uint32_t step = gridDim.x * 256u;
    for (uint32_t g = blockIdx.x * 256u + threadIdx.x; g < a.total; g += step) {
        const uint32_t m = fast_div(g, a.d_vpr), j = g - m * a.VPR;
        const uint32_t tap = fast_div(j, a.d_cv), cv = j - tap * a.CV;
        i32x4 v = {0, 0, 0, 0};
        if (tap < (uint32_t)a.RS) {
            const int r = (int)fast_div(tap, a.d_s), s = (int)tap - r * a.S;
            const uint32_t n = fast_div(m, a.d_howo), rem = m - n * a.HoWo;
            const int oh = (int)fast_div(rem, a.d_wo), ow = (int)rem - oh * a.Wo;
            const int ih = oh * a.stride - a.pad + r, iw = ow * a.stride - a.pad + s;
            if ((unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W)
                v = *reinterpret_cast<const i32x4*>(
                    a.x + (((int64_t)n * a.H + ih) * a.W + iw) * a.CB + cv * 16);
        }
        *reinterpret_cast<i32x4*>(a.a + (int64_t)g * 16) = v;
    }
}

}  // namespace igc

// Tap-fold kernel for convolutions with few output channels (C_out * R * S
// <= 32), such as a decoder's last layer to RGB (C_out = 3, 3x3).
//
// The implicit GEMM of the other kernels multiplies a C_out x (R*S*C_in)
// filter by (R*S*C_in) x pixels gathered columns: with C_out = 3 the 32-row
// MFMA blocks are 91% padding, and every input pixel is gathered R*S times.
// Here the rows of the MFMA are the C_out*R*S (output channel, tap) pairs
// and K is C_in alone:
//   P[(co, r, s)][q] = sum_ci W(r, s, ci, co) * x[q][ci]      for every input pixel q
// so each input pixel is multiplied once, by all taps of all channels (the
// A operand is read from the NK matrix: row co, columns (r*S + s)*C_in + ci,
// page "dispatch_fused_im2col_conv2d_apple", summary).  Each output then
// sums its R*S shifted partial products:
//   y[oh][ow][co] = sum_{r,s} P[(co, r, s)][(oh*st - p + r, ow*st - p + s)]
// which is the convolution's definition with the sum over ci done first.
//
// Work: a workgroup owns a strip of TW output columns and TH output rows of
// one image.  It streams the strip's PH = (TH - 1)*st + R input rows (PW =
// (TW - 1)*st + S pixels each, padding as zeros) through a ring of NSLOT
// row slots in LDS, filled by buffer-load-to-LDS NSLOT - 1 rows ahead.
// A slot holds its pixels unpadded, so every 1 KB request covers whole
// cache lines of the NHWC row (a 16-byte pad per pixel made each request
// straddle lines and cut the streaming rate from 5.5 to 3.2 TB/s,
// measured); the 16-byte units are instead permuted within each 256-byte
// window (stage_unit), which keeps the fragment reads of 16 consecutive
// pixels on 16 different bank groups.  Per
// input row, the 32-pixel blocks of P are computed (wave w takes blocks
// 3 - w, 7 - w, ...: a one-block row goes to wave 3, which neither loads
// nor, below 65 output columns, sums; 17.7 -> 17.4 us on the RGB layer) and
// written to a ring of R + 1 fp32 P rows; the output row whose
// last tap row this completes is summed, passed through the fused epilogue
// and stored.  Waves 0 and 1 issue the row requests and wait on their
// counter; waves 2 and 3 do the output sums and stores.  A wave that waits
// for its loads thus never has stores outstanding (the vector-memory counter
// counts both, and a store would hold up the wait), and the stores of one
// row leave while the next rows are multiplied.  Two barriers per input row.
// Short rows (at most TF_RPF_BLOCKS 1 KB blocks) take a second path: the
// loader waves fetch rows into registers two rows ahead and write each into
// its slot one row ahead, with one barrier per row; its first two rows are
// requested together with the NK rows.
#pragma once

#include "igemm_kernels.hpp"

namespace igc {

constexpr int TF_WAVES = 4;
constexpr int TF_RPF_BLOCKS = 8;   // register-staged rows: 1 KB blocks per row at most

// Position of 16-byte unit u (= pixel * cpp + chunk, cpp = 2^cl chunks per
// pixel) in a staged row: the unit's index within its 256-byte window is
// XORed with the window's index (the pixel's index for 512-byte pixels).  An
// involution that stays inside the window, so a request's 64 units are the
// same 64 units of the row either way, and 16 consecutive pixels that start
// at a multiple of 16 read chunk c from 16 different bank groups.
__device__ __forceinline__ int stage_unit(int u, int cl) {
    const int h = (u >> (cl > 4 ? cl : 4)) & 15;
    return (u & ~15) | ((u & 15) ^ h);
}

// KS: MFMA k-steps over C_in (the A fragments held in registers); T3: the
// filter is 3x3 (C_out <= 3), so the output sums unroll at compile time;
// RPF: the input rows go through the loader waves' registers (at most
// TF_RPF_BLOCKS 1 KB blocks per row), two rows in flight per workgroup, and
// the register count is held to four waves per SIMD (four workgroups per
// CU).
template <int DT, int KS, bool T3, bool RESID, bool RPF>
__global__ __launch_bounds__(TF_WAVES * 64)
__attribute__((amdgpu_waves_per_eu(RPF ? 4 : 1, 8))) void igemm_fwd_tapfold_kernel(ConvArgs a) {
    constexpr int E = DtTraits<DT>::E;
    constexpr int KSB = (DT == DT_FP8) ? 64 : 32;   // K bytes per 32x32 MFMA
    constexpr int FR = (DT == DT_FP8) ? 2 : 1;      // 16-byte chunks per fragment
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    lds_poison<TF_WAVES * 64>(lds, a.lds_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const int RS = a.R * a.S;
    const int cbytes = a.C * E;

    const int per_img = a.tiles_h * a.tiles_w;
    const int tile = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int n = tile / per_img;
    const int trem = tile - n * per_img;
    const int oh0 = (trem / a.tiles_w) * a.TH;
    const int ow0 = (trem % a.tiles_w) * a.TW;
    const int ih0 = oh0 * a.stride - a.pt;
    const int iw0 = ow0 * a.stride - a.pl;

    // ---- LDS: [coefficients: scale[32], bias[32]] [input row ring: NSLOT
    // slots of prow bytes] [P ring: R + 1 rows of PW pixels x spitch floats].
    // The NK rows are staged in the ring's space first: they are dead once
    // each lane holds its A fragments.
    float* coef = reinterpret_cast<float*>(lds);
    const int NK_OFF = a.patch_off;
    const int nk_bytes = a.F * a.kpitch * E;
    const int NSLOT = a.nslot;
    const int p_off = a.patch_off + NSLOT * a.prow;
    const int pslot = (a.PW * a.spitch * 4 + 15) & ~15;

    // ---- row requests (waves 0 and 1): input row q of the segment into ring
    // slot q % NSLOT.  Each wave instruction fills one 1 KB block of the
    // slot; lane t of block b fetches the 16-byte unit stage_unit(64 b + t).
    // Rows and pixels outside the image and rows past the segment read out
    // of range: zero, without touching memory.
    const int cpp = cbytes >> 4;
    const int cl = __builtin_ctz((unsigned)cpp);   // cpp is a power of two
    const int nrb = a.prow >> 10;   // 1 KB blocks per slot
    const int64_t img = (int64_t)a.H * a.W * cbytes;
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (int64_t)n * img, (uint32_t)img);
    const bool loader = wave < 2;
    auto issue_row = [&](int q) {
        const int ih = ih0 + q;
        const bool row_ok = (q < a.PH) & ((unsigned)ih < (unsigned)a.H);
        uint8_t* slot = lds + a.patch_off + (q % NSLOT) * a.prow;
        for (int b = wave; b < nrb; b += 2) {
            const int u = stage_unit(b * 64 + lane, cl);   // the unit this lane's slot holds
            const int px = u >> cl, pos = u & (cpp - 1);
            const int iw = iw0 + px;
            const bool ok = row_ok & (px < a.PW) & ((unsigned)iw < (unsigned)a.W);
            const uint32_t off = (uint32_t)((ih * a.W + iw) * cbytes + pos * 16);
            // non-temporal: each input line is read by this strip and at most
            // its neighbours
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (__attribute__((address_space(3))) void*)(slot + b * 1024), 16,
                off | ((uint32_t)!ok << 31), 0, 0, 2);
        }
    };
    constexpr int NBL = TF_RPF_BLOCKS / 2;
    i32x4 rbuf[2][NBL];
    auto load_row = [&](int q, i32x4 (&rb)[NBL]) {
        const int ih = ih0 + q;
        const bool row_ok = (q < a.PH) & ((unsigned)ih < (unsigned)a.H);
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int b = wave + 2 * j;
            const int u = stage_unit(b * 64 + lane, cl);
            const int px = u >> cl, pos = u & (cpp - 1);
            const int iw = iw0 + px;
            const bool ok = row_ok & (b < nrb) & (px < a.PW) & ((unsigned)iw < (unsigned)a.W);
            const uint32_t off = (uint32_t)((ih * a.W + iw) * cbytes + pos * 16);
            // non-temporal, as the ring requests
            rb[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  xrs, off | ((uint32_t)!ok << 31), 0, 2));
        }
    };
    auto store_row = [&](int q, const i32x4 (&rb)[NBL]) {
        uint8_t* slot = lds + a.patch_off + (q & 1) * a.prow;
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int b = wave + 2 * j;
            if (b < nrb) *reinterpret_cast<i32x4*>(slot + b * 1024 + lane * 16) = rb[j];
        }
    };
    // coefficients of the fused epilogue (1 and 0 when absent); loaded before
    // any row request, so their wait holds up nothing
    if (tid < a.F) {
        coef[tid] = a.scale ? a.scale[tid] : 1.0f;
        coef[32 + tid] = a.bias ? a.bias[tid] : 0.0f;
    }
    // the NK rows, by buffer-load-to-LDS
    {
        const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.nk, (uint32_t)nk_bytes);
        const int fblocks = (nk_bytes + 1023) >> 10;
        for (int b = wave; b < fblocks; b += TF_WAVES) {
            const uint32_t off = (uint32_t)(b * 1024 + lane * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                frs, (__attribute__((address_space(3))) void*)(lds + NK_OFF + b * 1024), 16,
                off < (uint32_t)nk_bytes ? off : OOB_OFFSET, 0, 0, 0);
        }
        if constexpr (RPF) {
            // rows 0 and 1 requested into registers behind the NK rows (the
            // ring is not written until the fragments are taken): the wait
            // covers the NK requests alone, loads completing in order
            if (loader) {
                load_row(0, rbuf[0]);
                load_row(1, rbuf[1]);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NBL) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }
    // (a plain barrier: a fence would also wait for the row requests)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // A fragments into registers: folded row j = (co, tap) of this lane, its
    // 8 (16 for fp8) channels of each k-step; rows past C_out*R*S are zero
    i32x4 fa[KS][FR];
    {
        const int j = frag_row;
        const int co = j / RS, tp = j - co * RS;
        const bool ok = co < a.F;
        const uint8_t* fp =
            lds + NK_OFF + (ok ? co * a.kpitch * E + tp * cbytes : 0) + half * 16 * FR;
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int f = 0; f < FR; ++f)
                fa[t][f] = ok ? *reinterpret_cast<const i32x4*>(fp + t * KSB + f * 16)
                              : i32x4{0, 0, 0, 0};
    }
    // every lane holds its fragments: the ring may be filled (a plain
    // barrier, which leaves the row requests in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const int nb = (a.PW + 31) >> 5;   // 32-pixel blocks per input row
    const int rp1 = a.R + 1;
    // the work on input row i between two barriers (row i in ring slot
    // i % NSLOT): its P row, and the output row P rows up to i - 1 complete
    auto row_work = [&](int i) {
        // ---- P of input row i into P-ring row i % (R + 1)
        if (i < a.PH) {
            const uint8_t* srow = lds + a.patch_off + (i % NSLOT) * a.prow;
            float* prow_p = reinterpret_cast<float*>(lds + p_off + (i % rp1) * pslot);
            for (int blk = TF_WAVES - 1 - wave; blk < nb; blk += TF_WAVES) {
                const int px = blk * 32 + frag_row;
                // pixels past the row read pixel 0 (kept 16-aligned for the
                // swizzle) and are never written
                const int u0 = (px < a.PW ? px : 0) << cl;
                // even and odd k-steps in two independent accumulator chains
                f32x16 acc2[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    i32x4 bf[FR];
#pragma unroll
                    for (int f = 0; f < FR; ++f)
                        bf[f] = *reinterpret_cast<const i32x4*>(
                            srow + 16 * stage_unit(u0 + t * (KSB / 16) + half * FR + f, cl));
                    acc2[t & 1] = mfma32<DT>(fa[t], bf, acc2[t & 1]);
                }
                const f32x16 acc = acc2[0] + acc2[1];
                fp8_accumulator_margin<DT>();
                if (px < a.PW) {
                    float* pp = prow_p + px * a.spitch + 4 * half;
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int e = 0; e < 4; ++e) pp[8 * g + e] = acc[4 * g + e];
                }
            }
        }
        // ---- the output row completed by P rows up to i - 1 (waves 2, 3)
        if (!loader && i >= 1) {
            const int q0 = i - a.R;   // its first P row
            if (q0 >= 0 && q0 % a.stride == 0) {
                const int oh = q0 / a.stride;
                if (oh < a.TH && oh0 + oh < a.Ho) {
                    for (int tw = tid - 128; tw < a.TW; tw += 128) {
                        if (ow0 + tw >= a.Wo) break;
                        const int64_t obase =
                            ((int64_t)(n * a.Ho + oh0 + oh) * a.Wo + ow0 + tw) * a.F;
                        // pixel (tw*st + s) of P row q0 + r, folded row
                        // (co*R + r)*S + s
                        const float* pr[T3 ? 3 : 1];
                        if constexpr (T3) {
#pragma unroll
                            for (int r = 0; r < 3; ++r)
                                pr[r] = reinterpret_cast<const float*>(
                                            lds + p_off + ((q0 + r) % rp1) * pslot) +
                                        tw * a.stride * a.spitch;
                        }
                        auto sum = [&](int co) {
                            float v = 0.0f;
                            if constexpr (T3) {
#pragma unroll
                                for (int r = 0; r < 3; ++r)
#pragma unroll
                                    for (int s = 0; s < 3; ++s)
                                        v += pr[r][s * a.spitch + co * 9 + r * 3 + s];
                            } else {
                                for (int r = 0; r < a.R; ++r) {
                                    const float* q = reinterpret_cast<const float*>(
                                                         lds + p_off + ((q0 + r) % rp1) * pslot) +
                                                     tw * a.stride * a.spitch + co * RS + r * a.S;
                                    for (int s = 0; s < a.S; ++s) v += q[s * a.spitch + s];
                                }
                            }
                            return v;
                        };
                        auto finish = [&](int co, float v) {
                            if (a.epi) v = __builtin_fmaf(coef[co], v, coef[32 + co]);
                            if constexpr (RESID)
                                v = __builtin_fmaf(a.beta, out_to_f32(a.src[obase + co], ODT), v);
                            if (a.epi) v = epi_act(a, v);
                            a.y[obase + co] = f32_to_out(v, ODT);
                        };
                        if constexpr (T3) {
                            // all three sums first (27 reads in flight; rows
                            // past C_out*9 are in the P row, just unused)
                            float v[3];
#pragma unroll
                            for (int co = 0; co < 3; ++co) v[co] = sum(co);
#pragma unroll
                            for (int co = 0; co < 3; ++co)
                                if (co < a.F) finish(co, v[co]);
                        } else {
                            for (int co = 0; co < a.F; ++co) finish(co, sum(co));
                        }
                    }
                }
            }
        }
    };

    if constexpr (RPF) {
        // Register-staged rows (NSLOT == 2, at most TF_RPF_BLOCKS blocks per
        // row): loader lane l holds the 16-byte units it would have
        // requested, NBL per row, for two rows: row i + 1 arriving and row
        // i + 2 just requested.  In step i the loaders request row i + 2,
        // wait for row i + 1 and write it into its ring slot (free since
        // step i - 1's barrier), while every wave works on row i; one
        // barrier per row.  With one row in flight per workgroup the row's
        // HBM latency was waited out every step (RGB layer: 22.2 -> 18.4 us).
        // Rows 0 and 1 were requested with the NK rows (18.7 -> 17.7 us).
        if (loader) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NBL) : "memory");   // row 0 arrived
            store_row(0, rbuf[0]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // step i with rbuf[PB] free (row i, written) and rbuf[1 - PB] row i + 1
        auto step = [&](int i, auto pc) {
            constexpr int PB = decltype(pc)::value;
            if (loader) {
                load_row(i + 2, rbuf[PB]);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NBL) : "memory");   // row i + 1 arrived
                store_row(i + 1, rbuf[1 - PB]);
            }
            row_work(i);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        };
        for (int i = 0; i <= a.PH; i += 2) {
            step(i, IntC<0>{});
            if (i + 1 <= a.PH) step(i + 1, IntC<1>{});
        }
    } else {
        const int nrb_w = loader ? (nrb - wave + 1) / 2 : 0;   // this wave's requests per row
        if (loader)
            for (int q = 0; q < NSLOT - 1; ++q) issue_row(q);
        for (int i = 0; i <= a.PH; ++i) {
            if (loader && i < a.PH) {
                issue_row(i + NSLOT - 1);
                wait_vmcnt_le((NSLOT - 1) * nrb_w);   // row i has landed
            }
            asm volatile("s_barrier" ::: "memory");
            row_work(i);
            asm volatile("s_barrier" ::: "memory");
        }
    }
}

}  // namespace igc

// Patch-resident kernel for wide layers (C_out > 64) with a spatial filter.
//
// The wide kernel stages every k-tile's pixel rows afresh, so with an R x S
// filter each input line reaches LDS R*S times per tile.  Here a workgroup
// owns an output tile of TH x TW pixels of one image (BPX = WPX*TN*32 pixel
// slots, its 32-pixel blocks in row-major order over the tile) and BCO
// output channels, and keeps the tile's input patch in LDS: PH = (TH - 1)*st
// + R rows of PW = (TW - 1)*st + S pixels (padding as zeros), one 128-byte
// chunk of C_in at a time, at a pitch of 144 bytes per pixel.  Only the
// filter streams: one k-tile per (chunk, tap), BCO NK rows x 128 bytes, by
// buffer-load-to-LDS through NSTAGE stages as in the wide kernel.  The MFMA
// B fragments of tap (r, s) are the patch pixels r rows and s columns
// further on, a uniform offset added to per-lane bases; A fragments come
// from the filter stage.  This is the page's online gather (page
// "dispatch_fused_im2col_conv2d_apple", summary) with the gathered columns
// of all taps served from one staged patch.  A grouped launch runs several
// problems of one shape (the phases of a transposed convolution), storing
// through the output map.
//
// K runs in the order (chunk, tap, channel in chunk) instead of the NK
// matrix's (tap, channel): the same products, summed in another order.
// After the last tap of a chunk every wave has read its last fragments of
// the patch (the barrier of that k-tile), so the next chunk's patch is
// requested into the same place there, under that k-tile's last MFMAs, and
// waited for before the next k-tile's first fragment reads.
//
// The 144-byte pixel pitch keeps fragment reads conflict-free for every
// start pixel: 16 lanes on 16 consecutive pixels at one chunk land on 16
// different 16-byte bank groups of the 64 banks (9 p mod 16 is distinct for
// 16 consecutive p), and a row pad ((prow - TW*144) % 256 == 0) keeps that
// true where a block's 32 pixels wrap to the next tile row.  (An XOR swizzle
// would make the tap offset depend on the lane.)
#pragma once

#include "igemm_kernels.hpp"

namespace igc {

template <int DT, int TM, int TN, int WCO, int WPX, int NSTAGE, bool RESID>
__global__ __launch_bounds__(WCO * WPX * 64) void igemm_fwd_patch_kernel(ConvArgs a) {
    constexpr int E = DtTraits<DT>::E;
    constexpr int KTB = 128;                 // K bytes per k-tile: one chunk at one tap
    constexpr int CPR = KTB / 16;            // 16-byte chunks per staged filter row
    constexpr int RPI = 64 / CPR;            // filter rows per DMA instruction
    constexpr int NW = WCO * WPX;
    constexpr int BCO = WCO * TM * 32;
    constexpr int AI = BCO / (RPI * NW);     // filter DMA instructions per wave per k-tile
    constexpr int KSB = WideStep<DT>::KSB;   // k bytes per MFMA step
    constexpr int FR = KSB / 32;             // 16-byte chunks per fragment
    constexpr int KS = KTB / KSB;            // MFMA steps per k-tile
    constexpr int STAGE = BCO * KTB;
    constexpr int PP = PATCH_PP;
    constexpr int WAITN = (NSTAGE - 2) * AI;   // filter requests left in flight at a k-tile's wait
    static_assert(AI * RPI * NW == BCO && AI % 2 == 0, "whole DMA rows per wave, even count");
    static_assert(NSTAGE >= 2 && (NSTAGE - 1) * AI < 40, "stage count within the wait counter");
    static_assert(KS % 2 == 0, "fragment buffers alternate within a k-tile");
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    lds_poison<NW * 64>(lds, a.lds_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wco = wave / WPX, wpx = wave % WPX;

    // tile: co_tiles channel tiles of each pixel tile are consecutive (one
    // XCD); a grouped launch (the phases of a transposed convolution) runs
    // `groups` such problems, group_block moving NK, output, source and
    // padding to this workgroup's
    const int per_img = a.tiles_h * a.tiles_w;
    const int ntile = a.px_tiles * a.co_tiles;   // px_tiles = N * per_img
    const int tile = xcd_remap(group_block(a, ntile), ntile);
    const int co_tile = tile % a.co_tiles;
    const int ptile = tile / a.co_tiles;
    const int n = ptile / per_img;
    const int trem = ptile - n * per_img;
    const int oh0 = (trem / a.tiles_w) * a.TH;
    const int ow0 = (trem - (trem / a.tiles_w) * a.tiles_w) * a.TW;
    const int co0 = co_tile * BCO;
    const int cbytes = a.C * E;

    // ---- filter requests (as the wide kernel): row co0 + (wave*AI + i)*8 +
    // sub of k-tile kt, chunk dch(i) at this lane's slot; rows >= C_out out
    // of range (zero).  Chunk d of stage row r sits at d ^ swz(r).
    auto swz = [](int r) { return (r >> 1) & 7; };
    const int sub = lane / CPR;
    const int dch0 = (lane % CPR) ^ swz(sub);
    auto dch = [&](int i) { return dch0 ^ ((i & 1) << 2); };
    const uint32_t nk_bytes = (uint32_t)a.F * (uint32_t)a.kpitch * (uint32_t)E;
    const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.nk, nk_bytes);
    uint32_t aoff[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int co = co0 + (wave * AI + i) * RPI + sub;
        aoff[i] = co < a.F ? (uint32_t)co * (uint32_t)(a.kpitch * E) + dch(i) * 16 : OOB_OFFSET;
    }
    auto dma = [](__amdgpu_buffer_rsrc_t rs, uint8_t* dst, uint32_t off) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
    };
    // non-temporal (cache policy NT)
    auto dma_nt = [](__amdgpu_buffer_rsrc_t rs, uint8_t* dst, uint32_t off) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 2);
    };

    // ---- patch requests: LDS [PH][prow], pixel pw of row ph at pw*144;
    // each wave instruction fills one 1 KB block (lane t -> 16-byte slot t of
    // the block), so each lane fetches the chunk that belongs at its slot:
    // slot r of a row is chunk r % 9 of pixel r / 9 (slot 8 is the pixel's
    // pad), and the pad slots, the row pad and padding pixels read out of
    // range (zero).
    const int64_t img = (int64_t)a.H * a.W * cbytes;
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (int64_t)n * img, (uint32_t)img);
    const int ih0 = oh0 * a.stride - a.pt;
    const int iw0 = ow0 * a.stride - a.pl;
    const int rs = a.prow >> 4;                 // slots per patch row
    const int pblocks = (a.PH * rs + 63) >> 6;  // 1 KB blocks of the patch
    uint8_t* patch = lds + a.patch_off;
    auto issue_patch = [&](int cc) {
        const int sl = wave * 64 + lane;
        int ph = sl / rs, rem = sl - (sl / rs) * rs;
        const int dph = (NW * 64) / rs, drem = (NW * 64) % rs;
        const float inv9 = 1.0f / 9.0f;
        for (int b = wave; b < pblocks; b += NW) {
            const int pw = small_div(rem, 9, inv9), pos = rem - pw * 9;
            const int ih = ih0 + ph, iw = iw0 + pw;
            const bool ok = (pos < 8) & (pw < a.PW) & (ph < a.PH) &
                            ((unsigned)ih < (unsigned)a.H) & ((unsigned)iw < (unsigned)a.W);
            const uint32_t off = (uint32_t)((ih * a.W + iw) * cbytes + cc * KTB + pos * 16);
            // non-temporal, as the band kernel's patch: each input line is
            // wanted by this tile and its neighbours only, while the filter
            // is read by every workgroup
            dma_nt(xrs, patch + b * 1024, off | ((uint32_t)!ok << 31));
            rem += drem;
            const int car = rem >= rs ? 1 : 0;
            rem -= car ? rs : 0;
            ph += dph + car;
        }
    };

    const int nchunk = cbytes / KTB;
    const int RS = a.R * a.S;
    const int nkt = nchunk * RS;
    // request the next filter k-tile into stage st (fully masked past the
    // end, so every wave's wait counts stay uniform); k-tile (cc, tap) is NK
    // byte tap*cbytes + cc*128 of each row
    int kt_next = 0, i_tap = 0, i_cc = 0, i_koff = 0;
    auto issue = [&](int st) {
        const uint32_t past = kt_next < nkt ? 0u : OOB_OFFSET;
        ++kt_next;
        uint8_t* sb = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            dma(frs, sb + (wave * AI + i) * 1024, (aoff[i] + (uint32_t)i_koff) | past);
        if (++i_tap == RS) {
            i_tap = 0;
            ++i_cc;
            i_koff = i_cc * KTB;
        } else {
            i_koff += cbytes;
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // fragment addresses.  A: row (lane & 31) of each 32-row block of the
    // stage, chunk ks*2*FR + half*FR + h at its swizzled position.  B: tile
    // pixel p = (wpx*TN + j)*32 + (lane & 31) at patch pixel (tp*st, tq*st)
    // (slots past the tile read pixel 0 and are never stored), bytes
    // half*FR*16 + ks*KSB + h*16 of the chunk, plus the tap's offset.
    const int frow = lane & 31, half = lane >> 5;
    int xa[KS][FR];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int h = 0; h < FR; ++h)
            xa[ks][h] = frow * KTB + (((ks * 2 * FR + half * FR + h) ^ swz(frow)) << 4) +
                        wco * TM * 32 * KTB;
    const int P = a.TH * a.TW;
    int pbv[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int p = (wpx * TN + j) * 32 + frow;
        const int tp = p / a.TW, tq = p - (p / a.TW) * a.TW;
        pbv[j] = a.patch_off + half * FR * 16 +
                 (p < P ? tp * a.stride * a.prow + tq * a.stride * PP : 0);
    }
    i32x4 af[2][TM][FR], bfr[2][TN][FR];
    auto read_b = [&](int toff, int ks, int fb) {
        const uint8_t* pb = lds + toff;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int h = 0; h < FR; ++h)
                bfr[fb][j][h] = *reinterpret_cast<const i32x4*>(pb + pbv[j] + ks * KSB + h * 16);
    };
    auto read_frags = [&](int st, int toff, int ks, int fb) {
        const uint8_t* sb = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int h = 0; h < FR; ++h)
                af[fb][i][h] = *reinterpret_cast<const i32x4*>(sb + xa[ks][h] + i * 32 * KTB);
        read_b(toff, ks, fb);
    };
    auto mma = [&](int fb) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i][j] = mfma32<DT>(af[fb][i], bfr[fb][j], acc[i][j]);
    };
    constexpr int MPG = (TM * TN + TM + TN - 1) / (TM + TN);
    auto interleave = [&]() {
#pragma unroll
        for (int g = 0; g < TM + TN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);   // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, MPG, 0);  // MFMAs
        }
    };
    // last step of a k-tile: the filter requests between the first DMAM
    // MFMAs, the next k-tile's first fragment reads between the rest
    constexpr int DMAM = TM * TN / 2;
    constexpr int DMAG = (AI + DMAM - 1) / DMAM;
    constexpr int VALUG = 3 * DMAG;
    constexpr int RDG = ((TM + TN) * FR + TM * TN - DMAM - 1) / (TM * TN - DMAM);

    int cur = 0;                 // stage of the k-tile being multiplied
    int m_r = 0, m_s = 0;        // its tap
    int toff = 0;                // the tap's patch offset: r*prow + s*144
    // One k-tile.  SW: the last tap of a chunk that another chunk follows.
    // The body is one basic block for every k-tile but those (a branch in it
    // would let the compiler sink the MFMAs below the barrier and the
    // requests, away from the reads they are interleaved with).
    auto ktile = [&](auto swc, int next_cc) {
        constexpr bool SW = decltype(swc)::value;
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            read_frags(cur, toff, ks + 1, (ks + 1) & 1);
            mma(ks & 1);
            interleave();
        }
        // the next k-tile's filter complete in this wave's part and this
        // wave's reads of this k-tile finished; then a bare barrier
        // (__syncthreads would also drain the requests still in flight)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(WAITN) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int freed = cur;   // free in every wave now: receives k-tile kt + NSTAGE
        cur = cur + 1 == NSTAGE ? 0 : cur + 1;
        // the next tap (after the last one of a chunk, tap 0 of the next)
        const int s1 = m_s + 1 == a.S ? 0 : m_s + 1;
        const int r1 = s1 == 0 ? (m_r + 1 == a.R ? 0 : m_r + 1) : m_r;
        m_s = s1;
        m_r = r1;
        toff = r1 * a.prow + s1 * PP;
        // SW: every wave is past its last read of this chunk's patch (the
        // barrier above), so the next chunk's patch goes to the same place,
        // requested before the filter k-tile so that one wait below (all
        // but the last AI requests complete; requests complete in order)
        // covers it; the B fragments read meanwhile from the old patch are
        // read again once it has arrived.
        if constexpr (SW) issue_patch(next_cc);
        issue(freed);
        read_frags(cur, toff, 0, 0);   // past the last k-tile: a harmless read
        mma((KS - 1) & 1);
#pragma unroll
        for (int g = 0; g < DMAM; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
            __builtin_amdgcn_sched_group_barrier(0x010, DMAG, 0);    // buffer loads to LDS
            __builtin_amdgcn_sched_group_barrier(0x002, VALUG, 0);   // their address math
        }
#pragma unroll
        for (int g = DMAM; g < TM * TN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, RDG, 0);     // DS reads
        }
        if constexpr (SW) {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(AI) : "memory");
            __builtin_amdgcn_sched_barrier(0);
            read_b(toff, 0, 0);
        }
    };

    if (nkt > 0) {
        issue_patch(0);
#pragma unroll
        for (int st = 0; st < NSTAGE; ++st) issue(st);
        // the patch and stage 0 complete (the later stages may still be in
        // flight), in every wave
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((NSTAGE - 1) * AI) : "memory");
        read_frags(0, 0, 0, 0);
        for (int cc = 0; cc < nchunk; ++cc) {
            const bool more = cc + 1 < nchunk;
            const int nt = more ? RS - 1 : RS;
            for (int t = 0; t < nt; ++t) ktile(IntC<0>{}, 0);
            if (more) ktile(IntC<1>{}, cc + 1);
        }
    }
    fp8_accumulator_margin<DT>();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // masked tail requests
    __syncthreads();   // stages and patch no longer read or written

    // ---- epilogue through a private LDS region per wave (as the wide
    // kernel): the wave's fp32 32-pixel block in [pixel][channel] order,
    // read back with LPP consecutive lanes on one pixel's channels; 8-byte
    // stores (4 channels), range-checked buffer accesses over this image's
    // output, so pixels past the tile or the image are dropped.  The host
    // guarantees C_out % 4 == 0 and an image's output below 2^31 bytes.
    constexpr int ODT = (DT == DT_FP16) ? DT_FP16 : DT_BF16;
    constexpr int WCH = TM * 32;                 // channels per wave
    constexpr int EP = WCH * 4 + 16;             // bytes per pixel row (padded)
    constexpr int LPP = WCH / 4;                 // lanes per pixel on read-back
    constexpr int PPI = 64 / LPP;                // pixels per read-back instruction
    constexpr int NI = 32 / PPI;                 // read-back instructions per block
    uint8_t* ereg = lds + wave * 32 * EP;
    const int c4 = lane % LPP, pl = lane / LPP;
    const int co = co0 + wco * WCH + c4 * 4;     // this lane's first channel
    float esc[4], ebi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) epi_coef(a, co + e, &esc[e], &ebi[e]);
    // output pixel (n, oh, ow) is pixel (n, oh*ysh, ow*ysw) of Hy x Wy images
    // (the identity without an output map)
    const int64_t oimg = (int64_t)a.Hy * a.Wy * a.F;   // output elements per image
    const __amdgpu_buffer_rsrc_t yrs = make_rsrc(a.y + (int64_t)n * oimg, (uint32_t)(oimg * 2));
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(RESID ? a.src + (int64_t)n * oimg : a.y, RESID ? (uint32_t)(oimg * 2) : 0u);
    const uint32_t cmask = co < a.F ? 0u : OOB_OFFSET;
    const int th_n = min(a.TH, a.Ho - oh0);
    const int tw_n = min(a.TW, a.Wo - ow0);
    // this lane's pixels in block j: tile pixel p0 + q*PPI for q < NI, a
    // run walked column by column (tq wraps at TW); byte offsets in the
    // image's output, out of range for pixels past the tile or the image.
    // 24-bit multiplies: an image has fewer than 2^24 pixels and a pixel
    // row of the output fewer than 2^24 bytes.
    uint32_t off[2][NI];
    const uint32_t orow = (uint32_t)(a.ysh * a.Wy) * (uint32_t)a.F * 2u;   // bytes per tile row
    const uint32_t opix = (uint32_t)a.ysw * (uint32_t)a.F * 2u;            // bytes per tile column
    auto offsets = [&](int j, uint32_t (&o)[NI]) {
        const int p0 = (wpx * TN + j) * 32 + pl;
        int tp = p0 / a.TW, tq = p0 - (p0 / a.TW) * a.TW;
#pragma unroll
        for (int q = 0; q < NI; ++q) {
            const bool ok = (p0 + q * PPI < P) & (tp < th_n) & (tq < tw_n);
            const uint32_t v = __umul24((uint32_t)(oh0 + tp), orow) +
                               __umul24((uint32_t)(ow0 + tq), opix) + (uint32_t)co * 2u;
            o[q] = ok ? (v | cmask) : OOB_OFFSET;
            tq += PPI;
            const bool wrap = tq >= a.TW;
            tq -= wrap ? a.TW : 0;
            tp += wrap ? 1 : 0;
        }
    };
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
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 sv[2][NI];
    auto load_src = [&](int j) {
#pragma unroll
        for (int q = 0; q < NI; ++q)
            // non-temporal: the source is read exactly once
            sv[j & 1][q] = __builtin_amdgcn_raw_buffer_load_b64(srs, off[j & 1][q], 0, 2);
    };
    // EPI: the scale / bias / activation path, chosen once for the whole
    // epilogue (a per-element select would cost its VALU work every time)
    auto run = [&](auto epic) {
        constexpr bool EPI = decltype(epic)::value;
        offsets(0, off[0]);
        if constexpr (RESID) load_src(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if (j + 1 < TN) {
                offsets(j + 1, off[(j + 1) & 1]);
                if constexpr (RESID) load_src(j + 1);
            }
            stage_block(j);
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const f32x4 v4 =
                    *reinterpret_cast<const f32x4*>(ereg + (q * PPI + pl) * EP + c4 * 16);
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
                // non-temporal: written once, 128 or 256 contiguous bytes
                // per pixel per instruction
                __builtin_amdgcn_raw_buffer_store_b64(ov, yrs, off[j & 1][q], 0, 2);
            }
        }
    };
    if (a.epi) run(IntC<1>{});
    else run(IntC<0>{});
}

}  // namespace igc

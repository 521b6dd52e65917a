// ssd_tile16.h -- chunk tile for 16-bit inputs (bf16 / fp16) on gfx950.
//
// Same arithmetic as chunk_tile in ssd_device.h (page keys are listed there), organised
// around three gfx950 features:
//   * buffer_load_dwordx4 ... lds: x, B and C chunks are copied from HBM straight into LDS
//     (no register round trip), each lane moving one 16-byte piece; the buffer resource's
//     record count makes tokens past the end of the sequence read as zeros;
//   * ds_read_b64_tr_b16: LDS tiles stay in their HBM row layout ([token][column]) and the
//     token-major MFMA operands (x and B with k = token) are read transposed;
//   * rows are stored with their 16-byte pieces XOR-permuted (swizzled) so the transposed
//     reads of 16 rows do not pile onto the same LDS banks.
// The x operand of the chunk-state product is kept in registers and reused (unscaled)
// by the diagonal-block product of chunk_scan; L = CB * decay * dt is formed directly in
// registers from CB; y is produced 16 rows at a time.
#pragma once

#include "ssd_device.h"


namespace ssd {

constexpr float LOG2E = 1.4426950408889634f;

#define SSD_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T, int P, int N, int Q> struct Geo16 {
    static constexpr int PW = P < 32 ? P : 32;  // p columns per wave
    static constexpr int WPH = P / PW;          // waves per head
    static constexpr int HPT = 4 / WPH;         // heads per tile
    static constexpr int MBP = PW / 16;
    // p columns of the accumulator layout: lane r16 of p block pb holds column pcol(pb, r16)
    // of its wave's PW.  The interleave gives output lane q of y^T the 4 MBP consecutive columns
    // 4 MBP q .. +4 MBP - 1 across its p blocks, so y and the D x term move as one piece per lane.
    static constexpr int pcol(int pb, int r16) { return (r16 >> 2) * 4 * MBP + 4 * pb + (r16 & 3); }
    static constexpr int NB = N / 16;
    static constexpr int KS = Q / 32;  // 32-token k-steps
    static constexpr int QB = Q / 16;  // 16-token row blocks
    static constexpr int SZ_X = HPT * Q * P * 2;
    static constexpr int SZ_BC = Q * N * 2;
    static constexpr int SZ_V = (3 * HPT + 1) * Q * 4;  // dt, acs, chunk-state weights; seg
    // CB (fp32) staged in LDS as 32-row bands holding only the columns the diagonal block
    // reads: band r (rows 32r .. 32r+31) keeps columns [0, 32(r+1)) in rows of 8(r+1)+1
    // 16-byte pieces (the odd pitch spreads 16 consecutive rows over all bank groups), each
    // band padded to whole 1 KB copy instructions.  Only for Q <= 128 (it would not fit at 256).
    static constexpr bool CB_LDS = Q <= 128;
    static constexpr int band_pieces(int r) { return ((32 * (8 * r + 9) + 63) / 64) * 64; }
    static constexpr int cb_pieces() {
        int t = 0;
        for (int r = 0; r < Q / 32; ++r) t += band_pieces(r);
        return t;
    }
    static constexpr int SZ_CB = CB_LDS ? cb_pieces() * 16 : 0;
    static constexpr int SZ_R1 = SZ_X > SZ_CB ? SZ_X : SZ_CB;  // x, later CB (and L)
    // L_h[i][j] = CB[i][j] exp(acs_i - acs_j) dt_j (j <= i, else 0) of every head of the tile,
    // in T, staged as 32-row bands of the lower triangle: band r keeps columns [0, 32(r+1)) in
    // rows of 4(r+1)+1 16-byte pieces (odd pitch: 16 consecutive rows hit distinct bank groups).
    // Built once per tile over the CB bands when it fits in their space.
    static constexpr int lband_pitch(int r) { return 4 * (r + 1) + 1; }
    static constexpr int lband_base(int r) { return 32 * r * (2 * r + 3); }  // pieces before band r
    static constexpr int SZ_LH = lband_base(KS) * 16;                          // bytes per head
    static constexpr bool L_LDS = CB_LDS && HPT * SZ_LH <= SZ_R1;
    static constexpr int SMEM = SZ_R1 + SZ_BC + SZ_V;
    // fused kernel's workgroups per CU: 64-token chunks leave room (LDS and, at most 168, registers)
    // for three
    static constexpr int OCC = Q == 64 ? 3 : 2;
    static_assert(Q % 32 == 0 && Q <= 256, "Q must be a multiple of 32, at most 256");
    // OCC is the register budget's hint; the LDS decides the real count (hipOccupancy at launch).
    // They agree for P >= 64 at Q <= 128; Q = 256 and the 4-head tiles at N = 128, Q = 128 hold
    // one workgroup per CU by their LDS.
    static_assert(!(P >= 64 && Q <= 128) || OCC * SMEM <= 160 * 1024, "OCC workgroups must fit in 160 KB of LDS");
    static_assert(N % 32 == 0, "N % 32 == 0");
};

// Swizzle of the 16-byte piece index inside a row of CH pieces.  A transposed operand read
// touches rows k0 + 8q + m (q, m = 0..3, k0 a multiple of 32; the second read adds 4), each lane
// 8 bytes, the four lanes of a row 32 contiguous bytes before the swizzle.  The LDS serves such a
// read (and ds_read_b64) 32 lanes per cycle -- lanes 0-31 are the rows with q = 0, 1 -- from 64
// four-byte banks (a 256-byte bank line); measured on MI355X with rocprofv3's
// SQ_LDS_BANK_CONFLICT.  So the swizzle must spread the 8 rows of each half-wave apart:
//   CH = 16 (256-byte rows, one bank line each): s = 2m + 8(q & 1) + (q >> 1) puts those 8 rows
//           on 8 distinct 32-byte pairs of pieces (a row's two pieces stay one aligned pair);
//   CH = 8 (128-byte rows, two per line): s = 2(m >> 1) + 4(q & 1) + (q >> 1) with the row's
//           line half (bit 0) spreads them over the line's 16 pieces;
// the 16-row row-wise reads of the D x term (16 bytes a lane) measured conflict-free with the
// CH = 8 form too.  Neither depends on row bit 2 (the +4) or bits 5 and up (k0).
template <int CH> __device__ inline int swz(int row) {
    const int m = row & 3, q = (row >> 3) & 3;
    if constexpr (CH >= 16) return ((m << 1) | ((q & 1) << 3) | (q >> 1)) & (CH - 1);
    else if constexpr (CH == 8) return ((m >> 1) << 1) | ((q & 1) << 2) | (q >> 1);
    else if constexpr (CH == 4) return (row >> 3) & 3;                        // 4 rows per bank line
    else return (row >> 3) & 1;
}

// Tiles read row-wise (C in chunk_scan: 16 consecutive rows per read) use the low row bits.
template <int CH> __device__ inline int swz_row(int row) { return row & (CH - 1); }

enum : int { SWZ_TR = 0, SWZ_ROW = 1 };

// Element offset of (row, col) in a swizzled [rows][COLS] 16-bit LDS tile.
template <int COLS, int KIND = SWZ_TR> __device__ inline int sw_off(int row, int col) {
    constexpr int CH = COLS / 8;
    const int sz = KIND == SWZ_TR ? swz<CH>(row) : swz_row<CH>(row);
    return row * COLS + (((col >> 3) ^ sz) << 3) + (col & 7);
}

// rows [0, rows) of a row-major slice (row r at byte r * rs) -> swizzled LDS tile [rows][COLS];
// the four waves split the 1 KB copy instructions.
template <int COLS, int KIND = SWZ_TR, int AUX = 0>
__device__ inline void dma_rows(void* lds_tile, __amdgpu_buffer_rsrc_t rs_src, int rows, uint32_t rs) {
    constexpr int CH = COLS / 8;
    constexpr int RPI = 64 / CH;  // rows per 1 KB instruction
    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ninst = rows / RPI;
    for (int k = wave; k < ninst; k += 4) {
        const int row = k * RPI + lane / CH;
        const int c = (lane % CH) ^ (KIND == SWZ_TR ? swz<CH>(row) : swz_row<CH>(row));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_src, SSD_LDS(void, (char*)lds_tile + k * 1024), 16,
                                                 row * rs + c * 16, 0, 0, AUX);
    }
}

// Token-major MFMA operands from a swizzled [tokens][COLS] tile via transposed reads.  Lane l
// of 16-lane group q points at row k0 + 8q + m (m = (l & 15) >> 2) and columns col0 + 4 (l & 3)
// .. +3; the read hands lane l column col0 + (l & 15) of rows k0 + 8q .. +3, and a second read
// 4 rows down completes the 8 tokens of the MFMA k slots.  The swizzle of those rows does not
// depend on k0 (a multiple of 32) nor on the +4, so the lane offset for k0 = 0 is computed once
// per column block and each k step is a constant offset.
// tr_lane_offs: the lane offsets of column blocks 0, 16, .. 16 (NBK - 1); tr_lane_offs_p: those
// of the x operand's p blocks 0 .. MBP - 1 in the interleaved column order of Geo16::pcol (the
// four column quads of p block pb start at c0 + 4 MBP jj + 4 pb).  One read of the lane id
// each, so the compiler shares the row part.
template <int COLS, int NBK> __device__ inline void tr_lane_offs(int (&off)[NBK]) {
    const int lane = tid_here() & 63;
    const int q = lane >> 4, m = (lane & 15) >> 2, jj = lane & 3;
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) off[nb] = sw_off<COLS>(8 * q + m, nb * 16 + 4 * jj);
}
template <int COLS, int MBP> __device__ inline void tr_lane_offs_p(int c0, int (&off)[MBP]) {
    const int lane = tid_here() & 63;
    const int q = lane >> 4, m = (lane & 15) >> 2, jj = lane & 3;
#pragma unroll
    for (int pb = 0; pb < MBP; ++pb) off[pb] = sw_off<COLS>(8 * q + m, c0 + 4 * MBP * jj + 4 * pb);
}

template <typename T, int COLS> __device__ inline typename TT<T>::frag tr_frag_at(const T* tile, int lane_off, int k0) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SSD_LDS(s16x4, tile + lane_off + k0 * COLS));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SSD_LDS(s16x4, tile + lane_off + (k0 + 4) * COLS));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename TT<T>::frag, w);
}

// 8 fp32 values -> one 16-bit MFMA fragment.
template <typename T> __device__ inline typename TT<T>::frag pack8(f32x4 lo, f32x4 hi) {
    return __builtin_shufflevector(cvt4<T>(lo), cvt4<T>(hi), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Copy the CB rows/columns the diagonal block reads (bands of the lower triangle, see
// Geo16) from HBM into LDS.  AUX = AUX_L2 when CB was written by another workgroup of the
// same launch (on the same XCD).  ES: CB element size (4, or 2 for the relaxed 16-bit CB);
// a 16-byte piece holds 16 / ES elements, so a band row of 32 (band + 1) columns is
// 32 (band + 1) ES / 16 pieces plus one of padding.
template <int ES> __host__ __device__ constexpr int cb_pitch(int band) { return 32 * (band + 1) * ES / 16 + 1; }
// es is a run-time value: one copy loop for both CB types, so no control flow on the type
// sits next to the MFMAs whose accumulators are read around it (see cb_widen_sel).
template <int Q, int AUX> __device__ inline void dma_cb_bands(float* lds, const float* cb, int es) {
    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(cb, (uint32_t)(Q * Q * es));
    const int epp = 16 / es;  // elements per piece
    int base = 0;  // pieces
#pragma unroll
    for (int band = 0; band < Q / 32; ++band) {
        const int pitch = 32 * (band + 1) * es / 16 + 1;
        const int used = 32 * pitch;
        const int ninst = (used + 63) / 64;
        for (int k = wave; k < ninst; k += 4) {
            const int f = k * 64 + lane;  // piece index inside the band
            const int row = f / pitch, pc = f - row * pitch;
            const bool ok = f < used && pc < pitch - 1;
            const uint32_t voff = ok ? (uint32_t)(((32 * band + row) * Q + epp * pc) * es) : 0x40000000u;  // past num_records: reads as zeros
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SSD_LDS(void, (char*)lds + (base + k * 64) * 16), 16, voff, 0, 0, AUX);
        }
        base += ((used + 63) / 64) * 64;
    }
}

// Byte offset of CB[i][j] in the banded LDS copy, i in band `band` (a compile-time value where
// the caller unrolls its row blocks), for either CB type: the band's base and pitch for both
// element sizes are constants, so the type only selects between scalars (no control flow).
template <int Q> __device__ inline int cb_byte_off(int band, int i, int j, bool cb16) {
    int base2 = 0, base4 = 0;  // pieces before the band
#pragma unroll
    for (int r = 0; r < Q / 32; ++r)
        if (r < band) {
            base2 += ((32 * cb_pitch<2>(r) + 63) / 64) * 64;
            base4 += ((32 * cb_pitch<4>(r) + 63) / 64) * 64;
        }
    const int base = cb16 ? base2 : base4, pitch = cb16 ? cb_pitch<2>(band) : cb_pitch<4>(band);
    return (base + (i & 31) * pitch) * 16 + j * (cb16 ? 2 : 4);
}

// 8 consecutive CB values as two fp32 vectors, from either CB type: fp32 CB arrives as (lo, hi);
// 16-bit CB arrives with all 8 values in lo, which are then widened.  Both results are formed
// and one is selected, without a branch: the compiler let a uniform branch on the CB type sit
// between a row block's MFMAs and the VALU reads of their accumulators, and on the short side
// of it those reads came fewer wait states after the MFMAs than the hardware needs (stale
// accumulator values).
template <typename T> __device__ inline void cb_widen_sel(bool cb16, f32x4& lo, f32x4& hi) {
    const typename TT<T>::frag v = __builtin_bit_cast(typename TT<T>::frag, lo);
    const f32x4 wl = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    const f32x4 wh = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
    lo = cb16 ? wl : lo;
    hi = cb16 ? wh : hi;
}

// Piece offset (16-byte units) of L_h[i][8 jp .. 8 jp + 7] inside one head's bands.
template <typename G_> __device__ inline int lband_off(int i, int jp) {
    const int r = i >> 5;
    return G_::lband_base(r) + (i & 31) * G_::lband_pitch(r) + jp;
}

// The L bands of every valid head of the tile, built once per tile from CB.  Items are
// (row i, 8-column piece jp) of the lower 32-row bands, of three kinds:
//   factored: j's 16-token block ends before row i (all of a 32-block left of the diagonal,
//             and the lower-left 16x16 of a diagonal 32-block): L = CB * exp(acs_i - acs_m) *
//             sF[j], with m = the last token of j's 16-block and sF[j] = exp(acs_m - acs_j) dt_j.
//             Both factors are at most 1 when dt A <= 0 (acs does not increase along the chunk),
//             so nothing overflows; a factor underflows only when the exact product is below
//             e^-87.  Packed input: i and j are in one sequence exactly when j and m are and m
//             and i are (sequences are contiguous), so sF[j] carries the first test and the row
//             factor the second;
//   diagonal: i and j in the same 16-token block: L = CB * exp(acs_i - acs_j) * dt_j, masked to
//             j <= i (and, packed, to seg[j] == seg[i]) -- a product with dt_j, so any sign of dt
//             is handled;
//   zero:     the upper-right 16x16 of a diagonal 32-block.
// load() reads this thread's CB pieces from HBM/L2 into registers (issued early, so the reads
// overlap other work); store() writes the L pieces of every valid head into LDS.
template <typename T, typename G_, int AUX> struct LBuild {
    static constexpr int KS = G_::KS, Q = KS * 32, HPT = G_::HPT;
    static constexpr int NF = 64 * KS * (KS - 1) + 32 * KS;  // factored items, all bands
    static constexpr int ND = 64 * KS, NZ = 32 * KS;         // diagonal, zero items
    static constexpr int FI = (NF + 255) / 256, DI = (ND + 255) / 256;
    typedef typename TT<T>::frag frag;
    f32x4 cf[FI][2], cd[DI][2];
    int fi[FI], fj[FI];

    // factored item k -> (i, jp): band b holds rows 0..31 x pieces [0, 4b), then rows 16..31 x
    // pieces {4b, 4b + 1}
    __device__ static inline void f_item(int k, int& i, int& jp) {
        int b = 0, base = 0;
#pragma unroll
        for (int bb = 1; bb < KS; ++bb) {
            const int fb = 64 * bb * (bb - 1) + 32 * bb;
            if (k >= fb) {
                b = bb;
                base = fb;
            }
        }
        const int kl = k - base;
        if (kl < 128 * b) {
            // row = kl / (4b) for b in 1..3 (kl < 384): multiply by 2^16 / b, rounded up
            const int mul = b == 1 ? 65536 : (b == 2 ? 32768 : 21846);
            const int row = ((kl >> 2) * mul) >> 16;
            jp = kl - row * 4 * b;
            i = 32 * b + row;
        } else {
            const int kz = kl - 128 * b;
            i = 32 * b + 16 + (kz >> 1);
            jp = 4 * b + (kz & 1);
        }
    }
    __device__ static inline void d_item(int k, int& i, int& jp) {
        const int b = k >> 6, kl = k & 63;
        i = 32 * b + (kl < 32 ? kl >> 1 : 16 + ((kl - 32) >> 1));
        jp = 4 * b + (kl < 32 ? 0 : 2) + (kl & 1);
    }

    // cb16: CB holds the 16-bit input type; the 8 values of an item then arrive in the first
    // load and the second goes to an empty buffer range (zeros, no memory access), so both
    // storage types issue the same loads into the same registers.
    __device__ inline void load(const float* cbp, int tid, bool cb16) {
        const int es = cb16 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(cbp, (uint32_t)(Q * Q * es));
        const __amdgpu_buffer_rsrc_t r2 = cb16 ? make_rsrc(cbp, 0u) : r;
#pragma unroll
        for (int it = 0; it < FI; ++it) {
            const int k = tid + it * 256;
            int i = 0, jp = 0;
            if (k < NF) f_item(k, i, jp);
            fi[it] = i;
            fj[it] = jp;
            const uint32_t off = k < NF ? (uint32_t)(i * Q + 8 * jp) * es : 0x40000000u;  // past the end: zeros
            cf[it][0] = bload_f32x4<AUX>(r, off);
            cf[it][1] = bload_f32x4<AUX>(r2, off + 16);
        }
#pragma unroll
        for (int it = 0; it < DI; ++it) {
            const int k = tid + it * 256;
            int i = 0, jp = 0;
            if (k < ND) d_item(k, i, jp);
            const uint32_t off = k < ND ? (uint32_t)(i * Q + 8 * jp) * es : 0x40000000u;
            cd[it][0] = bload_f32x4<AUX>(r, off);
            cd[it][1] = bload_f32x4<AUX>(r2, off + 16);
        }
    }

    __device__ inline void store(T* sL, const float* sA2, const float* sF, const float* sDt, const int* sSeg,
                                 bool varlen, bool cb16, int nvh, int tid) {
        // widen in place (here, not in load(), so the loads stay in flight until now): with 16-bit
        // CB the 8 values of each item into its two fp32 vectors
#pragma unroll
        for (int it = 0; it < FI; ++it) cb_widen_sel<T>(cb16, cf[it][0], cf[it][1]);
#pragma unroll
        for (int it = 0; it < DI; ++it) cb_widen_sel<T>(cb16, cd[it][0], cd[it][1]);
#pragma unroll
        for (int it = 0; it < FI; ++it) {
            const int k = tid + it * 256;
            if (k < NF) {
                const int i = fi[it], jp = fj[it], j0 = 8 * jp;
                const int o = lband_off<G_>(i, jp) * 8;
                const bool row_same = !varlen || sSeg[i] == sSeg[j0 | 15];
#pragma unroll
                for (int hh = 0; hh < HPT; ++hh) {
                    if (hh < nvh) {
                        const float gx = __builtin_amdgcn_exp2f(sA2[hh * Q + i] - sA2[hh * Q + (j0 | 15)]);
                        const float g = row_same ? gx : 0.f;
                        const f32x4 f0 = *(const f32x4*)(sF + hh * Q + j0) * g;
                        const f32x4 f1 = *(const f32x4*)(sF + hh * Q + j0 + 4) * g;
                        *(frag*)(sL + (size_t)hh * (G_::SZ_LH / sizeof(T)) + o) = pack8<T>(cf[it][0] * f0, cf[it][1] * f1);
                    }
                }
            }
        }
#pragma unroll
        for (int it = 0; it < DI; ++it) {
            const int k = tid + it * 256;
            if (k < ND) {
                int i, jp;
                d_item(k, i, jp);
                const int j0 = 8 * jp;
                const int o = lband_off<G_>(i, jp) * 8;
                bool keep[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) keep[e] = j0 + e <= i && (!varlen || sSeg[j0 + e] == sSeg[i]);
#pragma unroll
                for (int hh = 0; hh < HPT; ++hh) {
                    if (hh < nvh) {
                        const float ai = sA2[hh * Q + i];
                        const f32x4 a0 = *(const f32x4*)(sA2 + hh * Q + j0);
                        const f32x4 a1 = *(const f32x4*)(sA2 + hh * Q + j0 + 4);
                        const f32x4 d0 = *(const f32x4*)(sDt + hh * Q + j0);
                        const f32x4 d1 = *(const f32x4*)(sDt + hh * Q + j0 + 4);
                        f32x4 l0, l1;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            l0[e] = keep[e] ? cd[it][0][e] * __builtin_amdgcn_exp2f(ai - a0[e]) * d0[e] : 0.f;
                            l1[e] = keep[e + 4] ? cd[it][1][e] * __builtin_amdgcn_exp2f(ai - a1[e]) * d1[e] : 0.f;
                        }
                        *(frag*)(sL + (size_t)hh * (G_::SZ_LH / sizeof(T)) + o) = pack8<T>(l0, l1);
                    }
                }
            }
        }
        for (int k = tid; k < NZ; k += 256) {
            const int bb = k >> 5, kl = k & 31;
            const int o = lband_off<G_>(32 * bb + (kl >> 1), 4 * bb + 2 + (kl & 1)) * 8;
#pragma unroll
            for (int hh = 0; hh < HPT; ++hh)
                if (hh < nvh) *(frag*)(sL + (size_t)hh * (G_::SZ_LH / sizeof(T)) + o) = vzero<frag>();
        }
    }
};

// Per-sequence states at the chunk's state hand-off (packed input with per-sequence states):
//   inj:      the chunk's last segment starts inside it, so the state it passes on also carries
//             that sequence's initial state, decayed from just before its first token to the
//             chunk end (the chunk-state sum itself is already masked to the segment);
//   done0:    segment 0 (begun in an earlier chunk) ends inside this chunk: its final state is
//             the partial sum written by the chunk-state step plus S_c decayed to its last token;
//   last_ends: the chunk's last segment ends at the chunk end (or the row's): its final state
//             is the state passed on.
// apply() adds these for one lane's 4 state elements (p, n .. n+3); sv = S_c, snew = S_{c+1}.
struct SeqEnds {
    bool any = false, inj = false, done0 = false, last_ends = false;
    int qk = 0, q0 = 0, ql = 0;
    float deck = 0.f, dec0 = 0.f;
    __device__ inline void apply(const SsdArgs& a, int h, int p, int n, int P, int N, f32x4 sv, f32x4& snew) const {
        const int sdt = a.state_dtype;
        if (inj) snew += deck * load_state4(a.seq_h0, sdt, seq_state_off(a, qk, h, p, n, P, N));
        if (done0) {
            const size_t o = seq_state_off(a, q0, h, p, n, P, N);
            store_state4(a.seq_fin, sdt, o, load_state4(a.seq_fin, sdt, o) + dec0 * sv);
        }
        if (last_ends) store_state4(a.seq_fin, sdt, seq_state_off(a, ql, h, p, n, P, N), snew);
    }
};

// The hand-off facts of chunk c of row b for head h (a2_h = acs log2 e of the head); with_inj:
// the caller forms S_{c+1} itself (the fused hop), else the state-passing step already did.
__device__ inline SeqEnds seq_ends(const SsdArgs& a, int b, int c, int h, const int* sSeg, const float* a2_h,
                                   int Q, int valid, bool with_inj) {
    SeqEnds r;
    const int tok0 = c * Q, L = a.seqlen;
    const int Kc = sSeg[Q - 1];
    const int sK = Kc >= 1 ? seg_first(sSeg, Q, Kc) : 0;
    r.qk = Kc >= 1 ? seq_at(a, b, tok0 + sK) : 0;
    r.inj = with_inj && Kc >= 1 && a.seq_h0 && r.qk >= 0 && r.qk < a.nseq;
    r.deck = __builtin_amdgcn_exp2f(a2_h[Q - 1] - (sK > 0 ? a2_h[sK - 1] : 0.f));
    r.q0 = seq_at(a, b, tok0);
    if (sSeg[0] == 0 && Kc >= 1 && r.q0 >= 0 && r.q0 < a.nseq) {
        r.done0 = true;
        r.dec0 = __builtin_amdgcn_exp2f(a2_h[seg_first(sSeg, Q, 1) - 1]);
        wait_vm_all();  // this wave's partial sum of q0 (the chunk-state step, same lanes) is stored
    }
    const int tn = tok0 + valid;
    r.ql = Kc >= 1 ? r.qk : r.q0;
    r.last_ends = (tn >= L || seq_at(a, b, tn) != seq_at(a, b, tn - 1)) && r.ql >= 0 && r.ql < a.nseq;
    r.any = r.inj || r.done0 || r.last_ends;
    return r;
}

// Block form: the convolution before the SSD applied in place to the tile's x rows in LDS
// (raw xBC rows, copied in by round 1), before any x operand is read.  An item is one 8-channel
// piece of one head over 8 tokens; it needs the 3 raw rows above its first token (from LDS, or
// from the previous chunk's rows / the conv state in memory for the first 8 tokens).  Items are
// processed in rounds of 256 from the last rows up, each round reading all its inputs before a
// barrier and writing after it, so no round overwrites a row a later round still reads raw.
// Rows past the sequence end become zeros.
template <typename T, int P, int Q, int HPT>
__device__ void conv_x_tile(const ConvSrc<T> src, int b, int tok0, int valid, int head0, T* sX) {
    typedef typename TT<T>::v8 v8;
    constexpr int NPC = P / 8, SEGS = Q / 8, ITEMS = HPT * NPC * SEGS;
    constexpr int ROUNDS = (ITEMS + 255) / 256;
    static_assert(ITEMS % 256 == 0 || ROUNDS == 1, "a round must cover whole segments");
    const int tid = tid_here();
#pragma unroll 1
    for (int rnd = ROUNDS - 1; rnd >= 0; --rnd) {
        const int it = rnd * 256 + tid;
        const bool act = it < ITEMS;
        const int seg = it / (HPT * NPC), rem = it - seg * (HPT * NPC);
        const int hh = rem / NPC, pc = rem - hh * NPC;
        const int ch0 = (head0 + hh) * P + pc * 8;
        T* tile = sX + hh * Q * P;
        v8 raw[11];
        ConvTaps k;
        if (act) {
            k.load(src.w, src.bias, ch0);
#pragma unroll
            for (int r = 0; r < 11; ++r) {
                const int row = seg * 8 - 3 + r;
                if (row >= 0) {
                    raw[r] = *(const v8*)(tile + sw_off<P>(row, pc * 8));
                } else {
                    float v[8];
                    src.raw(b, tok0 + row, ch0, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) raw[r][e] = (T)v[e];
                }
            }
        }
        __syncthreads();  // this round's inputs are read
        if (act) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = seg * 8 + i;
                v8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float s = k.bias[e] + k.w[0][e] * (float)raw[i][e] + k.w[1][e] * (float)raw[i + 1][e] +
                                    k.w[2][e] * (float)raw[i + 2][e] + k.w[3][e] * (float)raw[i + 3][e];
                    o[e] = row < valid ? (T)silu_f(s) : (T)0.f;
                }
                *(v8*)(tile + sw_off<P>(row, pc * 8)) = o;
            }
        }
    }
    __syncthreads();
}

// Block form with the norm in the launch, part 1 (end of the chunk tile): the tile's y rows
// (HPT heads, staged in LDS as whole token rows of PPR 16-byte pieces, XOR-swizzled by the
// token, already rounded to T as y would leave) go to out in whole rows; each token's sum of
// g^2, g = y silu(z), over the tile's channels goes to nsum (one float atomic per token), then
// the tile counts itself in ncount.  No wait: norm_item finishes the rows a chunk later, from
// the same rounded y (so the result is the one the separate norm kernel gives on y).
template <typename T, int P, int Q, int PPR>
__device__ void norm_rows(const SsdArgs& a, int b, int c, int g, int head0, int tok0, int valid, const char* sY) {
    typedef typename TT<T>::v8 v8;
    constexpr int ROWB = PPR * 16, KN = Q * PPR / 256;
    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = a.seqlen, H = a.nheads, Gn = a.ngroups;
    const uint32_t rs = (uint32_t)H * P * 2;  // bytes between token rows of z and out
    const size_t row0 = ((size_t)b * L + tok0) * H * P + (size_t)head0 * P;
    const __amdgpu_buffer_rsrc_t zr = make_rsrc((const T*)a.z + row0, (uint32_t)(valid - 1) * rs + ROWB);
    const __amdgpu_buffer_rsrc_t orow = make_rsrc((T*)a.out + row0, (uint32_t)(valid - 1) * rs + ROWB);
    float* nsum = a.nsum + ((size_t)b * L + tok0) * Gn + g;
#pragma unroll
    for (int k = 0; k < KN; ++k) {
        const int f = (k * 4 + wave) * 64 + lane, t = f / PPR, pc = f % PPR;
        const v8 yv = *(const v8*)(sY + t * ROWB + ((pc ^ (t & (PPR - 1))) << 4));
        const v8 zv = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(zr, (uint32_t)t * rs + (uint32_t)pc * 16, 0, 0));
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = (float)yv[e] * silu_f((float)zv[e]);
            ss += v * v;
        }
#pragma unroll
        for (int m = PPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);  // the row's PPR lanes
        if (t < valid) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, yv), orow, (uint32_t)t * rs + (uint32_t)pc * 16, 0, 0);
            if (pc == 0) atomicAdd(nsum + (size_t)t * Gn, ss);
        }
    }
    wait_vm_all();  // this wave's rows and sums have reached the L2
    __syncthreads();
    if (tid == 0) atomicAdd(a.ncount + ((size_t)b * a.nchunks + c) * Gn + g, 1u);
}

// Block form with the norm in the launch, part 2: a norm item for the tile (b, c, g, tig) waits
// until all tpg tiles of its (b, g) pair have counted for chunk c (in the queue it comes a
// chunk after them), then turns its tile's y rows in out into out = g / sqrt(nsum / (H/G * P)
// + eps) * norm_w, g = y silu(z).  Same XCD as the tiles (one partition), so the rows and sums
// come from its L2.
template <typename T, int P, int HPT, int Q>
__device__ void norm_item(const SsdArgs& a, int b, int c, int g, int tig) {
    typedef typename TT<T>::v8 v8;
    constexpr int PPR = HPT * P / 8;  // 16-byte pieces of a token row of the tile
    constexpr int KN = Q * PPR / 256;  // pieces per thread
    const int tid = tid_here();
    const int L = a.seqlen, H = a.nheads, Gn = a.ngroups;
    const int head0 = g * a.hpg + tig * HPT, tok0 = c * Q;
    const int valid = L - tok0 < Q ? L - tok0 : Q;
    uint32_t* cnt = a.ncount + ((size_t)b * a.nchunks + c) * Gn + g;
    if (tid < 64) wait_flag(cnt, a, (uint32_t)a.tpg);
    __syncthreads();
    const uint32_t rs = (uint32_t)H * P * 2;
    const size_t row0 = ((size_t)b * L + tok0) * H * P + (size_t)head0 * P;
    // rows past the sequence end read as zeros and are not written
    const __amdgpu_buffer_rsrc_t orow = make_rsrc((T*)a.out + row0, (uint32_t)(valid - 1) * rs + PPR * 16);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc((const T*)a.z + row0, (uint32_t)(valid - 1) * rs + PPR * 16);
    const __amdgpu_buffer_rsrc_t ns = make_rsrc(a.nsum + ((size_t)b * L + tok0) * Gn + g, (uint32_t)(valid * Gn * 4));
    const float inv = 1.f / (float)(a.hpg * P);
    // every load first, then the arithmetic and the stores (one wait for all of them)
    v8 yv[KN], zv[KN];
    float r[KN];
#pragma unroll
    for (int k = 0; k < KN; ++k) {
        const int f = k * 256 + tid, t = f / PPR, pc = f % PPR;
        const uint32_t off = (uint32_t)t * rs + (uint32_t)pc * 16;
        yv[k] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(orow, off, 0, AUX_L2));
        zv[k] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(zr, off, 0, 0));
        r[k] = bload_f32<AUX_L2>(ns, (uint32_t)(t * Gn) * 4);
    }
#pragma unroll
    for (int k = 0; k < KN; ++k) {
        const int f = k * 256 + tid, t = f / PPR, pc = f % PPR;
        const float rk = __builtin_amdgcn_rsqf(r[k] * inv + a.norm_eps);
        const f32x4 w0 = *(const f32x4*)(a.norm_w + head0 * P + pc * 8);
        const f32x4 w1 = *(const f32x4*)(a.norm_w + head0 * P + pc * 8 + 4);
        v8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (T)((float)yv[k][e] * silu_f((float)zv[k][e]) * rk * (e < 4 ? w0[e] : w1[e - 4]));
        if (t < valid)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), orow, (uint32_t)t * rs + (uint32_t)pc * 16, 0, 2);
    }
}

// `hook` (fused form): claim() after the round-2 reads are issued; see ClaimHook.
// VL: 0 plain input; 1 packed variable-length input (a.seq_idx set: the decays are masked by
// sequence); 2 packed input with per-sequence states (a.seqstates).  Separate instantiations, so
// each kernel carries only the code of its own mode.
// BLK (fused form only): the block form -- x convolved from the raw xBC rows in LDS before
// use, B and C read from the bmm tiles' convolved copies, and with a.norm_fused the gated norm
// applied to y before it leaves (norm_rows).
template <typename T, int P, int N, int Q, int MODE, int VL, int BLK = 0, typename Hook>
__device__ void chunk_tile16(const SsdArgs& a, int b, int c, int g, int tig, char* smem, const float* cbp,
                             const Hook& hook) {
    typedef Geo16<T, P, N, Q> G_;
    constexpr int PW = G_::PW, WPH = G_::WPH, HPT = G_::HPT, MBP = G_::MBP, NB = G_::NB, KS = G_::KS,
                  QB = G_::QB;
    constexpr int AUX = MODE == MODE_FUSED ? AUX_L2 : 0;  // dt/acs and CB written inside one launch
    constexpr int CB_AUX = AUX;
    constexpr bool CB_LDS = G_::CB_LDS;
    typedef typename TT<T>::frag frag;
    typedef typename TT<T>::v4 v4;

    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int hs = wave / WPH, ph = wave % WPH;
    const int L = a.seqlen, H = a.nheads, Gn = a.ngroups, nc = a.nchunks, hpg = a.hpg;
    const int head0 = g * hpg + tig * HPT;
    const int h = head0 + hs;
    const bool hvalid = (tig * HPT + hs) < hpg;
    const int tok0 = c * Q;
    const int valid = L - tok0 < Q ? L - tok0 : Q;  // tokens of this chunk inside the sequence

    T* sX = (T*)smem;                                     // R1: [HPT][Q][P] x, later CB bands
    float* sCB = (float*)smem;
    T* sBC = (T*)(smem + G_::SZ_R1);                      // R2: [Q][N] B, later C
    // per-token vectors, [HPT][Q] each: sA2 = acs * log2(e); sW = chunk-state weights
    // exp(acs[Q-1] - acs_j) dt_j, later replaced by sF (see below); sDt = dt; then [Q] sSeg =
    // the sequence starts among chunk tokens 0 .. i (packed input only, shared by the heads)
    float* sA2 = (float*)(smem + G_::SZ_R1 + G_::SZ_BC);
    float* sW = sA2 + HPT * Q;
    float* sDt = sW + HPT * Q;
    float* sF = sW;
    int* sSeg = (int*)(sDt + HPT * Q);
    constexpr bool varlen = VL != 0;
    const bool cb16 = a.cb16 != 0;  // relaxed intermediates: CB in T

    // read now: a load issued just before its use in the y loop would make every row block wait
    // for all of the tile's outstanding memory operations
    const float Dh = (MODE != MODE_STATE && a.D && hvalid) ? a.D[h] : 0.f;
    const uint32_t xrs = (uint32_t)H * P * 2, bcrs = (uint32_t)Gn * N * 2;  // y rows; B, C rows
    const size_t xel = BLK ? (size_t)a.x_stride : (size_t)H * P;            // x rows, elements
    constexpr int BC_AUX = BLK ? AUX_L2 : 0;  // block form: B, C written inside the launch
    const uint32_t bc_bytes = (uint32_t)(valid - 1) * bcrs + N * 2;
    const size_t bc_off = (((size_t)b * L + tok0) * Gn + g) * N;

    // ---- round 1: x of every head of the tile, and B (or C), into LDS ----------------------
    for (int hh = 0; hh < HPT; ++hh) {
        const bool ok = (tig * HPT + hh) < hpg;
        const T* xb = (const T*)a.x + ((size_t)b * L + tok0) * xel + (size_t)(head0 + (ok ? hh : 0)) * P;
        const uint32_t bytes = ok ? (uint32_t)((valid - 1) * xel * 2) + P * 2 : 0u;
        dma_rows<P, SWZ_TR, 2>(sX + hh * Q * P, make_rsrc(xb, bytes), Q, (uint32_t)(xel * 2));  // nt: read once
    }
    if constexpr (MODE != MODE_SCAN)
        dma_rows<N, SWZ_TR, BC_AUX>(sBC, make_rsrc((const T*)a.B + bc_off, bc_bytes), Q, bcrs);
    else
        dma_rows<N, SWZ_ROW, BC_AUX>(sBC, make_rsrc((const T*)a.C + bc_off, bc_bytes), Q, bcrs);
    {
        // heads of the tile past the group read as zeros
        const int nvh = hpg - tig * HPT < HPT ? hpg - tig * HPT : HPT;
        const size_t off = (((size_t)b * nc + c) * H + head0) * Q;
        const __amdgpu_buffer_rsrc_t rdt = make_rsrc(a.dtf + off, (uint32_t)(nvh * Q * 4));
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.acs + off, (uint32_t)(nvh * Q * 4));
        for (int e = tid; e < HPT * Q; e += 256) {
            sDt[e] = bload_f32<AUX>(rdt, (uint32_t)e * 4);
            sA2[e] = bload_f32<AUX>(ra, (uint32_t)e * 4) * LOG2E;
        }
        if constexpr (varlen) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.seg + ((size_t)b * nc + c) * Q, (uint32_t)Q * 4);
            for (int e = tid; e < Q; e += 256) sSeg[e] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, e * 4, 0, AUX);
        }
    }
    lds_barrier();  // dt, acs (seg) in LDS (the x / B copies may still be in flight)
    // chunk-state weights; with packed input only the chunk's last sequence reaches its end
    for (int e = tid; e < HPT * Q; e += 256) {
        const int hh = e / Q;
        const float w = __builtin_amdgcn_exp2f(sA2[hh * Q + Q - 1] - sA2[e]) * sDt[e];
        sW[e] = (varlen && sSeg[e - hh * Q] != sSeg[Q - 1]) ? 0.f : w;
    }
    wait_vm_all();
    __syncthreads();
    if constexpr (BLK) conv_x_tile<T, P, Q, HPT>(ConvSrc<T>(a), b, tok0, valid, head0, sX);

    const float* a2_h = sA2 + hs * Q;
    // the state entering the chunk reaches its end unless a packed sequence starts inside it
    const bool carry = !varlen || sSeg[Q - 1] == 0;

    // x operand, token-major: xf[kk][pb] holds x[kk*32 + 8q .. +7][ph*PW + pcol(pb, r16)]
    frag xf[KS][MBP];
    {
        int xo[MBP];
        tr_lane_offs_p<P, MBP>(ph * PW, xo);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) xf[kk][pb] = tr_frag_at<T, P>(sX + hs * Q * P, xo[pb], kk * 32);
    }

    // S_c in accumulator layout, rounded to T: tile (nb, pb), lane -> S[p = ph*PW + pcol(pb, r16)][n = nb*16 + 4q + r]
    v4 scb[NB][MBP];
    LBuild<T, G_, AUX> lb;  // the L bands' CB pieces, read early (Q <= 128 with room for L)
    if constexpr (MODE != MODE_SCAN) {
        // ---- chunk_state: s^T[n][p] = sum_j B[j][n] (x[j][p] w_j) ----
        f32x4 acc[NB][MBP];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) acc[nb][pb] = vzero<f32x4>();
        int boff[NB];
        tr_lane_offs<N, NB>(boff);
        if constexpr (VL == 2) {
            if (a.seqstates && hvalid) {
                // Per-sequence final states of the segments that end before the chunk's last
                // one: the chunk state over the segment's tokens up to its last token e, plus (a
                // segment that starts here) its sequence's initial state decayed to e.  Segment 0
                // (begun in an earlier chunk) gets its partial sum here and the decayed entry state
                // S_c at the hop (chunk_scan in the unfused form).
                const int Kc = sSeg[Q - 1], k0 = sSeg[0] == 0 ? 0 : 1;
                const float* dt_h = sDt + hs * Q;
                for (int k = k0; k < Kc; ++k) {
                    const int s = k == 0 ? 0 : seg_first(sSeg, Q, k);
                    const int e = seg_first(sSeg, Q, k + 1) - 1;
                    const int qs = seq_at(a, b, tok0 + s);
                    const float a2e = a2_h[e];
                    f32x4 pacc[NB][MBP];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) pacc[nb][pb] = vzero<f32x4>();
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) {
                        if (kk * 32 > e || kk * 32 + 31 < s) continue;
                        frag af[NB];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) af[nb] = tr_frag_at<T, N>(sBC, boff[nb], kk * 32);
                        float w[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int j = kk * 32 + 8 * q + u;
                            w[u] = sSeg[j] == k ? __builtin_amdgcn_exp2f(a2e - a2_h[j]) * dt_h[j] : 0.f;
                        }
                        frag xw[MBP];
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb)
#pragma unroll
                            for (int u = 0; u < 8; ++u) xw[pb][u] = (T)((float)xf[kk][pb][u] * w[u]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int pb = 0; pb < MBP; ++pb) pacc[nb][pb] = TT<T>::mma(af[nb], xw[pb], pacc[nb][pb]);
                    }
                    if (qs >= 0 && qs < a.nseq) {
                        const float dec = (k >= 1 && a.seq_h0) ? __builtin_amdgcn_exp2f(a2e - (s > 0 ? a2_h[s - 1] : 0.f)) : 0.f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int pb = 0; pb < MBP; ++pb) {
                                const int p = ph * PW + G_::pcol(pb, r16), n = nb * 16 + 4 * q;
                                const size_t o = seq_state_off(a, qs, h, p, n, P, N);
                                f32x4 v = pacc[nb][pb];
                                if (dec != 0.f) v += dec * load_state4(a.seq_h0, a.state_dtype, o);
                                store_state4(a.seq_fin, a.state_dtype, o, v);
                            }
                    }
                }
            }
        }
        if (hvalid) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                // every B fragment of this k step is read before the first product, so the LDS
                // reads overlap one another instead of each waiting out its own latency
                frag af[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) af[nb] = tr_frag_at<T, N>(sBC, boff[nb], kk * 32);
                const f32x4 w0 = *(const f32x4*)(sW + hs * Q + kk * 32 + 8 * q);
                const f32x4 w1 = *(const f32x4*)(sW + hs * Q + kk * 32 + 8 * q + 4);
                frag xw[MBP];
#pragma unroll
                for (int pb = 0; pb < MBP; ++pb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xw[pb][e] = (T)((float)xf[kk][pb][e] * w0[e]);
                        xw[pb][e + 4] = (T)((float)xf[kk][pb][e + 4] * w1[e]);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) acc[nb][pb] = TT<T>::mma(af[nb], xw[pb], acc[nb][pb]);
            }
        }
        if constexpr (MODE == MODE_STATE) {
            if (hvalid) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) {
                        const int p = ph * PW + G_::pcol(pb, r16), n = nb * 16 + 4 * q;
                        *(f32x4*)(a.s + ((((size_t)b * nc + c) * H + h) * P + p) * N + n) = acc[nb][pb];
                    }
            }
            return;
        } else {
            // ---- round 2: C into LDS (B is no longer read) and CB -- into registers for the L
            // bands, else into LDS.  The reads are in flight while the hop below waits for and
            // updates the state.
            lds_barrier();  // every wave is done reading x and B
            dma_rows<N, SWZ_ROW, BC_AUX>(sBC, make_rsrc((const T*)a.C + bc_off, bc_bytes), Q, bcrs);
            if constexpr (G_::L_LDS) {
                lb.load(cbp, tid, cb16);
            } else if constexpr (CB_LDS) {
                dma_cb_bands<Q, CB_AUX>(sCB, cbp, cb16 ? 2 : 4);
            }
            hook.claim();
            if (a.relay && hook.relay_live()) {
                // relay form: s_c to the chain's relay item, S_c back
                if (hvalid) relay_handoff<T, NB, MBP>(a, b, c, h, ph, WPH, acc, scb);
            } else if (hvalid) {
                // state_passing hop: S_{c+1} = exp(acs[Q-1]) S_c + s_c, in place in the chain's slot.
                // In a relay-form launch whose partition runs no relay items, the chain's counter
                // starts at 0 and the state lives in the final-state slot 1 (S_0 in slot 0).
                uint32_t* fl = chain_counter(a, b, h, ph, WPH);
                const uint32_t base = a.relay ? 0u : 1u;
                wait_flag(fl, a, (uint32_t)c + base);
                const int K = a.slots;
                const int sin = a.relay ? (c > 0 ? 1 : 0) : c % K, sout = a.relay ? 1 : (c + 1) % K;
                const __amdgpu_buffer_rsrc_t rin =
                    ring_rsrc(a.states, a.state_dtype, ring_chain(b, sin, h, ph, K, H, WPH, NB * MBP), NB * MBP);
                const __amdgpu_buffer_rsrc_t rout =
                    ring_rsrc(a.states, a.state_dtype, ring_chain(b, sout, h, ph, K, H, WPH, NB * MBP), NB * MBP);
                const float dec = carry ? __builtin_amdgcn_exp2f(a2_h[Q - 1]) : 0.f;
                const bool zero0 = c == 0 && !a.has_h0;  // S_0 = 0: nothing to read
                SeqEnds se;
                if constexpr (VL == 2) {
                    if (a.seqstates) se = seq_ends(a, b, c, h, sSeg, a2_h, Q, valid, true);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) {
                        const uint32_t off = ((nb * MBP + pb) * 64 + lane) * 4;
                        const f32x4 sv = zero0 ? vzero<f32x4>() : ring_load(rin, a.state_dtype, off);
                        f32x4 snew = dec * sv + acc[nb][pb];
                        if constexpr (VL == 2) {
                            if (se.any) se.apply(a, h, ph * PW + G_::pcol(pb, r16), nb * 16 + 4 * q, P, N, sv, snew);
                        }
                        ring_store(rout, a.state_dtype, off, snew);
                        scb[nb][pb] = cvt4<T>(sv);
                    }
                publish_flag_wave(fl, (uint32_t)c + 1 + base);  // its wait covers the copies too
            }
            wait_vm_all();
            __syncthreads();  // C (and CB) are in LDS
        }
    } else {
        __syncthreads();
        // ---- round 2: CB (into registers for the L bands, else into LDS over x); S_c into registers
        __syncthreads();  // every wave holds its x operand in registers
        if constexpr (G_::L_LDS) {
            lb.load(cbp, tid, cb16);
        } else if constexpr (CB_LDS) {
            dma_cb_bands<Q, 0>(sCB, cbp, cb16 ? 2 : 4);
        }
        if (hvalid) {
            const int K = a.slots, slot = c % K;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int pb = 0; pb < MBP; ++pb) {
                    const int p = ph * PW + G_::pcol(pb, r16), n = nb * 16 + 4 * q;
                    scb[nb][pb] = cvt4<T>(load_state4(a.states, a.state_dtype, ((((size_t)b * K + slot) * H + h) * P + p) * N + n));
                }
            if constexpr (VL == 2) {
                if (a.seqstates) {
                    // per-sequence final states ending in this chunk, from the chunk-entry and
                    // chunk-end states the state-passing step left in slots c and c + 1
                    const SeqEnds se = seq_ends(a, b, c, h, sSeg, a2_h, Q, valid, false);
                    if (se.any) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int pb = 0; pb < MBP; ++pb) {
                                const int p = ph * PW + G_::pcol(pb, r16), n = nb * 16 + 4 * q;
                                const size_t o = ((((size_t)b * K + slot) * H + h) * P + p) * N + n;
                                const f32x4 sv = load_state4(a.states, a.state_dtype, o);
                                f32x4 snew = load_state4(a.states, a.state_dtype, o + (size_t)H * P * N);
                                se.apply(a, h, p, n, P, N, sv, snew);
                            }
                    }
                }
            }
        }
        wait_vm_all();
        __syncthreads();
    }

    if constexpr (MODE != MODE_STATE) {
        // ---- chunk_scan, 16 rows of y at a time ----
        // Per-token column factors, replacing sW in place (each element is rewritten by the
        // thread that reads it): sF[j] = exp(acs_r - acs_j) dt_j, r = the last token of j's
        // 32-token block (<= dt_j when dt A <= 0); packed input: 0 unless j and r are in one
        // sequence.  Off the diagonal (all of a 32-column block left of the 16 rows) L[i][j] is
        // split as exp(acs_i - acs_r) * exp(acs_r - acs_j) dt_j: both factors are at most 1 when
        // acs does not increase along the chunk, so nothing overflows, and a factor only
        // underflows when the exact product is below e^-87.  The column factor scales x once per
        // tile; the row factor is one exp per lane per block (packed: 0 unless r and i are in
        // one sequence).  On the diagonal, each element takes its own exp(acs_i - acs_j) * dt_j.
        // (With the L bands, the column factors end at 16-token blocks instead: see LBuild.)
        //
        // x for the D x term in the y layout (x[ib*16 + r16][ph*PW + 4 MBP q + 4 pb .. +3]).  While the
        // x tile is still in LDS (it is, unless the CB bands were copied over it) it comes from
        // there: with the L bands, which replace it next, every row block is read now; without
        // CB in LDS, at its use.  Otherwise it is read again from HBM/L2, two blocks ahead.
        constexpr bool XD_LDS = G_::L_LDS || !CB_LDS;
        constexpr int XDA = G_::L_LDS ? QB : (XD_LDS ? 1 : 2);
        const __amdgpu_buffer_rsrc_t xr =
            make_rsrc((const T*)a.x + (((size_t)b * L + tok0) * H + h) * P, (uint32_t)(valid - 1) * xrs + P * 2);
        const T* sX_h = sX + hs * Q * P;
        auto xd_load = [&](int ib, int pb) -> v4 {
            if constexpr (XD_LDS)
                return *(const v4*)(sX_h + sw_off<P>(ib * 16 + r16, ph * PW + 4 * MBP * q + 4 * pb));
            const uint32_t off = (uint32_t)(ib * 16 + r16) * xrs + (uint32_t)(ph * PW + 4 * MBP * q + 4 * pb) * 2;
            return __builtin_bit_cast(v4, __builtin_amdgcn_raw_buffer_load_b64(xr, off, 0, 0));
        };
        v4 xd[XDA][MBP];
        if (hvalid) {
#pragma unroll
            for (int ib = 0; ib < (XD_LDS && !G_::L_LDS ? 0 : XDA); ++ib)
#pragma unroll
                for (int pb = 0; pb < MBP; ++pb) xd[ib][pb] = xd_load(ib, pb);
        }
        for (int e = tid; e < HPT * Q; e += 256) {
            const int hh = e / Q, j = e - hh * Q;
            const int r = G_::L_LDS ? (j | 15) : (j | 31);
            const float f = __builtin_amdgcn_exp2f(sA2[hh * Q + r] - sA2[e]) * sDt[e];
            sF[e] = (varlen && sSeg[j] != sSeg[r]) ? 0.f : f;
        }
        lds_barrier();
        if constexpr (G_::L_LDS) {
            const int nvh = hpg - tig * HPT < HPT ? hpg - tig * HPT : HPT;
            lb.store((T*)smem, sA2, sF, sDt, sSeg, varlen, cb16, nvh, tid);  // over x (already in registers)
            lds_barrier();                                             // L is complete
        }
        if (!hvalid) return;
        // S_c as the A operand of C . S^T; k slots of step ks: n = 32ks + 4q + {0..3} and
        // 32ks + 16 + 4q + {0..3} (the accumulator layout), matched by the C reads below.
        frag sop[N / 32][MBP];
#pragma unroll
        for (int ks = 0; ks < N / 32; ++ks)
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb)
                sop[ks][pb] = __builtin_shufflevector(scb[2 * ks][pb], scb[2 * ks + 1][pb], 0, 1, 2, 3, 4, 5, 6, 7);
        // x scaled by the column factor, for the blocks left of the diagonal (without L bands)
        frag xs[KS][MBP];
        const float* f_h = sF + hs * Q;
        const float* dt_h = sDt + hs * Q;
        const T* sL_h = (const T*)smem + (size_t)hs * G_::SZ_LH / sizeof(T);
#pragma unroll
        for (int kk = 0; kk + 1 < (G_::L_LDS ? 0 : KS); ++kk) {
            const f32x4 f0 = *(const f32x4*)(f_h + kk * 32 + 8 * q);
            const f32x4 f1 = *(const f32x4*)(f_h + kk * 32 + 8 * q + 4);
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) {
                f32x4 lo, hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = (float)xf[kk][pb][e] * f0[e];
                    hi[e] = (float)xf[kk][pb][e + 4] * f1[e];
                }
                xs[kk][pb] = pack8<T>(lo, hi);
            }
        }
        const uint32_t ces = cb16 ? 2u : 4u;
        const __amdgpu_buffer_rsrc_t cbr = make_rsrc(cbp, (uint32_t)(Q * Q) * ces);
        const __amdgpu_buffer_rsrc_t cbr2 = cb16 ? make_rsrc(cbp, 0u) : cbr;
        // y: written once and never read here, so non-temporal (nt) stores keep it from
        // pushing the state slots and CB out of the L2
        const __amdgpu_buffer_rsrc_t yr =
            make_rsrc((T*)a.y + (((size_t)b * L + tok0) * H + h) * P, (uint32_t)(valid - 1) * xrs + P * 2);
        // this lane's C-row read offsets for k step ks (row r16 of a 16-row block; the row
        // swizzle of C repeats every 16 rows, so block ib adds ib * 16 * N)
        int clo[N / 32], chi[N / 32];
#pragma unroll
        for (int ks = 0; ks < N / 32; ++ks) {
            clo[ks] = sw_off<N, SWZ_ROW>(r16, ks * 32 + 4 * q);
            chi[ks] = sw_off<N, SWZ_ROW>(r16, ks * 32 + 16 + 4 * q);
        }
        v4 yo[QB][MBP];  // y rows of this lane, in T
#pragma unroll
        for (int ib = 0; ib < QB; ++ib) {
            const int i = ib * 16 + r16;  // this lane's output row (column of y^T)
            f32x4 accY[MBP];
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) accY[pb] = vzero<f32x4>();
            // The row block's offset is hidden from the compiler so that it keeps the C reads
            // single ds_read_b64 (32 lanes a cycle, conflict-free with the row swizzle) instead of
            // merging the reads of two row blocks into ds_read2st64_b64, which the LDS serves 16
            // lanes a cycle (measured: four times the cycles of the two reads apart).
            int cblk = ib * 16 * N;
            asm volatile("" : "+v"(cblk));
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) {
                const v4 lo = *(const v4*)(sBC + clo[ks] + cblk);
                const v4 hi = *(const v4*)(sBC + chi[ks] + cblk);
                const frag cf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int pb = 0; pb < MBP; ++pb) accY[pb] = TT<T>::mma(sop[ks][pb], cf, accY[pb]);
            }
            const float ai2 = a2_h[i];
            // S_c reaches row i only inside the chunk's first packed sequence
            const float ei = (varlen && sSeg[i] != 0) ? 0.f : __builtin_amdgcn_exp2f(ai2);
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) accY[pb] *= ei;
            if constexpr (VL == 2) {
                if (a.seqstates && a.seq_h0) {
                    // the sequences that start in these 16 rows enter with their initial states:
                    // + exp(acs_i - acs_{s-1}) C_i . h0_q for row i of the segment starting at s
                    const int klo = sSeg[ib * 16] > 1 ? sSeg[ib * 16] : 1, khi = sSeg[ib * 16 + 15];
                    for (int k = klo; k <= khi; ++k) {
                        const int s = seg_first(sSeg, Q, k);
                        const int qs = seq_at(a, b, tok0 + s);
                        if (qs < 0 || qs >= a.nseq) continue;
                        f32x4 tmp[MBP];
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) tmp[pb] = vzero<f32x4>();
#pragma unroll
                        for (int ks = 0; ks < N / 32; ++ks) {
                            const v4 lo = *(const v4*)(sBC + clo[ks] + ib * 16 * N);
                            const v4 hi = *(const v4*)(sBC + chi[ks] + ib * 16 * N);
                            const frag cf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                            for (int pb = 0; pb < MBP; ++pb) {
                                const int p = ph * PW + G_::pcol(pb, r16);
                                const f32x4 h_lo = load_state4(a.seq_h0, a.state_dtype, seq_state_off(a, qs, h, p, ks * 32 + 4 * q, P, N));
                                const f32x4 h_hi = load_state4(a.seq_h0, a.state_dtype, seq_state_off(a, qs, h, p, ks * 32 + 16 + 4 * q, P, N));
                                tmp[pb] = TT<T>::mma(pack8<T>(h_lo, h_hi), cf, tmp[pb]);
                            }
                        }
                        const float fi = sSeg[i] == k ? __builtin_amdgcn_exp2f(ai2 - (s > 0 ? a2_h[s - 1] : 0.f)) : 0.f;
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) accY[pb] += tmp[pb] * fi;
                    }
                }
            }
            const int kd = ib >> 1;  // the diagonal 32-column block of these 16 rows
            if constexpr (G_::L_LDS) {
                // L^T operand straight from the bands: lane (r16, q) takes L[i][32kk + 8q .. +7]
#pragma unroll
                for (int kk = 0; kk <= kd; ++kk) {
                    const frag lf = *(const frag*)(sL_h + lband_off<G_>(i, kk * 4 + q) * 8);
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) accY[pb] = TT<T>::mma(xf[kk][pb], lf, accY[pb]);
                }
            }
#pragma unroll
            for (int kk = 0; kk <= (G_::L_LDS ? -1 : kd); ++kk) {
                const int j0 = kk * 32 + 8 * q;
                f32x4 c0, c1;
                if constexpr (CB_LDS) {
                    // two 16-byte reads for either CB type at offsets selected before them (16-bit:
                    // the first holds all 8 values, the second reads the next piece of the band
                    // row, at most its padding piece, and is not used), then the 16-bit values are
                    // widened.  Control flow on the CB type here (a branch, or a second read that
                    // the compiler may skip when it repeats the first) lands between this row
                    // block's MFMAs and the reads of their accumulators; see cb_widen_sel.
                    const int o0 = cb_byte_off<Q>(ib >> 1, i, j0, cb16);
                    c0 = *(const f32x4*)((const char*)sCB + o0);
                    c1 = *(const f32x4*)((const char*)sCB + o0 + 16);
                    cb_widen_sel<T>(cb16, c0, c1);
                } else {
                    // the same two loads for either CB type (16-bit: all 8 values in the first, the
                    // second from an empty range), then the 16-bit values are widened; no control
                    // flow on the CB type (see cb_widen_sel)
                    c0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(cbr, (uint32_t)(i * Q + j0) * ces, 0, CB_AUX));
                    c1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(cbr2, (uint32_t)(i * Q + j0 + 4) * 4, 0, CB_AUX));
                    cb_widen_sel<T>(cb16, c0, c1);
                }
                if (kk < kd) {
                    const float gx = __builtin_amdgcn_exp2f(ai2 - a2_h[kk * 32 + 31]);
                    const float gi = (varlen && sSeg[i] != sSeg[kk * 32 + 31]) ? 0.f : gx;
                    const frag lf = pack8<T>(c0 * gi, c1 * gi);
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) accY[pb] = TT<T>::mma(xs[kk][pb], lf, accY[pb]);
                } else {
                    const f32x4 a0 = *(const f32x4*)(a2_h + j0), a1 = *(const f32x4*)(a2_h + j0 + 4);
                    const f32x4 d0 = *(const f32x4*)(dt_h + j0), d1 = *(const f32x4*)(dt_h + j0 + 4);
                    f32x4 l0, l1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v0 = c0[e] * __builtin_amdgcn_exp2f(ai2 - a0[e]) * d0[e];
                        const float v1 = c1[e] * __builtin_amdgcn_exp2f(ai2 - a1[e]) * d1[e];
                        const bool k0 = j0 + e <= i && (!varlen || sSeg[j0 + e] == sSeg[i]);
                        const bool k1 = j0 + 4 + e <= i && (!varlen || sSeg[j0 + 4 + e] == sSeg[i]);
                        l0[e] = k0 ? v0 : 0.f;
                        l1[e] = k1 ? v1 : 0.f;
                    }
                    const frag lf = pack8<T>(l0, l1);
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) accY[pb] = TT<T>::mma(xf[kk][pb], lf, accY[pb]);
                }
            }
            // y = acc + D x: 4 MBP consecutive p per lane (see Geo16::pcol)
            v4 xcur[MBP];
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) {
                if constexpr (G_::L_LDS) {
                    xcur[pb] = xd[ib][pb];
                } else if constexpr (XD_LDS) {
                    xcur[pb] = xd_load(ib, pb);
                } else {
                    xcur[pb] = xd[0][pb];
                    xd[0][pb] = xd[1][pb];
                    if (ib + 2 < QB) xd[1][pb] = xd_load(ib + 2, pb);
                }
            }
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) {
                f32x4 yv = accY[pb];
                yv[0] += Dh * (float)xcur[pb][0];
                yv[1] += Dh * (float)xcur[pb][1];
                yv[2] += Dh * (float)xcur[pb][2];
                yv[3] += Dh * (float)xcur[pb][3];
                yo[ib][pb] = cvt4<T>(yv);
            }
        }
        // y leaves in whole token rows: the tile's HPT heads of one token are adjacent in y
        // (HPT * P * 2 = 256 bytes for P >= 32), but each wave holds only its 32 p columns of a
        // head, so stored directly every row would go out as 64-byte pieces of 128-byte lines.
        // With every head of the tile valid (a tile-wide condition: the waves of a head past the
        // group's end have left already) the waves first put their pieces into LDS (R1: the L
        // bands, x and CB are no longer read), then each wave stores four whole token rows per
        // instruction.  16-byte pieces are XOR-swizzled by the token so neither pass conflicts.
        constexpr int ROWB = HPT * P * 2, PPR = ROWB / 16;
        static_assert(!BLK || (MBP == 2 && PPR == 16 && HPT * Q * P * 2 <= G_::SZ_R1 && XD_LDS),
                      "the block form stages whole y rows in LDS and keeps the convolved x there");
        const int nvh_y = hpg - tig * HPT < HPT ? hpg - tig * HPT : HPT;
        if (MBP == 2 && PPR == 16 && HPT * Q * P * 2 <= G_::SZ_R1 && nvh_y == HPT) {
            char* sY = smem;
            lds_barrier();  // every wave is done with R1
#pragma unroll
            for (int ib = 0; ib < QB; ++ib) {
                const int i = ib * 16 + r16;
                const int pc = (hs * P + ph * PW + 4 * MBP * q) >> 3;
                *(u32x4*)(sY + i * ROWB + ((pc ^ (i & (PPR - 1))) << 4)) =
                    __builtin_bit_cast(u32x4, __builtin_shufflevector(yo[ib][0], yo[ib][1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
            lds_barrier();
            if (BLK && a.norm_fused) {
                norm_rows<T, P, Q, PPR>(a, b, c, g, head0, tok0, valid, sY);
                return;
            }
            const __amdgpu_buffer_rsrc_t yrow =
                make_rsrc((T*)a.y + (((size_t)b * L + tok0) * H + head0) * P, (uint32_t)(valid - 1) * xrs + ROWB);
#pragma unroll
            for (int k = 0; k < Q * PPR / 256; ++k) {
                const int f = (k * 4 + wave) * 64 + lane, t = f / PPR, pc = f % PPR;
                const u32x4 v = *(const u32x4*)(sY + t * ROWB + ((pc ^ (t & (PPR - 1))) << 4));
                if (t < valid) __builtin_amdgcn_raw_buffer_store_b128(v, yrow, (uint32_t)t * xrs + (uint32_t)pc * 16, 0, 2);
            }
        } else {
            // The stores go out together after the loop: a store's registers stay reserved until
            // it completes, so reusing them block after block would make every block wait for the
            // previous block's store.  (yo takes the registers the D x operand frees.)
#pragma unroll
            for (int ib = 0; ib < QB; ++ib) {
                const int i = ib * 16 + r16;
                if (i < valid) {
                    const uint32_t yoff = (uint32_t)i * xrs + (uint32_t)(ph * PW + 4 * MBP * q) * 2;
                    if constexpr (MBP == 2)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(u32x4, __builtin_shufflevector(yo[ib][0], yo[ib][1], 0, 1, 2, 3, 4, 5, 6, 7)),
                            yr, yoff, 0, 2);
                    else
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, yo[ib][0]), yr, yoff, 0, 2);
                }
            }
        }
    }
}

}  // namespace ssd

// moe_gemm_mx.hip - grouped products with MXFP4 routed weights and MXFP8
// activations on gfx950's scaled f8f6f4 MFMA.
//
// Formats (DeepGEMM issue "GC MoE": FP8 activations with packed FP4 routed
// weights; the MegaKernel issue's ue8m0 scales per 32 elements for FP8 GEMM
// inputs; read as the OCP Microscaling formats): weights are E2M1, two per
// byte with element 2i in the low nibble, one E8M0 scale byte per 32 K
// elements of a row; activations and the re-quantised SwiGLU output are E4M3
// with one E8M0 byte per 32 elements.  The MFMA applies both scales itself,
// so the products accumulate in fp32 registers with no promotion step.
//
// Operand placement of v_mfma_scale_f32_32x32x64_f8f6f4 on gfx950 (measured
// with single-wave probes): lane (r, h) of an fp8 operand holds K [16h, 16h+16)
// in bytes 0-15 and K [32+16h, 48+16h) in bytes 16-31; of an fp4 operand K
// [32h, 32h+32) in 16 bytes, low nibble first; its scale byte applies to K
// block h (K [32h, 32h+32)) of row r.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_layer.h"

namespace moe {

constexpr int kMxThreads = 512;   // 8 waves
constexpr int kMxBM = 128;        // rows of an M tile
constexpr int kMxBK = 128;        // K elements of a sub-block: 128 fp8 bytes, 64 fp4 bytes per row
constexpr int kMxRegStages = 2;   // stages of operands loading ahead in registers

// LDS chunk (16 bytes) of a 64-byte fp4 row: 16 consecutive rows read at one
// logical chunk land on 16 distinct 4-bank groups.
__device__ __forceinline__ int lds_chunk4(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// One work item = (M tile of <= 128 rows of one expert) x (BN panel rows),
// the 8 waves a 4 (M) x 2 (N) grid of 32 x BN/2 wave tiles.  Per stage of KS
// 128-K sub-blocks a thread stages 2 KS A chunks (token rows, fp8), BN KS / 128
// B chunks (panel rows, fp4) and KS scale words (4 E8M0 bytes each: A scales
// for threads 0-127, B scales for threads 128-383) in registers, two stages
// ahead, and writes them into a 2-stage LDS ring.  Wave (wm, wn) owns tile
// rows [32 wm, 32 wm + 32) and panel rows [BN/2 wn, BN/2 (wn + 1)) as blocks
// of 32.
// SWIGLU: panel rows interleave gate/up in blocks of 32 (as the bf16 path), so
// blocks (0, 1) and (2, 3) of a wave are (gate, up) pairs; each pair gives 32
// h columns of one 32-wide MXFP8 block, whose row maximum is a reduction over
// the 32 lanes that hold the columns.  Otherwise y bf16 [P, n_out] in expert
// order.
// KS = 128-K sub-blocks per stage: with KS = 2 every weight row delivers a
// whole 128-byte line of E2M1 codes per stage (and every token row 256 bytes)
// instead of half a line.
// WM = 1 (decode batches): one 32-row block, the 8 waves side by side over a
// 512-row panel (32 x 64 each, one gate/up pair); every thread then stages the
// scale words of panel row t and of tile row t % 32.
template <int BN, bool SWIGLU, int KS, int WM = 4>
__global__ __launch_bounds__(kMxThreads) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const ExpertArray<uint8_t> B,
    const ExpertArray<uint8_t> Bs, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles_p,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ offsets, int E, int K,
    int n_out, int b_rows, int topk, uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cs,
    uint16_t* __restrict__ Cy) {
    constexpr int BM = 32 * WM, WN = 8 / WM;
    constexpr int NB = BN / (32 * WN);                // 32-row panel blocks per wave
    constexpr int ACH = 8 * KS, BCH = 4 * KS;         // 16-byte chunks per A / B row and stage
    constexpr int A_PER = BM * ACH / kMxThreads;      // 16-byte A chunks per thread and stage
    constexpr int B_PER = BN * BCH / kMxThreads;      // 16-byte B chunks per thread and stage
    static_assert((KS == 1 || KS == 2) && (WM == 4 || WM == 1) && A_PER >= 1 && B_PER >= 1 &&
                  (!SWIGLU || NB % 2 == 0) && (WM == 4 ? BM + BN <= kMxThreads : BN == kMxThreads),
                  "tile shape");
    __shared__ u32x4 a_lds[2][BM][ACH];
    __shared__ u32x4 b_lds[2][BN][BCH];
    __shared__ uint32_t sa_lds[2][KS][BM];
    __shared__ uint32_t sb_lds[2][KS][BN];
    // physical LDS chunk of logical chunk c of a row: KS = 1 as lds_chunk /
    // lds_chunk4; KS = 2 rows are 256 (A) and 128 (B) bytes, so 16 and 8
    // consecutive rows spread over the positions of a full-row XOR
    auto a_phys = [](int r, int c) { return KS == 1 ? lds_chunk(r, c) : c ^ (r & 15); };
    auto b_phys = [](int r, int c) { return KS == 1 ? lds_chunk4(r, c) : c ^ ((r >> 1) & 7); };

    // waves w and w + 4 share a SIMD: (wm, wn) = (w / 2, w % 2) puts the
    // waves of the first rows on four different SIMDs, so a tile of a few
    // rows (decode batches) still spreads its products over the CU
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = WM == 4 ? wave >> 1 : 0, wn = WM == 4 ? wave & 1 : wave;
    const int h = lane >> 5;
    const int ntiles = *ntiles_p;
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int items = ntiles * n_tiles_n;
    const int nks = K / (kMxBK * KS);
    const int kb_row = K / 32;                        // scale bytes per row

    auto panel_row = [&](int rr, int nt) {
        if (SWIGLU) {
            const int blk = rr >> 5;
            return ((blk & 1) ? n_out : 0) + nt * (BN / 2) + (blk >> 1) * 32 + (rr & 31);
        }
        return nt * BN + rr;
    };

    for (int it = xcd_slot(blockIdx.x, gridDim.x); it < items; it += gridDim.x) {
        const GroupedItem gi = grouped_item(it, tile_off, E, n_tiles_n);
        const int nt = gi.nt, e = gi.e;
        const int row0 = tiles[2 * gi.mt + 1];
        const int mrows = min(BM, offsets[e + 1] - row0);
        const bool active = 32 * wm < mrows;

        // sources (rows past the tile's end read row 0, never stored)
        const uint8_t* a_src[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int q = tid + kMxThreads * i;       // chunk id: row q / ACH, chunk q % ACH
            const int r = q / ACH;
            int64_t arow = 0;
            if (r < mrows) arow = SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
            a_src[i] = A + arow * K + (q % ACH) * 16;
        }
        const uint8_t* b_src[B_PER];
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int q = tid + kMxThreads * i;       // row q / BCH, chunk q % BCH
            b_src[i] = B.expert(e, (int64_t)b_rows * (K / 2)) + (int64_t)panel_row(q / BCH, nt) * (K / 2) + (q % BCH) * 16;
        }
        // scale words: WM = 4: thread t < 128 -> A row t, 128 <= t < 128 + BN
        // -> B row t - 128; WM = 1: B row t (s_src) and A row t % 32 (sa_src)
        const bool sa_t = tid < BM, sb_t = WM == 4 ? tid >= BM && tid < BM + BN : true;
        const uint8_t* s_src;
        const uint8_t* sa_src;
        {
            const int r = WM == 4 ? (sa_t ? tid : 0) : (tid & (BM - 1));
            int64_t arow = 0;
            if ((WM == 1 || sa_t) && r < mrows)
                arow = SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
            const uint8_t* sa = As + arow * kb_row;
            const uint8_t* sb = Bs.expert(e, (int64_t)b_rows * kb_row) + (int64_t)panel_row(sb_t ? (WM == 4 ? tid - BM : tid) : 0, nt) * kb_row;
            s_src = WM == 4 ? (sb_t ? sb : sa) : sb;
            sa_src = sa;
        }

        f32x16 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
        // kMxRegStages stages of operands in registers: stage ks is written to
        // the LDS ring, and its registers are refilled with stage
        // ks + kMxRegStages right after the barrier, before the wave computes
        // stage ks, so that kMxRegStages stages stay in flight through every
        // product
        u32x4 ra[kMxRegStages][A_PER], rb[kMxRegStages][B_PER];
        uint32_t rs[kMxRegStages][KS];
        uint32_t rsa[kMxRegStages][KS];   // WM = 1 only: the A word

        auto load = [&](u32x4 (&ra_)[A_PER], u32x4 (&rb_)[B_PER], uint32_t (&rs_)[KS],
                        uint32_t (&rsa_)[KS], int ks) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) ra_[i] = *(const u32x4*)(a_src[i] + ks * (kMxBK * KS));
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                // decode batches read each weight panel once: non-temporal,
                // so that the stream does not push the E8M0 rows out of L2
                const uint8_t* src = b_src[i] + ks * (kMxBK / 2 * KS);
                if constexpr (WM == 1) rb_[i] = __builtin_nontemporal_load((const u32x4*)src);
                else rb_[i] = *(const u32x4*)src;
            }
            // 4 scale bytes per 128-K sub-block (blocks 4 (KS ks + j) .. + 3)
            if constexpr (KS == 1) {
                rs_[0] = *(const uint32_t*)(s_src + ks * 4);
                if constexpr (WM == 1) rsa_[0] = *(const uint32_t*)(sa_src + ks * 4);
            } else {   // two words (the scale tensors need only 4-byte alignment)
                rs_[0] = *(const uint32_t*)(s_src + ks * 8);
                rs_[1] = *(const uint32_t*)(s_src + ks * 8 + 4);
                if constexpr (WM == 1) {
                    rsa_[0] = *(const uint32_t*)(sa_src + ks * 8);
                    rsa_[1] = *(const uint32_t*)(sa_src + ks * 8 + 4);
                }
            }
        };
        auto step = [&](int S, u32x4 (&ra_)[A_PER], u32x4 (&rb_)[B_PER], uint32_t (&rs_)[KS],
                        uint32_t (&rsa_)[KS], int ks) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) {
                const int q = tid + kMxThreads * i, r = q / ACH;
                a_lds[S][r][a_phys(r, q % ACH)] = ra_[i];
            }
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int q = tid + kMxThreads * i, r = q / BCH;
                b_lds[S][r][b_phys(r, q % BCH)] = rb_[i];
            }
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if constexpr (WM == 4) {
                    if (sa_t) sa_lds[S][j][tid] = rs_[j];
                    if (sb_t) sb_lds[S][j][tid - BM] = rs_[j];
                } else {
                    sb_lds[S][j][tid] = rs_[j];
                    if (sa_t) sa_lds[S][j][tid] = rsa_[j];
                }
            }
            lds_barrier();
            // refill (past the last stage: re-read the last one, an L2 hit)
            load(ra_, rb_, rs_, rsa_, min(ks + kMxRegStages, nks - 1));
            if (active && ks < nks) {
                const int ar = 32 * wm + (lane & 31);
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    const uint32_t sa = sa_lds[S][j][ar];
                    uint32_t sb[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) sb[nb] = sb_lds[S][j][(wn * NB + nb) * 32 + (lane & 31)];
#pragma unroll
                    for (int c = 0; c < 2; ++c) {   // two 64-K MFMA chunks per 128-K sub-block
                        const u32x4 lo = a_lds[S][ar][a_phys(ar, 8 * j + 4 * c + h)];
                        const u32x4 hi = a_lds[S][ar][a_phys(ar, 8 * j + 4 * c + 2 + h)];
                        const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        const int shift = 8 * (2 * c + h);   // this lane's 32-K block
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const int br = (wn * NB + nb) * 32 + (lane & 31);
                            const u32x4 bq = b_lds[S][br][b_phys(br, 4 * j + 2 * c + h)];
                            const u32x4 z = {0u, 0u, 0u, 0u};
                            const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(bq, z, 0, 1, 2, 3, 4, 5, 6, 7));
                            acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                a, b, acc[nb], 0 /* A fp8 */, 4 /* B fp4 */, 0, (int)(sa >> shift), 0,
                                (int)(sb[nb] >> shift));
                        }
                    }
                }
            }
        };

        static_assert(kMxRegStages == 2, "one register buffer per LDS stage");
        load(ra[0], rb[0], rs[0], rsa[0], 0);
        load(ra[1], rb[1], rs[1], rsa[1], min(1, nks - 1));
        for (int ks = 0; ks < nks; ks += 2) {
            // unconditional (an odd last step computes nothing): a path that
            // skipped it would leave the compiler's wait counts pessimistic
            step(0, ra[0], rb[0], rs[0], rsa[0], ks);
            step(1, ra[1], rb[1], rs[1], rsa[1], ks + 1);
        }

        if (SWIGLU) {
            // h for f = nt*(BN/2) + (wn*NB/2 + p)*32 + lane%32; one MXFP8 block per p
            const int nfb = n_out / 32;
            if (active) {
#pragma unroll
                for (int p = 0; p < NB / 2; ++p)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const float hv = silu_fast(acc[2 * p][q]) * acc[2 * p + 1][q];
                        const float amax = half_max32(fabsf(hv));
                        // shared exponent floor(log2(amax)) - 8 (a subnormal
                        // or zero amax ends below -127 and is clamped there)
                        const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;
                        const int se = max(-127, min(127, ex - 8));
                        const float v = fminf(fmaxf(__builtin_ldexpf(hv, -se), -448.0f), 448.0f);
                        const uint32_t code = f32x4_to_e4m3x4(v, 0.0f, 0.0f, 0.0f);
                        const int row = 32 * wm + acc_row(q, lane);
                        if (row < mrows) {
                            const int blk = nt * (BN / 64) + wn * (NB / 2) + p;
                            Cq[(int64_t)(row0 + row) * n_out + blk * 32 + (lane & 31)] = (uint8_t)code;
                            if ((lane & 31) == 0) Cs[(int64_t)(row0 + row) * nfb + blk] = (uint8_t)(se + 127);
                        }
                    }
            }
        } else if (active) {
            const bool odd = lane & 1;
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const int row = 32 * wm + acc_row(q, lane) + (odd ? 1 : 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float y0 = acc[nb][q], y1 = acc[nb][q + 1];
                    const float got = pair_swap(odd ? y0 : y1);
                    const int col = nt * BN + (wn * NB + nb) * 32 + (lane & 30);
                    if (row < mrows) {
                        const uint32_t v = odd ? pack_bf16x2_hw(got, y1) : pack_bf16x2_hw(y0, got);
                        *(uint32_t*)(Cy + (int64_t)(row0 + row) * n_out + col) = v;
                    }
                }
            }
        }
        lds_barrier();  // the LDS ring is reused by the next item
    }
}

// Wide variant for long M tiles (prefill): 128 rows x 512 panel rows, the 8
// waves a 2 (M) x 4 (N) grid of 64 x 128 wave tiles ((wm, wn) = (w / 4,
// w % 4): the two waves of a SIMD own the same panel rows and the two 64-row
// halves).  Each A fragment read from LDS now feeds 4 products and each B
// fragment 2, against 4 and 1 in the 32 x 128 tiles above: 16 instead of 24
// LDS bytes per lane and product, which the 128 x 256 kernel spends about as
// much time on as on its products.  Scales: every thread stages the word of
// panel row tid, threads < 128 also the word of tile row tid.
// The wide tiles' LDS arrays: separate variables, the same ones for the
// gate_up and the down loop of a one-launch layer.
struct MxWideRing {
    __device__ static u32x4 (&a())[2][kMxBM][8] {
        __shared__ u32x4 v[2][kMxBM][8];
        return v;
    }
    __device__ static u32x4 (&b())[2][512][4] {
        __shared__ u32x4 v[2][512][4];
        return v;
    }
    __device__ static uint32_t (&sa())[2][kMxBM] {
        __shared__ uint32_t v[2][kMxBM];
        return v;
    }
    __device__ static uint32_t (&sb())[2][512] {
        __shared__ uint32_t v[2][512];
        return v;
    }
};

// The persistent item loop of the wide tiles, with the scheduling hooks of
// moe_layer.h.
template <bool SWIGLU, class Sched>
__device__ __forceinline__ void mx_wide_loop(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const ExpertArray<uint8_t>& B,
    const ExpertArray<uint8_t>& Bs, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ offsets, int E, int K, int n_out, int b_rows, int topk,
    uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cs, uint16_t* __restrict__ Cy, Sched& sc) {
    constexpr int BN = 512;
    constexpr int NB = 4;                             // 32-row panel blocks per wave
    constexpr int MB = 2;                             // 32-row tile blocks per wave
    constexpr int A_PER = kMxBM * 8 / kMxThreads;     // 2
    constexpr int B_PER = BN * 4 / kMxThreads;        // 4
    auto& a_lds = MxWideRing::a();
    auto& b_lds = MxWideRing::b();
    auto& sa_lds = MxWideRing::sa();
    auto& sb_lds = MxWideRing::sb();

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int h = lane >> 5;
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int nks = K / kMxBK;
    const int kb_row = K / 32;
    const bool sa_t = tid < kMxBM;

    auto panel_row = [&](int rr, int nt) {
        if (SWIGLU) {
            const int blk = rr >> 5;
            return ((blk & 1) ? n_out : 0) + nt * (BN / 2) + (blk >> 1) * 32 + (rr & 31);
        }
        return nt * BN + rr;
    };

    for (int it = sc.first(); it >= 0; it = sc.next(it)) {
        const GroupedItem gi = grouped_item(it, tile_off, E, n_tiles_n);
        sc.wait_inputs(gi);
        const int nt = gi.nt, e = gi.e;
        const int row0 = tiles[2 * gi.mt + 1];
        const int mrows = min(kMxBM, offsets[e + 1] - row0);
        const bool active = 64 * wm < mrows;
        // rows past the tile's end read token row 0 or the tile's first row
        // (never stored)
        auto a_row = [&](int r) -> int64_t {
            if (r >= mrows) return SWIGLU ? 0 : row0;
            return SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
        };

        const uint8_t* a_src[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int q = tid + kMxThreads * i;
            a_src[i] = A + a_row(q >> 3) * K + (q & 7) * 16;
        }
        const uint8_t* b_src[B_PER];
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int q = tid + kMxThreads * i;
            b_src[i] = B.expert(e, (int64_t)b_rows * (K / 2)) + (int64_t)panel_row(q >> 2, nt) * (K / 2) + (q & 3) * 16;
        }
        const uint8_t* sa_src = As + a_row(tid & (kMxBM - 1)) * kb_row;
        const uint8_t* sb_src = Bs.expert(e, (int64_t)b_rows * kb_row) + (int64_t)panel_row(tid, nt) * kb_row;

        f32x16 acc[MB][NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
        u32x4 ra[2][A_PER], rb[2][B_PER];
        uint32_t rsa[2], rsb[2];

        auto load = [&](u32x4 (&ra_)[A_PER], u32x4 (&rb_)[B_PER], uint32_t& rsa_, uint32_t& rsb_,
                        int ks) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) ra_[i] = *(const u32x4*)(a_src[i] + ks * kMxBK);
#pragma unroll
            for (int i = 0; i < B_PER; ++i) rb_[i] = *(const u32x4*)(b_src[i] + ks * (kMxBK / 2));
            rsb_ = *(const uint32_t*)(sb_src + ks * 4);
            rsa_ = sc.load_scale_word(sa_src + ks * 4);
        };
        auto step = [&](int S, u32x4 (&ra_)[A_PER], u32x4 (&rb_)[B_PER], uint32_t& rsa_,
                        uint32_t& rsb_, int ks) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) {
                const int q = tid + kMxThreads * i, r = q >> 3;
                a_lds[S][r][lds_chunk(r, q & 7)] = ra_[i];
            }
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int q = tid + kMxThreads * i, r = q >> 2;
                b_lds[S][r][lds_chunk4(r, q & 3)] = rb_[i];
            }
            sb_lds[S][tid] = rsb_;
            if (sa_t) sa_lds[S][tid] = rsa_;
            lds_barrier();
            load(ra_, rb_, rsa_, rsb_, min(ks + 2, nks - 1));
            if (active && ks < nks) {
                uint32_t sa[MB], sb[NB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) sa[mb] = sa_lds[S][64 * wm + 32 * mb + (lane & 31)];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) sb[nb] = sb_lds[S][(wn * NB + nb) * 32 + (lane & 31)];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    i32x8 a[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const int ar = 64 * wm + 32 * mb + (lane & 31);
                        const int asw = (ar >> 1) & 7;
                        const u32x4 lo = a_lds[S][ar][(4 * c + h) ^ asw];
                        const u32x4 hi = a_lds[S][ar][(4 * c + 2 + h) ^ asw];
                        a[mb] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                    const int shift = 8 * (2 * c + h);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int br = (wn * NB + nb) * 32 + (lane & 31);
                        const u32x4 bq = b_lds[S][br][lds_chunk4(br, 2 * c + h)];
                        const u32x4 z = {0u, 0u, 0u, 0u};
                        const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(bq, z, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                a[mb], b, acc[mb][nb], 0, 4, 0, (int)(sa[mb] >> shift), 0,
                                (int)(sb[nb] >> shift));
                    }
                }
            }
        };

        load(ra[0], rb[0], rsa[0], rsb[0], 0);
        load(ra[1], rb[1], rsa[1], rsb[1], min(1, nks - 1));
        for (int ks = 0; ks < nks; ks += 2) {
            step(0, ra[0], rb[0], rsa[0], rsb[0], ks);
            step(1, ra[1], rb[1], rsa[1], rsb[1], ks + 1);
        }

        if (SWIGLU) {
            const int nfb = n_out / 32;
            if (active) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int p = 0; p < NB / 2; ++p)
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const float hv = silu_fast(acc[mb][2 * p][q]) * acc[mb][2 * p + 1][q];
                            const float amax = half_max32(fabsf(hv));
                            const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;
                            const int se = max(-127, min(127, ex - 8));
                            const float v = fminf(fmaxf(__builtin_ldexpf(hv, -se), -448.0f), 448.0f);
                            const uint32_t code = f32x4_to_e4m3x4(v, 0.0f, 0.0f, 0.0f);
                            const int row = 64 * wm + 32 * mb + acc_row(q, lane);
                            if (row < mrows) {
                                const int blk = nt * (BN / 64) + wn * (NB / 2) + p;
                                sc.store_u8(Cq + (int64_t)(row0 + row) * n_out + blk * 32 + (lane & 31), (uint8_t)code);
                                if ((lane & 31) == 0) sc.store_u8(Cs + (int64_t)(row0 + row) * nfb + blk, (uint8_t)(se + 127));
                            }
                        }
            }
        } else if (active) {
            const bool odd = lane & 1;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 16; q += 2) {
                    const int row = 64 * wm + 32 * mb + acc_row(q, lane) + (odd ? 1 : 0);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const float y0 = acc[mb][nb][q], y1 = acc[mb][nb][q + 1];
                        const float got = pair_swap(odd ? y0 : y1);
                        const int col = nt * BN + (wn * NB + nb) * 32 + (lane & 30);
                        if (row < mrows) {
                            const uint32_t v = odd ? pack_bf16x2_hw(got, y1) : pack_bf16x2_hw(y0, got);
                            sc.store_u32(Cy + (int64_t)(row0 + row) * n_out + col, v);
                        }
                    }
                }
        }
        lds_barrier();
        sc.stored(it);
    }
    sc.drained();
}

template <bool SWIGLU>
__global__ __launch_bounds__(kMxThreads) void gemm_mx_wide_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const ExpertArray<uint8_t> B,
    const ExpertArray<uint8_t> Bs, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles_p,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ offsets, int E, int K,
    int n_out, int b_rows, int topk, uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cs,
    uint16_t* __restrict__ Cy) {
    PlainSched sc{*ntiles_p * (SWIGLU ? n_out / 256 : n_out / 512)};
    mx_wide_loop<SWIGLU>(A, As, B, Bs, perm, tiles, tile_off, offsets, E, K, n_out, b_rows, topk,
                         Cq, Cs, Cy, sc);
}

// ------------------------------------------------------ one-launch layer
// moe_experts_mxfp4's grouped path for prefill shapes in one persistent
// launch (the hand-offs of moe_layer.h): the routing plan, then the wide
// tiles for both products (gate_up items statically, down items from the
// queue), then the combine.  The FP8 x FP4 precision pair of the DeepGEMM
// "Mega MoE" news item.
__global__ __launch_bounds__(kMxThreads) void layer_mx_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs, const ExpertArray<uint8_t> w13,
    const ExpertArray<uint8_t> w13s, const ExpertArray<uint8_t> w2, const ExpertArray<uint8_t> w2s,
    const int32_t* __restrict__ idx, int32_t* counts, int32_t* offsets, int32_t* perm,
    int32_t* inv, int32_t* tiles, int32_t* ntiles_p, int32_t* tile_off,
    const float* __restrict__ wts, const uint16_t* __restrict__ residual, int64_t T, int E, int H,
    int F, int k, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, uint16_t* __restrict__ y,
    uint16_t* __restrict__ out, LayerSync sy) {
    __shared__ int claim;
    // the routing plan, in the weight ring before its first use
    const uint64_t stamp = layer_plan((int*)&MxWideRing::b()[0][0][0], idx, (int)(T * k), E, kMxBM,
                                      counts, offsets, perm, inv, tiles, ntiles_p, tile_off,
                                      layer_gen(sy), sy);
    if (blockIdx.x == 0 && threadIdx.x < kXcds)   // this call's queues of down items
        st_dev_u64(sy.queue(threadIdx.x), (uint64_t)(uint32_t)stamp << 32);
    const int ntiles = *ntiles_p;
    const int npg = F / 256, npd = H / 512;
    const int NG = ntiles * npg, ND = ntiles * npd;
    LayerSched<true> sg{NG, NG, npg, 0, stamp, sy, tile_off, 0, nullptr, 0};
    mx_wide_loop<true>(x, xs, w13, w13s, perm, tiles, tile_off, offsets, E, H, F, 2 * F, k, hq, hs,
                       nullptr, sg);
    LayerSched<false, true> sd{ND, NG, npg, 0, stamp, sy, tile_off, 0, &claim, 0};
    mx_wide_loop<false>(hq, hs, w2, w2s, perm, tiles, tile_off, offsets, E, F, H, H, 1, nullptr,
                        nullptr, y, sd);
    // the scale ring is idle now: one of its words carries the error state
    layer_combine((int*)&MxWideRing::sb()[0][0], y, inv, wts, residual, T, k, H, out, stamp, sy);
}

// Decode batches (at most 32 rows per expert on average, K a multiple of 256
// for both products): 32-row tiles over 512-row panels, gemm_mx_kernel with
// WM = 1.  A 128-row tile would be mostly padding rows whose staging
// registers here hold twice the weight bytes in flight.
bool mx_use_narrow(int64_t P, int E, int H, int F) {
    return P <= 32 * (int64_t)E && H % 512 == 0 && F % 256 == 0;
}

int mx_tile_m(bool narrow) { return narrow ? 32 : kMxBM; }

template <int BN, bool SWIGLU, int KS, int WM = 4>
static int mx_grid() {
    static const int g = resident_grid((const void*)gemm_mx_kernel<BN, SWIGLU, KS, WM>, kMxThreads,
                                       device_cu_count());
    return capped_grid(g);
}

template <bool SWIGLU>
static int mx_wide_grid() {
    static const int g = resident_grid((const void*)gemm_mx_wide_kernel<SWIGLU>, kMxThreads,
                                       device_cu_count());
    return capped_grid(g);
}

bool mx_use_wide(int64_t P, int E, int H, int F) {
    return P > 64 * (int64_t)E && F % 256 == 0 && H % 512 == 0;
}

hipError_t launch_gateup_mx(const uint8_t* x, const uint8_t* xs, const ExpertArray<uint8_t>& w13,
                            const ExpertArray<uint8_t>& w13s, const GroupedPlan& pl, bool wide, bool narrow, int H,
                            int F, int k, uint8_t* hq, uint8_t* hs, hipStream_t s) {
    if (narrow) {
        MOE_LAUNCH((gemm_mx_kernel<512, true, 2, 1>), dim3(mx_grid<512, true, 2, 1>()), dim3(kMxThreads),
                   0, s, x, xs, w13, w13s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E,
                   H, F, 2 * F, k, hq, hs, (uint16_t*)nullptr);
        return hipGetLastError();
    }
    if (wide) {
        MOE_LAUNCH((gemm_mx_wide_kernel<true>), dim3(mx_wide_grid<true>()), dim3(kMxThreads), 0, s, x,
                   xs, w13, w13s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E, H, F,
                   2 * F, k, hq, hs, (uint16_t*)nullptr);
        return hipGetLastError();
    }
    if (H % 256 == 0)
        MOE_LAUNCH((gemm_mx_kernel<256, true, 2>), dim3(mx_grid<256, true, 2>()), dim3(kMxThreads), 0,
                   s, x, xs, w13, w13s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E,
                   H, F, 2 * F, k, hq, hs, (uint16_t*)nullptr);
    else
        MOE_LAUNCH((gemm_mx_kernel<256, true, 1>), dim3(mx_grid<256, true, 1>()), dim3(kMxThreads), 0,
                   s, x, xs, w13, w13s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E,
                   H, F, 2 * F, k, hq, hs, (uint16_t*)nullptr);
    return hipGetLastError();
}

bool layer_mx_fits(int64_t P, int E, int H, int F) {
    return !mx_use_narrow(P, E, H, F) && mx_use_wide(P, E, H, F);
}

hipError_t launch_layer_mx(const uint8_t* x, const uint8_t* xs, const ExpertArray<uint8_t>& w13,
                           const ExpertArray<uint8_t>& w13s, const ExpertArray<uint8_t>& w2,
                           const ExpertArray<uint8_t>& w2s, const int32_t* idx,
                           const LayerPlan& pl, const float* w, const uint16_t* residual,
                           int64_t T, int H, int F, int E, int k, uint8_t* hq, uint8_t* hs,
                           uint16_t* y, uint16_t* out, void* sync, hipStream_t s) {
    static const int g = std::min(
        resident_grid((const void*)layer_mx_kernel, kMxThreads, device_cu_count()), kLayerMaxGrid);
    MOE_LAUNCH(layer_mx_kernel, dim3(capped_grid(g)), dim3(kMxThreads), 0, s, x, xs, w13, w13s, w2,
               w2s, idx, pl.counts, pl.offsets, pl.perm, pl.inv, pl.tiles, pl.ntiles, pl.tile_off,
               w, residual, T, E, H, F, k, hq, hs, y, out, LayerSync{(uint64_t*)sync});
    return hipGetLastError();
}

hipError_t launch_down_mx(const uint8_t* hq, const uint8_t* hs, const ExpertArray<uint8_t>& w2,
                          const ExpertArray<uint8_t>& w2s, const GroupedPlan& pl, bool wide, bool narrow, int H, int F, uint16_t* y,
                          hipStream_t s) {
    if (narrow)
        MOE_LAUNCH((gemm_mx_kernel<512, false, 2, 1>), dim3(mx_grid<512, false, 2, 1>()),
                   dim3(kMxThreads), 0, s, hq, hs, w2, w2s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off,
                   pl.offsets, pl.E, F, H, H, 1, (uint8_t*)nullptr, (uint8_t*)nullptr, y);
    else if (wide)
        MOE_LAUNCH((gemm_mx_wide_kernel<false>), dim3(mx_wide_grid<false>()), dim3(kMxThreads), 0, s,
                   hq, hs, w2, w2s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E, F,
                   H, H, 1, (uint8_t*)nullptr, (uint8_t*)nullptr, y);
    else if (H % 256 == 0 && F % 256 == 0)
        MOE_LAUNCH((gemm_mx_kernel<256, false, 2>), dim3(mx_grid<256, false, 2>()), dim3(kMxThreads), 0,
                   s, hq, hs, w2, w2s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E, F,
                   H, H, 1, (uint8_t*)nullptr, (uint8_t*)nullptr, y);
    else if (H % 256 == 0)
        MOE_LAUNCH((gemm_mx_kernel<256, false, 1>), dim3(mx_grid<256, false, 1>()), dim3(kMxThreads), 0,
                   s, hq, hs, w2, w2s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E, F,
                   H, H, 1, (uint8_t*)nullptr, (uint8_t*)nullptr, y);
    else
        MOE_LAUNCH((gemm_mx_kernel<128, false, 1>), dim3(mx_grid<128, false, 1>()), dim3(kMxThreads), 0,
                   s, hq, hs, w2, w2s, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E, F,
                   H, H, 1, (uint8_t*)nullptr, (uint8_t*)nullptr, y);
    return hipGetLastError();
}

}  // namespace moe

// moe_gemm_fp8.hip - fp8 block-scaled grouped products of the routed-experts
// layer on gfx950 f8f6f4 MFMA, and the block-128 fp8 quantiser.
//
// Operands follow mirage issue "Supporting MegaKernel for DeepSeek Models",
// Layer Tensor Details: moe_w13_fp8_layer (input [B,H] E4M3 + fp32 scale
// [B,H/128]; weight [E,2F,H] E4M3 + fp32 scale [E,2F,H/128]),
// moe_silu_mul_layer, moe_w2_fp8_layer (input E4M3 + fp32 scale per 128 of F;
// weight [E,H,F] + scale [E,H,F/128]) and bf16_to_fp8_quantize (block 128).
// A 128-wide K block is one MFMA group: two 32x32x64 products into a fresh
// fp32 temporary, then acc += tmp * scale_a[row] * scale_b[col].
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_layer.h"

namespace moe {

constexpr int kFp8Threads = 512;  // 8 waves
constexpr int kFp8BK = 128;       // K bytes per stage == one scale block

// Block-128 quantisation (mirage issue "Supporting MegaKernel for DeepSeek
// Models", bf16_to_fp8_quantize, with moe_w2_fp8_layer's fp32 input scale):
// given the block's max |v| already reduced over its 128 values, this
// thread's (up to) four values become codes RNE_e4m3(clamp(v * (448/amax),
// +-448)) and the block's scale amax/448, all in fp32; an all-zero block
// gets scale 1 and zero codes.  The one routine behind both the SwiGLU
// epilogue of the gate_up product and the stand-alone quantiser.  Returns
// the scale; writes the four codes packed little-endian in *codes.
__device__ __forceinline__ float quant_block_codes(const float v[4], float amax, uint32_t* codes) {
    const bool zero = !(amax > 0.0f);
    const float scale = zero ? 1.0f : amax / 448.0f;
    const float mul = zero ? 0.0f : 448.0f / amax;
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(v[i] * mul, -448.0f), 448.0f);
    if (zero) {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = 0.0f;
    }
    *codes = f32x4_to_e4m3x4(q[0], q[1], q[2], q[3]);
    return scale;
}

// 128 values spread as 4 per lane over one 32-lane half (same row).
__device__ __forceinline__ float quant_block_half(const float v[4], float amax_local, uint32_t* codes) {
    return quant_block_codes(v, half_max32(amax_local), codes);
}

// Same work decomposition and data path as the bf16 products: one work item
// = (M tile of <= BM = 32*WM rows of one expert) x (BN panel rows); waves
// form a WM x WN grid, wave (wm, wn) owns rows [32wm, 32wm+32) and 32*NBW
// panel rows.  A 128-byte K step is one scale block.  The A bytes, the B
// panel and both operands' per-row scales go through an LDS ring (2 stages;
// 8 scale slots under SQ) fed by branch-free look-ahead loads two k-steps
// ahead.  Per block, two
// 32x32x64 MFMAs fill a fresh fp32 temporary that is promoted with
// scale_a[row] * scale_b[col] into the accumulator.
// SWIGLU: panel rows interleave gate/up in blocks of 32 (as the bf16 path);
// one item covers a whole 128-wide h block split over the WN = 2 column
// waves, which exchange per-row partial maxima through LDS before the
// block-128 re-quantisation.  Otherwise: y bf16 in expert order (row m of
// the plan holds slot perm[m]).
// SQ (K a multiple of 512): each thread reads its row's scales for four
// K blocks with one 16-byte load every fourth step into an 8-slot LDS ring.
// A scale read touches one cache line per row, against one line per eight
// lanes for the operand bytes, so one 4-byte read per step doubled the
// cache-line requests of a stage; SQ cuts that to a quarter.
// The LDS arrays of one tile shape: separate variables (each with its own
// base, so fragment reads keep constant offsets), the same ones for the
// gate_up and the down loop of a one-launch layer, which run one after the
// other.  SR: scale ring slots.
template <int WM, int BN, bool SQ>
struct Fp8Ring {
    static constexpr int BM = 32 * WM, SR = SQ ? 8 : 2;
    __device__ static u32x4 (&a())[2][BM][8] {
        __shared__ u32x4 v[2][BM][8];
        return v;
    }
    __device__ static u32x4 (&b())[2][BN][8] {
        __shared__ u32x4 v[2][BN][8];
        return v;
    }
    __device__ static float (&sa())[SR][BM] {
        __shared__ __attribute__((aligned(16))) float v[SR][BM];
        return v;
    }
    __device__ static float (&sb())[SR][BN] {
        __shared__ float v[SR][BN];
        return v;
    }
    // per-row partial maxima of the SwiGLU epilogue
    __device__ static float (&amax())[8 / WM][BM] {
        __shared__ float v[8 / WM][BM];
        return v;
    }
};

// The persistent item loop, with the scheduling hooks of moe_layer.h.
template <int WM, int BN, bool SWIGLU, bool SQ, class Sched>
__device__ __forceinline__ void fp8_loop(
    const uint8_t* __restrict__ A, const float* __restrict__ As,
    const ExpertArray<uint8_t>& B, const ExpertArray<float>& Bs, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ offsets, int E, int K, int n_out, int b_rows, int topk,
    uint8_t* __restrict__ Cq, float* __restrict__ Cs, uint16_t* __restrict__ Cy, Sched& sc) {
    constexpr int WN = 8 / WM;
    constexpr int BM = 32 * WM;
    constexpr int NBW = BN / (32 * WN);
    // 16-byte A chunks per thread and stage; a 32-row tile has 256 chunks for
    // 512 threads, so threads 256..511 repeat those of threads 0..255 (same
    // source, same LDS slot, same value)
    constexpr int A_PER = BM * 8 >= kFp8Threads ? BM * 8 / kFp8Threads : 1;
    constexpr int B_PER = BN * 8 / kFp8Threads;
    // SwiGLU: each wave holds PP (gate, up) block pairs = 32 PP h columns; a
    // 128-wide h block (one E4M3 scale) spans WB = 4 / PP waves
    constexpr int PP = NBW / 2;
    constexpr int WB = PP > 0 ? 4 / PP : 1;
    static_assert(WM * WN == 8 && NBW >= 1 && B_PER >= 1 && (BM * 8) % 256 == 0, "bad tile shape");
    static_assert(BM <= kFp8Threads && BN <= kFp8Threads, "one scale per thread");
    static_assert(!SWIGLU || (NBW % 2 == 0 && 4 % PP == 0 && WN % WB == 0),
                  "the SwiGLU epilogue needs whole gate/up pairs and whole 128-wide h blocks");
    using Ring = Fp8Ring<WM, BN, SQ>;
    auto& a_lds = Ring::a();
    auto& b_lds = Ring::b();
    auto& sa_lds = Ring::sa();
    auto& sb_lds = Ring::sb();

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    // waves w and w + 4 share a SIMD; they take turns at the higher issue
    // priority, one K step each, so that the promotion ALU work of one
    // overlaps the matrix products of the other instead of running in step
    // with them (fp8 prefill gate_up 1837 -> 1760 us on the Zipf T=4096 shape)
    const int wave_pair = __builtin_amdgcn_readfirstlane(wave) >> 2;
    const int chunk = tid & 7, row_t = tid >> 3;
    const int a_row_t = row_t & (BM - 1);   // BM = 32: rows 32..63 repeat rows 0..31
    const int g = lane >> 5;
    const int fsw = (lane >> 1) & 7;  // lds_chunk swizzle of fragment rows 32*b + lane%32
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int nkb = K / kFp8BK;

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
        const int nt = gi.nt, mt = gi.mt, e = gi.e;
        const int row0 = tiles[2 * mt + 1];
        const int mrows = min(BM, offsets[e + 1] - row0);
        const bool active = 32 * wm < mrows;

        // A rows (and A scale rows) past the tile's end read token row 0 or
        // the tile's first row
        const uint8_t* a_src[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int r = a_row_t + 64 * i;
            int64_t arow = SWIGLU ? 0 : row0;
            if (r < mrows) arow = SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
            a_src[i] = A + arow * K + chunk * 16;
        }
        const bool sa_ok = tid < BM, sb_ok = tid < BN;
        int64_t sarow = SWIGLU ? 0 : row0;
        if (sa_ok && tid < mrows)
            sarow = SWIGLU ? (int64_t)(perm[row0 + tid] / topk) : (int64_t)(row0 + tid);
        const float* as_src = As + sarow * nkb;
        const uint8_t* b_src = B.expert(e, (int64_t)b_rows * K) + (int64_t)panel_row(row_t, nt) * K + chunk * 16;
        const int64_t b_step = (int64_t)(SWIGLU ? 32 : 64) * K;
        const float* bs_src = Bs.expert(e, (int64_t)b_rows * nkb) + (int64_t)panel_row(sb_ok ? tid : 0, nt) * nkb;

        f32x16 acc[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb] = f32x16{};
        u32x4 ra0[A_PER], ra1[A_PER], rb0[B_PER], rb1[B_PER];
        float rsa0, rsa1, rsb0, rsb1;  // !SQ: the scales of one step
        float4 qa, qb;                 // SQ: the scales of four steps

#define MOE_FP8_LOAD(RA, RB, KB)                                                               \
    do {                                                                                       \
        _Pragma("unroll") for (int i = 0; i < A_PER; ++i) RA[i] =                              \
            *(const u32x4*)(a_src[i] + (KB) * kFp8BK);                                         \
        /* decode batches (WM == 1) read each weight panel once: non-temporal, */         \
        /* so that the stream does not push the scale rows out of L2 */                   \
        _Pragma("unroll") for (int i = 0; i < B_PER; ++i) {                                    \
            const u32x4* src_ = (const u32x4*)(b_src + i * b_step + (KB) * kFp8BK);            \
            if constexpr (WM == 1) RB[i] = __builtin_nontemporal_load(src_);                   \
            else RB[i] = *src_;                                                                \
        }                                                                                      \
    } while (0)

    /* J = KB % 4 (SQ); the scales of step KB sit in ring slot SS */                          \
#define MOE_FP8_STEP(S, J, RA, RB, RSA, RSB, KB)                                               \
    do {                                                                                       \
        _Pragma("unroll") for (int i = 0; i < A_PER; ++i) {                                    \
            const int rr = a_row_t + 64 * i;                                                   \
            a_lds[S][rr][lds_chunk(rr, chunk)] = RA[i];                                        \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < B_PER; ++i) {                                    \
            const int rr = row_t + 64 * i;                                                     \
            b_lds[S][rr][lds_chunk(rr, chunk)] = RB[i];                                        \
        }                                                                                      \
        const int SS = SQ ? ((KB) & 7) : S;                                                    \
        if constexpr (!SQ) {                                                                   \
            if (sa_ok) sa_lds[S][tid] = RSA;                                                   \
            if (sb_ok) sb_lds[S][tid] = RSB;                                                   \
        } else if constexpr (J == 0) {                                                         \
            if (sa_ok) {                                                                       \
                sa_lds[SS][tid] = qa.x; sa_lds[SS + 1][tid] = qa.y;                            \
                sa_lds[SS + 2][tid] = qa.z; sa_lds[SS + 3][tid] = qa.w;                        \
            }                                                                                  \
            if (sb_ok) {                                                                       \
                sb_lds[SS][tid] = qb.x; sb_lds[SS + 1][tid] = qb.y;                            \
                sb_lds[SS + 2][tid] = qb.z; sb_lds[SS + 3][tid] = qb.w;                        \
            }                                                                                  \
        }                                                                                      \
        lds_barrier(); /* LDS only: the next steps' loads stay in flight */                    \
        if (((KB) ^ wave_pair) & 1) __builtin_amdgcn_s_setprio(2);                             \
        else __builtin_amdgcn_s_setprio(0);                                                    \
        if (active && (KB) < nkb) {                                                            \
            const int ar = 32 * wm + (lane & 31);                                              \
            const i32x8 a0 = __builtin_bit_cast(i32x8, __builtin_shufflevector(                \
                a_lds[S][ar][(2 * g) ^ fsw], a_lds[S][ar][(2 * g + 1) ^ fsw],                   \
                0, 1, 2, 3, 4, 5, 6, 7));                                                      \
            const i32x8 a1 = __builtin_bit_cast(i32x8, __builtin_shufflevector(                \
                a_lds[S][ar][(4 + 2 * g) ^ fsw], a_lds[S][ar][(4 + 2 * g + 1) ^ fsw],           \
                0, 1, 2, 3, 4, 5, 6, 7));                                                      \
            float sa[16]; /* A scale of each accumulator row of this lane */                   \
            _Pragma("unroll") for (int qq = 0; qq < 4; ++qq) {                                 \
                const float4 v = *(const float4*)&sa_lds[SS][32 * wm + 8 * qq + 4 * g];         \
                sa[4 * qq] = v.x; sa[4 * qq + 1] = v.y; sa[4 * qq + 2] = v.z; sa[4 * qq + 3] = v.w; \
            }                                                                                  \
            _Pragma("unroll") for (int nb = 0; nb < NBW; ++nb) {                               \
                const int brow = (wn * NBW + nb) * 32 + (lane & 31);                           \
                const i32x8 b0 = __builtin_bit_cast(i32x8, __builtin_shufflevector(            \
                    b_lds[S][brow][(2 * g) ^ fsw], b_lds[S][brow][(2 * g + 1) ^ fsw],           \
                    0, 1, 2, 3, 4, 5, 6, 7));                                                  \
                const i32x8 b1 = __builtin_bit_cast(i32x8, __builtin_shufflevector(            \
                    b_lds[S][brow][(4 + 2 * g) ^ fsw], b_lds[S][brow][(4 + 2 * g + 1) ^ fsw],   \
                    0, 1, 2, 3, 4, 5, 6, 7));                                                  \
                f32x16 tmp = mfma_fp8_32x32x64(a0, b0, f32x16{});                              \
                tmp = mfma_fp8_32x32x64(a1, b1, tmp);                                          \
                const float sbv = sb_lds[SS][brow];                                            \
                _Pragma("unroll") for (int q = 0; q < 16; ++q) acc[nb][q] +=                   \
                    tmp[q] * (sa[q] * sbv);                                                    \
            }                                                                                  \
        }                                                                                      \
        MOE_FP8_LOAD(RA, RB, min((KB) + 2, nkb - 1));                                          \
        if constexpr (!SQ) {                                                                   \
            RSA = sc.load_scale(as_src + min((KB) + 2, nkb - 1));                              \
            RSB = bs_src[min((KB) + 2, nkb - 1)];                                              \
        } else if constexpr (J == 0) {                                                         \
            qa = sc.load_scale4(as_src + min((KB) + 4, nkb - 4));                              \
            qb = *(const float4*)(bs_src + min((KB) + 4, nkb - 4));                            \
        }                                                                                      \
    } while (0)

        // prologue loads in the loop's own issue order, so that the waits the
        // compiler derives at the loop head hold the look-ahead loads in flight
        if constexpr (SQ) {
            qa = sc.load_scale4(as_src);
            qb = *(const float4*)bs_src;
            MOE_FP8_LOAD(ra0, rb0, 0);
            MOE_FP8_LOAD(ra1, rb1, min(1, nkb - 1));
            for (int kb = 0; kb < nkb; kb += 4) {
                MOE_FP8_STEP(0, 0, ra0, rb0, rsa0, rsb0, kb);
                MOE_FP8_STEP(1, 1, ra1, rb1, rsa1, rsb1, kb + 1);
                MOE_FP8_STEP(0, 2, ra0, rb0, rsa0, rsb0, kb + 2);
                MOE_FP8_STEP(1, 3, ra1, rb1, rsa1, rsb1, kb + 3);
            }
        } else {
            MOE_FP8_LOAD(ra0, rb0, 0);
            rsa0 = sc.load_scale(as_src);
            rsb0 = bs_src[0];
            MOE_FP8_LOAD(ra1, rb1, min(1, nkb - 1));
            rsa1 = sc.load_scale(as_src + min(1, nkb - 1));
            rsb1 = bs_src[min(1, nkb - 1)];
            for (int kb = 0; kb < nkb; kb += 2) {
                MOE_FP8_STEP(0, 0, ra0, rb0, rsa0, rsb0, kb);
                MOE_FP8_STEP(1, 0, ra1, rb1, rsa1, rsb1, kb + 1);
            }
        }
#undef MOE_FP8_STEP
#undef MOE_FP8_LOAD
        __builtin_amdgcn_s_setprio(0);

        if (SWIGLU) {
            // h for f = nt*(BN/2) + (wn*PP + p)*32 + lane%32, p < PP; wave wn's
            // 128-wide h block is shared with the waves wb0 .. wb0 + WB - 1
            float hv[PP > 0 ? PP : 1][16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float m = 0.0f;
#pragma unroll
                for (int p = 0; p < PP; ++p) {
                    hv[p][q] = silu(acc[2 * p][q]) * acc[2 * p + 1][q];
                    m = fmaxf(m, fabsf(hv[p][q]));
                }
                m = half_max32(m);
                if ((lane & 31) == 0) Ring::amax()[wn][32 * wm + acc_row(q, lane)] = m;
            }
            lds_barrier();
            if (active) {
                const int nfb = n_out / 128;
                const int wb0 = wn - wn % WB;
                const int hblk = nt * (BN / 256) + wn / WB;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = 32 * wm + acc_row(q, lane);
                    float amax = Ring::amax()[wb0][row];
#pragma unroll
                    for (int j = 1; j < WB; ++j) amax = fmaxf(amax, Ring::amax()[wb0 + j][row]);
                    float vv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int p = 0; p < PP; ++p) vv[p] = hv[p][q];
                    uint32_t codes;
                    const float scale = quant_block_codes(vv, amax, &codes);
                    if (row < mrows) {
                        uint8_t* dst = Cq + (int64_t)(row0 + row) * n_out + nt * (BN / 2) + wn * PP * 32 + (lane & 31);
#pragma unroll
                        for (int p = 0; p < PP; ++p) sc.store_u8(dst + 32 * p, (uint8_t)(codes >> (8 * p)));
                        if (wn % WB == 0 && (lane & 31) == 0) sc.store_f32(Cs + (int64_t)(row0 + row) * nfb + hblk, scale);
                    }
                }
            }
        } else if (active) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * wm + acc_row(q, lane);
                if (row < mrows) {
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        const int col = nt * BN + (wn * NBW + nb) * 32 + (lane & 31);
                        sc.store_u16(Cy + (int64_t)(row0 + row) * n_out + col, (uint16_t)f32_to_bf16(acc[nb][q]));
                    }
                }
            }
        }
        lds_barrier();  // LDS (operand rings, amax) is reused by the next item
        sc.stored(it);
    }
    sc.drained();
}

template <int WM, int BN, bool SWIGLU, bool SQ>
__global__ __launch_bounds__(kFp8Threads) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const ExpertArray<uint8_t> B,
    const ExpertArray<float> Bs, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles_p,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ offsets, int E, int K,
    int n_out, int b_rows, int topk, uint8_t* __restrict__ Cq, float* __restrict__ Cs,
    uint16_t* __restrict__ Cy) {
    PlainSched sc{*ntiles_p * (SWIGLU ? n_out / (BN / 2) : n_out / BN)};
    fp8_loop<WM, BN, SWIGLU, SQ>(A, As, B, Bs, perm, tiles, tile_off, offsets, E, K, n_out, b_rows,
                                 topk, Cq, Cs, Cy, sc);
}

constexpr int kFp8WM = 4;  // 4 x 2 waves: 128-row M tiles
constexpr int kFp8TileM = 32 * kFp8WM;
// Decode batches (at most 32 rows per expert on average): 32-row M tiles and
// 512-row panels on 1 x 8 waves (32 x 64 each, one gate/up pair).  A 128-row
// tile would be mostly padding, and its accumulators would hold the registers
// that here stage twice the weight bytes per stage (two stages of 64 KB in
// flight per CU instead of 32 KB), which the weight stream is bound by.
constexpr int kFp8NarrowTileM = 32;

bool fp8_use_narrow(int64_t P, int E, int H, int F) {
    return P <= 32 * (int64_t)E && F % 256 == 0 && H % 512 == 0;
}

int fp8_tile_m(bool narrow) { return narrow ? kFp8NarrowTileM : kFp8TileM; }

template <int WM, int BN, bool SWIGLU, bool SQ>
static int fp8_grid() {
    static const int g = resident_grid((const void*)gemm_fp8_kernel<WM, BN, SWIGLU, SQ>,
                                       kFp8Threads, device_cu_count());
    return capped_grid(g);
}

// SQ (16-byte scale loads) needs K / 128 to be a multiple of 4
template <int WM, int BN, bool SWIGLU>
static void launch_fp8(const uint8_t* A, const float* As, const ExpertArray<uint8_t>& B,
                       const ExpertArray<float>& Bs,
                       const GroupedPlan& pl, int K, int n_out, int b_rows, int topk, uint8_t* Cq,
                       float* Cs, uint16_t* Cy, hipStream_t s) {
    if ((K / kFp8BK) % 4 == 0)
        MOE_LAUNCH((gemm_fp8_kernel<WM, BN, SWIGLU, true>), dim3(fp8_grid<WM, BN, SWIGLU, true>()),
                   dim3(kFp8Threads), 0, s, A, As, B, Bs, pl.perm, pl.tiles, pl.ntiles,
                   pl.tile_off, pl.offsets, pl.E, K, n_out, b_rows, topk, Cq, Cs, Cy);
    else
        MOE_LAUNCH((gemm_fp8_kernel<WM, BN, SWIGLU, false>), dim3(fp8_grid<WM, BN, SWIGLU, false>()),
                   dim3(kFp8Threads), 0, s, A, As, B, Bs, pl.perm, pl.tiles, pl.ntiles,
                   pl.tile_off, pl.offsets, pl.E, K, n_out, b_rows, topk, Cq, Cs, Cy);
}

hipError_t launch_gateup_fp8(const uint8_t* x, const float* xs, const ExpertArray<uint8_t>& w13,
                             const ExpertArray<float>& w13s, const GroupedPlan& pl, bool narrow, int H, int F,
                             int k, uint8_t* hq, float* hs, hipStream_t s) {
    if (narrow)
        launch_fp8<1, 512, true>(x, xs, w13, w13s, pl, H, F, 2 * F, k, hq, hs, nullptr, s);
    else
        launch_fp8<kFp8WM, 256, true>(x, xs, w13, w13s, pl, H, F, 2 * F, k, hq, hs, nullptr, s);
    return hipGetLastError();
}

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const ExpertArray<uint8_t>& w2,
                           const ExpertArray<float>& w2s, const GroupedPlan& pl, bool narrow, int H, int F, uint16_t* y,
                           hipStream_t s) {
    if (narrow)
        launch_fp8<1, 512, false>(hq, hs, w2, w2s, pl, F, H, H, 1, nullptr, nullptr, y, s);
    else if (H % 256 == 0)
        launch_fp8<kFp8WM, 256, false>(hq, hs, w2, w2s, pl, F, H, H, 1, nullptr, nullptr, y, s);
    else
        launch_fp8<kFp8WM, 128, false>(hq, hs, w2, w2s, pl, F, H, H, 1, nullptr, nullptr, y, s);
    return hipGetLastError();
}

// ------------------------------------------------------ one-launch layer
// moe_experts_fp8's grouped path in one persistent launch after the plan
// (the hand-offs of moe_layer.h): 128-row M tiles x 256-row panels for both
// products, whose 16-byte scale rings share one set of LDS arrays.
__global__ __launch_bounds__(kFp8Threads) void layer_fp8_kernel(
    const uint8_t* __restrict__ x, const float* __restrict__ xs, const ExpertArray<uint8_t> w13,
    const ExpertArray<float> w13s, const ExpertArray<uint8_t> w2, const ExpertArray<float> w2s,
    const int32_t* __restrict__ idx, int32_t* counts, int32_t* offsets, int32_t* perm,
    int32_t* inv, int32_t* tiles, int32_t* ntiles_p, int32_t* tile_off,
    const float* __restrict__ wts, const uint16_t* __restrict__ residual, int64_t T, int E, int H,
    int F, int k, uint8_t* __restrict__ hq, float* __restrict__ hs, uint16_t* __restrict__ y,
    uint16_t* __restrict__ out, LayerSync sy) {
    __shared__ int claim;
    // the routing plan, in the weight ring before its first use
    const uint64_t stamp =
        layer_plan((int*)&Fp8Ring<kFp8WM, 256, true>::b()[0][0][0], idx, (int)(T * k), E, kFp8TileM,
                   counts, offsets, perm, inv, tiles, ntiles_p, tile_off, layer_gen(sy), sy);
    if (blockIdx.x == 0 && threadIdx.x < kXcds)   // this call's queues of down items
        st_dev_u64(sy.queue(threadIdx.x), (uint64_t)(uint32_t)stamp << 32);
    const int ntiles = *ntiles_p;
    const int npg = F / 128, npd = H / 256;
    const int NG = ntiles * npg, ND = ntiles * npd;
    LayerSched<true> sg{NG, NG, npg, 0, stamp, sy, tile_off, 0, nullptr, 0};
    fp8_loop<kFp8WM, 256, true, true>(x, xs, w13, w13s, perm, tiles, tile_off, offsets, E, H, F,
                                       2 * F, k, hq, hs, nullptr, sg);
    // down items from the queue: many per workgroup, of uneven lengths
    LayerSched<false, true> sd{ND, NG, npg, 0, stamp, sy, tile_off, 0, &claim, 0};
    fp8_loop<kFp8WM, 256, false, true>(hq, hs, w2, w2s, perm, tiles, tile_off, offsets, E, F, H,
                                        H, 1, nullptr, nullptr, y, sd);
    // the scale ring is idle now: one of its words carries the error state
    layer_combine((int*)&Fp8Ring<kFp8WM, 256, true>::sb()[0][0], y, inv, wts, residual, T, k, H,
                  out, stamp, sy);
}

// Prefill shapes whose K blocks come four per scale load in both products.
bool layer_fp8_fits(int64_t P, int E, int H, int F) {
    return !fp8_use_narrow(P, E, H, F) && H % 512 == 0 && F % 512 == 0;
}

hipError_t launch_layer_fp8(const uint8_t* x, const float* xs, const ExpertArray<uint8_t>& w13,
                            const ExpertArray<float>& w13s, const ExpertArray<uint8_t>& w2,
                            const ExpertArray<float>& w2s, const int32_t* idx,
                            const LayerPlan& pl, const float* w, const uint16_t* residual,
                            int64_t T, int H, int F, int E, int k, uint8_t* hq, float* hs,
                            uint16_t* y, uint16_t* out, void* sync, hipStream_t s) {
    static const int g = std::min(
        resident_grid((const void*)layer_fp8_kernel, kFp8Threads, device_cu_count()), kLayerMaxGrid);
    MOE_LAUNCH(layer_fp8_kernel, dim3(capped_grid(g)), dim3(kFp8Threads), 0, s, x, xs, w13, w13s,
               w2, w2s, idx, pl.counts, pl.offsets, pl.perm, pl.inv, pl.tiles, pl.ntiles,
               pl.tile_off, w, residual, T, E, H, F, k, hq, hs, y, out,
               LayerSync{(uint64_t*)sync});
    return hipGetLastError();
}

// ------------------------------------------------------- stand-alone quantiser
// Block-128 quantisation with a power-of-two scale (mirage issue "Supporting
// MegaKernel for DeepSeek Models", bf16_to_fp8_quantize: "FP8 E4M3 + scale
// ue8m0", block 128).  The page gives no rule; the one taken: e is the
// smallest integer with amax <= 448 * 2^e, clamped to [-127, 127]; codes are
// RNE_e4m3(clamp(v * 2^-e, +-448)) (v * 2^-e is exact, so the e4m3 rounding
// is the only one) and the scale byte is e + 127.  An all-zero block gets
// byte 127 (scale 1) and zero codes.  With amax = m * 2^E, m in [1, 2):
// 448 = 1.75 * 2^8, so e = E - 8 when m <= 1.75 and E - 7 otherwise.
__device__ __forceinline__ uint8_t quant_block_ue8m0(const float v[4], float amax, uint32_t* codes) {
    int e = 0;
    if (amax > 0.0f) {
        int x;
        const float f = frexpf(amax, &x);   // amax = f * 2^x, f in [0.5, 1)
        e = (x - 1) - 8 + (2.0f * f > 1.75f ? 1 : 0);
        e = min(max(e, -127), 127);
    }
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(ldexpf(v[i], -e), -448.0f), 448.0f);
    *codes = f32x4_to_e4m3x4(q[0], q[1], q[2], q[3]);
    return (uint8_t)(e + 127);
}

// One 32-lane half per 128-value block: lane i of the half takes values
// i, i+32, i+64, i+96 (the same spread as the epilogue's accumulators).
// UE8M0: power-of-two scale bytes instead of fp32 scales.
template <bool UE8M0>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ in, int in_is_bf16,
                                                       int64_t nblocks, int K,
                                                       uint8_t* __restrict__ codes,
                                                       void* __restrict__ scales) {
    const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
    const int l = threadIdx.x & 31;
    const bool live = blk < nblocks;
    const int64_t b = live ? blk : 0;
    const int nkb = K / 128;
    const int64_t row = b / nkb;
    const int kb = (int)(b - row * nkb);
    const int64_t base = row * K + kb * 128;
    float v[4];
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t i = base + p * 32 + l;
        v[p] = in_is_bf16 ? bf16_to_f32(((const uint16_t*)in)[i]) : ((const float*)in)[i];
        amax = fmaxf(amax, fabsf(v[p]));
    }
    uint32_t c;
    if constexpr (UE8M0) {
        const uint8_t sb = quant_block_ue8m0(v, half_max32(amax), &c);
        if (live && l == 0) ((uint8_t*)scales)[b] = sb;
    } else {
        const float scale = quant_block_half(v, amax, &c);
        if (live && l == 0) ((float*)scales)[b] = scale;
    }
    if (live) {
#pragma unroll
        for (int p = 0; p < 4; ++p) codes[base + p * 32 + l] = (uint8_t)(c >> (8 * p));
    }
}

hipError_t launch_quantize_fp8(const void* in, int in_is_bf16, int64_t rows, int K, uint8_t* codes,
                               void* scales, bool ue8m0, hipStream_t s) {
    const int64_t nblocks = rows * (K / 128);
    const int64_t threads = nblocks * 32;
    const int blocks = (int)((threads + 255) / 256);
    if (ue8m0)
        MOE_LAUNCH(quantize_kernel<true>, dim3(blocks), dim3(256), 0, s, in, in_is_bf16, nblocks, K,
                   codes, scales);
    else
        MOE_LAUNCH(quantize_kernel<false>, dim3(blocks), dim3(256), 0, s, in, in_is_bf16, nblocks, K,
                   codes, scales);
    return hipGetLastError();
}

}  // namespace moe

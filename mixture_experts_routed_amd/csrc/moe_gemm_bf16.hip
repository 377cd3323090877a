// moe_gemm_bf16.hip - grouped bf16 products of the routed-experts layer on
// gfx950 MFMA, and the router-weighted combine.
//
// Model card "DeepSeek-OCR-2 MoE experts": the prefill op is a grouped GEMM
// over experts with a plain SiLU SwiGLU between the two products, then a
// router-weighted scatter-add; "Usage" fixes gate_up_proj [E,2F,H] and
// down_proj [E,H,F] (both K-contiguous, so C = A * B^T with both operands
// K-major, the layout MFMA wants).  The combine follows mirage issue
// "Supporting MegaKernel for DeepSeek Models", moe_local_reduction, without
// its residual, done as a gather in slot order (no float atomics).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kGemmThreads = 512;  // 8 waves
constexpr int kBK = 64;            // bf16 K elements per stage (128 bytes per row)

// One work item = (M tile of <= BM = 32*WM rows of one expert) x (BN rows of
// the expert's weight panel).  Waves form a WM x WN grid; wave (wm, wn) owns
// rows [32wm, 32wm+32) and 32*NBW panel rows.  Both operands go through a
// 2-stage LDS ring: every thread moves whole 16-byte chunks with 8 lanes per
// 128-byte row segment (coalesced global reads), chunks XOR-swizzled for the
// 64-bank LDS; the MFMA fragments are then read from LDS.  Loads run NREG
// k-steps ahead in NREG register stages (named arrays with constant
// indices, no branch around any load, so the compiler waits for exactly the
// stage it consumes).  Rows past an M tile's end load row 0 (valid memory) and their
// outputs are never stored.
// SWIGLU: panel rows are interleaved in blocks of 32 as gate, up, gate, up,
// ... so each wave holds matching gate/up accumulators lane for lane, and the
// epilogue writes h = silu(gate) * up as bf16 [P, F] in expert order.
// Otherwise the epilogue writes y[slot, col] bf16 with slot = perm[row].
template <int WM, int BN, bool SWIGLU, int NREG>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ offsets, int E, int K, int n_out, int b_rows, int topk,
    uint16_t* __restrict__ C) {
    constexpr int WN = 8 / WM;
    constexpr int BM = 32 * WM;
    constexpr int NBW = BN / (32 * WN);  // 32-wide accumulator blocks per wave
    constexpr int A_PER = BM * 8 / kGemmThreads;
    constexpr int B_PER = BN * 8 / kGemmThreads;
    static_assert(WM * WN == 8 && NBW >= 1 && A_PER >= 1 && B_PER >= 1, "bad tile shape");
    static_assert(!SWIGLU || NBW % 2 == 0, "SwiGLU needs gate/up block pairs per wave");
    static_assert(NREG == 2 || NREG == 3, "two or three register stages");
    __shared__ u32x4 a_lds[2][BM][8];
    __shared__ u32x4 b_lds[2][BN][8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int chunk = tid & 7, row_t = tid >> 3;
    const int ntiles = *ntiles_p;
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int items = ntiles * n_tiles_n;
    const int nks = K / kBK;
    const int fsw = (lane >> 1) & 7;  // lds_chunk swizzle of fragment rows 32*b + lane%32

    for (int it = xcd_slot(blockIdx.x, gridDim.x); it < items; it += gridDim.x) {
        const GroupedItem gi = grouped_item(it, tile_off, E, n_tiles_n);
        const int nt = gi.nt, mt = gi.mt, e = gi.e;
        const int row0 = tiles[2 * mt + 1];
        const int mrows = min(BM, offsets[e + 1] - row0);
        const bool active = 32 * wm < mrows;

        const uint16_t* a_src[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int r = row_t + 64 * i;
            int64_t arow = 0;
            if (r < mrows) arow = SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
            a_src[i] = A + arow * K + chunk * 8;
        }
        // thread rows row_t + 64 i of the panel: 64 panel rows are 32 weight
        // rows apart when gate/up interleave in blocks of 32, else 64
        int brow0;
        if (SWIGLU) {
            const int blk = row_t >> 5;
            brow0 = ((blk & 1) ? n_out : 0) + nt * (BN / 2) + (blk >> 1) * 32 + (row_t & 31);
        } else {
            brow0 = nt * BN + row_t;
        }
        const uint16_t* b_src = B + ((int64_t)e * b_rows + brow0) * K + chunk * 8;
        const int64_t b_step = (int64_t)(SWIGLU ? 32 : 64) * K;

        f32x16 acc[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb] = f32x16{};
        u32x4 ra0[A_PER], ra1[A_PER], ra2[A_PER], rb0[B_PER], rb1[B_PER], rb2[B_PER];

#define MOE_BF16_LOAD(RA, RB, KS)                                                             \
    do {                                                                                      \
        _Pragma("unroll") for (int i = 0; i < A_PER; ++i) RA[i] =                             \
            *(const u32x4*)(a_src[i] + (KS) * kBK);                                           \
        _Pragma("unroll") for (int i = 0; i < B_PER; ++i) RB[i] =                             \
            *(const u32x4*)(b_src + i * b_step + (KS) * kBK);                                 \
    } while (0)

#define MOE_BF16_STEP(S, RA, RB, KS)                                                          \
    do {                                                                                      \
        _Pragma("unroll") for (int i = 0; i < A_PER; ++i) {                                   \
            const int rr = row_t + 64 * i;                                                    \
            a_lds[S][rr][lds_chunk(rr, chunk)] = RA[i];                                       \
        }                                                                                     \
        _Pragma("unroll") for (int i = 0; i < B_PER; ++i) {                                   \
            const int rr = row_t + 64 * i;                                                    \
            b_lds[S][rr][lds_chunk(rr, chunk)] = RB[i];                                       \
        }                                                                                     \
        __syncthreads();                                                                      \
        if (active && (KS) < nks) {                                                           \
            _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                \
                const int c = (kk * 2 + (lane >> 5)) ^ fsw;                                   \
                const u32x4 af = a_lds[S][32 * wm + (lane & 31)][c];                          \
                u32x4 bf[NBW];                                                                \
                _Pragma("unroll") for (int nb = 0; nb < NBW; ++nb) bf[nb] =                   \
                    b_lds[S][(wn * NBW + nb) * 32 + (lane & 31)][c];                          \
                _Pragma("unroll") for (int nb = 0; nb < NBW; ++nb) acc[nb] =                  \
                    mfma_bf16_32x32x16(af, bf[nb], acc[nb]);                                  \
            }                                                                                 \
        }                                                                                     \
        MOE_BF16_LOAD(RA, RB, min((KS) + NREG, nks - 1));                                     \
    } while (0)

        // NREG register stages (loads run NREG k-steps ahead) over a two-stage
        // LDS ring: LDS stage ks % 2, register stage ks % NREG
        MOE_BF16_LOAD(ra0, rb0, 0);
        MOE_BF16_LOAD(ra1, rb1, min(1, nks - 1));
        if constexpr (NREG == 2) {
            for (int ks = 0; ks < nks; ks += 2) {
                MOE_BF16_STEP(0, ra0, rb0, ks);
                MOE_BF16_STEP(1, ra1, rb1, ks + 1);
            }
        } else {
            MOE_BF16_LOAD(ra2, rb2, min(2, nks - 1));
            for (int ks = 0; ks < nks; ks += 6) {
                MOE_BF16_STEP(0, ra0, rb0, ks);
                MOE_BF16_STEP(1, ra1, rb1, ks + 1);
                if (ks + 2 >= nks) break;
                MOE_BF16_STEP(0, ra2, rb2, ks + 2);
                MOE_BF16_STEP(1, ra0, rb0, ks + 3);
                if (ks + 4 >= nks) break;
                MOE_BF16_STEP(0, ra1, rb1, ks + 4);
                MOE_BF16_STEP(1, ra2, rb2, ks + 5);
            }
        }
#undef MOE_BF16_STEP
#undef MOE_BF16_LOAD
        __syncthreads();  // the next item's first LDS write must not overtake these reads

        if (active) {
            if (SWIGLU) {
#pragma unroll
                for (int p = 0; p < NBW / 2; ++p) {
                    const int f = nt * (BN / 2) + (wn * NBW / 2 + p) * 32 + (lane & 31);
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int row = 32 * wm + acc_row(q, lane);
                        if (row < mrows) {
                            const float hv = silu(acc[2 * p][q]) * acc[2 * p + 1][q];
                            C[(int64_t)(row0 + row) * n_out + f] = (uint16_t)f32_to_bf16(hv);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = 32 * wm + acc_row(q, lane);
                    if (row < mrows) {
                        const int64_t slot = perm[row0 + row];
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) {
                            const int col = nt * BN + (wn * NBW + nb) * 32 + (lane & 31);
                            C[slot * n_out + col] = (uint16_t)f32_to_bf16(acc[nb][q]);
                        }
                    }
                }
            }
        }
    }
}

// Tile shape of the bf16 products: 128-row M tiles (4 x 2 waves), 256 panel
// rows per item (halves the token-row re-reads per flop compared with 128),
// three register stages; one workgroup per CU (96 KB of LDS).
constexpr int kBf16WM = 4;
constexpr int kBf16TileM = 32 * kBf16WM;
constexpr int kBf16NReg = 3;

int bf16_tile_m() { return kBf16TileM; }

template <int WM, int BN, bool SWIGLU, int NREG>
static int gemm_grid() {
    static const int g = resident_grid((const void*)gemm_bf16_kernel<WM, BN, SWIGLU, NREG>,
                                       kGemmThreads, device_cu_count());
    return g;
}

template <int BN, bool SWIGLU>
static void launch_bf16(const uint16_t* A, const uint16_t* B, const GroupedPlan& pl, int K,
                        int n_out, int b_rows, int topk, uint16_t* C, hipStream_t s) {
    hipLaunchKernelGGL((gemm_bf16_kernel<kBf16WM, BN, SWIGLU, kBf16NReg>),
                       dim3(gemm_grid<kBf16WM, BN, SWIGLU, kBf16NReg>()), dim3(kGemmThreads), 0, s,
                       A, B, pl.perm, pl.tiles, pl.ntiles, pl.tile_off, pl.offsets, pl.E, K, n_out,
                       b_rows, topk, C);
}

hipError_t launch_gateup_bf16(const uint16_t* x, const uint16_t* w13, const GroupedPlan& pl,
                              int H, int F, int k, uint16_t* h, hipStream_t s) {
    if (F % 128 == 0) launch_bf16<256, true>(x, w13, pl, H, F, 2 * F, k, h, s);
    else launch_bf16<128, true>(x, w13, pl, H, F, 2 * F, k, h, s);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const uint16_t* h, const uint16_t* w2, const GroupedPlan& pl, int H,
                            int F, uint16_t* y, hipStream_t s) {
    if (H % 256 == 0) launch_bf16<256, false>(h, w2, pl, F, H, H, 1, y, s);
    else if (H % 128 == 0) launch_bf16<128, false>(h, w2, pl, F, H, H, 1, y, s);
    else launch_bf16<64, false>(h, w2, pl, F, H, H, 1, y, s);
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// One thread per (token, 8 columns): out = sum_j w[t,j] * y[t*k+j] in slot
// order, fp32, one rounding to bf16.  Dropped slots contribute nothing.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ w, int64_t T,
                                                      int k, int E, int H,
                                                      uint16_t* __restrict__ out) {
    const int cpr = H / 8;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= T * cpr) return;
    const int64_t t = g / cpr;
    const int c = (int)(g - t * cpr) * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
        const int e = idx[t * k + j];
        if ((unsigned)e >= (unsigned)E) continue;
        const float wt = w[t * k + j];
        const uint4 v = *(const uint4*)(y + (t * k + j) * H + c);
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wt * f[i];
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *(uint4*)(out + t * H + c) = o;
}

hipError_t launch_combine(const uint16_t* y, const int32_t* idx, const float* w, int64_t T, int k,
                          int E, int H, uint16_t* out, hipStream_t s) {
    const int64_t n = T * (H / 8);
    const int blocks = (int)((n + 255) / 256);
    hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, y, idx, w, T, k, E, H, out);
    return hipGetLastError();
}

}  // namespace moe

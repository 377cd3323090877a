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

constexpr int kGemmThreads = 512;  // 8 waves; wave w owns tile rows [32w, 32w+32)
constexpr int kBK = 64;            // bf16 K elements per stage (128 bytes per row)

// One work item = (M tile of <= 256 rows of one expert) x (BN output columns).
// SWIGLU: B rows are interleaved in blocks of 32 as gate, up, gate, up, ...
// so that each wave holds matching gate/up accumulators lane for lane, and
// the epilogue writes h = silu(gate) * up as bf16 [P, F] in expert order.
// Otherwise the epilogue writes y[slot, col] bf16 with slot = perm[row].
template <int BN, bool SWIGLU>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, const int32_t* __restrict__ offsets, int K,
    int n_out, int b_rows, int topk, uint16_t* __restrict__ C) {
    constexpr int NB = BN / 32;                       // 32-wide accumulator blocks per wave
    constexpr int A_PER = kTileM * 8 / kGemmThreads;  // 16-byte chunks per thread
    constexpr int B_PER = BN * 8 / kGemmThreads;
    static_assert(B_PER >= 1, "BN too small");
    __shared__ uint4 a_lds[2][kTileM][8];
    __shared__ uint4 b_lds[2][BN][8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk = tid & 7, row_t = tid >> 3;
    const int ntiles = *ntiles_p;
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int items = ntiles * n_tiles_n;
    const int nks = K / kBK;

    for (int it = xcd_slot(blockIdx.x, gridDim.x); it < items; it += gridDim.x) {
        const int nt = it / ntiles, mt = it - nt * ntiles;
        const int e = tiles[2 * mt], row0 = tiles[2 * mt + 1];
        const int mrows = min(kTileM, offsets[e + 1] - row0);

        const uint16_t* a_src[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int r = row_t + 64 * i;
            a_src[i] = nullptr;
            if (r < mrows) {
                const int64_t arow = SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
                a_src[i] = A + arow * K + chunk * 8;
            }
        }
        const uint16_t* b_src[B_PER];
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int rr = row_t + 64 * i;
            int brow;
            if (SWIGLU) {
                const int blk = rr >> 5;
                brow = ((blk & 1) ? n_out : 0) + nt * (BN / 2) + (blk >> 1) * 32 + (rr & 31);
            } else {
                brow = nt * BN + rr;
            }
            b_src[i] = B + ((int64_t)e * b_rows + brow) * K + chunk * 8;
        }

        uint4 a_reg[A_PER], b_reg[B_PER];
        auto load_stage = [&](int ks) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i)
                a_reg[i] = a_src[i] ? *(const uint4*)(a_src[i] + ks * kBK) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < B_PER; ++i) b_reg[i] = *(const uint4*)(b_src[i] + ks * kBK);
        };
        auto store_stage = [&](int buf) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) {
                const int r = row_t + 64 * i;
                a_lds[buf][r][chunk ^ (r & 7)] = a_reg[i];
            }
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int rr = row_t + 64 * i;
                b_lds[buf][rr][chunk ^ (rr & 7)] = b_reg[i];
            }
        };

        f32x16 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
        const bool active = wave * 32 < mrows;
        const int my_row = wave * 32 + (lane & 31);
        const int sw = lane & 7;  // == my_row & 7 == (nb*32 + lane%32) & 7

        load_stage(0);
        store_stage(0);
        __syncthreads();
        for (int ks = 0; ks < nks; ++ks) {
            const int buf = ks & 1;
            if (ks + 1 < nks) load_stage(ks + 1);
            if (active) {
#pragma unroll
                for (int kk = 0; kk < kBK / 16; ++kk) {
                    const int c = kk * 2 + (lane >> 5);
                    const uint4 a = a_lds[buf][my_row][c ^ sw];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const uint4 b = b_lds[buf][nb * 32 + (lane & 31)][c ^ sw];
                        acc[nb] = mfma_bf16_32x32x16(a, b, acc[nb]);
                    }
                }
            }
            if (ks + 1 < nks) store_stage(buf ^ 1);
            __syncthreads();
        }

        if (active) {
            if (SWIGLU) {
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    const int f = nt * (BN / 2) + p * 32 + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wave * 32 + acc_row(r, lane);
                        if (row < mrows) {
                            const float hv = silu(acc[2 * p][r]) * acc[2 * p + 1][r];
                            C[(int64_t)(row0 + row) * n_out + f] = (uint16_t)f32_to_bf16(hv);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wave * 32 + acc_row(r, lane);
                    if (row < mrows) {
                        const int64_t slot = perm[row0 + row];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const int col = nt * BN + nb * 32 + (lane & 31);
                            C[slot * n_out + col] = (uint16_t)f32_to_bf16(acc[nb][r]);
                        }
                    }
                }
            }
        }
    }
}

static int gemm_grid() {
    int g = device_cu_count();
    return ((g + kXcds - 1) / kXcds) * kXcds;
}

hipError_t launch_gateup_bf16(const uint16_t* x, const uint16_t* w13, const int32_t* perm,
                              const int32_t* tiles, const int32_t* ntiles, const int32_t* offsets,
                              int64_t, int H, int F, int k, uint16_t* h, hipStream_t s) {
    hipLaunchKernelGGL((gemm_bf16_kernel<128, true>), dim3(gemm_grid()), dim3(kGemmThreads), 0, s,
                       x, w13, perm, tiles, ntiles, offsets, H, F, 2 * F, k, h);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const uint16_t* h, const uint16_t* w2, const int32_t* perm,
                            const int32_t* tiles, const int32_t* ntiles, const int32_t* offsets,
                            int64_t, int H, int F, uint16_t* y, hipStream_t s) {
    if (H % 128 == 0)
        hipLaunchKernelGGL((gemm_bf16_kernel<128, false>), dim3(gemm_grid()), dim3(kGemmThreads), 0,
                           s, h, w2, perm, tiles, ntiles, offsets, F, H, H, 1, y);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<64, false>), dim3(gemm_grid()), dim3(kGemmThreads), 0,
                           s, h, w2, perm, tiles, ntiles, offsets, F, H, H, 1, y);
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

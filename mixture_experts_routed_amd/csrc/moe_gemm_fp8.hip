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
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kFp8Threads = 512;  // 8 waves; wave w owns tile rows [32w, 32w+32)
constexpr int kFp8BK = 128;       // K bytes per stage == one scale block

// Block-128 quantisation of 128 values spread as 4 per lane over one 32-lane
// half (same row): shared by the layer's epilogue and the stand-alone kernel.
// Returns the scale; writes the four codes packed little-endian in *codes.
__device__ __forceinline__ float quant_block_half(const float v[4], float amax_local, uint32_t* codes) {
    const float amax = half_max32(amax_local);
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

template <int BN, bool SWIGLU>
__global__ __launch_bounds__(kFp8Threads, 1) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles_p,
    const int32_t* __restrict__ offsets, int K, int n_out, int b_rows, int topk,
    uint8_t* __restrict__ Cq, float* __restrict__ Cs, uint16_t* __restrict__ Cy) {
    constexpr int NB = BN / 32;
    constexpr int A_PER = kTileM * 8 / kFp8Threads;
    constexpr int B_PER = BN * 8 / kFp8Threads;
    static_assert(!SWIGLU || BN == 256, "the SwiGLU epilogue needs a full 128-column h block");
    __shared__ uint4 a_lds[2][kTileM][8];
    __shared__ uint4 b_lds[2][BN][8];
    __shared__ __attribute__((aligned(16))) float sa_lds[2][kTileM];
    __shared__ __attribute__((aligned(16))) float sb_lds[2][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk = tid & 7, row_t = tid >> 3;
    const int ntiles = *ntiles_p;
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int items = ntiles * n_tiles_n;
    const int nkb = K / kFp8BK;

    for (int it = xcd_slot(blockIdx.x, gridDim.x); it < items; it += gridDim.x) {
        const int nt = it / ntiles, mt = it - nt * ntiles;
        const int e = tiles[2 * mt], row0 = tiles[2 * mt + 1];
        const int mrows = min(kTileM, offsets[e + 1] - row0);

        const uint8_t* a_src[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int r = row_t + 64 * i;
            a_src[i] = nullptr;
            if (r < mrows) {
                const int64_t arow = SWIGLU ? (int64_t)(perm[row0 + r] / topk) : (int64_t)(row0 + r);
                a_src[i] = A + arow * K + chunk * 16;
            }
        }
        const uint8_t* b_src[B_PER];
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
            b_src[i] = B + ((int64_t)e * b_rows + brow) * K + chunk * 16;
        }
        // scale rows: threads [0,256) -> A rows, [256, 256+BN) -> B rows
        const float* s_src = nullptr;
        int s_stride = 0;
        if (tid < kTileM) {
            if (tid < mrows) {
                const int64_t arow = SWIGLU ? (int64_t)(perm[row0 + tid] / topk) : (int64_t)(row0 + tid);
                s_src = As + arow * nkb;
                s_stride = 1;
            }
        } else if (tid - kTileM < BN) {
            const int rr = tid - kTileM;
            int brow;
            if (SWIGLU) {
                const int blk = rr >> 5;
                brow = ((blk & 1) ? n_out : 0) + nt * (BN / 2) + (blk >> 1) * 32 + (rr & 31);
            } else {
                brow = nt * BN + rr;
            }
            s_src = Bs + ((int64_t)e * b_rows + brow) * nkb;
            s_stride = 1;
        }

        uint4 a_reg[A_PER], b_reg[B_PER];
        float s_reg = 0.0f;
        auto load_stage = [&](int kb) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i)
                a_reg[i] = a_src[i] ? *(const uint4*)(a_src[i] + kb * kFp8BK) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < B_PER; ++i) b_reg[i] = *(const uint4*)(b_src[i] + kb * kFp8BK);
            s_reg = s_src ? s_src[kb * s_stride] : 0.0f;
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
            if (tid < kTileM) sa_lds[buf][tid] = s_reg;
            else if (tid - kTileM < BN) sb_lds[buf][tid - kTileM] = s_reg;
        };

        f32x16 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
        const bool active = wave * 32 < mrows;
        const int my_row = wave * 32 + (lane & 31);
        const int sw = lane & 7;
        const int g = lane >> 5;

        load_stage(0);
        store_stage(0);
        __syncthreads();
        for (int kb = 0; kb < nkb; ++kb) {
            const int buf = kb & 1;
            if (kb + 1 < nkb) load_stage(kb + 1);
            if (active) {
                i32x8 a0, a1;
                {
                    const uint4 c0 = a_lds[buf][my_row][(2 * g) ^ sw];
                    const uint4 c1 = a_lds[buf][my_row][(2 * g + 1) ^ sw];
                    const uint4 c2 = a_lds[buf][my_row][(4 + 2 * g) ^ sw];
                    const uint4 c3 = a_lds[buf][my_row][(4 + 2 * g + 1) ^ sw];
                    a0 = i32x8{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
                    a1 = i32x8{(int)c2.x, (int)c2.y, (int)c2.z, (int)c2.w, (int)c3.x, (int)c3.y, (int)c3.z, (int)c3.w};
                }
                float sa[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *(const float4*)&sa_lds[buf][wave * 32 + 8 * q + 4 * g];
                    sa[4 * q + 0] = v.x; sa[4 * q + 1] = v.y; sa[4 * q + 2] = v.z; sa[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int brow = nb * 32 + (lane & 31);
                    const uint4 d0 = b_lds[buf][brow][(2 * g) ^ sw];
                    const uint4 d1 = b_lds[buf][brow][(2 * g + 1) ^ sw];
                    const uint4 d2 = b_lds[buf][brow][(4 + 2 * g) ^ sw];
                    const uint4 d3 = b_lds[buf][brow][(4 + 2 * g + 1) ^ sw];
                    const i32x8 b0{(int)d0.x, (int)d0.y, (int)d0.z, (int)d0.w, (int)d1.x, (int)d1.y, (int)d1.z, (int)d1.w};
                    const i32x8 b1{(int)d2.x, (int)d2.y, (int)d2.z, (int)d2.w, (int)d3.x, (int)d3.y, (int)d3.z, (int)d3.w};
                    f32x16 tmp = mfma_fp8_32x32x64(a0, b0, f32x16{});
                    tmp = mfma_fp8_32x32x64(a1, b1, tmp);
                    const float sbv = sb_lds[buf][brow];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[nb][r] += tmp[r] * (sa[r] * sbv);
                }
            }
            if (kb + 1 < nkb) store_stage(buf ^ 1);
            __syncthreads();
        }

        if (active) {
            if (SWIGLU) {
                // h block of 128 columns: f = nt*128 + p*32 + lane%32, p = 0..3
                const int fblk = nt;
                const int nfb = n_out / 128;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wave * 32 + acc_row(r, lane);
                    float hv[4];
                    float amax = 0.0f;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        hv[p] = silu(acc[2 * p][r]) * acc[2 * p + 1][r];
                        amax = fmaxf(amax, fabsf(hv[p]));
                    }
                    uint32_t codes;
                    const float scale = quant_block_half(hv, amax, &codes);
                    if (row < mrows) {
                        uint8_t* dst = Cq + (int64_t)(row0 + row) * n_out + fblk * 128 + (lane & 31);
#pragma unroll
                        for (int p = 0; p < 4; ++p) dst[p * 32] = (uint8_t)(codes >> (8 * p));
                        if ((lane & 31) == 0) Cs[(int64_t)(row0 + row) * nfb + fblk] = scale;
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
                            Cy[slot * n_out + col] = (uint16_t)f32_to_bf16(acc[nb][r]);
                        }
                    }
                }
            }
        }
    }
}

static int fp8_grid() {
    int g = device_cu_count();
    return ((g + kXcds - 1) / kXcds) * kXcds;
}

hipError_t launch_gateup_fp8(const uint8_t* x, const float* xs, const uint8_t* w13,
                             const float* w13s, const int32_t* perm, const int32_t* tiles,
                             const int32_t* ntiles, const int32_t* offsets, int64_t, int H, int F,
                             int k, uint8_t* hq, float* hs, hipStream_t s) {
    hipLaunchKernelGGL((gemm_fp8_kernel<256, true>), dim3(fp8_grid()), dim3(kFp8Threads), 0, s, x,
                       xs, w13, w13s, perm, tiles, ntiles, offsets, H, F, 2 * F, k, hq, hs,
                       (uint16_t*)nullptr);
    return hipGetLastError();
}

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* w2, const float* w2s,
                           const int32_t* perm, const int32_t* tiles, const int32_t* ntiles,
                           const int32_t* offsets, int64_t, int H, int F, uint16_t* y,
                           hipStream_t s) {
    hipLaunchKernelGGL((gemm_fp8_kernel<128, false>), dim3(fp8_grid()), dim3(kFp8Threads), 0, s,
                       hq, hs, w2, w2s, perm, tiles, ntiles, offsets, F, H, H, 1,
                       (uint8_t*)nullptr, (float*)nullptr, y);
    return hipGetLastError();
}

// ------------------------------------------------------- stand-alone quantiser
// One 32-lane half per 128-value block: lane i of the half takes values
// i, i+32, i+64, i+96 (the same spread as the epilogue's accumulators).
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ in, int in_is_bf16,
                                                       int64_t nblocks, int K,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
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
    const float scale = quant_block_half(v, amax, &c);
    if (live) {
#pragma unroll
        for (int p = 0; p < 4; ++p) codes[base + p * 32 + l] = (uint8_t)(c >> (8 * p));
        if (l == 0) scales[b] = scale;
    }
}

hipError_t launch_quantize_fp8(const void* in, int in_is_bf16, int64_t rows, int K, uint8_t* codes,
                               float* scales, hipStream_t s) {
    const int64_t nblocks = rows * (K / 128);
    const int64_t threads = nblocks * 32;
    const int blocks = (int)((threads + 255) / 256);
    hipLaunchKernelGGL(quantize_kernel, dim3(blocks), dim3(256), 0, s, in, in_is_bf16, nblocks, K,
                       codes, scales);
    return hipGetLastError();
}

}  // namespace moe

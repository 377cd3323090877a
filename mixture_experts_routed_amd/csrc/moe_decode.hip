// moe_decode.hip - gather-GEMV form of the routed-experts layer for a
// handful of tokens.  Model card "DeepSeek-OCR-2 MoE experts", description:
// the decode op handles about 1-4 tokens with two persistent-shape kernels,
// without a per-expert host loop and without a device-to-host sync.  Here:
//   phase 1: every (distinct selected expert, f) pair streams gate row f and
//            up row F+f once and writes h[slot, f] = silu(g) * u in fp32 for
//            every slot that selected the expert;
//   phase 2: every output column c streams down row c of each selected
//            expert and forms out[t, c] = sum_j w[t,j] * (down[e_j][c] . h)
//            in slot order (the combine, fused, no atomics).
// Only the selected experts' weights are read from HBM, each row once.
//
// The kernel boundary is the only device-wide synchronisation.  On MI355X a
// launch boundary costs about 1.5 us, while an in-kernel grid barrier costs
// 7-45 us (same-address atomics serialise at about 15 ns each) and the
// agent-scope cache write-back/invalidate a flag-based hand-off needs made a
// single fused launch slower than two.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecCh = 8;         // 16-byte chunks per lane of a gate/up row: H <= 2048

// The routing of all P <= 32 slots, held by the lanes of one wave: lane s
// has slot s's expert (or -1) and weight.  `first` marks the lanes that are
// the first slot of a distinct expert (distinct experts are numbered in order
// of first appearance); `u` is the distinct index of the lane's slot.
struct WaveRouting {
    int e;
    float w;
    int u;
    uint64_t first;
    int n;
};

__device__ __forceinline__ WaveRouting wave_routing(const int32_t* __restrict__ idx,
                                                    const float* __restrict__ wts, int P, int E) {
    const int lane = threadIdx.x & 63;
    WaveRouting r;
    int e = lane < P ? idx[lane] : -1;
    r.w = (wts != nullptr && lane < P) ? wts[lane] : 0.0f;
    const bool valid = (unsigned)e < (unsigned)E;
    if (!valid) e = -1;
    int first = lane;
    for (int s = 0; s < P; ++s) {
        const int es = __shfl(e, s, kWave);
        if (s < first && es == e) first = s;
    }
    const bool is_first = valid && first == lane;
    r.first = __ballot(is_first);
    r.n = __popcll(r.first);
    r.u = valid ? __popcll(r.first & ((1ull << first) - 1ull)) : -1;
    r.e = e;
    return r;
}

// One (expert, f) pair: gate row f in lanes [0,32), up row F+f in lanes
// [32,64), already loaded; h[s, f] for every slot s of the expert.
__device__ __forceinline__ void gateup_pair(const uint16_t* __restrict__ x, const uint4 (&wv)[kDecCh],
                                            uint64_t slots, int k, int H, int F, int f,
                                            float* __restrict__ h) {
    const int lane = threadIdx.x & 63, l32 = lane & 31;
    const int nch = H / 8;
    while (slots) {
        const int s = __builtin_ctzll(slots);
        slots &= slots - 1ull;
        const uint16_t* xr = x + (int64_t)(s / k) * H;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < kDecCh; ++i) {
            const int c = l32 + 32 * i;
            if (c < nch) {
                const uint4 xv = *(const uint4*)(xr + c * 8);
                float a[8], b[8];
                unpack8(wv[i], a);
                unpack8(xv, b);
#pragma unroll
                for (int q = 0; q < 8; ++q) part += a[q] * b[q];
            }
        }
        part = half_sum32(part);
        const float up = __shfl(part, 32, kWave);
        if (lane == 0) h[(int64_t)s * F + f] = silu(part) * up;
    }
}

// Slots [s0, s0+8) of the down rows: dot each valid slot's row chunk with
// h[slot] and add w[slot] * dot to its token's accumulator, in slot order.
template <int CPL>
__device__ __forceinline__ void down_group(const float* __restrict__ h, const uint4 (&wv)[8][CPL],
                                           const int (&es)[8], const WaveRouting& R, int s0, int P,
                                           int k, int F, float (&acc)[kDecodeMaxT]) {
    const int lane = threadIdx.x & 63;
    const int nch = F / 8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int s = s0 + jj;
        const float ws = __shfl(R.w, s < P ? s : 0, kWave);
        if (es[jj] < 0) continue;  // dropped slot or past the end (wave-uniform)
        const float* hr = h + (int64_t)s * F;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            if (ch < nch) {
                const float4 h0 = *(const float4*)(hr + ch * 8);
                const float4 h1 = *(const float4*)(hr + ch * 8 + 4);
                float a[8];
                unpack8(wv[jj][i], a);
                part += a[0] * h0.x + a[1] * h0.y + a[2] * h0.z + a[3] * h0.w +
                        a[4] * h1.x + a[5] * h1.y + a[6] * h1.z + a[7] * h1.w;
            }
        }
        const int t = s / k;
#pragma unroll
        for (int tt = 0; tt < kDecodeMaxT; ++tt)
            if (tt == t) acc[tt] += ws * part;
    }
}

template <int CPL>
__device__ __forceinline__ void down_load(const uint16_t* __restrict__ w2, const WaveRouting& R,
                                          int s0, int P, int H, int F, int c, uint4 (&wv)[8][CPL],
                                          int (&es)[8]) {
    const int lane = threadIdx.x & 63;
    const int nch = F / 8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int s = s0 + jj;
        es[jj] = __shfl(R.e, s < P ? s : 0, kWave);
        if (s >= P || c >= H) es[jj] = -1;
        const uint16_t* row = w2 + ((int64_t)(es[jj] >= 0 ? es[jj] : 0) * H + (c < H ? c : 0)) * F;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            wv[jj][i] = (es[jj] >= 0 && ch < nch) ? load_nt16(row + ch * 8) : make_uint4(0, 0, 0, 0);
        }
    }
}

// Phase 1: one (distinct expert u, f) pair per wave, pair = 4 * b + wave.
// Every wave is short-lived and all of a call's row loads are in flight at
// once: at decode sizes the stream is latency-bound, and on MI355X spreading
// it over the most waves beats fewer, longer-lived pipelined waves.
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ idx, int P, int k, int E, int H, int F,
    float* __restrict__ h) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const WaveRouting R = wave_routing(idx, nullptr, P, E);
    const int64_t pair = (int64_t)blockIdx.x * (kDecThreads / kWave) + wave;
    const int u = (int)(pair / F), f = (int)(pair - (int64_t)u * F);
    if (u >= R.n) return;  // fewer distinct experts than slots
    uint64_t fm = R.first;
    for (int i = 0; i < u; ++i) fm &= fm - 1ull;
    const int e = __shfl(R.e, __builtin_ctzll(fm), kWave);
    const uint64_t slots = __ballot(R.u == u);
    const int half = lane >> 5, l32 = lane & 31;
    const int nch = H / 8;
    const uint16_t* row = w13 + ((int64_t)e * 2 * F + (int64_t)half * F + f) * H;
    uint4 wv[kDecCh];
#pragma unroll
    for (int i = 0; i < kDecCh; ++i) {
        const int c = l32 + 32 * i;
        wv[i] = c < nch ? load_nt16(row + c * 8) : make_uint4(0, 0, 0, 0);
    }
    gateup_pair(x, wv, slots, k, H, F, f, h);
}

// Phase 2: one wave per output column c = 4 * b + wave.
template <int CPL>
__global__ __launch_bounds__(kDecThreads) void decode_down_kernel(
    const float* __restrict__ h, const uint16_t* __restrict__ w2, const int32_t* __restrict__ idx,
    const float* __restrict__ wts, int T, int k, int E, int H, int F, uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int P = T * k;
    const WaveRouting R = wave_routing(idx, wts, P, E);
    const int c = blockIdx.x * (kDecThreads / kWave) + wave;
    if (c >= H) return;
    uint4 wv[8][CPL];
    int es[8];
    float acc[kDecodeMaxT];
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) acc[t] = 0.0f;
    for (int s0 = 0; s0 < P; s0 += 8) {
        down_load<CPL>(w2, R, s0, P, H, F, c, wv, es);
        down_group<CPL>(h, wv, es, R, s0, P, k, F, acc);
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) {
        if (t >= T) break;
        const float v = wave_sum(acc[t]);
        if (lane == 0) out[(int64_t)t * H + c] = (uint16_t)f32_to_bf16(v);
    }
}

hipError_t launch_decode(const uint16_t* x, const uint16_t* w13, const uint16_t* w2,
                         const int32_t* idx, const float* w, int T, int k, int E, int H, int F,
                         float* h, uint16_t* out, hipStream_t s) {
    const DecodeGeometry g = decode_geometry(T, k, E, H, F);
    const int64_t pairs = (int64_t)g.umax * F;
    const int wpb = kDecThreads / kWave;
    hipLaunchKernelGGL(decode_gateup_kernel, dim3((unsigned)((pairs + wpb - 1) / wpb)),
                       dim3(kDecThreads), 0, s, x, w13, idx, T * k, k, E, H, F, h);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid((unsigned)g.nw2), block(kDecThreads);
    switch ((F / 8 + 63) / 64) {
        case 1: hipLaunchKernelGGL(decode_down_kernel<1>, grid, block, 0, s, h, w2, idx, w, T, k, E, H, F, out); break;
        case 2: hipLaunchKernelGGL(decode_down_kernel<2>, grid, block, 0, s, h, w2, idx, w, T, k, E, H, F, out); break;
        case 3: hipLaunchKernelGGL(decode_down_kernel<3>, grid, block, 0, s, h, w2, idx, w, T, k, E, H, F, out); break;
        case 4: hipLaunchKernelGGL(decode_down_kernel<4>, grid, block, 0, s, h, w2, idx, w, T, k, E, H, F, out); break;
        default: return hipErrorInvalidValue;  // F > 2048 is routed to the grouped path by the caller
    }
    return hipGetLastError();
}

}  // namespace moe

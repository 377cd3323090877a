// moe_plan.hip - deterministic routing plan (expert histogram, exclusive
// prefix, stable scatter) for the grouped products of the routed-experts
// layer.  The model card "DeepSeek-OCR-2 MoE experts" describes its prefill
// op as a grouped GEMM over experts; the mirage issue "Supporting MegaKernel
// for DeepSeek Models" passes the per-expert prefix as an [E+1] int32 tensor
// (moe_w13_fp8_layer "masks").  Slots s = t*k + j are ordered by expert with
// ties in ascending s; ids outside [0,E) are dropped.
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_route.h"
#include "../../include/moe_experts.h"

namespace moe {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanRegs = 32;  // slots per lane loaded together (one round trip per 2048-slot chunk)

// One workgroup.  Wave w owns a contiguous, 64-aligned run of slots, so the
// order (wave, position in run) is the slot order.  Pass 1 counts per
// (wave, expert) with LDS integer atomics (exact, order-free).  Each expert's
// per-wave counts then become running bases, and pass 2 walks the slots again
// in order: lanes with the same expert in one 64-slot step find each other by
// OR-ing their lane bits into a per-(wave, expert) LDS mask (order-free, so
// deterministic) and take consecutive positions by lane rank.  (A ballot per
// id bit costs about 7 vector instructions per bit and step, which on one CU
// shared by 16 waves made this pass the kernel's main cost.)
// The plan of one workgroup of kPlanThreads threads (shared by the plan
// kernel and the fused router + plan kernel).
__device__ __forceinline__ void plan_body(
    const int32_t* __restrict__ idx, int P, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles, int32_t* __restrict__ tile_off,
    int tile_m) {
    __shared__ int base[kPlanWaves][MOE_MAX_EXPERTS];
    __shared__ unsigned long long lanes_of[kPlanWaves][MOE_MAX_EXPERTS];  // pass 2, zero between steps
    __shared__ int tot[MOE_MAX_EXPERTS];
    __shared__ int off_sh[MOE_MAX_EXPERTS + 1];
    __shared__ int tile_sh[MOE_MAX_EXPERTS + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kPlanWaves * MOE_MAX_EXPERTS; i += kPlanThreads) {
        (&base[0][0])[i] = 0;
        (&lanes_of[0][0])[i] = 0ull;
    }
    __syncthreads();

    const int run = ((P + kPlanWaves * kWave - 1) / (kPlanWaves * kWave)) * kWave;
    const int s0 = wave * run;
    const int s1 = min(P, s0 + run);

    for (int cb = s0; cb < s1; cb += kWave * kPlanRegs) {
        int ev[kPlanRegs];
#pragma unroll
        for (int i = 0; i < kPlanRegs; ++i) {
            const int s = cb + kWave * i + lane;
            ev[i] = s < s1 ? idx[s] : -1;
        }
#pragma unroll
        for (int i = 0; i < kPlanRegs; ++i) {
            if (cb + kWave * i >= s1) break;  // wave-uniform: past this wave's run
            if ((unsigned)ev[i] < (unsigned)E) atomicAdd(&base[wave][ev[i]], 1);
        }
    }
    __syncthreads();

    for (int e = tid; e < E; e += kPlanThreads) {
        int acc = 0;
        for (int w = 0; w < kPlanWaves; ++w) {
            const int c = base[w][e];
            base[w][e] = acc;
            acc += c;
        }
        tot[e] = acc;
    }
    __syncthreads();

    if (wave == 0) {  // exclusive prefix of counts and of M tiles over experts
        const int per = (E + kWave - 1) / kWave;
        const int e0 = lane * per;
        int c_sum = 0, t_sum = 0;
        for (int i = 0; i < per; ++i) {
            const int e = e0 + i;
            if (e < E) {
                c_sum += tot[e];
                t_sum += (tot[e] + tile_m - 1) / tile_m;
            }
        }
        int c_inc = c_sum, t_inc = t_sum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int cu = __shfl_up(c_inc, o, kWave);
            const int tu = __shfl_up(t_inc, o, kWave);
            if (lane >= o) { c_inc += cu; t_inc += tu; }
        }
        int c_run = c_inc - c_sum, t_run = t_inc - t_sum;
        for (int i = 0; i < per; ++i) {
            const int e = e0 + i;
            if (e < E) {
                off_sh[e] = c_run;
                tile_sh[e] = t_run;
                c_run += tot[e];
                t_run += (tot[e] + tile_m - 1) / tile_m;
            }
        }
        if (lane == kWave - 1) {
            off_sh[E] = c_inc;
            tile_sh[E] = t_inc;
        }
    }
    __syncthreads();

    for (int e = tid; e <= E; e += kPlanThreads) {
        offsets[e] = off_sh[e];
        tile_off[e] = tile_sh[e];
        if (e < E) {
            counts[e] = tot[e];
            const int nt = tile_sh[e + 1] - tile_sh[e];
            for (int i = 0; i < nt; ++i) {
                tiles[2 * (tile_sh[e] + i)] = e;
                tiles[2 * (tile_sh[e] + i) + 1] = off_sh[e] + i * tile_m;
            }
        }
    }
    if (tid == 0) *ntiles = tile_sh[E];
    // absolute base of each (wave, expert) run: one LDS read per scatter step
    for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) base[i / E][i % E] += off_sh[i % E];
    __syncthreads();

    // pass 2: stable scatter in slot order; each wave only touches its own
    // row of `base`
    for (int cb = s0; cb < s1; cb += kWave * kPlanRegs) {
        int ev[kPlanRegs];
#pragma unroll
        for (int i = 0; i < kPlanRegs; ++i) {
            const int s = cb + kWave * i + lane;
            ev[i] = s < s1 ? idx[s] : -1;
        }
#pragma unroll
        for (int i = 0; i < kPlanRegs; ++i) {
            if (cb + kWave * i >= s1) break;  // wave-uniform: past this wave's run
            const int s = cb + kWave * i + lane;
            const int e = ev[i];
            const bool valid = (unsigned)e < (unsigned)E;
            // the lanes of this step that hold expert e (LDS operations of
            // one wave complete in issue order: the ORs land before the read,
            // the read before the clear)
            if (valid) atomicOr(&lanes_of[wave][e], 1ull << lane);
            __builtin_amdgcn_wave_barrier();
            const uint64_t same = valid ? lanes_of[wave][e] : 0ull;
            __builtin_amdgcn_wave_barrier();
            if (valid) lanes_of[wave][e] = 0ull;
            int rank = 0, pos = -1;
            if (valid) {
                rank = __popcll(same & ((1ull << lane) - 1ull));
                pos = base[wave][e] + rank;
                perm[pos] = s;
            }
            if (s < s1) inv[s] = pos;
            // every lane has read base[wave][*] above before the group leader
            // bumps it (LDS operations of one wave complete in issue order)
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) base[wave][e] += __popcll(same);
            __builtin_amdgcn_wave_barrier();
        }
    }
    for (int i = off_sh[E] + tid; i < P; i += kPlanThreads) perm[i] = -1;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ idx, int P, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles, int32_t* __restrict__ tile_off,
    int tile_m) {
    plan_body(idx, P, E, counts, offsets, perm, inv, tiles, ntiles, tile_off, tile_m);
}

// ------------------------------------------------------------------ routers
// (the per-token routine is in moe_route.h)

template <int EP>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a, int64_t T, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // whole waves leave together
    route_token<EP>(a, t, threadIdx.x & 63, idx, w);
}

// Router and plan in one launch of one workgroup (small batches): the 16
// waves route the tokens, then the same workgroup builds the plan from the
// ids it has just written.
template <int EP>
__global__ __launch_bounds__(kPlanThreads) void route_plan_kernel(
    RouteArgs a, int T, int32_t* __restrict__ idx, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles,
    int32_t* __restrict__ tile_off, int tile_m) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int t = wave; t < T; t += kPlanWaves) route_token<EP>(a, t, lane, idx, w);
    __threadfence_block();
    __syncthreads();   // the ids are visible to every wave of the workgroup
    plan_body(idx, T * a.k, a.E, counts, offsets, perm, inv, tiles, ntiles, tile_off, tile_m);
}

template <int EP>
static hipError_t launch_route_ep(const RouteArgs& a, int64_t T, int32_t* idx, float* w,
                                  hipStream_t s) {
    MOE_LAUNCH(route_kernel<EP>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, a, T, idx, w);
    return hipGetLastError();
}

template <int EP>
static hipError_t launch_route_plan_ep(const RouteArgs& a, int T, int32_t* idx, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int32_t* tiles, int32_t* ntiles,
                                       int32_t* tile_off, int tile_m, hipStream_t s) {
    MOE_LAUNCH(route_plan_kernel<EP>, dim3(1), dim3(kPlanThreads), 0, s, a, T, idx, w, counts,
               offsets, perm, inv, tiles, ntiles, tile_off, tile_m);
    return hipGetLastError();
}

hipError_t launch_route(const void* logits, const void* bias, int bf16, int mode, int64_t T, int E,
                        int k, int num_groups, int topk_group, int group_top, float scale,
                        int32_t* idx, float* w, hipStream_t s) {
    const RouteArgs a{logits, bias, bf16, mode, E, k, num_groups, topk_group, group_top, scale};
    if (E <= 64) return launch_route_ep<1>(a, T, idx, w, s);
    if (E <= 128) return launch_route_ep<2>(a, T, idx, w, s);
    if (E <= 256) return launch_route_ep<4>(a, T, idx, w, s);
    return launch_route_ep<8>(a, T, idx, w, s);
}

hipError_t launch_route_plan(const void* logits, const void* bias, int bf16, int mode, int T,
                             int E, int k, int num_groups, int topk_group, int group_top,
                             float scale, int32_t* idx, float* w, int32_t* counts,
                             int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles,
                             int32_t* ntiles, int32_t* tile_off, int tile_m, hipStream_t s) {
    const RouteArgs a{logits, bias, bf16, mode, E, k, num_groups, topk_group, group_top, scale};
#define MOE_RP(EP) launch_route_plan_ep<EP>(a, T, idx, w, counts, offsets, perm, inv, tiles, ntiles, tile_off, tile_m, s)
    if (E <= 64) return MOE_RP(1);
    if (E <= 128) return MOE_RP(2);
    if (E <= 256) return MOE_RP(4);
    return MOE_RP(8);
#undef MOE_RP
}

hipError_t launch_plan(const int32_t* idx, int P, int E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* ntiles,
                       int32_t* tile_off, int tile_m, hipStream_t s) {
    MOE_LAUNCH(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, idx, P, E, counts,
                       offsets, perm, inv, tiles, ntiles, tile_off, tile_m);
    return hipGetLastError();
}

// ----------------------------------------------------- shared experts
// Routing with the S shared experts appended as always-on slots: slot j < k
// keeps the router's choice (an id outside [0, E) becomes -1, dropped, so it
// can never name a shared expert), slots k .. k+S-1 name experts E .. E+S-1
// with weight 1.  One thread per augmented slot.
__global__ __launch_bounds__(256) void augment_routing_kernel(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ w,
                                                              int64_t T, int k, int E, int S,
                                                              int32_t* __restrict__ idx2,
                                                              float* __restrict__ w2) {
    const int k2 = k + S;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * k2) return;
    const int64_t t = i / k2;
    const int j = (int)(i - t * k2);
    if (j < k) {
        const int e = idx[t * k + j];
        idx2[i] = (unsigned)e < (unsigned)E ? e : -1;
        w2[i] = w[t * k + j];
    } else {
        idx2[i] = E + (j - k);
        w2[i] = 1.0f;
    }
}

hipError_t launch_augment_routing(const int32_t* idx, const float* w, int64_t T, int k, int E,
                                  int S, int32_t* idx2, float* w2, hipStream_t s) {
    const int64_t n = T * (k + S);
    MOE_LAUNCH(augment_routing_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, w,
               T, k, E, S, idx2, w2);
    return hipGetLastError();
}

}  // namespace moe

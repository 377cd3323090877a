// moe_plan.hip - deterministic routing plan (expert histogram, exclusive
// prefix, stable scatter) for the grouped products of the routed-experts
// layer.  The model card "DeepSeek-OCR-2 MoE experts" describes its prefill
// op as a grouped GEMM over experts; the mirage issue "Supporting MegaKernel
// for DeepSeek Models" passes the per-expert prefix as an [E+1] int32 tensor
// (moe_w13_fp8_layer "masks").  Slots s = t*k + j are ordered by expert with
// ties in ascending s; ids outside [0,E) are dropped.
#include "moe_device.h"
#include "moe_internal.h"
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
// One wave routes one token.  Expert e sits in lane e % 64, register e / 64
// (coalesced loads of the logits row).  Two rules:
//  - softmax (model card "DeepSeek-OCR-2 MoE experts": fp32 softmax, greedy
//    top-k, weights scaled by routed_scaling_factor): softmax is increasing
//    in the logit, so the k largest logits are chosen (decided exactly on the
//    input values); weight = exp(l - max) / sum exp(l - max) in fp32, times
//    the factor, not renormalised;
//  - group-aware sigmoid (MegaKernel issue, moe_topk_sigmoid_routing_layer:
//    logits + bias, num_groups, topk_group, routed_scaling_factor):
//    s = sigmoid(l) and the choice score c = s + bias, in fp64; a group's
//    score is the sum of its group_top (1 or 2) largest c; the topk_group best
//    groups are kept; the k largest c among their experts are chosen; weights
//    are the chosen s renormalised to sum 1, times the factor.
// Ties go to the lower expert (or group) id; a NaN score ranks below every
// number.  The chosen ids are written largest score first.

__device__ __forceinline__ bool route_better(double a, int ia, double b, int ib) {
    return a > b || (a == b && ia < ib);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const long long b = __double_as_longlong(v);
    const int lo = __shfl_xor((int)(b & 0xffffffffll), m, kWave);
    const int hi = __shfl_xor((int)(b >> 32), m, kWave);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ double shfl_f64(double v, int src) {
    const long long b = __double_as_longlong(v);
    const int lo = __shfl((int)(b & 0xffffffffll), src, kWave);
    const int hi = __shfl((int)(b >> 32), src, kWave);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

struct RouteArgs {
    const void* logits;
    const void* bias;
    int bf16;          // logits and bias are bf16 (else fp32)
    int mode;          // MOE_ROUTE_*
    int E, k, num_groups, topk_group, group_top;
    float scale;
};

__device__ __forceinline__ float route_load(const void* p, int bf16, int64_t i) {
    return bf16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

template <int EP>
__device__ __forceinline__ void route_token(const RouteArgs& a, int64_t t, int lane,
                                            int32_t* __restrict__ idx_out,
                                            float* __restrict__ w_out) {
    const int E = a.E;
    const bool sig = a.mode == MOE_ROUTE_SIGMOID_GROUP;
    float lg[EP];
    double c[EP], sv[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) {
        const int e = lane + kWave * i;
        lg[i] = e < E ? route_load(a.logits, a.bf16, t * E + e) : 0.0f;
        if (sig) {
            sv[i] = 1.0 / (1.0 + exp(-(double)lg[i]));
            c[i] = sv[i] + (double)(e < E ? route_load(a.bias, a.bf16, e) : 0.0f);
        } else {
            sv[i] = 0.0;
            c[i] = (double)lg[i];
        }
        if (c[i] != c[i] || e >= E) c[i] = -INFINITY;   // NaN ranks lowest; no expert past E
    }

    // allowed experts: those of the kept groups (every expert for softmax)
    unsigned long long kept = ~0ull;
    int gsize = E;
    if (sig) {
        gsize = E / a.num_groups;
        double my_gscore = -INFINITY;
        for (int g = 0; g < a.num_groups; ++g) {
            double m1 = -INFINITY, m2 = -INFINITY;   // two largest c of group g held here
#pragma unroll
            for (int i = 0; i < EP; ++i) {
                const int e = lane + kWave * i;
                if (e < E && e / gsize == g) {
                    const double v = c[i];
                    if (v > m1) { m2 = m1; m1 = v; } else if (v > m2) { m2 = v; }
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const double p1 = shfl_xor_f64(m1, o), p2 = shfl_xor_f64(m2, o);
                const double n1 = fmax(m1, p1);
                m2 = fmax(fmin(m1, p1), fmax(m2, p2));
                m1 = n1;
            }
            const double gs = a.group_top == 2 ? m1 + m2 : m1;
            if (lane == g) my_gscore = gs;
        }
        // rank of group `lane` among the groups
        int rank = 0;
        for (int h = 0; h < a.num_groups; ++h) {
            const double o = shfl_f64(my_gscore, h);
            if (route_better(o, h, my_gscore, lane)) ++rank;
        }
        kept = __ballot(lane < a.num_groups && rank < a.topk_group);
    }

    bool taken[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) {
        const int e = lane + kWave * i;
        taken[i] = e >= E || !((kept >> (e / gsize)) & 1ull);
    }
    int my_id = -1;      // lane j < k: the j-th chosen expert
    double my_s = 0.0;   // its s (sigmoid) or logit (softmax)
    for (int j = 0; j < a.k; ++j) {
        double best = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EP; ++i) {
            const int e = lane + kWave * i;
            if (!taken[i] && route_better(c[i], e, best, bi)) { best = c[i]; bi = e; }
        }
        // (scores are never NaN here, so any untaken expert beats the
        // starting (-inf, INT_MAX): a valid id wins even among -inf scores)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const double ob = shfl_xor_f64(best, o);
            const int oi = __shfl_xor(bi, o, kWave);
            if (route_better(ob, oi, best, bi)) { best = ob; bi = oi; }
        }
        const int owner = bi & (kWave - 1), slot = bi >> 6;
        double val = 0.0;
#pragma unroll
        for (int i = 0; i < EP; ++i)
            if (i == slot) val = sig ? sv[i] : (double)lg[i];
        val = shfl_f64(val, owner);
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EP; ++i)
                if (i == slot) taken[i] = true;
        }
        if (lane == j) { my_id = bi; my_s = val; }
    }

    float w;
    if (sig) {
        double sum = lane < a.k ? my_s : 0.0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sum += shfl_xor_f64(sum, o);
        w = (float)(my_s / sum * (double)a.scale);
    } else {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < EP; ++i)
            if (lane + kWave * i < E) mx = fmaxf(mx, lg[i]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        float se = 0.0f;
#pragma unroll
        for (int i = 0; i < EP; ++i)
            if (lane + kWave * i < E) se += expf(lg[i] - mx);
        se = wave_sum(se);
        w = expf((float)my_s - mx) / se * a.scale;
    }
    if (lane < a.k) {
        idx_out[t * a.k + lane] = my_id;
        w_out[t * a.k + lane] = w;
    }
}

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

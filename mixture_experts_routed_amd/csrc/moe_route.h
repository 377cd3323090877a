// moe_route.h - the per-token router routine (internal header), shared by
// the router kernels and the decode kernel that routes for itself.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"
#include "../../include/moe_experts.h"

namespace moe {

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

__device__ __forceinline__ float route_load(const void* p, int bf16, int64_t i) {
    return bf16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// Lane j < k receives the j-th chosen id and its weight.
template <int EP>
__device__ __forceinline__ void route_token_lanes(const RouteArgs& a, int64_t t, int lane,
                                                  int& id_out, float& w_out) {
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
    id_out = my_id;
    w_out = w;
}

template <int EP>
__device__ __forceinline__ void route_token(const RouteArgs& a, int64_t t, int lane,
                                            int32_t* __restrict__ idx_out,
                                            float* __restrict__ w_out) {
    int id;
    float w;
    route_token_lanes<EP>(a, t, lane, id, w);
    if (lane < a.k) {
        idx_out[t * a.k + lane] = id;
        w_out[t * a.k + lane] = w;
    }
}

}  // namespace moe

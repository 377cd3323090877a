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
// Order-preserving 64-bit key of a double (a larger key is a larger value,
// -0 and +0 share one key); 0 is below every number's key.
__device__ __forceinline__ uint64_t route_key(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x + 0.0);   // -0 + 0 = +0
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(v & 0xffffffffull), l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Lane j < k receives the j-th chosen id and its weight.  The choice is a
// radix select on 64-bit keys with one ballot per key bit (no LDS round
// trips): the k-th largest key p is found bit by bit, keys above p are
// chosen, and keys equal to p fill the remaining places in ascending expert
// order; the chosen are then ranked by (key, lower id) with scalar reads.
template <int EP>
__device__ __forceinline__ void route_token_lanes(const RouteArgs& a, int64_t t, int lane,
                                                  int& id_out, float& w_out) {
    const int E = a.E;
    const bool sig = a.mode == MOE_ROUTE_SIGMOID_GROUP;
    float lg[EP];
    double c[EP], sv[EP];
    bool valid[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) {
        const int e = lane + kWave * i;
        valid[i] = e < E;
        lg[i] = valid[i] ? route_load(a.logits, a.bf16, t * E + e) : 0.0f;
        if (sig) {
            sv[i] = 1.0 / (1.0 + exp(-(double)lg[i]));
            c[i] = sv[i] + (double)(valid[i] ? route_load(a.bias, a.bf16, e) : 0.0f);
        } else {
            sv[i] = 0.0;
            c[i] = (double)lg[i];
        }
        if (c[i] != c[i] || !valid[i]) c[i] = -INFINITY;   // NaN ranks lowest
    }

    // allowed experts: those of the kept groups (every expert for softmax)
    unsigned long long kept = ~0ull;
    int gsize = E;
    if (sig) {
        const int G = a.num_groups;
        gsize = E / G;
        double my_gscore = -INFINITY;   // lane g < G: the score of group g
        if (gsize <= kWave && kWave % gsize == 0) {
            // in every register slot the lanes form aligned runs of gsize that
            // each hold one group: a segmented top-2 merge over the run
            double m1[EP], m2[EP];
#pragma unroll
            for (int i = 0; i < EP; ++i) { m1[i] = c[i]; m2[i] = -INFINITY; }
            for (int o = gsize >> 1; o >= 1; o >>= 1) {
#pragma unroll
                for (int i = 0; i < EP; ++i) {
                    const double p1 = shfl_xor_f64(m1[i], o), p2 = shfl_xor_f64(m2[i], o);
                    const double n1 = fmax(m1[i], p1);
                    m2[i] = fmax(fmin(m1[i], p1), fmax(m2[i], p2));
                    m1[i] = n1;
                }
            }
            const int first = (lane * gsize) & (kWave - 1), slot = (lane * gsize) >> 6;
#pragma unroll
            for (int i = 0; i < EP; ++i) {
                const double gs = a.group_top == 2 ? m1[i] + m2[i] : m1[i];
                const double v = shfl_f64(gs, first);
                if (lane < G && i == slot) my_gscore = v;
            }
        } else {
            for (int g = 0; g < G; ++g) {
                double m1 = -INFINITY, m2 = -INFINITY;   // two largest c of group g held here
#pragma unroll
                for (int i = 0; i < EP; ++i) {
                    const int e = lane + kWave * i;
                    if (valid[i] && e / gsize == g) {
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
        }
        // rank of group `lane` among the groups (scalar reads of each score)
        int rank = 0;
        for (int h = 0; h < G; ++h) {
            const double o = readlane_f64(my_gscore, h);
            if (route_better(o, h, my_gscore, lane)) ++rank;
        }
        kept = __ballot(lane < G && rank < a.topk_group);
    }

    uint64_t key[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) {
        const int e = lane + kWave * i;
        const bool allowed = valid[i] && ((kept >> (e / gsize)) & 1ull);
        key[i] = allowed ? route_key(c[i]) : 0ull;
    }
    // p = the k-th largest key (at least k experts are allowed, all keys > 0)
    const int k = a.k;
    uint64_t p = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = p | (1ull << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < EP; ++i) n += __popcll(__ballot(key[i] >= cand));
        if (n >= k) p = cand;
    }
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < EP; ++i) n_gt += __popcll(__ballot(key[i] > p));
    int need = k - n_gt;   // keys equal to p, taken in ascending expert order
    bool chosen[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) {
        const uint64_t m = __ballot(key[i] == p);
        const int take = min(need, __popcll(m));
        const bool eq = (m >> lane) & 1ull;
        const int below = __popcll(m & ((1ull << lane) - 1ull));
        chosen[i] = key[i] > p || (eq && below < take);
        need -= take;
    }
    // rank of each chosen expert among the chosen: larger key, or equal key
    // and lower id, goes first
    int rk[EP];
    uint64_t cm[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) { rk[i] = 0; cm[i] = __ballot(chosen[i]); }
#pragma unroll
    for (int i2 = 0; i2 < EP; ++i2) {
        uint64_t m = cm[i2];
        while (m) {
            const int l2 = __builtin_ctzll(m);
            m &= m - 1ull;
            const uint64_t ky = readlane_u64(key[i2], l2);
            const int ey = l2 + kWave * i2;
#pragma unroll
            for (int i = 0; i < EP; ++i) {
                const int e = lane + kWave * i;
                if (ky > key[i] || (ky == key[i] && ey < e)) ++rk[i];
            }
        }
    }
    // lane j receives the expert of rank j and its s (sigmoid) or logit
    int my_id = -1;
    double my_s = 0.0;
#pragma unroll
    for (int i = 0; i < EP; ++i) {
        uint64_t m = cm[i];
        const double val = sig ? sv[i] : (double)lg[i];
        while (m) {
            const int l2 = __builtin_ctzll(m);
            m &= m - 1ull;
            const int r = __builtin_amdgcn_readlane(rk[i], l2);
            const double v = readlane_f64(val, l2);
            if (lane == r) { my_id = l2 + kWave * i; my_s = v; }
        }
    }

    float w;
    if (sig) {
        double sum = lane < k ? my_s : 0.0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sum += shfl_xor_f64(sum, o);
        w = (float)(my_s / sum * (double)a.scale);
    } else {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < EP; ++i)
            if (valid[i]) mx = fmaxf(mx, lg[i]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        float se = 0.0f;
#pragma unroll
        for (int i = 0; i < EP; ++i)
            if (valid[i]) se += expf(lg[i] - mx);
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

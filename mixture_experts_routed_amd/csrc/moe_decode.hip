// moe_decode.hip - gather-GEMV form of the routed-experts layer for a
// handful of tokens, in one persistent launch.  Model card "DeepSeek-OCR-2
// MoE experts", description: the decode op handles about 1-4 tokens with two
// persistent-shape phases, without a per-expert host loop and without a
// device-to-host sync, streaming only the selected experts' weights.
//
// One workgroup per compute unit (all resident), 8 waves:
//  - phase 1 (waves 0-4): the (distinct selected expert u, f) pairs, n_u * F
//    of them, are split evenly over the workgroups (wave 4, which also
//    polls, takes a smaller share of its workgroup's).  A wave streams the
//    gate row f and the up row F + f of expert u (each byte read once, two
//    steps of rows in flight), dots them with every token's row (branch-free:
//    this phase is bound by the weight stream) and, for each token that
//    chose u, stores W * silu(gate . x) * (up . x) as bf16 into the
//    workspace row of the (expert, token)'s representative slot, with
//    device-scope stores (W is the summed routing weight of the token's
//    slots on u);
//  - hand-off: once all five waves' stores have completed, wave 4 stores
//    the workgroup's flag (a 64-bit word made from the call's stamp) and
//    polls the flags of the whole grid (bounded by a clock limit), then
//    copies all of h into LDS with device-scope loads and raises an LDS
//    flag.  The stamp comes from a generation word that workgroup 0
//    advances once every flag is seen, so consecutive calls (also replays of
//    a captured graph) never match an old flag;
//  - phase 2: the H output rows are split evenly over the grid, and a
//    workgroup's (row, expert) tasks over waves 0-3 and 5-7.  Waves 5-7
//    request their down rows at kernel start and hold them in registers;
//    waves 0-3 request theirs after their gate/up work.  A step dots a
//    batch of down rows with the h rows of the expert's representatives
//    (from LDS; tokens that did not choose the expert are skipped) and sums
//    all of them across the wave at once (register-swap and DPP moves);
//    y[row][representative] goes to LDS;
//  - out[t][c] = sum of y over token t's representatives in slot order
//    (+ residual), written once.
// So the layer is one launch: no partial sums, no combine kernel, no float
// atomics, and the result does not depend on timing or grid size.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_route.h"

namespace moe {

constexpr int kDecThreads = 512;
constexpr int kDecUpWaves = 5;                    // waves 0-4: gate/up rows and h
constexpr int kDecDownWaves = 8 - kDecUpWaves;    // waves 5-7: down rows from kernel start
constexpr int kDecPollWave = kDecUpWaves - 1;     // wave 4: the hand-off
constexpr int kDecP2Waves = 7;                    // waves with down-phase tasks
constexpr int kDecUpShare = 3;                    // phase-1 share of waves 0-3 ...
constexpr int kDecUpTotal = 4 * kDecUpShare + 2;  // ... and of wave 4 (2), out of 14
// gate/up row pairs per wave step (two steps in flight): three for one token
// and H <= 1536, otherwise two (the token rows take more registers)
template <int NT, int NCH>
constexpr int pair_batch() { return NT == 1 && NCH <= 3 ? 3 : 2; }

// More device-scope (sc1) stores, next to those of moe_device.h.
__device__ __forceinline__ void st_dev_f32(float* p, float v) {
    __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u16(uint16_t* p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Weight rows are read through buffer resources: a load past the resource's
// size returns zeros without a memory access.  A resource of size 0 serves
// the tasks of a step past the end of a wave's work, and an offset beyond
// the size serves the lanes past the end of a row, so no load sits behind a
// branch (the waits the compiler derives stay exact) and none costs traffic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset `off`, marked as streamed once (nt = 2).
__device__ __forceinline__ uint4 load_nt16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// Sum over the 64 lanes of each of the N = 2^n values v[0..N): afterwards
// lane l holds the total of value l >> (6 - n).  Each halving step pairs
// every lane with one whose lane bit b differs and trades half of the values
// with it: the lanes with bit b clear keep the lower half, the others the
// upper.  Bits 5 and 4 use the gfx950 row-swap moves (v_permlane32_swap:
// upper half of one register <-> lower half of the other; v_permlane16_swap:
// odd rows of one <-> even rows of the other), which need no selects; bits
// 3 .. 0 use DPP moves within a row (mirror, half-mirror, quad permutes),
// whose pairings also differ in exactly that bit.  N values take N - 1 moves
// plus 6 - n for the last one, all without LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_level(float lo, float hi, bool upper) {
    const float keep = upper ? hi : lo, send = upper ? lo : hi;
    return keep + dpp_f<CTRL>(send);
}
// one halving level at lane bit B (5 .. 0)
template <int B>
__device__ __forceinline__ float trade(float lo, float hi, int lane) {
    if constexpr (B == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (B == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        constexpr int ctrl = B == 3 ? 0x140 : B == 2 ? 0x141 : B == 1 ? 0x4E : 0xB1;
        // both operands as plain registers: a select between two array
        // elements would otherwise become an indexed access
        asm("" : "+v"(lo), "+v"(hi));
        return dpp_level<ctrl>(lo, hi, (lane >> B) & 1);
    }
}
// t + the t of the partner lane at lane bit B
template <int B>
__device__ __forceinline__ float fold(float t) {
    if constexpr (B == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (B == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        return t + dpp_f<B == 3 ? 0x140 : B == 2 ? 0x141 : B == 1 ? 0x4E : 0xB1>(t);
    }
}
// the sum over lane bits B .. 0
template <int B>
__device__ __forceinline__ float fold_down(float t) {
    if constexpr (B < 0) return t;
    else return fold_down<B - 1>(fold<B>(t));
}
template <int N, int B = 5>
__device__ __forceinline__ float transpose_sum(float (&v)[N], int lane) {
    if constexpr (N == 1) {
        return fold_down<B>(v[0]);
    } else {
        float w[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) w[i] = trade<B>(v[i], v[i + N / 2], lane);
        return transpose_sum<N / 2, B - 1>(w, lane);
    }
}

// acc + the dot product of 8 bf16 pairs by four v_dot2c_f32_bf16 (the bf16
// products are exact in fp32; only the accumulation rounds).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
    return acc;
}

// The flag word of a call's stamp: the splitmix64 finaliser of the stamp.
// It is a bijection, so consecutive stamps (the generation word counts up by
// one per call) never share a flag word; and the small integers another
// entry point leaves in a shared workspace (counts, offsets) cannot pass for
// one the way the stamp itself could: after a grouped call whose routing
// gives experts 0, 1, 2 the counts 0, 1, 0, the word at the generation's
// offset plus one equals the second flag word its offsets left behind.
__device__ __forceinline__ uint64_t flag_word(uint64_t stamp) {
    uint64_t z = stamp;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// Workspace of the gather-GEMV form (all offsets fixed, see decode_ws_bytes).
struct DecodeWs {
    uint64_t* gen;     // generation word
    uint64_t* flags;   // one per workgroup
    uint32_t* err;     // set when a hand-off wait timed out
    uint16_t* h;       // [P][F] bf16
};

// Routing of the P <= 32 slots as every wave holds it: lane l describes slot
// l % 32 (both halves of the wave alike) and, for l < n_u, distinct expert l.
// The h row of (expert u, token t) is stored once, in the row of the first
// slot with that expert and token (its representative), already multiplied
// by W = the sum of the weights of u's slots of token t (a token naming an
// expert twice gets both weights), so the down phase needs no weights.
struct DecRouting {
    int n_u;        // distinct experts, in order of first appearance
    int u_s;        // this lane's slot: its distinct expert (-1 dropped)
    int t_s;        // its token
    bool rep;       // it is the representative of (u_s, t_s)
    float W;        // the summed weight of (u_s, t_s) (on representatives)
    int ue;         // lane u < n_u: expert id of u
    uint32_t repm;  // lane u < n_u: representative slots of u
};

// The distinct experts of the routing, which is all the first weight
// requests need.  e: the expert (-1 dropped) of slot lane % 32 (lanes of
// slots >= P: -1).
struct DecExperts {
    int n_u;      // distinct experts, in order of first appearance
    int u_s;      // this lane's slot: its distinct expert (-1 dropped)
    int ue;       // lane u < n_u: expert id of u (-1 otherwise)
};
__device__ __forceinline__ DecExperts dec_experts(const int e, int P) {
    const int lane = threadIdx.x & 63, ls = lane & 31;
    DecExperts x;
    int first = ls;
    for (int q = 0; q < P; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        if (q < first && eq == e) first = q;
    }
    uint32_t fm = (uint32_t)__ballot(e >= 0 && first == ls);   // first slots (lanes 0-31)
    x.n_u = __popc(fm);
    x.u_s = e >= 0 ? __popc(fm & ((1u << first) - 1u)) : -1;
    x.ue = -1;
    for (int u = 0; fm; ++u) {   // u-th set bit of fm: the first slot of expert u
        const int eq = __builtin_amdgcn_readlane(e, __builtin_ctz(fm));
        fm &= fm - 1u;
        if (lane == u) x.ue = eq;
    }
    return x;
}

// The rest of the routing, derived while the first weight requests are in
// flight.  wsl: the weight of slot lane % 32 (lanes of slots >= P: 0).
__device__ __forceinline__ DecRouting dec_routing(const int e, const float wsl, int P, int k,
                                                  const DecExperts& x) {
    const int lane = threadIdx.x & 63, ls = lane & 31;
    DecRouting r;
    r.n_u = x.n_u;
    r.u_s = x.u_s;
    r.ue = x.ue;
    r.t_s = ls / k;
    int rep = ls;
    float W = 0.0f;
    for (int q = 0; q < P; ++q) {   // slot order: a fixed summation order
        const int uq = __builtin_amdgcn_readlane(r.u_s, q);
        const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsl), q));
        if (uq == r.u_s && q / k == r.t_s) {
            rep = min(rep, q);
            W += wq;
        }
    }
    r.rep = e >= 0 && rep == ls;
    r.W = W;
    r.repm = 0u;
    for (int q = 0; q < r.n_u; ++q) {
        const uint32_t m = (uint32_t)__ballot(r.rep && r.u_s == q);
        if (lane == q) r.repm = m;
    }
    return r;
}

// One workgroup per CU.  NT = 1 (one token) or 4 (2-4 tokens; token rows
// past T are zero); NCH = 16-byte chunks per lane of an H row (H <= 512 NCH);
// NCF = chunks per lane of an F row; ROUTED: the workgroup routes the tokens
// itself from router logits first.
template <int NT, int NCH, int NCF, bool ROUTED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const uint16_t* __restrict__ x, const ExpertWeights w13, const ExpertWeights w2,
    const int32_t* __restrict__ idx, const float* __restrict__ wts,
    const uint16_t* __restrict__ residual, int T, int k, int E, int H, int F, int S,
    uint16_t* __restrict__ out, DecodeWs ws, uint64_t spin_ticks,
    const RouteArgs ra, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
    constexpr int DB = 16 / NCF;                    // down rows per phase-2 step
    constexpr int kPairBatch = pair_batch<NT, NCH>();
    __shared__ u32x4 h_lds[kDecodeHBytes / 16];     // h rows [P][F], bf16
    __shared__ float y_lds[kDecodeMaxRows][kDecodeMaxSlots];   // per (row, representative slot)
    __shared__ int32_t slot_e[kDecodeMaxSlots];     // expert of each slot (-1 dropped)
    __shared__ float slot_w[kDecodeMaxSlots];       // routing weight of each slot
    __shared__ int rep_tab[kDecodeMaxSlots][kDecodeMaxT];   // representative slot of (u, token), -1 none
    __shared__ int arrive, timed_out, h_ready;

    // the wave index as a scalar: everything derived from it (task ranges,
    // buffer resources) stays in scalar registers instead of being
    // re-derived per lane around every load
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, b = blockIdx.x;
    const int P = T * k;
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();

    // ---------------------------------------------------------------- set-up
    // Request order: the routing (the first weight requests depend on it),
    // then the token rows, and neither is used before both are requested,
    // so the two round trips overlap.
    // Given ids: every wave loads slot lane % 32 into its own lanes (no LDS
    // staging, so the barrier below does not wait for these loads).  k
    // counts the S shared slots of each token (experts E-S .. E-1, weight 1)
    // after its k-S routed ones, read from idx / wts [T, k-S].
    // (the pointers these requests need come with the first scalar loads
    // of the arguments, not one round trip later)
    asm volatile("" ::"s"(idx), "s"(wts), "s"(x), "s"(S));
    const int ls = lane & 31, kr = k - S, t_ls = ls / k, j_ls = ls - t_ls * k;
    int e_raw = -1;
    float w_raw = 0.0f;
    if (!ROUTED && ls < P && j_ls < kr) {
        e_raw = idx[t_ls * kr + j_ls];
        w_raw = wts[t_ls * kr + j_ls];
    }
    // the token rows (phase-1 waves), through a buffer resource: chunks past
    // a row's end and tokens past T read zeros (an offset beyond the bound)
    // instead of being selected out, which would wait for the loads here
    uint4 xv[NT][NCH];
    const int nch = H / 8;
    if (wave < kDecUpWaves) {
        const rsrc_t xr = make_rsrc(x, (uint32_t)(T * H * 2));
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = lane + 64 * i;
                const bool ok = t < T && c < nch;
                xv[t][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    xr, ok ? (uint32_t)(t * H + c * 8) * 2 : 0x80000000u, 0, 0));
            }
    }
    // this call's generation (read by the poll wave after its first weight
    // requests; every workgroup reads it before its flag goes out, and
    // workgroup 0 advances it only after seeing every flag)
    uint64_t gen = 0;
    // the weight arguments: loaded now, while the routing is in flight (the
    // compiler would otherwise load them next to their first use, the first
    // weight requests, and wait for them there)
    asm volatile("" ::"s"(w13.base), "s"(w13.shared), "s"(w13.n_routed), "s"(w2.base), "s"(w2.shared),
                 "s"(w2.n_routed));
    if (ROUTED) {
        if (wave < T) {
            int id;
            float wt;
            if (ra.E <= 64) route_token_lanes<1>(ra, wave, lane, id, wt);
            else if (ra.E <= 128) route_token_lanes<2>(ra, wave, lane, id, wt);
            else route_token_lanes<8>(ra, wave, lane, id, wt);
            if (lane < k) {
                slot_e[wave * k + lane] = (unsigned)id < (unsigned)E ? id : -1;
                slot_w[wave * k + lane] = wt;
                if (b == 0) {
                    idx_out[wave * k + lane] = id;
                    w_out[wave * k + lane] = wt;
                }
            }
        }
    }
    int e_l = -1;
    float w_l = 0.0f;
    if (!ROUTED && ls < P) {
        e_l = j_ls < kr ? ((unsigned)e_raw < (unsigned)(E - S) ? e_raw : -1) : E - S + (j_ls - kr);
        w_l = j_ls < kr ? w_raw : 1.0f;
    }
    if (tid == 0) {
        arrive = 0;
        timed_out = 0;
        h_ready = 0;
    }
    lds_barrier();
    if (ROUTED && (lane & 31) < P) {
        e_l = slot_e[lane & 31];
        w_l = slot_w[lane & 31];
    }
    const DecExperts X = dec_experts(e_l, P);
    const int n_u = X.n_u;
    // The rest of the routing and the tables of the products, once a wave's
    // first weight requests are out: the representatives, their weights,
    // lane u < n_u: the representative slot of (u, token t) (-1 if none).
    DecRouting R;
    int rep_of[NT];
    auto finish_routing = [&]() {
        R = dec_routing(e_l, w_l, P, k, X);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t tm = t < T ? R.repm & (uint32_t)(((1ull << k) - 1ull) << (t * k)) : 0u;
            rep_of[t] = tm ? __builtin_ctz(tm) : -1;
        }
        if (tid < kDecodeMaxSlots * kDecodeMaxT) {   // waves 0-1
            const int u = tid / kDecodeMaxT, t = tid % kDecodeMaxT;
            const uint32_t m = (uint32_t)__shfl(R.repm, u, kWave);
            const uint32_t tm = t < T ? m & (uint32_t)(((1ull << k) - 1ull) << (t * k)) : 0u;
            rep_tab[u][t] = u < n_u && tm ? __builtin_ctz(tm) : -1;
        }
    };

    // Phase-2 tasks (row r of [c0, c1), expert u), u fastest, in contiguous
    // ranges.  Waves 5, 6, 7 fetch their rows at kernel start and hold them
    // in registers; waves 0-3 fetch theirs after their gate/up work; wave 4
    // polls the flags.  When every wave needs at most one step, the tasks go
    // out in whole steps of DB rows, waves 5-7 first, then waves 0-3 (a
    // step's rows past the end would still be loaded and multiplied);
    // otherwise waves 5-7 take two steps each first and waves 0-3 split the
    // rest.
    // (32-bit quotients: b * H < 2^21 and b * N1 < 2^26 at the decode limits)
    // (worked out by each wave where it first needs them: the gate/up
    // waves after their first weight requests)
    int c0 = 0, c1 = 0, ta = 0, ntask = 0;
    auto down_tasks = [&]() {
        c0 = (int)((uint32_t)(b * H) / (uint32_t)G);
        c1 = (int)((uint32_t)((b + 1) * H) / (uint32_t)G);
        const int ntask_wg = (c1 - c0) * n_u;
        const int npre = min(ntask_wg, kDecDownWaves * 2 * DB);
        int tb = 0;
        if (ntask_wg <= kDecP2Waves * DB) {
            if (wave != kDecPollWave) {
                const int q = wave >= kDecUpWaves ? wave - kDecUpWaves : wave + kDecDownWaves;   // 0..6
                ta = min(q * DB, ntask_wg);
                tb = min((q + 1) * DB, ntask_wg);
            }
        } else if (wave >= kDecUpWaves) {
            const int q = wave - kDecUpWaves;
            ta = npre * q / kDecDownWaves;
            tb = npre * (q + 1) / kDecDownWaves;
        } else if (wave != kDecPollWave) {
            const int rest = ntask_wg - npre;
            ta = npre + rest * wave / kDecPollWave;
            tb = npre + rest * (wave + 1) / kDecPollWave;
        }
        ntask = tb - ta;
    };
    const int nchf = F / 8;
    uint4 da[DB][NCF], db[DB][NCF];
    auto load_down = [&](uint4 (&buf)[DB][NCF], int step) {
        const int t0 = ta + step * DB;
        int rr = t0 / max(n_u, 1), u = t0 - rr * max(n_u, 1);
#pragma unroll
        for (int i = 0; i < DB; ++i) {
            const bool real = step * DB + i < ntask;
            // a task past the end reads through an empty resource (zeros)
            const rsrc_t m = make_rsrc(w2.expert(__builtin_amdgcn_readlane(X.ue, real ? u : 0), (int64_t)H * F),
                                       real ? (uint32_t)H * F * 2 : 0u);
            const uint32_t row = (uint32_t)(c0 + rr) * F;
#pragma unroll
            for (int j = 0; j < NCF; ++j) {
                // chunks past the row end read zeros (offset beyond the bound)
                const int ch = lane + 64 * j;
                buf[i][j] = load_nt16(m, ch < nchf ? (row + ch * 8) * 2 : 0x80000000u);
            }
            if (++u == n_u) {
                u = 0;
                ++rr;
            }
        }
    };

    // --------------------------------------------------------------- phase 1
    // (the prefetch of waves 5-7 is the other branch, so that the two sets
    // of staging registers are never live together)
    if (wave < kDecUpWaves) {
        const int N1 = n_u * F;
        const int p0 = (int)((uint32_t)(b * N1) / (uint32_t)G), p1 = (int)((uint32_t)((b + 1) * N1) / (uint32_t)G);
        // shares 3, 3, 3, 3, 2 (of 14): wave 4 shares a SIMD with wave 0, so
        // it issues only in wave 0's idle slots and sends its first requests
        // behind those of the other seven waves; with an even share it ended
        // phase 1 last in every workgroup (T=4: 27 us against 21.5 us).
        // The shares are whole batches of kPairBatch pairs, so that only the
        // workgroup's last batch can be partial: a partial batch still issues
        // its loads past the end (through empty resources, to keep the waits
        // exact), and at T=1 cutting pairs instead of batches left a partial
        // batch in four waves of every workgroup (27 pair loads for 21 pairs)
        const int cq0 = kDecUpShare * wave, cq1 = wave + 1 < kDecUpWaves ? cq0 + kDecUpShare : kDecUpTotal;
        const int nbt = (p1 - p0 + kPairBatch - 1) / kPairBatch;   // the workgroup's batches
        const int q0 = p0 + (int)((uint32_t)(nbt * cq0) / kDecUpTotal) * kPairBatch;
        const int q1 = min(p0 + (int)((uint32_t)(nbt * cq1) / kDecUpTotal) * kPairBatch, p1);
        const int nstep = (q1 - q0 + kPairBatch - 1) / kPairBatch;
        const int u0 = n_u > 0 ? q0 / F : 0, f0 = q0 - u0 * F;
        // pair q0 + i is (u, f): f0 + i carried into the following experts
        auto pair_uf = [&](int i, int& u, int& f) {
            f = f0 + i;
            u = u0;
            while (f >= F) {
                f -= F;
                ++u;
            }
        };
        uint4 wa[kPairBatch][2][NCH], wb[kPairBatch][2][NCH];
        auto load_pairs = [&](uint4 (&buf)[kPairBatch][2][NCH], int step) {
#pragma unroll
            for (int j = 0; j < kPairBatch; ++j) {
                const int i = step * kPairBatch + j;
                const bool real = q0 + i < q1;
                int u, f;
                pair_uf(real ? i : 0, u, f);
                // a pair past the end reads through an empty resource (zeros)
                const rsrc_t m = make_rsrc(w13.expert(__builtin_amdgcn_readlane(X.ue, u), (int64_t)2 * F * H),
                                           real ? (uint32_t)F * H * 4 : 0u);
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const uint32_t row = (uint32_t)(r ? F + f : f) * H;
#pragma unroll
                    for (int i2 = 0; i2 < NCH; ++i2) {
                        // a chunk past the row end repeats the last one and
                        // meets a zeroed token chunk
                        const int ch = min(lane + 64 * i2, nch - 1);
                        buf[j][r][i2] = load_nt16(m, (row + ch * 8) * 2);
                    }
                }
            }
        };
        // value (j * 2 + r) * NT + t of a step: row r (gate, up) of pair j
        // dotted with token t
        constexpr int NV1 = kPairBatch * 2 * NT;
        constexpr int NVP1 = NV1 <= 8 ? 8 : NV1 <= 16 ? 16 : NV1 <= 32 ? 32 : 64;
        constexpr int LB1 = 6 - __builtin_ctz(NVP1);
        auto compute_pairs = [&](const uint4 (&buf)[kPairBatch][2][NCH], int step) {
            float v[NVP1];
#pragma unroll
            for (int i = NV1; i < NVP1; ++i) v[i] = 0.0f;
#pragma unroll
            for (int j = 0; j < kPairBatch; ++j)
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        float acc = 0.0f;
#pragma unroll
                        for (int i = 0; i < NCH; ++i) acc = dot8_bf16(buf[j][r][i], xv[t][i], acc);
                        v[(j * 2 + r) * NT + t] = acc;
                    }
            const float tot = transpose_sum<NVP1>(v, lane);
            // lane (j, s): pair j of the step, slot s (its representative row)
            const int sl = lane & 31, ts = min(R.t_s, NT - 1);
#pragma unroll
            for (int jb = 0; jb < kPairBatch; jb += 2) {
                const int j = jb + (lane >> 5);
                const float g = __shfl(tot, ((j * 2) * NT + ts) << LB1, kWave);
                const float up = __shfl(tot, ((j * 2 + 1) * NT + ts) << LB1, kWave);
                const int i = step * kPairBatch + j;
                if (j < kPairBatch && q0 + i < q1 && R.rep) {
                    int u, f;
                    pair_uf(i, u, f);
                    if (R.u_s == u)
                        st_dev_u16(ws.h + (int64_t)sl * F + f, (uint16_t)f32_to_bf16(R.W * (silu(g) * up)));
                }
            }
        };
        // two buffers in turn: a step's rows are requested two steps ahead
        // (the conditions are wave-uniform)
        if (nstep > 0) load_pairs(wa, 0);
        if (nstep > 1) load_pairs(wb, 1);
        finish_routing();
        down_tasks();
        if (wave == kDecPollWave) gen = ld_dev_u64(ws.gen);
        for (int st = 0; st < nstep; st += 2) {
            compute_pairs(wa, st);
            if (st + 2 < nstep) load_pairs(wa, st + 2);
            if (st + 1 < nstep) compute_pairs(wb, st + 1);
            if (st + 3 < nstep) load_pairs(wb, st + 3);
        }
        wait_vm_all();   // this wave's h stores have completed
        if (lane == 0) atomicAdd(&arrive, 1);
        if (wave == kDecPollWave) {
            // once the other four have stored their h: publish this
            // workgroup's, then wait for every workgroup's
            while (__hip_atomic_load(&arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kDecUpWaves)
                __builtin_amdgcn_s_sleep(1);
            // (gen enters arithmetic only here: computed where it was loaded,
            // the wave would wait there for every load before it)
            uint64_t g = gen;
            asm volatile("" : "+v"(g));
            const uint64_t stamp = g + 1;
            const uint64_t flag = flag_word(stamp);
            if (lane == 0) st_dev_u64(ws.flags + b, flag);
            bool ok = false;
            if (G <= 4 * kWave) {
                // two polls in flight, each read while the other's loads are
                // out, so the last flag to land is seen about half a round
                // trip sooner than by polls one after the other
                uint64_t pa[4], pb[4];
                auto issue = [&](uint64_t (&f)[4]) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) f[i] = ld_dev_u64(ws.flags + min(lane + kWave * i, G - 1));
                };
                auto seen = [&](const uint64_t (&f)[4]) {
                    bool all = true;
#pragma unroll
                    for (int i = 0; i < 4; ++i) all &= f[i] == flag;
                    return __all(all);
                };
                issue(pa);
                __builtin_amdgcn_s_sleep(8);
                issue(pb);
                while (true) {
                    if (seen(pa)) {
                        ok = true;
                        break;
                    }
                    issue(pa);
                    if (seen(pb)) {
                        ok = true;
                        break;
                    }
                    issue(pb);
                    if (__builtin_amdgcn_s_memrealtime() - t_start > spin_ticks) break;
                }
            } else {
                while (true) {
                    bool all = true;
                    for (int q = lane; q < G; q += 64) all &= ld_dev_u64(ws.flags + q) == flag;
                    if (__all(all)) {
                        ok = true;
                        break;
                    }
                    if (__builtin_amdgcn_s_memrealtime() - t_start > spin_ticks) break;
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (!ok && lane == 0) {
                timed_out = 1;
                atomicOr(ws.err, 1u);
            }
            // every workgroup has read this call's generation: advance it
            if (b == 0 && lane == 0) st_dev_u64(ws.gen, stamp);
            // h of every slot into LDS (device-scope loads), 1 KB per instruction
            const int nkb = (P * F * 2 + 1023) / 1024;
            for (int q = 0; q < nkb; ++q)
                dma16_dev((const char*)ws.h + (int64_t)q * 1024 + lane * 16, (char*)h_lds + q * 1024);
            wait_vm_all();
            __hip_atomic_store(&h_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else if (ntask > 0) {
            load_down(da, 0);
            if (ntask > DB) load_down(db, 1);
        }
    } else {
        down_tasks();
        if (ntask > 0) {
            load_down(da, 0);
            if (ntask > DB) load_down(db, 1);
        }
        finish_routing();
    }

    // --------------------------------------------------------------- phase 2
    if (ntask > 0) {
        // value i * NT + t of a step: task i's down row dotted with the h row
        // of its expert's representative slot for token t (zero weights past
        // the end; a missing representative gives a value that is dropped)
        constexpr int NV = DB * NT;
        constexpr int NVP = NV <= 8 ? 8 : NV <= 16 ? 16 : NV <= 32 ? 32 : 64;
        constexpr int LB = 6 - __builtin_ctz(NVP);   // lanes per value: 1 << LB
        int hch[NCF];   // this lane's h chunks (tail lanes: the last one, times zero weights)
#pragma unroll
        for (int j = 0; j < NCF; ++j) hch[j] = min(lane + 64 * j, nchf - 1);
        auto compute_down = [&](const uint4 (&buf)[DB][NCF], int step) {
            const int t0 = ta + step * DB;
            int rr = t0 / n_u, u = t0 - rr * n_u;
            float v[NVP];
#pragma unroll
            for (int i = NV; i < NVP; ++i) v[i] = 0.0f;
#pragma unroll
            for (int i = 0; i < DB; ++i) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    // scalar: the h row of u's representative for token t;
                    // with 2-4 tokens an expert is usually routed for only
                    // some of them, and the others' values would be dropped
                    // (a uniform branch: no h read, no dot products)
                    const int rraw = __builtin_amdgcn_readlane(rep_of[t], u);
                    float part = 0.0f;
                    if (NT == 1 || rraw >= 0) {
                        const u32x4* hs = h_lds + max(rraw, 0) * (F / 8);
#pragma unroll
                        for (int j = 0; j < NCF; ++j) {
                            const u32x4 hv = hs[hch[j]];
                            part = dot8_bf16(buf[i][j], make_uint4(hv.x, hv.y, hv.z, hv.w), part);
                        }
                    }
                    v[i * NT + t] = part;
                }
                if (++u == n_u) {
                    u = 0;
                    ++rr;
                }
            }
            const float tot = transpose_sum<NVP>(v, lane);
            const int vi = lane >> LB;
            if ((lane & ((1 << LB) - 1)) == 0 && vi < NV) {
                const int i = vi / NT, t = vi - (vi / NT) * NT;
                if (step * DB + i < ntask) {
                    const int task = t0 + i;
                    const int rw = task / n_u, uw = task - rw * n_u;
                    const int r = rep_tab[uw][t];
                    if (r >= 0) y_lds[rw][r] = tot;
                }
            }
        };
        const int nsteps = (ntask + DB - 1) / DB;
        // the poll wave's signal that h is in LDS (it always comes: the
        // poll is bounded)
        while (__hip_atomic_load(&h_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
            __builtin_amdgcn_s_sleep(1);
        for (int st = 0; st < nsteps; st += 2) {
            compute_down(da, st);
            if (st + 2 < nsteps) load_down(da, st + 2);
            if (st + 1 < nsteps) compute_down(db, st + 1);
            if (st + 3 < nsteps) load_down(db, st + 3);
        }
    }
    lds_barrier();   // every row's values are in LDS (and timed_out is final)

    // out[t][c] = sum over token t's representative slots (ascending) of
    // y[c][slot], + residual; one thread per (token, row)
    const uint32_t reps = (uint32_t)__ballot(R.rep);   // lanes 0-31: slots 0-31
    for (int q = tid; q < T * (c1 - c0); q += kDecThreads) {
        const int t = q / (c1 - c0), rr = q - t * (c1 - c0);
        uint32_t tm = reps & (((1u << k) - 1u) << (t * k));   // token t's representative slots
        float o = 0.0f;
        while (tm) {
            const int r = __builtin_ctz(tm);
            tm &= tm - 1u;
            o += y_lds[rr][r];
        }
        if (residual) o += bf16_to_f32(residual[(int64_t)t * H + c0 + rr]);
        out[(int64_t)t * H + c0 + rr] = (uint16_t)f32_to_bf16(timed_out ? __builtin_nanf("") : o);
    }
}

template <int NT, int NCH, int NCF, bool ROUTED>
static int decode_grid() {
    static const int g = std::min(resident_grid((const void*)decode_kernel<NT, NCH, NCF, ROUTED>,
                                                kDecThreads, device_cu_count()),
                                  kDecodeMaxGrid);
    return capped_grid(g);
}

// The wait for the other workgroups' flags gives up after this many ticks of
// the 100 MHz constant clock (100 ms): a wait that long means the grid is
// not resident (other work holds the CUs); the rows then come out NaN and
// the workspace's error word is set.
constexpr uint64_t kSpinTicks = 10000000ull;

template <int NT, int NCH, int NCF, bool ROUTED>
static void launch_one(const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                       const int32_t* idx, const float* w, const uint16_t* residual, int T, int k,
                       int E, int H, int F, uint16_t* out, const DecodeWs& dws, hipStream_t s,
                       const RouteArgs& ra, int32_t* io, float* wo, int S) {
    // at most kDecodeMaxRows output rows per workgroup
    const int G = std::max(decode_grid<NT, NCH, NCF, ROUTED>(), (H + kDecodeMaxRows - 1) / kDecodeMaxRows);
    // (the arguments the first requests need, S included, lie in the first
    // 128 bytes of the argument block: one scalar round trip fetches them)
    MOE_LAUNCH((decode_kernel<NT, NCH, NCF, ROUTED>), dim3(G), dim3(kDecThreads), 0, s, x, w13, w2, idx, w, residual, T, k, E, H, F, S,
               out, dws, kSpinTicks, ra, io, wo);
}

template <int NT, int NCH, bool ROUTED>
static hipError_t launch_ncf(int ncf, const uint16_t* x, const ExpertWeights& w13,
                             const ExpertWeights& w2, const int32_t* idx, const float* w,
                             const uint16_t* residual, int T, int k, int E, int H, int F,
                             uint16_t* out, const DecodeWs& d, hipStream_t s, const RouteArgs& ra,
                             int32_t* io, float* wo, int S) {
    switch (ncf) {
        case 1: launch_one<NT, NCH, 1, ROUTED>(x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S); break;
        case 2: launch_one<NT, NCH, 2, ROUTED>(x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S); break;
        default: launch_one<NT, NCH, 4, ROUTED>(x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S); break;
    }
    return hipGetLastError();
}

template <bool ROUTED>
static hipError_t launch_decode_t(const uint16_t* x, const ExpertWeights& w13,
                                  const ExpertWeights& w2, const int32_t* idx, const float* w,
                                  const uint16_t* residual, int T, int k, int E, int H, int F,
                                  uint16_t* out, void* ws, hipStream_t s, const RouteArgs& ra,
                                  int32_t* io, float* wo, int S) {
    char* base = (char*)ws;
    const DecodeWs d{(uint64_t*)base, (uint64_t*)(base + 256), (uint32_t*)(base + 256 + 8 * kDecodeMaxGrid),
                     (uint16_t*)(base + kDecodeHOffset)};
    const int nch = (H / 8 + 63) / 64;
    const int ncf = (F / 8 + 63) / 64;   // 1, 2, 3 (as 4) or 4
    if (T == 1) {
        switch (nch) {
            case 1: return launch_ncf<1, 1, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
            case 2: return launch_ncf<1, 2, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
            case 3: return launch_ncf<1, 3, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
            case 4: return launch_ncf<1, 4, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
            default: return hipErrorInvalidValue;
        }
    }
    switch (nch) {
        case 1: return launch_ncf<4, 1, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
        case 2: return launch_ncf<4, 2, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
        case 3: return launch_ncf<4, 3, ROUTED>(ncf, x, w13, w2, idx, w, residual, T, k, E, H, F, out, d, s, ra, io, wo, S);
        default: return hipErrorInvalidValue;   // excluded by decode_fast_path
    }
}

hipError_t launch_decode(const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                         const int32_t* idx, const float* w, const uint16_t* residual, int T, int k,
                         int E, int H, int F, uint16_t* out, void* ws, hipStream_t s,
                         const RouteArgs& ra, int32_t* idx_out, float* w_out, int S) {
    if (ra.logits)
        return launch_decode_t<true>(x, w13, w2, idx, w, residual, T, k, E, H, F, out, ws, s, ra,
                                     idx_out, w_out, 0);
    return launch_decode_t<false>(x, w13, w2, idx, w, residual, T, k, E, H, F, out, ws, s, ra,
                                  idx_out, w_out, S);
}

}  // namespace moe

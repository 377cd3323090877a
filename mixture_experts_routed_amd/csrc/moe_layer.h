// moe_layer.h - scheduling of the grouped products shared by the
// stage-by-stage kernels and the one-launch layers (bf16 and fp8), and the
// router-weighted combine.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"
#include "../../include/moe_experts.h"

namespace moe {

// Hooks of the stand-alone kernels: workgroup b takes item xcd_slot(b) and
// then every G-th (consecutive items run on one XCD), stores are plain and
// nothing is waited for (the kernel boundaries order the stages).
struct PlainSched {
    int items;
    __device__ int first() const {
        const int it = xcd_slot(blockIdx.x, gridDim.x);
        return it < items ? it : -1;
    }
    __device__ int next(int it) const {
        return it + (int)gridDim.x < items ? it + (int)gridDim.x : -1;
    }
    __device__ void wait_inputs(const GroupedItem&) const {}
    __device__ void store_u32(void* p, uint32_t v) const { *(uint32_t*)p = v; }
    __device__ void store_u16(uint16_t* p, uint16_t v) const { *p = v; }
    __device__ void store_u8(uint8_t* p, uint8_t v) const { *p = v; }
    __device__ void store_f32(float* p, float v) const { *p = v; }
    // per-row scales of the A operand (one, or four K blocks at once)
    __device__ float load_scale(const float* p) const { return *p; }
    __device__ float4 load_scale4(const float* p) const { return *(const float4*)p; }
    __device__ uint32_t load_scale_word(const uint8_t* p) const { return *(const uint32_t*)p; }
    __device__ void stored(int) const {}
    __device__ void drained() const {}
};

// ------------------------------------------------------------------ combine
// Unit g = (token t, 8 columns c): out = sum_j w[t,j] * y[inv[t*k+j]] in
// slot order, plus the residual if any, in fp32, one rounding to bf16.  y is
// in expert order; inv (from the plan) is -1 for dropped slots, which
// contribute nothing.
__device__ __forceinline__ void combine_unit(const uint16_t* __restrict__ y,
                                             const int32_t* __restrict__ inv,
                                             const float* __restrict__ w,
                                             const uint16_t* __restrict__ residual, int64_t g,
                                             int k, int H, bool nan_out,
                                             uint16_t* __restrict__ out) {
    const int cpr = H / 8;
    const int64_t t = g / cpr;
    const int c = (int)(g - t * cpr) * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
        const int r = inv[t * k + j];
        if (r < 0) continue;
        const float wt = w[t * k + j];
        const uint4 v = *(const uint4*)(y + (int64_t)r * H + c);
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wt * f[i];
    }
    if (residual) {
        float r[8];
        unpack8(*(const uint4*)(residual + t * H + c), r);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += r[i];
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    if (nan_out) o = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
    *(uint4*)(out + t * H + c) = o;
}

// NU units per thread at once with every slot's loads in flight (k <= KM):
// the same sums as combine_unit, for a grid with few waves per CU.
template <int KM, int NU>
__device__ __forceinline__ void combine_units(const uint16_t* __restrict__ y,
                                              const int32_t* __restrict__ inv,
                                              const float* __restrict__ w,
                                              const uint16_t* __restrict__ residual, int64_t g0,
                                              int64_t gstep, int64_t gend, int k, int H,
                                              bool nan_out, uint16_t* __restrict__ out) {
    const int cpr = H / 8;
    int64_t t[NU];
    int c[NU], r[NU][KM];
    float wt[NU][KM];
    uint4 v[NU][KM];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int64_t g = min(g0 + u * gstep, gend - 1);
        t[u] = g / cpr;
        c[u] = (int)(g - t[u] * cpr) * 8;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            r[u][j] = j < k ? inv[t[u] * k + j] : -1;
            wt[u][j] = j < k ? w[t[u] * k + j] : 0.0f;
        }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int j = 0; j < KM; ++j)
            v[u][j] = r[u][j] >= 0 ? *(const uint4*)(y + (int64_t)r[u][j] * H + c[u]) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        if (g0 + u * gstep >= gend) break;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (r[u][j] < 0) continue;
            float f[8];
            unpack8(v[u][j], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += wt[u][j] * f[i];
        }
        if (residual) {
            float rs[8];
            unpack8(*(const uint4*)(residual + t[u] * H + c[u]), rs);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += rs[i];
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        if (nan_out) o = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
        *(uint4*)(out + t[u] * H + c[u]) = o;
    }
}

// ------------------------------------------------------ one-launch layer
// A grouped path in one persistent launch after the plan: gate_up items,
// then down items, then the combine, handed over between workgroups through
// flags in the workspace instead of kernel boundaries (the single-kernel
// idea of the DeepGEMM "Mega MoE" news item, on one GPU).  Workgroup b walks
// the sequence xcd_slot(b) + j G over [gate_up items | down items], so the
// workgroups with one gate_up item fewer start the down items first, and a
// workgroup only ever waits for items earlier in the sequence, held by
// resident workgroups: the waits end.
//  - a gate_up item stores its h tile (and its scales, for quantised h)
//    with device-scope stores; once they
//    have completed in every wave (right after the epilogue) it stores its
//    flag (the call's stamp);
//  - a down item first waits for the flags of its M tile's gate_up items,
//    then reads h rows as usual: no copy of them is in any L2 yet, so the
//    reads fetch the stored values;
//  - a workgroup past its down items stores its down flag; the combine
//    waits for every workgroup's down flag, then sums its share of tokens
//    exactly as combine_kernel does.
// The stamp is the generation word + 1; workgroup 0 advances the word at
// the end, once every workgroup has acknowledged reading it, so flags of
// earlier calls never match.  Waits are bounded by a clock limit: a grid that
// is not resident together gives NaN outputs and sets the error word.
// Hand-off words (64-bit) in the workspace, from one base pointer:
struct LayerSync {
    uint64_t* base;
    __device__ uint64_t* gen() const { return base; }        // generation word
    __device__ uint64_t* err() const { return base + 1; }    // = stamp when a wait timed out
    // dynamic down items, one queue per XCD: (stamp << 32) | items handed out
    __device__ uint64_t* queue(int x) const { return base + 2 + x; }
    __device__ uint64_t* ack() const { return base + 32; }   // [G] workgroup read the generation
    __device__ uint64_t* dflag() const { return base + 32 + kLayerMaxGrid; }   // [G] down items done
    // [kLayerPlanChunks] each: chunk counted / chunk scattered
    __device__ uint64_t* pcount() const { return base + 32 + 2 * kLayerMaxGrid; }
    __device__ uint64_t* pdone() const { return pcount() + kLayerPlanChunks; }
    // [E][kLayerPlanChunks] per-chunk expert counts (expert-major)
    __device__ int32_t* pcnt() const { return (int32_t*)(pdone() + kLayerPlanChunks); }
    __device__ uint64_t* gflag() const {   // [gate_up items]
        return pdone() + kLayerPlanChunks + kLayerPlanChunks * MOE_MAX_EXPERTS / 2;
    }
};

// wave 0 waits until flags[i * stride], i < n, all equal stamp (each wait
// bounded by kLayerSpinTicks of the 100 MHz clock; past it the error word
// takes the stamp); then the whole workgroup passes a barrier
__device__ __forceinline__ void wait_flags(const uint64_t* flags, int n, int stride,
                                           uint64_t stamp, LayerSync sy) {
    if (threadIdx.x < 64) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (true) {
            bool all = true;
            for (int i = threadIdx.x; i < n; i += 64) all &= ld_dev_u64(flags + (int64_t)i * stride) == stamp;
            if (__all(all)) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kLayerSpinTicks) {
                if (threadIdx.x == 0) st_dev_u64(sy.err(), stamp);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    lds_barrier();
}

// gate_up phase (GATE) or down phase of the one-launch layer.
// Slot s = xcd_slot(b) takes gate_up items s, s + G, ... (q + 1 of them for
// s < r, q for s >= r, with NG = q G + r), then its down items.  Down items
// are numbered like gate_up items (expert by expert), and the k-th down item
// of slot s is the item whose number is:
//  - for s >= r and k < c ("early" items, started while the last round of
//    gate_up items still runs): k (G - r) + (s - r), so these come from the
//    first experts, whose gate_up items finished in the earlier rounds;
//  - otherwise c (G - r) + the rank of the slot's sequence position
//    s + (nG(s) + k) G among the positions not taken by early items.
// c = how many down items fit in one gate_up item's time, bounded so that
// the early items stay within the tiles of finished rounds.  Any order is
// deadlock-free: down items wait only for gate_up items, and every
// workgroup runs all its gate_up items first.
// DYN (down phase): items are handed out in order from queue words instead,
// each workgroup claiming one item ahead (its claim for the next item is
// issued before the current item's first loads, so its latency hides
// behind theirs); workgroups that finish their gate_up items early take
// more down items, whatever the items' lengths.  One queue per XCD, over
// blocks of 32 consecutive items (block c on XCD c mod 8, as the stand-alone
// kernels map items), so that the items sharing an expert's weight panels
// and h rows run under one L2; a workgroup whose queue has run dry takes
// items from the next XCD's queue, so that the XCDs finish together.
template <bool GATE, bool DYN = false>
struct LayerSched {
    int items, NG, npg, c;   // npg: gate_up items per M tile
    uint64_t stamp;
    LayerSync sy;
    const int32_t* tile_off;
    int k;
    int* claim;       // DYN: LDS word handing thread 0's claim to every wave
    uint32_t ahead;   // DYN: thread 0's claim for the next item
    int qx = 0;       // DYN: the queue thread 0 takes items from
    // the next item of queue x (0xffffffff when the queue word does not
    // carry this call's stamp)
    __device__ uint32_t claim_from(int x) const {
        const uint64_t old = atomicAdd((unsigned long long*)sy.queue(x), 1ull);
        if ((uint32_t)(old >> 32) != (uint32_t)stamp) return 0xffffffffu;
        const uint32_t kq = (uint32_t)old;
        return (kq / 32) * (32 * kXcds) + 32 * (uint32_t)x + (kq % 32);
    }
    __device__ uint32_t claim_one() const { return claim_from(qx); }
    // items in queue x
    __device__ uint32_t queue_len(int x) const {
        const uint32_t full = (uint32_t)items / (32 * kXcds), rest = (uint32_t)items % (32 * kXcds);
        return full * 32 + (uint32_t)min(max((int)rest - 32 * x, 0), 32);
    }
    // v, or, if v is past the end (queue qx has run dry), an item of the
    // queue with the most items left (its words read at once; synchronous,
    // only at the end of the phase)
    __device__ uint32_t steal_if_dry(uint32_t v) {
        while (v >= (uint32_t)items) {
            uint64_t w[kXcds];
#pragma unroll
            for (int x = 0; x < kXcds; ++x) w[x] = ld_dev_u64(sy.queue(x));
            int best = -1;
            uint32_t most = 0;
#pragma unroll
            for (int x = 0; x < kXcds; ++x) {
                const uint32_t kq = (uint32_t)w[x], n = queue_len(x);
                if ((uint32_t)(w[x] >> 32) == (uint32_t)stamp && kq < n && n - kq > most) {
                    most = n - kq;
                    best = x;
                }
            }
            if (best < 0) break;   // every queue is dry
            qx = best;
            v = claim_from(qx);
        }
        return v;
    }
    __device__ int take(uint32_t v) const {
        if (threadIdx.x == 0) *claim = (int)min(v, (uint32_t)items);
        lds_barrier();
        const int it = *claim;
        return it < items ? it : -1;
    }
    __device__ int down_item(int kk) const {
        const int G = gridDim.x, s = xcd_slot(blockIdx.x, G);
        const int q = NG / G, r = NG % G, nf = G - r;
        if (c > 0 && s >= r && kk < c) return kk * nf + (s - r);
        const int j = (s < r ? q + 1 : q) + kk;            // the position's round
        const int jr = q + 1, jf = q + (c > 0 ? c : 0);    // first rounds not early
        int64_t rank = (int64_t)r * max(0, j - jr) + (int64_t)nf * max(0, j - jf);
        if (j >= jr) rank += min(s, r);
        if (j >= jf) rank += max(0, s - r);
        const int64_t it = (int64_t)c * nf + rank;
        return it < items ? (int)it : -1;
    }
    __device__ int first() {
        const int G = gridDim.x, seq0 = xcd_slot(blockIdx.x, G);
        if (GATE) return seq0 < items ? seq0 : -1;
        if (DYN) {
            uint32_t v = 0xffffffffu;
            if (threadIdx.x == 0) {
                // the queue word carries this call's stamp once workgroup 0
                // has set it (at its start)
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                bool ok = true;
                while ((uint32_t)(ld_dev_u64(sy.queue(blockIdx.x % kXcds)) >> 32) != (uint32_t)stamp) {
                    if (__builtin_amdgcn_s_memrealtime() - t0 > kLayerSpinTicks) {
                        st_dev_u64(sy.err(), stamp);
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (ok) {
                    qx = blockIdx.x % kXcds;
                    v = steal_if_dry(claim_one());
                    ahead = v < (uint32_t)items ? claim_one() : 0xffffffffu;
                } else {
                    ahead = 0xffffffffu;
                }
            }
            return take(v);
        }
        k = 0;
        return down_item(0);
    }
    __device__ int next(int it) {
        if (GATE) return it + (int)gridDim.x < items ? it + (int)gridDim.x : -1;
        if (DYN) {
            uint32_t v = 0;
            if (threadIdx.x == 0) {
                v = ahead == 0xffffffffu ? ahead : steal_if_dry(ahead);
                ahead = v < (uint32_t)items ? claim_one() : 0xffffffffu;
            }
            return take(v);
        }
        return down_item(++k);
    }
    __device__ void wait_inputs(const GroupedItem& gi) const {
        if (GATE) return;
        const int t0e = tile_off[gi.e], mtiles = tile_off[gi.e + 1] - t0e;
        // gate_up items of M tile gi.mt: npg * t0e + panel * mtiles + (mt - t0e)
        wait_flags(sy.gflag() + (int64_t)npg * t0e + (gi.mt - t0e), npg, mtiles, stamp, sy);
    }
    __device__ void store_u32(void* p, uint32_t v) const { st_dev_u32((uint32_t*)p, v); }
    __device__ void store_u16(uint16_t* p, uint16_t v) const {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void store_u8(uint8_t* p, uint8_t v) const {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void store_f32(float* p, float v) const { st_dev_u32((uint32_t*)p, __float_as_uint(v)); }
    // Per-row scales of the A operand.  In the down phase they are the
    // gate_up epilogue's h scales, whose rows are shorter than a cache line:
    // a line can hold rows of two M tiles, and a workgroup that read it for
    // one tile must not keep an old copy of the other tile's rows, so these
    // loads bypass the L2 (device scope).  h codes are read normally: their
    // rows are whole lines, first touched after the tile's flags.
    __device__ float load_scale(const float* p) const {
        if (GATE) return *p;
        return __uint_as_float(__hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT));
    }
    __device__ float4 load_scale4(const float* p) const {
        if (GATE) return *(const float4*)p;
        return make_float4(load_scale(p), load_scale(p + 1), load_scale(p + 2), load_scale(p + 3));
    }
    // four E8M0 scale bytes of the A operand (same reason)
    __device__ uint32_t load_scale_word(const uint8_t* p) const {
        if (GATE) return *(const uint32_t*)p;
        return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // a gate_up item's flag, once its stores have completed in every wave
    // (the next item's first loads, issued before them, have landed too)
    __device__ void stored(int it) const {
        if (!GATE) return;
        wait_vm_all();
        lds_barrier();
        if (threadIdx.x == 0) st_dev_u64(sy.gflag() + it, stamp);
    }
    __device__ void drained() const {
        if (GATE) return;
        wait_vm_all();
        lds_barrier();
        if (threadIdx.x == 0) st_dev_u64(sy.dflag() + blockIdx.x, stamp);
    }
};

// This call's generation word, requested by wave 0 and not waited for
// here: the plan's first loads go out before the wait, so the two round
// trips overlap.
__device__ __forceinline__ uint64_t layer_gen(LayerSync sy) {
    return threadIdx.x < 64 ? ld_dev_u64(sy.gen()) : 0ull;
}
// This call's stamp (the generation word + 1) from layer_gen's value, kept
// in scalar registers (the other waves hold 0 and never use it); the
// workgroup's acknowledgement that it has read the word.
__device__ __forceinline__ uint64_t layer_stamp(uint64_t g, LayerSync sy) {
    uint64_t stamp = 0;
    if (threadIdx.x < 64) {
        asm volatile("" : "+v"(g));   // the load is waited for here, not at its issue
        stamp = g + 1;
        if (threadIdx.x == 0) st_dev_u64(sy.ack() + blockIdx.x, stamp);
    }
    return ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(stamp >> 32)) << 32) |
           __builtin_amdgcn_readfirstlane((uint32_t)stamp);
}

// The routing plan as the layer's first phase, the same arrays as the plan
// kernel's (the ordering rule fixes every entry): the first Gp = min(G,
// kLayerPlanChunks) workgroups each take a contiguous chunk of slots,
//  1. count their slots per (wave, expert) and publish the chunk's counts;
//  2. once every chunk is counted, each sums the counts of all chunks (the
//     totals, their exclusive prefix = offsets and the M-tile prefix) and of
//     the chunks before its own, and scatters its slots in slot order, lanes
//     of one 64-slot step that share an expert ranked by an OR-ed lane mask
//     (as the plan kernel);
//  3. workgroup 0 writes counts, offsets, the tiles and their prefix.
// Every workgroup then waits until every chunk is scattered.  All plan
// stores are device-scope; the arrays are first read after that wait.
// `ldsi`: 56 KB of idle LDS; `gen`: layer_gen's value.  Returns the call's
// stamp (layer_stamp).
__device__ __forceinline__ uint64_t layer_plan(int* ldsi, const int32_t* __restrict__ idx, int P,
                                               int E, int tile_m, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ perm,
                                               int32_t* __restrict__ inv,
                                               int32_t* __restrict__ tiles,
                                               int32_t* __restrict__ ntiles,
                                               int32_t* __restrict__ tile_off, uint64_t gen,
                                               LayerSync sy) {
    constexpr int NW = 8;   // waves of a 512-thread workgroup
    const int G = gridDim.x, b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Gp = min(G, kLayerPlanChunks);
    uint64_t stamp = 0;
    if (b < Gp) {
        int* base = ldsi;                                               // [NW][E]
        unsigned long long* lanes_of = (unsigned long long*)(ldsi + NW * MOE_MAX_EXPERTS);  // [NW][E]
        int* tot = ldsi + 3 * NW * MOE_MAX_EXPERTS;                     // [E]
        int* off = tot + MOE_MAX_EXPERTS;                               // [E + 1]
        int* tsh = off + MOE_MAX_EXPERTS + 1;                           // [E + 1]
        for (int i = tid; i < NW * MOE_MAX_EXPERTS; i += blockDim.x) {
            base[i] = 0;
            lanes_of[i] = 0ull;
        }
        lds_barrier();
        // the chunk, and each wave's 64-aligned run of it
        const int c0 = (int)((int64_t)P * b / Gp), c1 = (int)((int64_t)P * (b + 1) / Gp);
        const int run = ((c1 - c0 + NW * kWave - 1) / (NW * kWave)) * kWave;
        const int s0 = min(c1, c0 + wave * run), s1 = min(c1, s0 + run);
        for (int s = s0 + lane; s < s1; s += kWave) {
            const int e = idx[s];
            if ((unsigned)e < (unsigned)E) atomicAdd(&base[wave * E + e], 1);
        }
        lds_barrier();
        for (int e = tid; e < E; e += blockDim.x) {
            int acc = 0;
            for (int w = 0; w < NW; ++w) acc += base[w * E + e];
            st_dev_u32((uint32_t*)(sy.pcnt() + e * kLayerPlanChunks + b), (uint32_t)acc);
        }
        stamp = layer_stamp(gen, sy);
        wait_vm_all();
        lds_barrier();
        if (tid == 0) st_dev_u64(sy.pcount() + b, stamp);
        wait_flags(sy.pcount(), Gp, 1, stamp, sy);
        // totals, and this chunk's base per expert (chunks before it, then
        // the waves before each wave's run): a thread per expert reads the
        // expert's row of chunk counts in 16-byte loads, all in flight
        // (normal loads: no workgroup reads the counts before every chunk's
        // flag, so no L2 holds an older copy)
        for (int e = tid; e < E; e += blockDim.x) {
            const uint4* row = (const uint4*)(sy.pcnt() + e * kLayerPlanChunks);
            uint4 q[kLayerPlanChunks / 4];
#pragma unroll
            for (int i = 0; i < kLayerPlanChunks / 4; ++i) q[i] = row[i];
            int t = 0, pre = 0;
#pragma unroll
            for (int i = 0; i < kLayerPlanChunks / 4; ++i) {
                const int v4[4] = {(int)q[i].x, (int)q[i].y, (int)q[i].z, (int)q[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 4 * i + j;
                    const int v = c < Gp ? v4[j] : 0;
                    t += v;
                    pre += c < b ? v : 0;
                }
            }
            tot[e] = t;
            for (int w = 0; w < NW; ++w) {
                const int cw = base[w * E + e];
                base[w * E + e] = pre;
                pre += cw;
            }
        }
        lds_barrier();
        if (wave == 0) {   // exclusive prefix of the totals and of the M tiles
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
                if (lane >= o) {
                    c_inc += cu;
                    t_inc += tu;
                }
            }
            int c_run = c_inc - c_sum, t_run = t_inc - t_sum;
            for (int i = 0; i < per; ++i) {
                const int e = e0 + i;
                if (e < E) {
                    off[e] = c_run;
                    tsh[e] = t_run;
                    c_run += tot[e];
                    t_run += (tot[e] + tile_m - 1) / tile_m;
                }
            }
            if (lane == kWave - 1) {
                off[E] = c_inc;
                tsh[E] = t_inc;
            }
        }
        lds_barrier();
        if (b == 0) {
            for (int e = tid; e <= E; e += blockDim.x) {
                st_dev_u32((uint32_t*)(offsets + e), (uint32_t)off[e]);
                st_dev_u32((uint32_t*)(tile_off + e), (uint32_t)tsh[e]);
                if (e < E) {
                    st_dev_u32((uint32_t*)(counts + e), (uint32_t)tot[e]);
                    for (int i = 0; i < tsh[e + 1] - tsh[e]; ++i) {
                        st_dev_u32((uint32_t*)(tiles + 2 * (tsh[e] + i)), (uint32_t)e);
                        st_dev_u32((uint32_t*)(tiles + 2 * (tsh[e] + i) + 1), (uint32_t)(off[e] + i * tile_m));
                    }
                }
            }
            if (tid == 0) st_dev_u32((uint32_t*)ntiles, (uint32_t)tsh[E]);
        }
        for (int i = tid; i < NW * E; i += blockDim.x) base[i] += off[i % E];
        lds_barrier();
        // stable scatter of the wave's run, 64 slots per step
        for (int sb = s0; sb < s1; sb += kWave) {
            const int s = sb + lane;
            const int e = s < s1 ? idx[s] : -1;
            const bool valid = (unsigned)e < (unsigned)E;
            if (valid) atomicOr(&lanes_of[wave * E + e], 1ull << lane);
            __builtin_amdgcn_wave_barrier();
            const unsigned long long same = valid ? lanes_of[wave * E + e] : 0ull;
            __builtin_amdgcn_wave_barrier();
            if (valid) lanes_of[wave * E + e] = 0ull;
            int rank = 0, pos = -1;
            if (valid) {
                rank = __popcll(same & ((1ull << lane) - 1ull));
                pos = base[wave * E + e] + rank;
                st_dev_u32((uint32_t*)(perm + pos), (uint32_t)s);
            }
            if (s < s1) st_dev_u32((uint32_t*)(inv + s), (uint32_t)pos);
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) base[wave * E + e] += __popcll(same);
            __builtin_amdgcn_wave_barrier();
        }
        // this chunk's share of the dropped-slot tail of perm
        const int d0 = off[E] + (int)((int64_t)(P - off[E]) * b / Gp);
        const int d1 = off[E] + (int)((int64_t)(P - off[E]) * (b + 1) / Gp);
        for (int i = d0 + tid; i < d1; i += blockDim.x) st_dev_u32((uint32_t*)(perm + i), 0xffffffffu);
        wait_vm_all();
        lds_barrier();
        if (tid == 0) st_dev_u64(sy.pdone() + b, stamp);
    } else {
        stamp = layer_stamp(gen, sy);
    }
    wait_flags(sy.pdone(), Gp, 1, stamp, sy);
    return stamp;
}

// c of LayerSched: how many down items a slot with one gate_up item fewer
// runs in one gate_up item's time (work_g, work_d: products per item),
// within the down items of the tiles finished in the earlier rounds.
__device__ __forceinline__ int layer_early_down(int NG, int ND, int npg, int npd, int64_t work_g,
                                                int64_t work_d) {
    const int G = gridDim.x, q = NG / G, nf = G - NG % G;
    if (NG % G == 0) return 0;
    const int c = (int)((work_g + work_d - 1) / work_d);
    return min(c, min(ND, q * G / npg * npd) / nf);
}

// The combine of the one-launch layer: once every workgroup's down items are
// stored, workgroup b sums its share of the (token, 8 columns) units;
// workgroup 0 advances the generation word.  `scratch`: an idle LDS word.
__device__ __forceinline__ void layer_combine(int* scratch, const uint16_t* __restrict__ y,
                                              const int32_t* __restrict__ inv,
                                              const float* __restrict__ wts,
                                              const uint16_t* __restrict__ residual, int64_t T,
                                              int k, int H, uint16_t* __restrict__ out,
                                              uint64_t stamp, LayerSync sy) {
    const int b = blockIdx.x, G = gridDim.x, nt = blockDim.x;
    wait_flags(sy.dflag(), G, 1, stamp, sy);
    if (threadIdx.x == 0) *scratch = ld_dev_u64(sy.err()) == stamp;
    if (b == 0 && threadIdx.x < 64) {
        // every workgroup has read the generation word (each stored its
        // acknowledgement at its start): advance it
        bool all;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        do {
            all = true;
            for (int i = threadIdx.x; i < G; i += 64) all &= ld_dev_u64(sy.ack() + i) == stamp;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kLayerSpinTicks) break;
        } while (!__all(all));
        if (threadIdx.x == 0) st_dev_u64(sy.gen(), stamp);
    }
    lds_barrier();
    const bool bad = *scratch;
    const int64_t U = T * (H / 8), u0 = U * b / G, u1 = U * (b + 1) / G;
    if (k <= 8) {
        // two units per thread at a time, all their slot loads in flight
        for (int64_t g = u0 + threadIdx.x; g < u1; g += 2 * nt)
            combine_units<8, 2>(y, inv, wts, residual, g, nt, u1, k, H, bad, out);
    } else {
        for (int64_t g = u0 + threadIdx.x; g < u1; g += nt)
            combine_unit(y, inv, wts, residual, g, k, H, bad, out);
    }
}

}  // namespace moe

// moe_decode.hip - gather-GEMV form of the routed-experts layer for a
// handful of tokens.  Model card "DeepSeek-OCR-2 MoE experts", description:
// the decode op handles about 1-4 tokens without a per-expert host loop and
// without a device-to-host sync, streaming only the selected experts'
// weights.  Here the F dimension is cut into 32-wide slices and one
// workgroup owns one (selected expert, slice):
//   - it streams the slice's 32 gate rows and 32 up rows (one read each),
//     forms h[slot, f] = silu(gate . x) * (up . x) for every slot that chose
//     the expert, and keeps h in LDS;
//   - it multiplies h into the slice's columns of the expert's down matrix
//     (all H rows, 64 bytes each, prefetched into LDS when the workgroup
//     starts) and writes one fp32 partial sum per (slot, slice, column).
// A second, small kernel adds the partial sums of every slot in a fixed
// order, applies the router weights and adds the residual if any (the
// combine): deterministic, no float atomics.  Every weight byte of a selected expert is read from HBM
// once, and the whole weight stream runs in a single launch: on MI355X a
// short stream pays a fixed start-up cost of several microseconds, so one
// long stream beats two short ones, and splitting F (not H) lets the down
// product start without any device-wide synchronisation.
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_route.h"

namespace moe {

constexpr int kDecThreads = 512;  // 8 waves

// Loads below never sit behind a branch: an out-of-range chunk or row loads
// a valid address (index clamped), so the compiler's waits count exactly the
// loads a use depends on.  Token chunks past the row end are zeroed.
__device__ __forceinline__ uint4 zero_unless(bool keep, uint4 v) {
    return keep ? v : make_uint4(0, 0, 0, 0);
}

// The routing of all P <= 32 slots, held by the lanes of one wave: lane s
// has slot s's expert (or -1) and weight.  `first` marks the lanes that are
// the first slot of a distinct expert (distinct experts are numbered in order
// of first appearance); `u` is the distinct index of the lane's slot.
struct WaveRouting {
    int e;
    int u;
    uint64_t first;
    int n;
};

__device__ __forceinline__ WaveRouting wave_routing(const int32_t* __restrict__ idx, int P, int E) {
    const int lane = threadIdx.x & 63;
    WaveRouting r;
    int e = lane < P ? idx[lane] : -1;
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

// Sum over the 64 lanes of each of the N = 2^n values v[0..N): after the
// call lane l holds the total of value (l >> (6 - n)).  Each halving step
// trades half of the values with the partner lane, so it takes
// N - 1 + (6 - n) shuffles instead of 6 N.
template <int N>
__device__ __forceinline__ float transpose_sum(float (&v)[N]) {
    const int lane = threadIdx.x & 63;
    int bit = 32;
#pragma unroll
    for (int step = N / 2; step >= 1; step /= 2, bit /= 2) {
        const bool hi = lane & bit;
#pragma unroll
        for (int i = 0; i < step; ++i) {
            // both operands as plain registers: a select between two array
            // elements would otherwise become an indexed (scratch) access
            float lo_v = v[i], hi_v = v[i + step];
            asm("" : "+v"(lo_v), "+v"(hi_v));
            const float keep = hi ? hi_v : lo_v;
            const float send = hi ? lo_v : hi_v;
            v[i] = keep + __shfl_xor(send, bit, kWave);
        }
    }
    float s = v[0];
    for (; bit >= 1; bit /= 2) s += __shfl_xor(s, bit, kWave);
    return s;
}

// acc + the dot product of 8 bf16 pairs (one 16-byte chunk each), by four
// v_dot2c_f32_bf16: the bf16 products are exact in fp32, so only the
// accumulation rounds, as with fp32 FMAs on the unpacked values, at a third
// of the vector instructions.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
    return acc;
}

// One workgroup per (distinct selected expert u, F slice sl), block index
// u * nslices + sl.  S = slice width (16 or 32), NCH = 16-byte chunks per
// lane of an H row (H <= 512 NCH), NT = number of tokens.
// With ra.logits set the workgroup routes the NT tokens itself first (waves
// 0 .. NT-1, one token each, into LDS; workgroup 0 also stores the ids and
// weights for the combine), so a decode call from router logits needs no
// router launch.
template <int S, int NCH, int NT>
__global__ __launch_bounds__(kDecThreads) void decode_slice_kernel(
    const uint16_t* __restrict__ x, const ExpertWeights w13,
    const ExpertWeights w2, const int32_t* __restrict__ idx, int k, int E, int H,
    int F, int nslices, float* __restrict__ part, const RouteArgs ra,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
    constexpr int kSlice = S;
    constexpr int kRowsPerWave = 2 * S / 8;     // gate/up panel rows per wave
    constexpr int CPR = S / 8;                  // 16-byte chunks of a down-slice row
    constexpr int NV = kRowsPerWave * NT;       // dot products per wave
    // down slice in registers when they allow it (H <= 1536, few tokens):
    // its rows are then used as they arrive; otherwise it goes through LDS
    constexpr bool W2REG = NCH <= 3 && NCH * NT <= 8;
    constexpr int W2ROWS = (3 * 512 + kDecThreads / CPR - 1) / (kDecThreads / CPR);
    constexpr int NVP = NV <= 8 ? 8 : NV <= 16 ? 16 : 32;  // padded to a power of two
    static_assert(NV <= 32, "at most 32 dot products per wave");
    __shared__ u32x4 w2s[W2REG ? 1 : kDecodeMaxDim * CPR];  // down[e][c][f0 .. f0+S): CPR chunks per row
    __shared__ float dots[2][NT][kSlice];                 // gate / up dot products
    __shared__ float hs[kDecodeMaxSlots][kSlice];
    __shared__ int32_t idx_sh[kDecodeMaxSlots];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = NT * k;
    // Work w = u * nslices + sl.  Blocks go to XCDs round-robin; mapping
    // w to XCD-contiguous runs of even length keeps the two 32-wide slices
    // that share a 128-byte line of the down matrix in one L2.
    const int per_xcd = gridDim.x / kXcds;
    const int w = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const int u = w / nslices, sl = w - u * nslices;
    if (u >= kDecodeMaxSlots) return;  // grid padding
    const int nch = H / 8;
    // the token rows first: they do not depend on the routing
    uint4 xv[NT][NCH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = lane + 64 * i;
            xv[t][i] = zero_unless(c < nch, *(const uint4*)(x + (int64_t)t * H + min(c, nch - 1) * 8));
        }
    const int32_t* ids = idx;
    if (ra.logits) {   // uniform over the grid
        if (wave < NT) {
            int id;
            float wt;
            if (ra.E <= 64) route_token_lanes<1>(ra, wave, lane, id, wt);
            else if (ra.E <= 128) route_token_lanes<2>(ra, wave, lane, id, wt);
            else route_token_lanes<8>(ra, wave, lane, id, wt);
            if (lane < k) {
                idx_sh[wave * k + lane] = id;
                if (blockIdx.x == 0) {
                    idx_out[wave * k + lane] = id;
                    w_out[wave * k + lane] = wt;
                }
            }
        }
        lds_barrier();
        ids = idx_sh;
    }
    const WaveRouting R = wave_routing(ids, P, E);
    if (u >= R.n) return;  // fewer distinct experts than slots (uniform over the workgroup)
    uint64_t fm = R.first;
    for (int i = 0; i < u; ++i) fm &= fm - 1ull;
    const int e = __shfl(R.e, __builtin_ctzll(fm), kWave);
    const uint64_t slots = __ballot(R.u == u);
    const int f0 = sl * kSlice;

    // 1. (large variants) the slice of the down matrix, straight into LDS:
    //    row c of w2s holds down[e][c][f0 .. f0+S) as CPR chunks; one wave
    //    load covers 64/CPR rows
    if constexpr (!W2REG) {
        constexpr int RPI = 64 / CPR;
        const int r = lane / CPR, ch = lane % CPR;
        const uint16_t* src = w2.expert(e, (int64_t)H * F) + (int64_t)r * F + f0 + ch * 8;
        for (int j = wave; j < H / RPI; j += kDecThreads / kWave)
            __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)j * RPI * F),
                                             (lds_void*)&w2s[j * 64], 16, 0, 0);
    }

    // 2./3. this wave's gate/up rows (panel row p in [0, 2S) is gate row f0 + p
    //    for p < S, else up row F + f0 + p - S; lane chunks c = lane + 64 i),
    //    dotted with every token.
    constexpr int RB = kRowsPerWave;
    uint4 w2r[W2REG ? W2ROWS : 1];
    float v[NVP];
#pragma unroll
    for (int i = NV; i < NVP; ++i) v[i] = 0.0f;
#pragma unroll
    for (int rb = 0; rb < kRowsPerWave; rb += RB) {
        uint4 wv[RB][NCH];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int p = kRowsPerWave * wave + rb + r;
            const int row = p < kSlice ? f0 + p : F + f0 + (p - kSlice);
            const uint16_t* src = w13.expert(e, (int64_t)2 * F * H) + (int64_t)row * H;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = lane + 64 * i;
                // a chunk past the row end repeats the last one; it meets a
                // zeroed token chunk, so it adds nothing
                wv[r][i] = load_nt16(src + min(c, nch - 1) * 8);
            }
        }
        // (small variants) this thread's rows of the down slice, requested
        // after the gate/up rows so that the dot products need not wait for
        // them: rows c = tid / CPR + (512 / CPR) j, chunk tid % CPR
        if constexpr (W2REG) {
            const uint16_t* src = w2.expert(e, (int64_t)H * F) + (int64_t)(tid / CPR) * F + f0 + (tid % CPR) * 8;
#pragma unroll
            for (int j = 0; j < W2ROWS; ++j) {
                const int c = tid / CPR + (kDecThreads / CPR) * j;
                // a row past H repeats row H - 1 and is never stored
                w2r[j] = load_nt16(src + (int64_t)(min(c, H - 1) - tid / CPR) * F);
            }
        }
        // every weight load is in flight before the first dot product
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < NCH; ++i) acc = dot8_bf16(wv[r][i], xv[t][i], acc);
                v[(rb + r) * NT + t] = acc;
            }
    }
    const float tot = transpose_sum<NVP>(v);
    {
        constexpr int n = __builtin_ctz(NVP);
        const int vi = lane >> (6 - n);
        if ((lane & ((1 << (6 - n)) - 1)) == 0 && vi < NV) {  // one lane per value
            const int r = vi / NT, t = vi - r * NT;
            const int p = kRowsPerWave * wave + r;
            dots[p < kSlice ? 0 : 1][t][p & (kSlice - 1)] = tot;
        }
    }
    lds_barrier();

    // 4. h for every slot of the expert (slot s belongs to token s / k)
    for (int i = tid; i < kDecodeMaxSlots * kSlice; i += kDecThreads) {
        const int s = i / kSlice, f = i - s * kSlice;
        if (s < P && ((slots >> s) & 1ull)) {
            const int t = s / k;
            hs[s][f] = silu(dots[0][t][f]) * dots[1][t][f];
        }
    }
    if constexpr (W2REG) {
        lds_barrier();  // h is complete
    } else {
        // the down slice has landed (this wave's loads), then every wave's
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // 5. partial down products: CPR lanes per row c, 8 values of the slice each
    const int q = tid % CPR;
#pragma unroll
    for (int j = 0; j < (W2REG ? W2ROWS : (kDecodeMaxDim * CPR + kDecThreads - 1) / kDecThreads); ++j) {
        const int c = tid / CPR + (kDecThreads / CPR) * j;
        if (c >= H) break;
        float wf[8];
        if constexpr (W2REG) {
            unpack8(w2r[j], wf);
        } else {
            const u32x4 wc = w2s[c * CPR + q];
            unpack8(make_uint4(wc.x, wc.y, wc.z, wc.w), wf);
        }
        uint64_t sm = slots;
        while (sm) {
            const int s = __builtin_ctzll(sm);
            sm &= sm - 1ull;
            const float* hr = &hs[s][q * 8];
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += wf[j] * hr[j];
            acc += pair_swap(acc);  // lanes q ^ 1
            if (CPR == 4)           // lanes q ^ 2
                acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xF, 0xF, false));
            if (q == 0) part[((int64_t)s * nslices + sl) * H + c] = acc;
        }
    }
}

// out[t, c] = sum_j w[t, j] * sum_sl part[t*k + j, sl, c] over valid slots.
// A workgroup owns 16 columns; its 16 column groups split the (slot, slice)
// pairs (pair = g + 16 i, pair = slot * nslices + slice) and their sums are
// added in group order, so the result does not depend on timing.  Loads go
// out in batches of 16 with no dependences between them; dropped slots have
// weight zero (no branch in the loop).
// The batch B of loads a thread has in flight is 16, or 64 when there are
// more than 16 x 16 pairs, so that up to 1024 pairs take one round trip.
constexpr int kCombCols = 16, kCombGroups = 16;  // many small workgroups: latency-bound
constexpr int kCombThreads = kCombCols * kCombGroups;
template <int kCombBatch>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ idx, const float* __restrict__ wts,
    const uint16_t* __restrict__ residual, int T, int k, int E, int H, int nslices,
    uint16_t* __restrict__ out) {
    // per slot: the routing weight's bits (0 for a dropped slot), a mask
    // that is all ones for a valid slot, zero for a dropped one, and the token
    __shared__ int4 wsl[kDecodeMaxSlots];
    __shared__ float red[kCombGroups][kDecodeMaxT][kCombCols];
    const int cl = threadIdx.x % kCombCols, g = threadIdx.x / kCombCols;
    const int c = blockIdx.x * kCombCols + cl;
    const int P = T * k;
    const int npairs = P * nslices;
    // the first batch of partial sums is requested before the slot weights
    // are read (no dependence between them)
    float v[kCombBatch];
#pragma unroll
    for (int i = 0; i < kCombBatch; ++i) {
        const int pr = min(g + kCombGroups * i, npairs - 1);
        v[i] = part[(int64_t)pr * H + c];
    }
    if (threadIdx.x < kDecodeMaxSlots) {
        const int sc = min((int)threadIdx.x, P - 1);  // both loads unconditional
        const int e = idx[sc];
        const float wv = wts[sc];
        const bool valid = (int)threadIdx.x < P && (unsigned)e < (unsigned)E;
        wsl[threadIdx.x] = make_int4(valid ? __float_as_int(wv) : 0, valid ? -1 : 0, sc / k, 0);
    }
    __syncthreads();
    float acc[kDecodeMaxT] = {0.0f, 0.0f, 0.0f, 0.0f};
    // slot s and slice sl of pair g + kCombGroups j, stepped without
    // divisions: each step adds dq slots and dr slices
    const int dq = kCombGroups / nslices, dr = kCombGroups - dq * nslices;
    int s = g / nslices, sl = g - s * nslices;
    for (int base = g; base < npairs; base += kCombGroups * kCombBatch) {
        if (base != g) {
#pragma unroll
            for (int i = 0; i < kCombBatch; ++i) {
                const int pr = min(base + kCombGroups * i, npairs - 1);
                v[i] = part[(int64_t)pr * H + c];
            }
        }
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i)
            if (base + kCombGroups * i >= npairs) v[i] = 0.0f;
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            // a dropped slot's partial sums are never written: masked out,
            // not multiplied by zero (stale memory may hold NaN); pairs past
            // the end hold 0 and read the last slot's entry
            const int4 ws = wsl[min(s, P - 1)];
            const float wv = __int_as_float(__float_as_int(v[i] * __int_as_float(ws.x)) & ws.y);
#pragma unroll
            for (int tt = 0; tt < kDecodeMaxT; ++tt)
                if (tt == ws.z) acc[tt] += wv;
            sl += dr;
            s += dq;
            if (sl >= nslices) {
                sl -= nslices;
                ++s;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) red[g][t][cl] = acc[t];
    __syncthreads();
    if (threadIdx.x < kCombCols * kDecodeMaxT) {
        const int t = threadIdx.x / kCombCols, cc = threadIdx.x % kCombCols;
        if (t < T) {
            float o = 0.0f;
#pragma unroll
            for (int i = 0; i < kCombGroups; ++i) o += red[i][t][cc];
            const int64_t oi = (int64_t)t * H + blockIdx.x * kCombCols + cc;
            if (residual) o += bf16_to_f32(residual[oi]);
            out[oi] = (uint16_t)f32_to_bf16(o);
        }
    }
}

template <int S, int NCH>
static void launch_slices(dim3 grid, const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                          const int32_t* idx, int T, int k, int E, int H, int F, int ns, float* part,
                          hipStream_t s, const RouteArgs& ra, int32_t* io, float* wo) {
    if (NCH * T > kDecodeMaxChunkTokens) return;  // excluded by decode_fast_path
    switch (T) {
        case 1: MOE_LAUNCH((decode_slice_kernel<S, NCH, 1>), grid, dim3(kDecThreads), 0, s, x, w13, w2, idx, k, E, H, F, ns, part, ra, io, wo); break;
        case 2: MOE_LAUNCH((decode_slice_kernel<S, NCH, 2>), grid, dim3(kDecThreads), 0, s, x, w13, w2, idx, k, E, H, F, ns, part, ra, io, wo); break;
        case 3: MOE_LAUNCH((decode_slice_kernel<S, NCH, 3>), grid, dim3(kDecThreads), 0, s, x, w13, w2, idx, k, E, H, F, ns, part, ra, io, wo); break;
        case 4: MOE_LAUNCH((decode_slice_kernel<S, NCH < 4 ? NCH : 3, 4>), grid, dim3(kDecThreads), 0, s, x, w13, w2, idx, k, E, H, F, ns, part, ra, io, wo); break;
        default: break;
    }
}

template <int S>
static hipError_t launch_width(const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                               const int32_t* idx, int T, int k, int E, int H, int F, int umax,
                               float* part, hipStream_t s, const RouteArgs& ra, int32_t* io,
                               float* wo) {
    const int ns = F / S;
    // padded to a multiple of 16 (even runs per XCD); padding blocks map to
    // u >= umax, where the routing has no distinct expert
    const dim3 grid((unsigned)((umax * ns + 15) / 16 * 16));
    switch ((H / 8 + 63) / 64) {
        case 1: launch_slices<S, 1>(grid, x, w13, w2, idx, T, k, E, H, F, ns, part, s, ra, io, wo); break;
        case 2: launch_slices<S, 2>(grid, x, w13, w2, idx, T, k, E, H, F, ns, part, s, ra, io, wo); break;
        case 3: launch_slices<S, 3>(grid, x, w13, w2, idx, T, k, E, H, F, ns, part, s, ra, io, wo); break;
        case 4: launch_slices<S, 4>(grid, x, w13, w2, idx, T, k, E, H, F, ns, part, s, ra, io, wo); break;
        default: return hipErrorInvalidValue;  // H > 2048 is routed to the grouped path by the caller
    }
    return hipGetLastError();
}

hipError_t launch_decode_slices(const uint16_t* x, const ExpertWeights& w13,
                                const ExpertWeights& w2, const int32_t* idx, int T, int k, int E,
                                int H, int F, float* part, hipStream_t s, const RouteArgs& ra,
                                int32_t* idx_out, float* w_out) {
    const DecodeGeometry g = decode_geometry(T, k, E, H, F);
    return g.slice == 16
               ? launch_width<16>(x, w13, w2, idx, T, k, E, H, F, g.umax, part, s, ra, idx_out, w_out)
               : launch_width<32>(x, w13, w2, idx, T, k, E, H, F, g.umax, part, s, ra, idx_out, w_out);
}

hipError_t launch_decode_combine(const float* part, const int32_t* idx, const float* w,
                                 const uint16_t* residual, int T, int k, int E, int H, int F,
                                 uint16_t* out, hipStream_t s) {
    const DecodeGeometry g = decode_geometry(T, k, E, H, F);
    if (T * k * g.nslices > kCombGroups * 16)
        MOE_LAUNCH(decode_combine_kernel<64>, dim3((unsigned)(H / kCombCols)), dim3(kCombThreads), 0,
                   s, part, idx, w, residual, T, k, E, H, g.nslices, out);
    else
        MOE_LAUNCH(decode_combine_kernel<16>, dim3((unsigned)(H / kCombCols)), dim3(kCombThreads), 0,
                   s, part, idx, w, residual, T, k, E, H, g.nslices, out);
    return hipGetLastError();
}

}  // namespace moe

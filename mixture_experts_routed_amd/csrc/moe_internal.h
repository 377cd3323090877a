// moe_internal.h - host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Every kernel launch goes through MOE_LAUNCH.  While the stage-timing
// recorder has armed an event pair for the calling thread, the launch carries
// them on its own dispatch (so they time the kernel's execution, not the
// dispatch queue), and the pair is disarmed; otherwise it is a plain launch.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming& launch_timing();  // per host thread

#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ...)                                     \
    do {                                                                                        \
        ::moe::LaunchTiming& lt_ = ::moe::launch_timing();                                      \
        if (lt_.start) {                                                                        \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, lt_.start, lt_.stop, 0u,  \
                                  __VA_ARGS__);                                                 \
            lt_ = ::moe::LaunchTiming{};                                                        \
        } else {                                                                                \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                \
        }                                                                                       \
    } while (0)

// The plan cuts every expert's rows into M tiles of at most tile_m rows
// (the grouped products' tile height; never below kMinTileM).
constexpr int kMinTileM = 32;
// Tile height of the stand-alone plan entry points (their tile list is not
// read by any product).
constexpr int kPlanTileM = 128;
int bf16_tile_m();
// fp8 decode batches (at most 32 rows per expert on average) take 32-row
// tiles (fp8_use_narrow), others 128.
bool fp8_use_narrow(int64_t P, int E, int H, int F);
int fp8_tile_m(bool narrow);

// Largest number of M tiles a plan over P slots and E experts can produce.
inline int64_t max_m_tiles(int64_t P, int E) { return (P + kMinTileM - 1) / kMinTileM + E; }

// tiles[2i], tiles[2i+1] = (expert, first row) of M tile i (expert order);
// tile_off[E+1] = prefix of M tiles per expert; *ntiles = tile_off[E].
hipError_t launch_plan(const int32_t* idx, int P, int E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* ntiles,
                       int32_t* tile_off, int tile_m, hipStream_t s);

// Per-expert weight matrices of `stride` elements: the E routed experts in
// one tensor, optionally followed by S shared experts in a tensor of their
// own (expert ids E .. E+S-1, see the shared-expert entry points).  Without
// shared experts `shared` is unused (n_routed covers every id).
struct ExpertWeights {
    const uint16_t* base;
    const uint16_t* shared;
    int n_routed;
    __host__ __device__ const uint16_t* expert(int e, int64_t stride) const {
        return e < n_routed ? base + (int64_t)e * stride : shared + (int64_t)(e - n_routed) * stride;
    }
};
inline ExpertWeights routed_only(const uint16_t* w, int E) { return ExpertWeights{w, w, E}; }

// Augmented routing for S shared experts: idx2/w2 [T, k+S] hold the routed
// slots (ids outside [0, E) as -1, i.e. dropped) followed by S slots naming
// experts E .. E+S-1 with weight 1.
hipError_t launch_augment_routing(const int32_t* idx, const float* w, int64_t T, int k, int E,
                                  int S, int32_t* idx2, float* w2, hipStream_t s);

// Router arguments as the kernels take them (logits NULL: no routing).
struct RouteArgs {
    const void* logits;
    const void* bias;
    int bf16;          // logits and bias are bf16 (else fp32)
    int mode;          // MOE_ROUTE_*
    int E, k, num_groups, topk_group, group_top;
    float scale;
};

// Grouped-GEMM inputs produced by the plan.
struct GroupedPlan {
    const int32_t* perm;
    const int32_t* tiles;
    const int32_t* ntiles;
    const int32_t* tile_off;
    const int32_t* offsets;
    int E;
};

// gate_up product with SwiGLU epilogue -> h bf16 [P, F] (expert order).
hipError_t launch_gateup_bf16(const uint16_t* x, const ExpertWeights& w13, const GroupedPlan& plan,
                              int H, int F, int k, uint16_t* h, hipStream_t s);

// down product -> y bf16 [P, H] in expert order (row = position in perm).
hipError_t launch_down_bf16(const uint16_t* h, const ExpertWeights& w2, const GroupedPlan& plan,
                            int P, int H, int F, uint16_t* y, hipStream_t s);

// out[t] = sum_j w[t,j] * y[inv[t*k+j]] over valid slots (fp32, slot order)
// + residual[t] when residual is not null.
hipError_t launch_combine(const uint16_t* y, const int32_t* inv, const float* w,
                          const uint16_t* residual, int64_t T, int k, int H, uint16_t* out,
                          hipStream_t s);

// Decode gather-GEMV (T small): one launch streams the selected experts'
// weights in 32-wide F slices and writes fp32 partial down products
// part[slot][slice][H]; a second small launch adds them up with the router
// weights.  Limits of this form: T <= 4, T*k <= 32, H <= 2048, F <= 2048
// and T * ceil(H / 512) <= 12 (the token rows and weight rows of a wave stay
// in registers); larger calls take the grouped path.
constexpr int kDecodeMaxT = 4;
constexpr int kDecodeMaxSlots = 32;
constexpr int kDecodeMaxDim = 2048;
constexpr int kDecodeMaxChunkTokens = 12;

struct DecodeGeometry {
    int umax;     // most distinct experts a call can select: min(T*k, E)
    int slice;    // F values per workgroup
    int nslices;  // F / slice
};

inline DecodeGeometry decode_geometry(int64_t T, int k, int E, int H, int F) {
    (void)H;
    DecodeGeometry g;
    const int P = (int)(T * k);
    g.umax = P < E ? P : E;
    g.slice = 32;  // 16-wide slices (more workgroups) measured slower at T = 1
    g.nslices = F / g.slice;
    return g;
}

// Bytes of the partial sums of the decode form.
inline size_t decode_partial_bytes(int64_t T, int k, int E, int H, int F) {
    const DecodeGeometry g = decode_geometry(T, k, E, H, F);
    return (size_t)(T * k) * (size_t)g.nslices * (size_t)H * sizeof(float);
}

// With ra.logits set, the kernel routes the T tokens itself (every
// workgroup, redundantly; workgroup 0 also writes idx_out / w_out for the
// combine and the caller) and `idx` is unused.
hipError_t launch_decode_slices(const uint16_t* x, const ExpertWeights& w13,
                                const ExpertWeights& w2, const int32_t* idx, int T, int k, int E,
                                int H, int F, float* part, hipStream_t s,
                                const RouteArgs& ra = RouteArgs{}, int32_t* idx_out = nullptr,
                                float* w_out = nullptr);
hipError_t launch_decode_combine(const float* part, const int32_t* idx, const float* w,
                                 const uint16_t* residual, int T, int k, int E, int H, int F,
                                 uint16_t* out, hipStream_t s);

// fp8 gate_up product with SwiGLU + block-128 re-quantisation epilogue.
hipError_t launch_gateup_fp8(const uint8_t* x, const float* xs, const uint8_t* w13,
                             const float* w13s, const GroupedPlan& plan, bool narrow, int H, int F,
                             int k, uint8_t* hq, float* hs, hipStream_t s);

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* w2, const float* w2s,
                           const GroupedPlan& plan, bool narrow, int H, int F, uint16_t* y,
                           hipStream_t s);

hipError_t launch_quantize_fp8(const void* in, int in_is_bf16, int64_t rows, int K, uint8_t* codes,
                               float* scales, hipStream_t s);

// MXFP4 x MXFP8 products (E2M1 weights two per byte, E4M3 activations, E8M0
// scales per 32 K elements): gate_up with SwiGLU + MXFP8 re-quantisation
// (hq [P, F] E4M3, hs [P, F/32] E8M0, expert order), and down -> y bf16
// [P, H] in expert order.  H, F multiples of 128 (F also of 128 per h tile).
// `wide` (mx_use_wide: many rows per expert, F % 256 == 0, H % 512 == 0)
// selects 128 x 512 tiles of 64 x 128 wave tiles instead of 128 x 256 tiles;
// `narrow` (mx_use_narrow: decode batches, H % 512 == 0, F % 256 == 0) 32-row
// tiles over 512-row panels.  The plan's tile height is mx_tile_m(narrow).
bool mx_use_narrow(int64_t P, int E, int H, int F);
int mx_tile_m(bool narrow);
bool mx_use_wide(int64_t P, int E, int H, int F);
hipError_t launch_gateup_mx(const uint8_t* x, const uint8_t* xs, const uint8_t* w13,
                            const uint8_t* w13s, const GroupedPlan& plan, bool wide, bool narrow,
                            int H, int F, int k, uint8_t* hq, uint8_t* hs, hipStream_t s);
hipError_t launch_down_mx(const uint8_t* hq, const uint8_t* hs, const uint8_t* w2,
                          const uint8_t* w2s, const GroupedPlan& plan, bool wide, bool narrow, int H,
                          int F, uint16_t* y, hipStream_t s);

// Routers (logits -> ids, weights), alone or followed by the plan in the
// same launch (one workgroup; small batches).
hipError_t launch_route(const void* logits, const void* bias, int bf16, int mode, int64_t T, int E,
                        int k, int num_groups, int topk_group, int group_top, float scale,
                        int32_t* idx, float* w, hipStream_t s);
hipError_t launch_route_plan(const void* logits, const void* bias, int bf16, int mode, int T,
                             int E, int k, int num_groups, int topk_group, int group_top,
                             float scale, int32_t* idx, float* w, int32_t* counts,
                             int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles,
                             int32_t* ntiles, int32_t* tile_off, int tile_m, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe

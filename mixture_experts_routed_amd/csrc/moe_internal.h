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
template <typename T>
struct ExpertArray {
    const T* base;
    const T* shared;
    int n_routed;
    __host__ __device__ const T* expert(int e, int64_t stride) const {
        return e < n_routed ? base + (int64_t)e * stride : shared + (int64_t)(e - n_routed) * stride;
    }
};
using ExpertWeights = ExpertArray<uint16_t>;
template <typename T>
inline ExpertArray<T> routed_only(const T* w, int E) { return ExpertArray<T>{w, w, E}; }

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

// The whole layer in one persistent launch (see moe_layer.h): the routing
// plan, gate_up, down and the combine, for H and F multiples of 128; the
// plan arrays, h and y go through the workspace as in the stage-by-stage
// form and out is bit-for-bit the same.  `sync` holds layer_sync_bytes of
// hand-off words (no initialisation needed).
struct LayerPlan {   // the plan arrays in the workspace (written by the launch)
    int32_t *counts, *offsets, *perm, *inv, *tiles, *ntiles, *tile_off;
};
constexpr int kLayerMaxGrid = 1024;                  // flag slots per workgroup kind
constexpr uint64_t kLayerSpinTicks = 200000000ull;   // 2 s of the 100 MHz clock
constexpr int kLayerPlanChunks = 64;                 // workgroups of the in-launch routing plan
bool layer_bf16_fits(int H, int F);
size_t layer_sync_bytes(int64_t P, int E, int F);
hipError_t launch_layer_bf16(const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                             const int32_t* idx, const LayerPlan& plan, const float* w,
                             const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                             uint16_t* h, uint16_t* y, uint16_t* out, void* sync, hipStream_t s);

// out[t] = sum_j w[t,j] * y[inv[t*k+j]] over valid slots (fp32, slot order)
// + residual[t] when residual is not null.
hipError_t launch_combine(const uint16_t* y, const int32_t* inv, const float* w,
                          const uint16_t* residual, int64_t T, int k, int H, uint16_t* out,
                          hipStream_t s);

// Decode gather-GEMV (a few tokens): one persistent launch (see
// moe_decode.hip) streams the selected experts' gate/up rows into h, hands h
// over between workgroups through the workspace, then streams their down
// rows and writes out.  Limits of this form: T <= 4, T*k <= 32, H and F <=
// 2048, H <= 1536 when T > 1 (the token rows stay in registers), and
// h = T*k*F bf16 values within the LDS budget; larger calls take the
// grouped path.
constexpr int kDecodeMaxT = 4;
constexpr int kDecodeMaxSlots = 32;
constexpr int kDecodeMaxDim = 2048;
constexpr int kDecodeMaxGrid = 1024;      // flag slots in the workspace
constexpr int kDecodeHBytes = 96 << 10;   // LDS budget for h (bf16)
constexpr int kDecodeMaxRows = 64;        // output rows per workgroup (grid >= H / 64)
// workspace: generation word, flags [kDecodeMaxGrid] u64, error word, h [T*k][F] bf16
constexpr size_t kDecodeHOffset = 256 + 8 * (size_t)kDecodeMaxGrid + 256;
inline size_t decode_h_bytes(int64_t T, int k, int F) {
    return ((size_t)(T * k) * (size_t)F * 2 + 1023) / 1024 * 1024;   // whole 1 KB copies
}
inline size_t decode_ws_bytes(int64_t T, int k, int F) { return kDecodeHOffset + decode_h_bytes(T, k, F); }
inline bool decode_fits(int64_t T, int k, int H, int F) {
    const int nch = (H / 8 + 63) / 64;
    return T >= 1 && T <= kDecodeMaxT && T * k <= kDecodeMaxSlots && H <= kDecodeMaxDim &&
           F <= kDecodeMaxDim && (T == 1 ? nch <= 4 : nch <= 3) &&
           decode_h_bytes(T, k, F) <= (size_t)kDecodeHBytes;
}

// S > 0: the last S of the E experts are shared experts that every token
// passes with weight 1; k counts them (k - S routed slots per token, read
// from idx / w [T, k-S]); no router then.
// With ra.logits set, the kernel routes the T tokens itself (every
// workgroup, redundantly; workgroup 0 also writes idx_out / w_out) and
// idx / w are unused.  ws: decode_ws_bytes, 256-byte aligned.
hipError_t launch_decode(const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                         const int32_t* idx, const float* w, const uint16_t* residual, int T, int k,
                         int E, int H, int F, uint16_t* out, void* ws, hipStream_t s,
                         const RouteArgs& ra = RouteArgs{}, int32_t* idx_out = nullptr,
                         float* w_out = nullptr, int S = 0);

// fp8 gate_up product with SwiGLU + block-128 re-quantisation epilogue.
hipError_t launch_gateup_fp8(const uint8_t* x, const float* xs, const ExpertArray<uint8_t>& w13,
                             const ExpertArray<float>& w13s, const GroupedPlan& plan, bool narrow, int H, int F,
                             int k, uint8_t* hq, float* hs, hipStream_t s);

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const ExpertArray<uint8_t>& w2,
                           const ExpertArray<float>& w2s, const GroupedPlan& plan, bool narrow, int H, int F, uint16_t* y,
                           hipStream_t s);

hipError_t launch_quantize_fp8(const void* in, int in_is_bf16, int64_t rows, int K, uint8_t* codes,
                               void* scales, bool ue8m0, hipStream_t s);

// The MXFP4 layer in one persistent launch (as launch_layer_bf16), for
// prefill shapes that take the wide tiles.
bool layer_mx_fits(int64_t P, int E, int H, int F);
hipError_t launch_layer_mx(const uint8_t* x, const uint8_t* xs, const ExpertArray<uint8_t>& w13,
                           const ExpertArray<uint8_t>& w13s, const ExpertArray<uint8_t>& w2,
                           const ExpertArray<uint8_t>& w2s, const int32_t* idx,
                           const LayerPlan& plan, const float* w, const uint16_t* residual,
                           int64_t T, int H, int F, int E, int k, uint8_t* hq, uint8_t* hs,
                           uint16_t* y, uint16_t* out, void* sync, hipStream_t s);

// The fp8 layer in one persistent launch (as launch_layer_bf16), for
// prefill shapes with H and F multiples of 512.
bool layer_fp8_fits(int64_t P, int E, int H, int F);
hipError_t launch_layer_fp8(const uint8_t* x, const float* xs, const ExpertArray<uint8_t>& w13,
                            const ExpertArray<float>& w13s, const ExpertArray<uint8_t>& w2,
                            const ExpertArray<float>& w2s, const int32_t* idx,
                            const LayerPlan& plan, const float* w, const uint16_t* residual,
                            int64_t T, int H, int F, int E, int k, uint8_t* hq, float* hs,
                            uint16_t* y, uint16_t* out, void* sync, hipStream_t s);

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
hipError_t launch_gateup_mx(const uint8_t* x, const uint8_t* xs, const ExpertArray<uint8_t>& w13,
                            const ExpertArray<uint8_t>& w13s, const GroupedPlan& plan, bool wide, bool narrow,
                            int H, int F, int k, uint8_t* hq, uint8_t* hs, hipStream_t s);
hipError_t launch_down_mx(const uint8_t* hq, const uint8_t* hs, const ExpertArray<uint8_t>& w2,
                          const ExpertArray<uint8_t>& w2s, const GroupedPlan& plan, bool wide, bool narrow, int H,
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

// Measurement helper: a plain streaming read of `bytes` bytes (sink: 4 KB).
hipError_t launch_probe_read(const void* src, size_t bytes, int grid, void* sink, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Upper bound on the persistent grids (moe_set_grid_cap; 0 = none), so that
// tests can make every workgroup run many work items.
int grid_cap();
inline int capped_grid(int g) {
    const int cap = grid_cap();
    if (cap <= 0 || g <= cap) return g;
    return cap >= 8 ? cap / 8 * 8 : 8;   // a multiple of the 8 XCDs
}

}  // namespace moe

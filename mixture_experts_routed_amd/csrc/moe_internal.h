// moe_internal.h - host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// The plan cuts every expert's rows into M tiles of at most tile_m rows
// (the grouped products' tile height; never below kMinTileM).
constexpr int kMinTileM = 128;
int bf16_tile_m();
int fp8_tile_m();

// Largest number of M tiles a plan over P slots and E experts can produce.
inline int64_t max_m_tiles(int64_t P, int E) { return (P + kMinTileM - 1) / kMinTileM + E; }

// tiles[2i], tiles[2i+1] = (expert, first row) of M tile i (expert order);
// tile_off[E+1] = prefix of M tiles per expert; *ntiles = tile_off[E].
hipError_t launch_plan(const int32_t* idx, int P, int E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* ntiles,
                       int32_t* tile_off, int tile_m, hipStream_t s);

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
hipError_t launch_gateup_bf16(const uint16_t* x, const uint16_t* w13, const GroupedPlan& plan,
                              int H, int F, int k, uint16_t* h, hipStream_t s);

// down product -> y bf16 [P, H] in expert order (row = position in perm).
hipError_t launch_down_bf16(const uint16_t* h, const uint16_t* w2, const GroupedPlan& plan, int H,
                            int F, uint16_t* y, hipStream_t s);

// out[t] = sum_j w[t,j] * y[inv[t*k+j]] over valid slots, fp32 in slot order.
hipError_t launch_combine(const uint16_t* y, const int32_t* inv, const float* w, int64_t T, int k,
                          int H, uint16_t* out, hipStream_t s);

// Decode gather-GEMV (T small): phase 1 writes h fp32 [T*k, F] by slot id,
// phase 2 does the down rows and the combine.  Limits of this form: T <= 4,
// T*k <= 32, H <= 2048, F <= 2048 (larger calls take the grouped path).
constexpr int kDecodeMaxT = 4;
constexpr int kDecodeMaxSlots = 32;
constexpr int kDecodeMaxDim = 2048;

struct DecodeGeometry {
    int umax;  // most distinct experts a call can select: min(T*k, E)
    int nw2;   // phase-2 workgroups (4 output columns each)
};

inline DecodeGeometry decode_geometry(int64_t T, int k, int E, int H, int F) {
    (void)F;
    DecodeGeometry g;
    const int P = (int)(T * k);
    g.umax = P < E ? P : E;
    g.nw2 = (H + 3) / 4;
    return g;
}

hipError_t launch_decode(const uint16_t* x, const uint16_t* w13, const uint16_t* w2,
                         const int32_t* idx, const float* w, int T, int k, int E, int H, int F,
                         float* h, uint16_t* out, hipStream_t s);

// fp8 gate_up product with SwiGLU + block-128 re-quantisation epilogue.
hipError_t launch_gateup_fp8(const uint8_t* x, const float* xs, const uint8_t* w13,
                             const float* w13s, const GroupedPlan& plan, int H, int F, int k,
                             uint8_t* hq, float* hs, hipStream_t s);

hipError_t launch_down_fp8(const uint8_t* hq, const float* hs, const uint8_t* w2, const float* w2s,
                           const GroupedPlan& plan, int H, int F, uint16_t* y, hipStream_t s);

hipError_t launch_quantize_fp8(const void* in, int in_is_bf16, int64_t rows, int K, uint8_t* codes,
                               float* scales, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe

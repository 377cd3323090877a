// moe_api.hip - C ABI of the routed-experts layer: argument checks, the
// workspace layout and the launch sequence of each entry point.  Every entry
// point validates on the host, then only enqueues kernels on the caller's
// stream (no allocation, no synchronisation, no host<->device copies).
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "moe_internal.h"
#include "../../include/moe_experts.h"

namespace moe {

// ---------------------------------------------------------------- device info
// Read-only per-device facts, filled once per device on first use.
namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu[kMaxDevices];      // 0 = unknown
std::atomic<int> g_is950[kMaxDevices];   // 0 = unknown, 1 = yes, 2 = no

int query_device(int* dev_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
    if (g_is950[dev].load(std::memory_order_acquire) == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
        g_cu[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_is950[dev].store(ok ? 1 : 2, std::memory_order_release);
    }
    *dev_out = dev;
    return g_is950[dev].load(std::memory_order_acquire) == 1 ? MOE_OK : MOE_ERR_DEVICE;
}
}  // namespace

std::atomic<int> g_grid_cap{0};
int grid_cap() { return g_grid_cap.load(std::memory_order_relaxed); }

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    const int n = g_cu[dev].load(std::memory_order_relaxed);
    return n > 0 ? n : 256;
}

// ---------------------------------------------------------------- stage timing
// Optional instrumentation (moe_profile_begin / moe_profile_end): while on,
// each layer call takes the next free call slot, and before each of its
// kernel launches arms a start/stop event pair that the launch carries.
LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}

namespace {
constexpr int kProfStages = MOE_PROFILE_MAX_STAGES;

struct Profiler {
    std::mutex mu;
    bool on = false;
    int cap = 0, used = 0;
    std::vector<hipEvent_t> ev;  // cap * kProfStages * 2 (start, stop)
    std::vector<int> ids;        // cap * kProfStages, -1 = no kernel timed
};
Profiler g_prof;

class StageClock {
  public:
    explicit StageClock(hipStream_t) {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (g_prof.on && g_prof.used < g_prof.cap) call_ = g_prof.used++;
    }
    // right before the launch of the kernel of stage `stage` (MOE_STAGE_*)
    void mark(int stage) {
        settle();
        if (call_ < 0 || n_ >= kProfStages) return;
        const size_t i = (size_t)call_ * kProfStages + n_;
        launch_timing() = LaunchTiming{g_prof.ev[2 * i], g_prof.ev[2 * i + 1]};
        pending_ = stage;
    }
    ~StageClock() { settle(); }
    StageClock(const StageClock&) = delete;
    StageClock& operator=(const StageClock&) = delete;

  private:
    // the armed pair was taken by a launch: the stage is timed
    void settle() {
        if (pending_ < 0) return;
        if (!launch_timing().start) g_prof.ids[(size_t)call_ * kProfStages + n_++] = pending_;
        launch_timing() = LaunchTiming{};
        pending_ = -1;
    }
    int call_ = -1;
    int n_ = 0;
    int pending_ = -1;
};
}  // namespace

// ---------------------------------------------------------------- layout
namespace {
constexpr size_t kNone = (size_t)-1;

struct Layout {
    size_t counts = kNone, offsets = kNone, perm = kNone, inv = kNone, tiles = kNone,
           ntiles = kNone, tile_off = kNone, h = kNone, hs = kNone, y = kNone, part = kNone,
           xq = kNone, xs = kNone, aug_idx = kNone, aug_w = kNone, sync = kNone, total = 0;
    bool decode_fast = false;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool decode_fast_path(int64_t T, int H, int F, int k) { return decode_fits(T, k, H, F); }

Layout make_layout(int variant, int64_t T, int H, int F, int E, int k) {
    Layout L;
    const int64_t P = T * k;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + (bytes ? bytes : 1));
        return at;
    };
    if (variant == MOE_VARIANT_DECODE && decode_fast_path(T, H, F, k)) {
        L.decode_fast = true;
        L.part = take(decode_ws_bytes(T, k, F));
        L.total = off;
        return L;
    }
    if (variant == MOE_VARIANT_PLAN) {
        L.tiles = take((size_t)max_m_tiles(P, E) * 2 * sizeof(int32_t));
        L.ntiles = take(sizeof(int32_t));
        L.tile_off = take((size_t)(E + 1) * sizeof(int32_t));
        L.total = off;
        return L;
    }
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.perm = take((size_t)P * 4);
    L.inv = take((size_t)P * 4);
    L.tiles = take((size_t)max_m_tiles(P, E) * 2 * sizeof(int32_t));
    L.ntiles = take(sizeof(int32_t));
    L.tile_off = take((size_t)(E + 1) * sizeof(int32_t));
    if (variant == MOE_VARIANT_FP8 || variant == MOE_VARIANT_FP8_BF16IN) {
        L.h = take((size_t)P * F);
        L.hs = take((size_t)P * (F / 128) * sizeof(float));
    } else if (variant == MOE_VARIANT_MXFP4) {
        L.h = take((size_t)P * F);
        L.hs = take((size_t)P * (F / 32));
    } else {
        L.h = take((size_t)P * F * 2);
    }
    L.y = take((size_t)P * H * 2);
    if (variant == MOE_VARIANT_PREFILL || variant == MOE_VARIANT_FP8 ||
        variant == MOE_VARIANT_FP8_BF16IN || variant == MOE_VARIANT_MXFP4)   // one-launch forms
        L.sync = take(layer_sync_bytes(P, E, F));
    if (variant == MOE_VARIANT_FP8_BF16IN) {  // the quantised hidden states
        L.xq = take((size_t)T * H);
        L.xs = take((size_t)T * (H / 128) * sizeof(float));
    }
    L.total = off;
    return L;
}

// Shared experts: the layout of the same variant over E + S experts and
// k + S slots, followed by the augmented routing [T, k+S] (ids, weights).
Layout make_shared_layout(int variant, int64_t T, int H, int F, int E, int k, int S) {
    Layout L = make_layout(variant, T, H, F, E + S, k + S);
    const size_t n = (size_t)(T * (k + S)) * 4;
    L.aug_idx = L.total;
    L.aug_w = align256(L.aug_idx + (n ? n : 1));
    L.total = align256(L.aug_w + (n ? n : 1));
    return L;
}

int check_shape(int variant, int64_t T, int H, int F, int E, int k) {
    if (variant < MOE_VARIANT_PREFILL || variant > MOE_VARIANT_MXFP4) return MOE_ERR_SHAPE;
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
    if (variant == MOE_VARIANT_PLAN) return MOE_OK;
    const bool fp8 = variant == MOE_VARIANT_FP8 || variant == MOE_VARIANT_FP8_BF16IN ||
                     variant == MOE_VARIANT_MXFP4;
    const int mult = fp8 ? 128 : 64;
    if (H < mult || F < mult || H % mult || F % mult) return MOE_ERR_SHAPE;
    if ((int64_t)E * 2 * F * (int64_t)H >= ((int64_t)1 << 47)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

int check_ws(const Layout& L, void* ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return MOE_ERR_WORKSPACE;
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

GroupedPlan plan_in(const Layout& L, void* ws, int E) {
    GroupedPlan p;
    p.perm = at<int32_t>(ws, L.perm);
    p.tiles = at<int32_t>(ws, L.tiles);
    p.ntiles = at<int32_t>(ws, L.ntiles);
    p.tile_off = at<int32_t>(ws, L.tile_off);
    p.offsets = at<int32_t>(ws, L.offsets);
    p.E = E;
    return p;
}

// Routing plan into the workspace, then the two grouped bf16 products and the combine.
int run_grouped_bf16(StageClock& clock, const Layout& L, const uint16_t* hidden,
                     const ExpertWeights& gate_up, const ExpertWeights& down, const int32_t* idx,
                     const float* w, const uint16_t* residual, int64_t T, int H, int F, int E,
                     int k, uint16_t* out, void* ws, hipStream_t s) {
    const int P = (int)(T * k);
    const GroupedPlan pl = plan_in(L, ws, E);
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* y = at<uint16_t>(ws, L.y);
    clock.mark(MOE_STAGE_PLAN);
    int rc = launched(launch_plan(idx, P, E, at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                                  at<int32_t>(ws, L.perm), at<int32_t>(ws, L.inv),
                                  at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                  at<int32_t>(ws, L.tile_off), bf16_tile_m(), s));
    if (rc) return rc;
    clock.mark(MOE_STAGE_GATE_UP);
    rc = launched(launch_gateup_bf16(hidden, gate_up, pl, H, F, k, h, s));
    if (rc) return rc;
    clock.mark(MOE_STAGE_DOWN);
    rc = launched(launch_down_bf16(h, down, pl, P, H, F, y, s));
    if (rc) return rc;
    clock.mark(MOE_STAGE_COMBINE);
    return launched(launch_combine(y, at<int32_t>(ws, L.inv), w, residual, T, k, H, out, s));
}

// The plan arrays of a layout, for the one-launch forms that write them.
LayerPlan layer_plan_in(const Layout& L, void* ws) {
    return LayerPlan{at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.perm),
                     at<int32_t>(ws, L.inv),    at<int32_t>(ws, L.tiles),   at<int32_t>(ws, L.ntiles),
                     at<int32_t>(ws, L.tile_off)};
}

// The same layer as run_grouped_bf16 in one persistent launch: the routing
// plan, gate_up, down and the combine (shapes that fit it; others take the
// stage-by-stage sequence).
int run_layer_bf16(StageClock& clock, const Layout& L, const uint16_t* hidden,
                   const ExpertWeights& gate_up, const ExpertWeights& down, const int32_t* idx,
                   const float* w, const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                   uint16_t* out, void* ws, hipStream_t s) {
    if (!layer_bf16_fits(H, F))
        return run_grouped_bf16(clock, L, hidden, gate_up, down, idx, w, residual, T, H, F, E, k,
                                out, ws, s);
    clock.mark(MOE_STAGE_LAYER);
    return launched(launch_layer_bf16(hidden, gate_up, down, idx, layer_plan_in(L, ws), w,
                                      residual, T, H, F, E, k, at<uint16_t>(ws, L.h),
                                      at<uint16_t>(ws, L.y), out, at<void>(ws, L.sync), s));
}

int check_bf16_args(const uint16_t* hidden, const uint16_t* gate_up, const uint16_t* down,
                    const int32_t* idx, const float* w, const uint16_t* residual, uint16_t* out) {
    if (!hidden || !gate_up || !down || !idx || !w || !out) return MOE_ERR_NULL;
    if (!aligned16(hidden) || !aligned16(gate_up) || !aligned16(down) || !aligned16(out) ||
        ((uintptr_t)idx & 3u) || ((uintptr_t)w & 3u) || (residual && !aligned16(residual)))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}
// Shared experts of the fp8 and mxfp4 layers: S experts stored like the
// routed ones (weights and block scales), passed by every token with weight
// 1, as extra experts E .. E+S-1 of the same grouped products.  S == 0: none.
struct SharedQ {
    int S;
    const uint8_t* gate_up;
    const void* gate_up_scale;
    const uint8_t* down;
    const void* down_scale;
};

// Checks common to the quantised layers with shared experts; fills the
// workspace layout (routed experts only when S == 0).
int check_sharedq(const SharedQ& sh, int variant, int64_t T, int H, int F, int E, int k, Layout* L) {
    if (sh.S < 0 || sh.S > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
    if (sh.S) {
        if (!sh.gate_up || !sh.gate_up_scale || !sh.down || !sh.down_scale) return MOE_ERR_NULL;
        const uintptr_t sa = variant == MOE_VARIANT_MXFP4 ? 3u : 15u;   // E8M0 bytes / fp32 scales
        if (!aligned16(sh.gate_up) || !aligned16(sh.down) ||
            (((uintptr_t)sh.gate_up_scale | (uintptr_t)sh.down_scale) & sa))
            return MOE_ERR_ALIGN;
    }
    const int rc = check_shape(variant, T, H, F, E + sh.S, k + sh.S);
    if (rc) return rc;
    *L = sh.S ? make_shared_layout(variant, T, H, F, E, k, sh.S) : make_layout(variant, T, H, F, E, k);
    return MOE_OK;
}

// With shared experts: the augmented routing [T, k+S] into the workspace;
// idx / w / E / k then describe the augmented problem.
int augment_if_shared(StageClock& clock, const SharedQ& sh, const Layout& L, void* ws, int64_t T,
                      const int32_t*& idx, const float*& w, int& E, int& k, hipStream_t stream) {
    if (!sh.S) return MOE_OK;
    int32_t* idx2 = at<int32_t>(ws, L.aug_idx);
    float* w2 = at<float>(ws, L.aug_w);
    clock.mark(MOE_STAGE_SHARED_ROUTE);
    const int rc = launched(launch_augment_routing(idx, w, T, k, E, sh.S, idx2, w2, stream));
    idx = idx2;
    w = w2;
    E += sh.S;
    k += sh.S;
    return rc;
}

// FP8 layer: the plan, the two grouped fp8 products and the combine; with
// `hidden` (bf16) set, its block-128 quantisation into the workspace first.
int run_fp8(int variant, const uint16_t* hidden, const uint8_t* x, const float* x_scale,
            const uint8_t* gate_up, const float* gate_up_scale, const uint8_t* down,
            const float* down_scale, const SharedQ& sh, const int32_t* top_k_index,
            const float* top_k_weights, const uint16_t* residual, int64_t T, int H, int F, int E,
            int k, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream,
            bool fused = false) {
    if (!gate_up || !gate_up_scale || !down || !down_scale || !top_k_index || !top_k_weights ||
        !out)
        return MOE_ERR_NULL;
    if (!aligned16(gate_up) || !aligned16(down) || !aligned16(out) || !aligned16(gate_up_scale) ||
        !aligned16(down_scale) || (residual && !aligned16(residual)) ||
        (((uintptr_t)top_k_index | (uintptr_t)top_k_weights) & 3u))
        return MOE_ERR_ALIGN;
    Layout L;
    int rc = check_sharedq(sh, variant, T, H, F, E, k, &L);
    if (rc) return rc;
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    const ExpertArray<uint8_t> w13{gate_up, sh.S ? sh.gate_up : gate_up, E};
    const ExpertArray<float> w13s{gate_up_scale, sh.S ? (const float*)sh.gate_up_scale : gate_up_scale, E};
    const ExpertArray<uint8_t> w2{down, sh.S ? sh.down : down, E};
    const ExpertArray<float> w2s{down_scale, sh.S ? (const float*)sh.down_scale : down_scale, E};
    uint8_t* hq = at<uint8_t>(ws, L.h);
    float* hs = at<float>(ws, L.hs);
    uint16_t* y = at<uint16_t>(ws, L.y);
    StageClock clock(stream);
    if (hidden) {
        x = at<uint8_t>(ws, L.xq);
        x_scale = at<float>(ws, L.xs);
        clock.mark(MOE_STAGE_QUANTIZE);
        rc = launched(launch_quantize_fp8(hidden, 1, T, H, (uint8_t*)x, (float*)x_scale, false, stream));
        if (rc) return rc;
    }
    const int32_t* idx = top_k_index;
    const float* w = top_k_weights;
    if ((rc = augment_if_shared(clock, sh, L, ws, T, idx, w, E, k, stream))) return rc;
    const int P = (int)(T * k);
    if (fused && layer_fp8_fits(P, E, H, F)) {
        clock.mark(MOE_STAGE_LAYER);
        return launched(launch_layer_fp8(x, x_scale, w13, w13s, w2, w2s, idx, layer_plan_in(L, ws),
                                         w, residual, T, H, F, E, k, hq, hs, y, out,
                                         at<void>(ws, L.sync), stream));
    }
    const GroupedPlan pl = plan_in(L, ws, E);
    clock.mark(MOE_STAGE_PLAN);
    const bool narrow = fp8_use_narrow(P, E, H, F);
    rc = launched(launch_plan(idx, P, E, at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                              at<int32_t>(ws, L.perm), at<int32_t>(ws, L.inv),
                              at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                              at<int32_t>(ws, L.tile_off), fp8_tile_m(narrow), stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_GATE_UP);
    rc = launched(launch_gateup_fp8(x, x_scale, w13, w13s, pl, narrow, H, F, k, hq, hs, stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_DOWN);
    rc = launched(launch_down_fp8(hq, hs, w2, w2s, pl, narrow, H, F, y, stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_COMBINE);
    return launched(launch_combine(y, at<int32_t>(ws, L.inv), w, residual, T, k, H, out, stream));
}
// MXFP4 layer: the plan, the two grouped MX products and the combine.
int run_mxfp4(const uint8_t* x, const uint8_t* x_scale, const uint8_t* gate_up,
              const uint8_t* gate_up_scale, const uint8_t* down, const uint8_t* down_scale,
              const SharedQ& sh, const int32_t* top_k_index, const float* top_k_weights,
              const uint16_t* residual, int64_t T, int H, int F, int E, int k, uint16_t* out,
              void* ws, size_t ws_bytes, hipStream_t stream, bool fused = false) {
    if (!x || !x_scale || !gate_up || !gate_up_scale || !down || !down_scale || !top_k_index ||
        !top_k_weights || !out)
        return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(gate_up) || !aligned16(down) || !aligned16(out) ||
        (residual && !aligned16(residual)) ||
        (((uintptr_t)x_scale | (uintptr_t)gate_up_scale | (uintptr_t)down_scale |
          (uintptr_t)top_k_index | (uintptr_t)top_k_weights) & 3u))
        return MOE_ERR_ALIGN;
    Layout L;
    int rc = check_sharedq(sh, MOE_VARIANT_MXFP4, T, H, F, E, k, &L);
    if (rc) return rc;
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    const ExpertArray<uint8_t> w13{gate_up, sh.S ? sh.gate_up : gate_up, E};
    const ExpertArray<uint8_t> w13s{gate_up_scale, sh.S ? (const uint8_t*)sh.gate_up_scale : gate_up_scale, E};
    const ExpertArray<uint8_t> w2{down, sh.S ? sh.down : down, E};
    const ExpertArray<uint8_t> w2s{down_scale, sh.S ? (const uint8_t*)sh.down_scale : down_scale, E};
    uint8_t* hq = at<uint8_t>(ws, L.h);
    uint8_t* hs = at<uint8_t>(ws, L.hs);
    uint16_t* y = at<uint16_t>(ws, L.y);
    StageClock clock(stream);
    const int32_t* idx = top_k_index;
    const float* w = top_k_weights;
    if ((rc = augment_if_shared(clock, sh, L, ws, T, idx, w, E, k, stream))) return rc;
    const int P = (int)(T * k);
    if (fused && layer_mx_fits(P, E, H, F)) {
        clock.mark(MOE_STAGE_LAYER);
        return launched(launch_layer_mx(x, x_scale, w13, w13s, w2, w2s, idx, layer_plan_in(L, ws), w,
                                        residual, T, H, F, E, k, hq, hs, y, out,
                                        at<void>(ws, L.sync), stream));
    }
    const GroupedPlan pl = plan_in(L, ws, E);
    clock.mark(MOE_STAGE_PLAN);
    const bool narrow = mx_use_narrow(P, E, H, F);
    rc = launched(launch_plan(idx, P, E, at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                              at<int32_t>(ws, L.perm), at<int32_t>(ws, L.inv),
                              at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                              at<int32_t>(ws, L.tile_off), mx_tile_m(narrow), stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_GATE_UP);
    const bool wide = !narrow && mx_use_wide(P, E, H, F);
    rc = launched(launch_gateup_mx(x, x_scale, w13, w13s, pl, wide, narrow, H, F, k, hq, hs, stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_DOWN);
    rc = launched(launch_down_mx(hq, hs, w2, w2s, pl, wide, narrow, H, F, y, stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_COMBINE);
    return launched(launch_combine(y, at<int32_t>(ws, L.inv), w, residual, T, k, H, out, stream));
}
// Router arguments (moe_route_topk / moe_route_plan).
int check_route(const void* logits, const void* bias, int logits_bf16, int mode, int64_t T, int E,
                int k, int num_groups, int topk_group, int group_top, const int32_t* idx,
                const float* w) {
    if (!logits || !idx || !w) return MOE_ERR_NULL;
    if (mode == MOE_ROUTE_SIGMOID_GROUP && !bias) return MOE_ERR_NULL;
    if ((logits_bf16 != 0 && logits_bf16 != 1) || T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 ||
        k > E || k > 32 || T * (int64_t)k >= ((int64_t)1 << 31) || T * (int64_t)E >= ((int64_t)1 << 40))
        return MOE_ERR_SHAPE;
    if (mode == MOE_ROUTE_SOFTMAX) {
        if (bias) return MOE_ERR_SHAPE;
    } else if (mode == MOE_ROUTE_SIGMOID_GROUP) {
        if (num_groups < 1 || num_groups > 64 || E % num_groups || topk_group < 1 ||
            topk_group > num_groups || (group_top != 1 && group_top != 2) ||
            (group_top == 2 && E / num_groups < 2) || k > topk_group * (E / num_groups))
            return MOE_ERR_SHAPE;
    } else {
        return MOE_ERR_SHAPE;
    }
    const uintptr_t a = logits_bf16 ? 1u : 3u;
    if (((uintptr_t)logits & a) || ((uintptr_t)bias & a) || (((uintptr_t)idx | (uintptr_t)w) & 3u))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

// The decode launch sequence (gather-GEMV for a few tokens, else the grouped
// path) over E experts (routed, then shared) and k slots per token.
int run_decode(StageClock& clock, const Layout& L, const uint16_t* hidden,
               const ExpertWeights& gate_up, const ExpertWeights& down, const int32_t* idx,
               const float* w, const uint16_t* residual, int64_t T, int H, int F, int E, int k,
               uint16_t* out, void* ws, hipStream_t stream) {
    if (!L.decode_fast)
        return run_grouped_bf16(clock, L, hidden, gate_up, down, idx, w, residual, T, H, F, E, k,
                                out, ws, stream);
    clock.mark(MOE_STAGE_DECODE);
    return launched(launch_decode(hidden, gate_up, down, idx, w, residual, (int)T, k, E, H, F, out,
                                  at<void>(ws, L.part), stream));
}

// Both shared-expert entry points: the augmented routing into the workspace,
// then the plain prefill or decode sequence over E + S experts.
int run_shared(int variant, const uint16_t* hidden, const uint16_t* gate_up, const uint16_t* down,
               const uint16_t* shared_gate_up, const uint16_t* shared_down,
               const int32_t* top_k_index, const float* top_k_weights, const uint16_t* residual,
               int64_t T, int H, int F, int E, int k, int S, uint16_t* out, void* ws,
               size_t ws_bytes, hipStream_t stream) {
    int rc = check_bf16_args(hidden, gate_up, down, top_k_index, top_k_weights, residual, out);
    if (rc) return rc;
    if (!shared_gate_up || !shared_down) return MOE_ERR_NULL;
    if (!aligned16(shared_gate_up) || !aligned16(shared_down)) return MOE_ERR_ALIGN;
    if (S < 1 || S > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
    if ((rc = check_shape(variant, T, H, F, E + S, k + S))) return rc;
    const Layout L = make_shared_layout(variant, T, H, F, E, k, S);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    int32_t* idx2 = at<int32_t>(ws, L.aug_idx);
    float* w2 = at<float>(ws, L.aug_w);
    StageClock clock(stream);
    const ExpertWeights gu{gate_up, shared_gate_up, E}, dn{down, shared_down, E};
    if (variant == MOE_VARIANT_DECODE && L.decode_fast) {
        // the gather-GEMV kernel appends the shared slots itself
        clock.mark(MOE_STAGE_DECODE);
        return launched(launch_decode(hidden, gu, dn, top_k_index, top_k_weights, residual, (int)T,
                                      k + S, E + S, H, F, out, at<void>(ws, L.part), stream,
                                      RouteArgs{}, nullptr, nullptr, S));
    }
    clock.mark(MOE_STAGE_SHARED_ROUTE);
    rc = launched(launch_augment_routing(top_k_index, top_k_weights, T, k, E, S, idx2, w2, stream));
    if (rc) return rc;
    if (variant == MOE_VARIANT_PREFILL)
        return run_grouped_bf16(clock, L, hidden, gu, dn, idx2, w2, residual, T, H, F, E + S,
                                k + S, out, ws, stream);
    return run_decode(clock, L, hidden, gu, dn, idx2, w2, residual, T, H, F, E + S, k + S, out, ws,
                      stream);
}
// ------------------------------------------------- allocation-free decode
// The workspace of moe_experts_decode_noalloc: a static device array, one
// copy per GPU for the life of the process.  In host code `scratch` only
// names the symbol; its device address (per device) comes from
// hipGetSymbolAddress and is the only way host code refers to its memory.
static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's `scratch` (looked up once per device, with
// that device current).
int scratch_ptr(int dev, void** out) {
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return MOE_OK;
}
}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer argument is NULL";
        case MOE_ERR_SHAPE: return "a size argument is outside the supported range";
        case MOE_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "workspace is NULL, not 256-byte aligned, or too small";
        case MOE_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case MOE_ERR_DEVICE: return "the current HIP device is not a gfx950 GPU";
        case MOE_ERR_SCRATCH:
            return "the call needs more scratch memory than the library's static buffer holds "
                   "(MOE_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int moe_workspace_size(int variant, int64_t T, int H, int F, int E, int k, size_t* bytes) {
    if (!bytes) return MOE_ERR_NULL;
    const int rc = check_shape(variant, T, H, F, E, k);
    if (rc) return rc;
    *bytes = make_layout(variant, T, H, F, E, k).total;
    return MOE_OK;
}

int moe_workspace_layout(int variant, int64_t T, int H, int F, int E, int k, size_t offs[8]) {
    if (!offs) return MOE_ERR_NULL;
    const int rc = check_shape(variant, T, H, F, E, k);
    if (rc) return rc;
    const Layout L = make_layout(variant, T, H, F, E, k);
    offs[0] = L.counts; offs[1] = L.offsets; offs[2] = L.perm; offs[3] = L.inv;
    offs[4] = L.h; offs[5] = L.hs; offs[6] = L.y; offs[7] = L.total;
    return MOE_OK;
}

int moe_routing_plan(const int32_t* top_k_index, int64_t T, int k, int E, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
    if (!top_k_index || !counts || !offsets || !perm || !inv) return MOE_ERR_NULL;
    int rc = check_shape(MOE_VARIANT_PLAN, T, 0, 0, E, k);
    if (rc) return rc;
    if (((uintptr_t)top_k_index | (uintptr_t)counts | (uintptr_t)offsets | (uintptr_t)perm |
         (uintptr_t)inv) & 3u)
        return MOE_ERR_ALIGN;
    const Layout L = make_layout(MOE_VARIANT_PLAN, T, 0, 0, E, k);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    return launched(launch_plan(top_k_index, (int)(T * k), E, counts, offsets, perm, inv,
                                at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                at<int32_t>(ws, L.tile_off), kPlanTileM, stream));
}

int moe_experts_prefill(const uint16_t* hidden, const uint16_t* gate_up, const uint16_t* down,
                        const int32_t* top_k_index, const float* top_k_weights,
                        const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                        uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_bf16_args(hidden, gate_up, down, top_k_index, top_k_weights, residual, out);
    if (rc) return rc;
    if ((rc = check_shape(MOE_VARIANT_PREFILL, T, H, F, E, k))) return rc;
    const Layout L = make_layout(MOE_VARIANT_PREFILL, T, H, F, E, k);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    return run_grouped_bf16(clock, L, hidden, routed_only(gate_up, E), routed_only(down, E),
                            top_k_index, top_k_weights, residual, T, H, F, E, k, out, ws, stream);
}

int moe_experts_prefill_fused(const uint16_t* hidden, const uint16_t* gate_up,
                              const uint16_t* down, const int32_t* top_k_index,
                              const float* top_k_weights, const uint16_t* residual, int64_t T,
                              int H, int F, int E, int k, uint16_t* out, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    int rc = check_bf16_args(hidden, gate_up, down, top_k_index, top_k_weights, residual, out);
    if (rc) return rc;
    if ((rc = check_shape(MOE_VARIANT_PREFILL, T, H, F, E, k))) return rc;
    const Layout L = make_layout(MOE_VARIANT_PREFILL, T, H, F, E, k);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    return run_layer_bf16(clock, L, hidden, routed_only(gate_up, E), routed_only(down, E),
                          top_k_index, top_k_weights, residual, T, H, F, E, k, out, ws, stream);
}

int moe_experts_decode(const uint16_t* hidden, const uint16_t* gate_up, const uint16_t* down,
                       const int32_t* top_k_index, const float* top_k_weights,
                       const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                       uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_bf16_args(hidden, gate_up, down, top_k_index, top_k_weights, residual, out);
    if (rc) return rc;
    if ((rc = check_shape(MOE_VARIANT_DECODE, T, H, F, E, k))) return rc;
    const Layout L = make_layout(MOE_VARIANT_DECODE, T, H, F, E, k);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    return run_decode(clock, L, hidden, routed_only(gate_up, E), routed_only(down, E), top_k_index,
                      top_k_weights, residual, T, H, F, E, k, out, ws, stream);
}

int moe_experts_decode_noalloc(const uint16_t* hidden, const uint16_t* gate_up,
                               const uint16_t* down, const int32_t* top_k_index,
                               const float* top_k_weights, const uint16_t* residual, int64_t T,
                               int H, int F, int E, int k, uint16_t* out, hipStream_t stream) {
    int rc = check_bf16_args(hidden, gate_up, down, top_k_index, top_k_weights, residual, out);
    if (rc) return rc;
    if ((rc = check_shape(MOE_VARIANT_DECODE, T, H, F, E, k))) return rc;
    const Layout L = make_layout(MOE_VARIANT_DECODE, T, H, F, E, k);
    if (L.total > MOE_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    void* ws = nullptr;
    if ((rc = scratch_ptr(dev, &ws))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    return run_decode(clock, L, hidden, routed_only(gate_up, E), routed_only(down, E), top_k_index,
                      top_k_weights, residual, T, H, F, E, k, out, ws, stream);
}

int moe_workspace_size_shared(int variant, int64_t T, int H, int F, int E, int k, int S,
                              size_t* bytes) {
    if (!bytes) return MOE_ERR_NULL;
    if ((variant != MOE_VARIANT_PREFILL && variant != MOE_VARIANT_DECODE &&
         variant != MOE_VARIANT_FP8 && variant != MOE_VARIANT_MXFP4) ||
        S < 1 || S > MOE_MAX_EXPERTS)
        return MOE_ERR_SHAPE;
    const int rc = check_shape(variant, T, H, F, E + S, k + S);
    if (rc) return rc;
    *bytes = make_shared_layout(variant, T, H, F, E, k, S).total;
    return MOE_OK;
}

int moe_experts_prefill_shared(const uint16_t* hidden, const uint16_t* gate_up,
                               const uint16_t* down, const uint16_t* shared_gate_up,
                               const uint16_t* shared_down, const int32_t* top_k_index,
                               const float* top_k_weights, const uint16_t* residual, int64_t T,
                               int H, int F, int E, int k, int S, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    return run_shared(MOE_VARIANT_PREFILL, hidden, gate_up, down, shared_gate_up, shared_down,
                      top_k_index, top_k_weights, residual, T, H, F, E, k, S, out, ws, ws_bytes,
                      stream);
}

int moe_experts_decode_shared(const uint16_t* hidden, const uint16_t* gate_up,
                              const uint16_t* down, const uint16_t* shared_gate_up,
                              const uint16_t* shared_down, const int32_t* top_k_index,
                              const float* top_k_weights, const uint16_t* residual, int64_t T,
                              int H, int F, int E, int k, int S, uint16_t* out, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    return run_shared(MOE_VARIANT_DECODE, hidden, gate_up, down, shared_gate_up, shared_down,
                      top_k_index, top_k_weights, residual, T, H, F, E, k, S, out, ws, ws_bytes,
                      stream);
}

int moe_experts_fp8(const uint8_t* x, const float* x_scale, const uint8_t* gate_up,
                    const float* gate_up_scale, const uint8_t* down, const float* down_scale,
                    const int32_t* top_k_index, const float* top_k_weights,
                    const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                    uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!x || !x_scale) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(x_scale)) return MOE_ERR_ALIGN;
    return run_fp8(MOE_VARIANT_FP8, nullptr, x, x_scale, gate_up, gate_up_scale, down, down_scale,
                   SharedQ{}, top_k_index, top_k_weights, residual, T, H, F, E, k, out, ws,
                   ws_bytes, stream);
}

int moe_experts_fp8_fused(const uint8_t* x, const float* x_scale, const uint8_t* gate_up,
                          const float* gate_up_scale, const uint8_t* down, const float* down_scale,
                          const int32_t* top_k_index, const float* top_k_weights,
                          const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                          uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!x || !x_scale) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(x_scale)) return MOE_ERR_ALIGN;
    return run_fp8(MOE_VARIANT_FP8, nullptr, x, x_scale, gate_up, gate_up_scale, down, down_scale,
                   SharedQ{}, top_k_index, top_k_weights, residual, T, H, F, E, k, out, ws,
                   ws_bytes, stream, true);
}

int moe_experts_fp8_shared(const uint8_t* x, const float* x_scale, const uint8_t* gate_up,
                           const float* gate_up_scale, const uint8_t* down,
                           const float* down_scale, const uint8_t* shared_gate_up,
                           const float* shared_gate_up_scale, const uint8_t* shared_down,
                           const float* shared_down_scale, const int32_t* top_k_index,
                           const float* top_k_weights, const uint16_t* residual, int64_t T, int H,
                           int F, int E, int k, int S, uint16_t* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    if (!x || !x_scale) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(x_scale)) return MOE_ERR_ALIGN;
    if (S < 1) return MOE_ERR_SHAPE;
    const SharedQ sh{S, shared_gate_up, shared_gate_up_scale, shared_down, shared_down_scale};
    return run_fp8(MOE_VARIANT_FP8, nullptr, x, x_scale, gate_up, gate_up_scale, down, down_scale,
                   sh, top_k_index, top_k_weights, residual, T, H, F, E, k, out, ws, ws_bytes,
                   stream);
}

int moe_experts_fp8_bf16in(const uint16_t* hidden, const uint8_t* gate_up,
                           const float* gate_up_scale, const uint8_t* down,
                           const float* down_scale, const int32_t* top_k_index,
                           const float* top_k_weights, const uint16_t* residual, int64_t T,
                           int H, int F, int E, int k, uint16_t* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    if (!hidden) return MOE_ERR_NULL;
    if (!aligned16(hidden)) return MOE_ERR_ALIGN;
    return run_fp8(MOE_VARIANT_FP8_BF16IN, hidden, nullptr, nullptr, gate_up, gate_up_scale, down,
                   down_scale, SharedQ{}, top_k_index, top_k_weights, residual, T, H, F, E, k, out,
                   ws, ws_bytes, stream);
}

int moe_experts_mxfp4(const uint8_t* x, const uint8_t* x_scale, const uint8_t* gate_up,
                      const uint8_t* gate_up_scale, const uint8_t* down, const uint8_t* down_scale,
                      const int32_t* top_k_index, const float* top_k_weights,
                      const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                      uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    return run_mxfp4(x, x_scale, gate_up, gate_up_scale, down, down_scale, SharedQ{}, top_k_index,
                     top_k_weights, residual, T, H, F, E, k, out, ws, ws_bytes, stream);
}

int moe_experts_mxfp4_fused(const uint8_t* x, const uint8_t* x_scale, const uint8_t* gate_up,
                            const uint8_t* gate_up_scale, const uint8_t* down,
                            const uint8_t* down_scale, const int32_t* top_k_index,
                            const float* top_k_weights, const uint16_t* residual, int64_t T, int H,
                            int F, int E, int k, uint16_t* out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    return run_mxfp4(x, x_scale, gate_up, gate_up_scale, down, down_scale, SharedQ{}, top_k_index,
                     top_k_weights, residual, T, H, F, E, k, out, ws, ws_bytes, stream, true);
}

int moe_experts_mxfp4_shared(const uint8_t* x, const uint8_t* x_scale, const uint8_t* gate_up,
                             const uint8_t* gate_up_scale, const uint8_t* down,
                             const uint8_t* down_scale, const uint8_t* shared_gate_up,
                             const uint8_t* shared_gate_up_scale, const uint8_t* shared_down,
                             const uint8_t* shared_down_scale, const int32_t* top_k_index,
                             const float* top_k_weights, const uint16_t* residual, int64_t T,
                             int H, int F, int E, int k, int S, uint16_t* out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    if (S < 1) return MOE_ERR_SHAPE;
    const SharedQ sh{S, shared_gate_up, shared_gate_up_scale, shared_down, shared_down_scale};
    return run_mxfp4(x, x_scale, gate_up, gate_up_scale, down, down_scale, sh, top_k_index,
                     top_k_weights, residual, T, H, F, E, k, out, ws, ws_bytes, stream);
}

int moe_route_topk(const void* logits, const void* bias, int logits_bf16, int mode, int64_t T,
                   int E, int k, int num_groups, int topk_group, int group_top,
                   float routed_scaling_factor, int32_t* top_k_index, float* top_k_weights,
                   hipStream_t stream) {
    int rc = check_route(logits, bias, logits_bf16, mode, T, E, k, num_groups, topk_group, group_top,
                         top_k_index, top_k_weights);
    if (rc) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    clock.mark(MOE_STAGE_ROUTER);
    return launched(launch_route(logits, bias, logits_bf16, mode, T, E, k, num_groups, topk_group,
                                 group_top, routed_scaling_factor, top_k_index, top_k_weights,
                                 stream));
}

int moe_route_plan(const void* logits, const void* bias, int logits_bf16, int mode, int64_t T,
                   int E, int k, int num_groups, int topk_group, int group_top,
                   float routed_scaling_factor, int32_t* top_k_index, float* top_k_weights,
                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
    int rc = check_route(logits, bias, logits_bf16, mode, T, E, k, num_groups, topk_group, group_top,
                         top_k_index, top_k_weights);
    if (rc) return rc;
    if (!counts || !offsets || !perm || !inv) return MOE_ERR_NULL;
    if (((uintptr_t)counts | (uintptr_t)offsets | (uintptr_t)perm | (uintptr_t)inv) & 3u)
        return MOE_ERR_ALIGN;
    const Layout L = make_layout(MOE_VARIANT_PLAN, T, 0, 0, E, k);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    if (T <= MOE_ROUTE_PLAN_FUSED_MAX_T) {
        clock.mark(MOE_STAGE_ROUTE_PLAN);
        return launched(launch_route_plan(logits, bias, logits_bf16, mode, (int)T, E, k, num_groups,
                                          topk_group, group_top, routed_scaling_factor,
                                          top_k_index, top_k_weights, counts, offsets, perm, inv,
                                          at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                          at<int32_t>(ws, L.tile_off), kPlanTileM, stream));
    }
    clock.mark(MOE_STAGE_ROUTER);
    rc = launched(launch_route(logits, bias, logits_bf16, mode, T, E, k, num_groups, topk_group,
                               group_top, routed_scaling_factor, top_k_index, top_k_weights,
                               stream));
    if (rc) return rc;
    clock.mark(MOE_STAGE_PLAN);
    return launched(launch_plan(top_k_index, (int)(T * k), E, counts, offsets, perm, inv,
                                at<int32_t>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                at<int32_t>(ws, L.tile_off), kPlanTileM, stream));
}

int moe_experts_decode_routed(const uint16_t* hidden, const void* logits, const void* bias,
                              int logits_bf16, int mode, int num_groups, int topk_group,
                              int group_top, float routed_scaling_factor, const uint16_t* gate_up,
                              const uint16_t* down, const uint16_t* residual, int64_t T, int H,
                              int F, int E, int k, uint16_t* out, int32_t* top_k_index,
                              float* top_k_weights, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
    int rc = check_bf16_args(hidden, gate_up, down, top_k_index, top_k_weights, residual, out);
    if (rc) return rc;
    if ((rc = check_route(logits, bias, logits_bf16, mode, T, E, k, num_groups, topk_group,
                          group_top, top_k_index, top_k_weights)))
        return rc;
    if ((rc = check_shape(MOE_VARIANT_DECODE, T, H, F, E, k))) return rc;
    const Layout L = make_layout(MOE_VARIANT_DECODE, T, H, F, E, k);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    int dev;
    if ((rc = query_device(&dev))) return rc;
    if (T == 0) return MOE_OK;
    StageClock clock(stream);
    const ExpertWeights gu = routed_only(gate_up, E), dn = routed_only(down, E);
    if (!L.decode_fast) {   // router launch, then the decode sequence on its ids
        clock.mark(MOE_STAGE_ROUTER);
        rc = launched(launch_route(logits, bias, logits_bf16, mode, T, E, k, num_groups, topk_group,
                                   group_top, routed_scaling_factor, top_k_index, top_k_weights,
                                   stream));
        if (rc) return rc;
        return run_decode(clock, L, hidden, gu, dn, top_k_index, top_k_weights, residual, T, H, F,
                          E, k, out, ws, stream);
    }
    const RouteArgs ra{logits, bias, logits_bf16, mode, E, k, num_groups, topk_group, group_top,
                       routed_scaling_factor};
    clock.mark(MOE_STAGE_DECODE);
    return launched(launch_decode(hidden, gu, dn, nullptr, nullptr, residual, (int)T, k, E, H, F,
                                  out, at<void>(ws, L.part), stream, ra, top_k_index,
                                  top_k_weights));
}

int moe_profile_begin(int max_calls) {
    if (max_calls < 1 || max_calls > MOE_PROFILE_MAX_CALLS) return MOE_ERR_SHAPE;
    int dev, rc;
    if ((rc = query_device(&dev))) return rc;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    const size_t need = (size_t)max_calls * kProfStages * 2;
    while (g_prof.ev.size() < need) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_LAUNCH;
        g_prof.ev.push_back(e);
    }
    g_prof.ids.assign((size_t)max_calls * kProfStages, -1);
    g_prof.cap = max_calls;
    g_prof.used = 0;
    g_prof.on = true;
    return MOE_OK;
}

int moe_profile_end(int max_calls, int* n_calls, float* ms, int* stage_ids) {
    if (!n_calls || !ms || !stage_ids) return MOE_ERR_NULL;
    if (max_calls < 0) return MOE_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.on = false;
    const int n = g_prof.used < max_calls ? g_prof.used : max_calls;
    for (int c = 0; c < n; ++c) {
        for (int i = 0; i < kProfStages; ++i) {
            const size_t j = (size_t)c * kProfStages + i;
            ms[j] = -1.0f;
            stage_ids[j] = -1;
            if (g_prof.ids[j] < 0) continue;
            float t = 0.0f;
            if (hipEventSynchronize(g_prof.ev[2 * j + 1]) != hipSuccess ||
                hipEventElapsedTime(&t, g_prof.ev[2 * j], g_prof.ev[2 * j + 1]) != hipSuccess)
                return MOE_ERR_LAUNCH;
            ms[j] = t;
            stage_ids[j] = g_prof.ids[j];
        }
    }
    *n_calls = n;
    g_prof.used = 0;
    return MOE_OK;
}

int moe_probe_stream_read(const void* src, size_t bytes, int grid, void* sink,
                          hipStream_t stream) {
    if (!src || !sink) return MOE_ERR_NULL;
    if (!aligned16(src) || !aligned16(sink)) return MOE_ERR_ALIGN;
    if (bytes < 16 || bytes % 16 || grid < 1 || grid > 65535) return MOE_ERR_SHAPE;
    int dev, rc;
    if ((rc = query_device(&dev))) return rc;
    StageClock clock(stream);
    clock.mark(MOE_STAGE_PROBE);
    return launched(launch_probe_read(src, bytes, grid, sink, stream));
}

int moe_set_grid_cap(int max_workgroups) {
    if (max_workgroups < 0) return MOE_ERR_SHAPE;
    g_grid_cap.store(max_workgroups, std::memory_order_relaxed);
    return MOE_OK;
}

int moe_quantize_fp8_block128(const void* in, int in_is_bf16, int64_t rows, int K, uint8_t* codes,
                              float* scales, hipStream_t stream) {
    if (!in || !codes || !scales) return MOE_ERR_NULL;
    if (rows < 0 || K < 128 || K % 128 || rows * (int64_t)(K / 128) * 32 >= ((int64_t)1 << 31))
        return MOE_ERR_SHAPE;
    if (((uintptr_t)in | (uintptr_t)scales) & 3u) return MOE_ERR_ALIGN;
    int dev, rc;
    if ((rc = query_device(&dev))) return rc;
    if (rows == 0) return MOE_OK;
    return launched(launch_quantize_fp8(in, in_is_bf16, rows, K, codes, scales, false, stream));
}

int moe_quantize_fp8_block128_ue8m0(const void* in, int in_is_bf16, int64_t rows, int K,
                                    uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    if (!in || !codes || !scales) return MOE_ERR_NULL;
    if (rows < 0 || K < 128 || K % 128 || rows * (int64_t)(K / 128) * 32 >= ((int64_t)1 << 31))
        return MOE_ERR_SHAPE;
    if ((uintptr_t)in & 3u) return MOE_ERR_ALIGN;
    int dev, rc;
    if ((rc = query_device(&dev))) return rc;
    if (rows == 0) return MOE_OK;
    return launched(launch_quantize_fp8(in, in_is_bf16, rows, K, codes, scales, true, stream));
}

}  // extern "C"

// moe_gemm_bf16.hip - grouped bf16 products of the routed-experts layer on
// gfx950 MFMA, and the router-weighted combine.
//
// Model card "DeepSeek-OCR-2 MoE experts": the prefill op is a grouped GEMM
// over experts with a plain SiLU SwiGLU between the two products, then a
// router-weighted scatter-add; "Usage" fixes gate_up_proj [E,2F,H] and
// down_proj [E,H,F] (both K-contiguous, so C = A * B^T with both operands
// K-major, the layout MFMA wants).  The combine follows mirage issue
// "Supporting MegaKernel for DeepSeek Models", moe_local_reduction, without
// its residual, done as a gather in slot order (no float atomics).
#include <algorithm>
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_layer.h"

namespace moe {

constexpr int kGemmThreads = 512;  // 8 waves; see WaveGrid for their tiles
constexpr int kBM = 256;           // rows of an M tile (about one expert's rows at prefill sizes)
constexpr int kBK = 64;            // bf16 K elements per stage: one 128-byte line per row
constexpr int kAStages = 2;        // token-row stages (L2 hits mostly): loads run 1 step ahead
constexpr int kBStages = 3;        // weight stages (HBM): loads run 2 steps ahead

// How the 8 waves split a 256 x BN tile.  Waves w and w + 4 of a workgroup
// share one SIMD (MI355X places the first four waves on the four SIMDs and
// the next four in the same order).  For 256-wide panels the grid is 2 (M) x
// 4 (N), laid out so that the two waves of a SIMD own the same panel columns
// and the two 128-row halves of the tile: a wave skips its 32-row blocks past
// the tile's last row, so each SIMD's matrix work follows the rows the tile
// really has (experts with 160-220 rows fill 256-row tiles only in part).
// Narrower panels keep a 4 (M) x 2 (N) grid (a SWIGLU wave needs a gate
// block and its up block).
template <int BN>
struct WaveGrid {
    static constexpr int WN = BN == 256 ? 4 : 2;   // waves along the panel
    static constexpr int WM = 8 / WN;              // waves along the rows
    static constexpr int MB = kBM / 32 / WM;       // 32-row blocks per wave
    static constexpr int NB = BN / 32 / WN;        // 32-row panel blocks per wave
    __device__ static int wm(int wave) { return WN == 4 ? wave >> 2 : wave & 3; }
    __device__ static int wn(int wave) { return WN == 4 ? wave & 3 : wave >> 2; }
};

// The persistent loop of a grouped product, shared by the stand-alone
// kernels and the one-launch layer, which differ in the Sched hooks: which
// items a workgroup takes, what it waits for before reading an item's
// operands, how it stores and what it signals once stores have completed.
// One work item = (M tile of <= 256 rows of one expert) x (BN rows of the
// expert's weight panel).  Wave (wm, wn) owns tile rows [32 MB wm, 32 MB
// (wm+1)) as MB 32-row blocks and panel rows [32 NB wn, 32 NB (wn+1)) as NB
// 32-row blocks.
// Operands stream through LDS rings filled by direct global->LDS loads, one
// whole 128-byte line per row and stage (on MI355X, half-line requests halve
// what L2 delivers per CU).  Each lane fetches the global chunk that belongs
// at its fixed LDS position, so the bank swizzle costs nothing.  The token
// rows have two stages and the weight rows three: weights come from HBM and
// need the longer lead; together they fill the 160 KB of LDS.  Rows past an
// M tile's end load a row of the tile (or token row 0) and their outputs are
// never stored.
// SWIGLU: panel rows are interleaved in blocks of 32 as gate, up, gate, up,
// ... so each wave holds matching gate/up accumulators lane for lane, and the
// epilogue writes h = silu(gate) * up as bf16 [P, F] in expert order.
// Otherwise the epilogue writes y bf16 [P, n_out] in expert order too (the
// combine finds a slot's row through the plan's inverse permutation).
template <int BN, bool SWIGLU, class Sched>
__device__ __forceinline__ void grouped_loop(
    u32x4* __restrict__ lds, const uint16_t* __restrict__ A, const ExpertWeights& B,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ offsets, int E, int K,
    int n_out, int b_rows, int topk, uint16_t* __restrict__ C, Sched& sc) {
    using WG = WaveGrid<BN>;
    constexpr int MB = WG::MB;
    constexpr int NB = WG::NB;
    constexpr int A_INST = kBM / 8 / 8;       // 8 rows per wave load; per wave and stage
    constexpr int B_INST = BN / 8 / 8;
    constexpr int A_STAGE = kBM * 8;          // u32x4 per stage
    constexpr int B_STAGE = BN * 8;
    constexpr int B_BASE = kAStages * A_STAGE;
    static_assert(NB >= 1 && B_INST >= 1 && (!SWIGLU || NB % 2 == 0), "bad panel width");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = WG::wm(wave), wn = WG::wn(wave);
    const int n_tiles_n = SWIGLU ? n_out / (BN / 2) : n_out / BN;
    const int nks = K / kBK;
    const int fsw = (lane >> 1) & 7;  // lds_chunk swizzle of fragment rows 32 b + lane % 32
    const int lrow = lane >> 3, lslot = lane & 7;

    // Per-item state: which tile, and every lane's row pointers for its
    // share of the LDS fills.
    struct Item {
        GroupedItem gi;
        int e, nt, row0, mrows;
        const uint16_t* a_src[A_INST];
        const uint16_t* b_src[B_INST];
    };
    auto setup = [&](int it, Item& m) {
        const GroupedItem gi = grouped_item(it, tile_off, E, n_tiles_n);
        m.gi = gi;
        m.e = gi.e;
        m.nt = gi.nt;
        m.row0 = tiles[2 * gi.mt + 1];
        m.mrows = min(kBM, offsets[m.e + 1] - m.row0);
        // token rows of the tile (all slot ids requested at once, no branch)
        int pr[A_INST];
#pragma unroll
        for (int i = 0; i < A_INST; ++i) {
            const int r = 8 * (A_INST * wave + i) + lrow;
            pr[i] = SWIGLU ? perm[m.row0 + min(r, m.mrows - 1)] : 0;
        }
#pragma unroll
        for (int i = 0; i < A_INST; ++i) {
            const int r = 8 * (A_INST * wave + i) + lrow;
            // rows past the tile's end repeat its first row (never stored)
            const int64_t arow = SWIGLU ? (r < m.mrows ? pr[i] / topk : 0) : m.row0 + (r < m.mrows ? r : 0);
            m.a_src[i] = A + arow * K + lds_chunk(r, lslot) * 8;
        }
        const uint16_t* Be = B.expert(m.e, (int64_t)b_rows * K);
#pragma unroll
        for (int i = 0; i < B_INST; ++i) {
            const int r = 8 * (B_INST * wave + i) + lrow;
            int brow;
            if (SWIGLU) {
                const int blk = r >> 5;
                brow = ((blk & 1) ? n_out : 0) + m.nt * (BN / 2) + (blk >> 1) * 32 + (r & 31);
            } else {
                brow = m.nt * BN + r;
            }
            m.b_src[i] = Be + (int64_t)brow * K + lds_chunk(r, lslot) * 8;
        }
    };
    // every wave issues the same number of loads per step, also when the
    // step index is clamped past the end (those fill unread slots)
    auto load_a = [&](const Item& m, int ks) {
        u32x4* dst = &lds[(ks & 1) * A_STAGE];
#pragma unroll
        for (int i = 0; i < A_INST; ++i) dma16(m.a_src[i] + ks * kBK, dst + (A_INST * wave + i) * 64);
    };
    auto load_b = [&](const Item& m, int ks) {
        u32x4* dst = &lds[B_BASE + (ks % kBStages) * B_STAGE];
#pragma unroll
        for (int i = 0; i < B_INST; ++i) dma16(m.b_src[i] + ks * kBK, dst + (B_INST * wave + i) * 64);
    };
    // the first stages of an item: A(0), B(0), B(1)
    auto prologue = [&](const Item& m) {
        load_a(m, 0);
        load_b(m, 0);
        load_b(m, min(1, nks - 1));
    };

    f32x16 acc[MB][NB];
    // The first NV row blocks of the wave, NV a compile-time count: the
    // fragment reads and products of blocks past the tile's last row are
    // skipped (their rows hold row-0 data and are never stored).
    auto compute_nv = [&](auto nv_c, int ks) {
        constexpr int NV = decltype(nv_c)::value;
        const u32x4* as = &lds[(ks & 1) * A_STAGE];
        const u32x4* bs = &lds[B_BASE + (ks % kBStages) * B_STAGE];
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int c = (kk * 2 + (lane >> 5)) ^ fsw;
            u32x4 af[NV], bf[NB];
#pragma unroll
            for (int mb = 0; mb < NV; ++mb) af[mb] = as[(32 * (MB * wm + mb) + (lane & 31)) * 8 + c];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bf[nb] = bs[((wn * NB + nb) * 32 + (lane & 31)) * 8 + c];
#pragma unroll
            for (int mb = 0; mb < NV; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = mfma_bf16_32x32x16(af[mb], bf[nb], acc[mb][nb]);
        }
    };
    // nv (the same in every lane of a wave) = row blocks of this wave that
    // hold tile rows
    auto compute = [&](int ks, int nv) {
        if (nv >= MB) compute_nv(std::integral_constant<int, MB>(), ks);
        else if (nv == 1) compute_nv(std::integral_constant<int, 1>(), ks);
        else if (MB > 2 && nv == 2) compute_nv(std::integral_constant<int, (MB > 2 ? 2 : 1)>(), ks);
        else if (MB > 3 && nv == 3) compute_nv(std::integral_constant<int, (MB > 3 ? 3 : 1)>(), ks);
    };

    // Stores of the finished tile.  Lanes l and l ^ 1 hold neighbouring
    // columns of the same rows; after one swap the even lane owns columns
    // (c, c+1) of row R(q) and the odd lane columns (c-1, c) of row R(q+1),
    // so every store writes a bf16 pair.
    auto epilogue = [&](const Item& m) {
        const bool odd = lane & 1;
        if (32 * MB * wm >= m.mrows) return;
        if (SWIGLU) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    const int f = m.nt * (BN / 2) + (wn * NB / 2 + p) * 32 + (lane & 31);
#pragma unroll
                    for (int q = 0; q < 16; q += 2) {
                        const float h0 = silu_fast(acc[mb][2 * p][q]) * acc[mb][2 * p + 1][q];
                        const float h1 = silu_fast(acc[mb][2 * p][q + 1]) * acc[mb][2 * p + 1][q + 1];
                        const float got = pair_swap(odd ? h0 : h1);
                        const int row = 32 * (MB * wm + mb) + acc_row(q, lane) + (odd ? 1 : 0);
                        if (row < m.mrows) {
                            const uint32_t v = odd ? pack_bf16x2_hw(got, h1) : pack_bf16x2_hw(h0, got);
                            sc.store_u32(C + (int64_t)(m.row0 + row) * n_out + (f & ~1), v);
                        }
                    }
                }
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 16; q += 2) {
                    const int row = 32 * (MB * wm + mb) + acc_row(q, lane) + (odd ? 1 : 0);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const float y0 = acc[mb][nb][q], y1 = acc[mb][nb][q + 1];
                        const float got = pair_swap(odd ? y0 : y1);
                        const int col = m.nt * BN + (wn * NB + nb) * 32 + (lane & 30);
                        if (row < m.mrows) {
                            const uint32_t v = odd ? pack_bf16x2_hw(got, y1) : pack_bf16x2_hw(y0, got);
                            sc.store_u32(C + (int64_t)(m.row0 + row) * n_out + col, v);
                        }
                    }
                }
        }
    };

    int it = sc.first();
    if (it < 0) {
        sc.drained();
        return;
    }
    Item cur, nxt;
    setup(it, cur);
    sc.wait_inputs(cur.gi);
    prologue(cur);
    while (true) {
        // The next item's row pointers are worked out while this item's first
        // stages load (their slot-id loads then cost no wait of their own).
        const int next = sc.next(it);
        const bool more = next >= 0;
        setup(more ? next : it, nxt);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
        const int nv = min(MB, max(0, (cur.mrows - 32 * MB * wm + 31) >> 5));
        // Issue order per step: A(ks+1), then B(ks+2); at step ks the newest
        // B_INST operations (B(ks+1)) may still be in flight.  Loads complete
        // in issue order, so at most B_INST operations in flight means A(ks)
        // and B(ks) have landed: at step 0 too, where the prologue's B(1) and
        // the previous item's epilogue stores are the newer operations.
        for (int ks = 0; ks < nks; ++ks) {
            stage_barrier<B_INST>();           // A(ks) and B(ks) have landed for every wave
            load_a(cur, min(ks + 1, nks - 1)); // refills the A slot read at step ks - 1
            load_b(cur, min(ks + 2, nks - 1)); // refills the B slot read at step ks - 1
            compute(ks, nv);
        }
        lds_barrier();  // every wave is done with the ring before the next item's fills

        // The next item's first stages load while this tile is stored (on the
        // last item the same tile is fetched again and never read).
        if (more) sc.wait_inputs(nxt.gi);
        prologue(nxt);
        epilogue(cur);
        sc.stored(it);
        if (!more) break;
        it = next;
        cur = nxt;
    }
    sc.drained();
    __builtin_amdgcn_s_waitcnt(0);  // no LDS fill may outlive the workgroup
}

// One work item = (M tile of <= 256 rows of one expert) x (BN rows of the
// expert's weight panel); the grid is persistent (see grouped_loop).
template <int BN, bool SWIGLU>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const ExpertWeights B,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ offsets, int E, int K, int n_out, int b_rows, int topk,
    uint16_t* __restrict__ C) {
    // one array for both operands (with fills into two arrays the compiler
    // adds a wait for all of them before every LDS read)
    __shared__ u32x4 lds[kAStages * kBM * 8 + kBStages * BN * 8];
    PlainSched sc{*ntiles_p * (SWIGLU ? n_out / (BN / 2) : n_out / BN)};
    grouped_loop<BN, SWIGLU>(lds, A, B, perm, tiles, tile_off, offsets, E, K, n_out, b_rows, topk,
                             C, sc);
}

int bf16_tile_m() { return kBM; }

template <int BN, bool SWIGLU>
static int gemm_grid() {
    static const int g = resident_grid((const void*)gemm_bf16_kernel<BN, SWIGLU>, kGemmThreads,
                                       device_cu_count());
    return capped_grid(g);
}

template <int BN, bool SWIGLU>
static void launch_bf16(const uint16_t* A, const ExpertWeights& B, const GroupedPlan& pl, int K,
                        int n_out, int b_rows, int topk, uint16_t* C, hipStream_t s) {
    MOE_LAUNCH((gemm_bf16_kernel<BN, SWIGLU>), dim3(gemm_grid<BN, SWIGLU>()),
                       dim3(kGemmThreads), 0, s, A, B, pl.perm, pl.tiles, pl.ntiles, pl.tile_off,
                       pl.offsets, pl.E, K, n_out, b_rows, topk, C);
}

hipError_t launch_gateup_bf16(const uint16_t* x, const ExpertWeights& w13, const GroupedPlan& pl,
                              int H, int F, int k, uint16_t* h, hipStream_t s) {
    if (F % 128 == 0) launch_bf16<256, true>(x, w13, pl, H, F, 2 * F, k, h, s);
    else launch_bf16<128, true>(x, w13, pl, H, F, 2 * F, k, h, s);
    return hipGetLastError();
}

// Rounds of a persistent grid of G workgroups over `items` equal items, in
// units of a 256-wide item (a BN-wide item costs BN/256 of one).
static double makespan(int64_t items, int G, int BN) {
    return (double)((items + G - 1) / G) * BN / 256.0;
}

hipError_t launch_down_bf16(const uint16_t* h, const ExpertWeights& w2, const GroupedPlan& pl,
                            int P, int H, int F, uint16_t* y, hipStream_t s) {
    // The M-tile count is only known on the device; about max(P/256, one
    // tile per touched expert) tiles: pick the panel width whose rounds of the
    // persistent grid finish first (256-wide items leave a mostly idle last
    // round when their count is a little above a multiple of the grid).
    const int64_t tiles = std::max<int64_t>((P + kBM - 1) / kBM, std::min<int64_t>(pl.E, P));
    const bool narrow = H % 256 != 0 ||
                        makespan(tiles * (H / 128), gemm_grid<128, false>(), 128) <
                            makespan(tiles * (H / 256), gemm_grid<256, false>(), 256);
    if (!narrow) launch_bf16<256, false>(h, w2, pl, F, H, H, 1, y, s);
    else if (H % 128 == 0) launch_bf16<128, false>(h, w2, pl, F, H, H, 1, y, s);
    else launch_bf16<64, false>(h, w2, pl, F, H, H, 1, y, s);
    return hipGetLastError();
}

// one thread per unit
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ residual,
                                                      int64_t T, int k, int H,
                                                      uint16_t* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= T * (H / 8)) return;
    combine_unit(y, inv, w, residual, g, k, H, false, out);
}

hipError_t launch_combine(const uint16_t* y, const int32_t* inv, const float* w,
                          const uint16_t* residual, int64_t T, int k, int H, uint16_t* out,
                          hipStream_t s) {
    const int64_t n = T * (H / 8);
    const int blocks = (int)((n + 255) / 256);
    MOE_LAUNCH(combine_kernel, dim3(blocks), dim3(256), 0, s, y, inv, w, residual, T, k, H, out);
    return hipGetLastError();
}

// The plan arrays (counts .. tile_off) are written by the plan phase and
// read afterwards, so they are not restrict-qualified here.
template <int BNG, int BND>
__global__ __launch_bounds__(kGemmThreads) void layer_bf16_kernel(
    const uint16_t* __restrict__ x, const ExpertWeights w13, const ExpertWeights w2,
    const int32_t* __restrict__ idx, int32_t* counts, int32_t* offsets, int32_t* perm,
    int32_t* inv, int32_t* tiles, int32_t* ntiles_p, int32_t* tile_off,
    const float* __restrict__ wts, const uint16_t* __restrict__ residual, int64_t T, int E, int H,
    int F, int k, uint16_t* __restrict__ h, uint16_t* __restrict__ y, uint16_t* __restrict__ out,
    LayerSync sy) {
    constexpr int BNMAX = BNG > BND ? BNG : BND;
    __shared__ u32x4 lds[kAStages * kBM * 8 + kBStages * BNMAX * 8];
    // the routing plan, in the operand ring before its first use
    const uint64_t stamp = layer_plan((int*)lds, idx, (int)(T * k), E, kBM, counts, offsets, perm,
                                      inv, tiles, ntiles_p, tile_off, layer_gen(sy), sy);
    const int ntiles = *ntiles_p;
    const int npg = F / (BNG / 2), npd = H / BND;
    const int NG = ntiles * npg;

    LayerSched<true> sg{NG, NG, npg, 0, stamp, sy, tile_off, 0, nullptr, 0};
    grouped_loop<BNG, true>(lds, x, w13, perm, tiles, tile_off, offsets, E, H, F, 2 * F, k, h, sg);
    const int ND = ntiles * npd;
    const int c = layer_early_down(NG, ND, npg, npd, (int64_t)H * BNG, (int64_t)F * BND);
    LayerSched<false> sd{ND, NG, npg, c, stamp, sy, tile_off, 0, nullptr, 0};
    grouped_loop<BND, false>(lds, h, w2, perm, tiles, tile_off, offsets, E, F, H, H, 1, y, sd);

    layer_combine((int*)lds, y, inv, wts, residual, T, k, H, out, stamp, sy);
}

// A whole number of 128-column h blocks and down panels (other shapes take
// the stand-alone kernels).
bool layer_bf16_fits(int H, int F) { return H % 128 == 0 && F % 128 == 0; }

size_t layer_sync_bytes(int64_t P, int E, int F) {
    return 8 * (32 + 2 * (size_t)kLayerMaxGrid + 2 * (size_t)kLayerPlanChunks +
                (size_t)kLayerPlanChunks * MOE_MAX_EXPERTS / 2 + (size_t)max_m_tiles(P, E) * (F / 128));
}

template <int BND>
static int layer_grid() {
    static const int g = std::min(
        resident_grid((const void*)layer_bf16_kernel<256, BND>, kGemmThreads, device_cu_count()),
        kLayerMaxGrid);
    return capped_grid(g);
}

hipError_t launch_layer_bf16(const uint16_t* x, const ExpertWeights& w13, const ExpertWeights& w2,
                             const int32_t* idx, const LayerPlan& pl, const float* w,
                             const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                             uint16_t* h, uint16_t* y, uint16_t* out, void* sync, hipStream_t s) {
    const LayerSync sy{(uint64_t*)sync};
    if (H % 256 == 0)
        MOE_LAUNCH((layer_bf16_kernel<256, 256>), dim3(layer_grid<256>()), dim3(kGemmThreads), 0,
                   s, x, w13, w2, idx, pl.counts, pl.offsets, pl.perm, pl.inv, pl.tiles,
                   pl.ntiles, pl.tile_off, w, residual, T, E, H, F, k, h, y, out, sy);
    else
        MOE_LAUNCH((layer_bf16_kernel<256, 128>), dim3(layer_grid<128>()), dim3(kGemmThreads), 0,
                   s, x, w13, w2, idx, pl.counts, pl.offsets, pl.perm, pl.inv, pl.tiles,
                   pl.ntiles, pl.tile_off, w, residual, T, E, H, F, k, h, y, out, sy);
    return hipGetLastError();
}

}  // namespace moe

// moe_device.h - device-side helpers shared by the gfx950 kernels of the
// routed-experts layer (internal header, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- vectors
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));
typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin over them

// 16-byte load that marks the line as streamed once (weights read a single time).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even by the gfx950 hardware convert (a NaN stays a NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Unpack 8 bf16 (one 16-byte chunk) into fp32.
__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// fp32 -> OCP E4M3FN with round to nearest even (gfx950 hardware convert).
// Callers clamp to +-448 first, so saturation behaviour never matters.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Two fp32 -> two bf16 in one word (lo in bits 0-15), round to nearest even
// by the gfx950 hardware convert.
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
    const uint16_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return (uint32_t)a | ((uint32_t)b << 16);
}

// SiLU for the grouped-product epilogues: z * 1 / (1 + 2^(-z log2 e)) with
// the hardware exp2 and reciprocal (about 1 ulp each, so a relative error
// near 1e-6, far below the bf16 rounding of the result).  Large negative z
// gives 2^+inf = inf and a zero reciprocal, i.e. -0; large positive z gives z.
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Value of lane l ^ 1 (swap within lane pairs; a DPP quad permutation).
__device__ __forceinline__ float pair_swap(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// ------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float half_sum32(float v) {  // sum within each 32-lane half
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float half_max32(float v) {  // max within each 32-lane half
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// ------------------------------------------------------------------ MFMA
// 32x32x16 bf16 -> fp32.  Lane l supplies row/col (l % 32) and K elements
// [8*(l/32), 8*(l/32)+8); accumulator register r of lane l holds element
// (row = 8*(r/4) + 4*(l/32) + r%4, col = l % 32).
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const uint4 a, const uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const u32x4 a, const u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x64 fp8(e4m3) x fp8(e4m3) -> fp32 with unit E8M0 block scales
// (127 encodes 2^0): lane l supplies 32 K bytes of row/col (l % 32).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(const i32x8 a, const i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ------------------------------------------------------- direct LDS fills
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: the wave writes
// 1 KB at `dst` (wave-uniform), lane L's bytes at dst + 16 L.  Counted by
// vmcnt like a load; no VGPRs are involved.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// 4 bytes per lane from global memory straight into LDS (lane L's word at
// dst + 4 L), counted by vmcnt like dma16.
__device__ __forceinline__ void dma4(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// Workgroup barrier once this wave has at most N vector-memory operations in
// flight (its older LDS fills have landed) and no LDS operation pending.  The
// empty asm statements keep the compiler from moving memory operations
// across it; the explicit wait replaces the vmcnt(0) a __syncthreads() fence
// would force while later stages are still loading.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier once this wave's LDS reads are done (vector-memory
// operations may stay in flight): closes an item, so that no wave refills a
// ring slot another wave is still reading.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------- device-scope accesses
// Relaxed atomics at agent scope (sc1): they bypass the non-coherent per-XCD
// L2, so data written by one workgroup is seen by any other once the store
// has completed (s_waitcnt).
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes per lane from global memory into LDS, device scope (sc1 = 16).
__device__ __forceinline__ void dma16_dev(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 16);
}
// every vector-memory operation of this wave has completed
__device__ __forceinline__ void wait_vm_all() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------- scheduling helpers
// Persistent grids walk work items i = round * G + slot.  Workgroup b runs on
// XCD b % 8; giving each XCD a contiguous run of slots keeps work items that
// share a weight panel (neighbouring M tiles of one expert) inside one L2.
__device__ __forceinline__ int xcd_slot(int b, int G) {
    // G is a multiple of 8 (see resident_grid)
    const int per = G / kXcds;
    return (b % kXcds) * per + (b / kXcds);
}

// Work items of a grouped product, numbered expert by expert: expert e owns
// items [n_tiles_n * tile_off[e], n_tiles_n * tile_off[e+1]), its M tiles
// varying fastest.  Together with xcd_slot this keeps all tiles of an expert
// (which share its token rows and its weight panels) inside one XCD's L2.
// Binary search over the M-tile prefix (E + 1 entries, cached reads).
struct GroupedItem {
    int e, mt, nt;
};
__device__ __forceinline__ GroupedItem grouped_item(int it, const int32_t* __restrict__ tile_off,
                                                    int E, int n_tiles_n) {
    int lo = 0, hi = E;  // find e with tile_off[e]*n <= it < tile_off[e+1]*n
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] * n_tiles_n <= it) lo = mid; else hi = mid;
    }
    const int t0 = tile_off[lo];
    const int mtiles = tile_off[lo + 1] - t0;
    const int local = it - t0 * n_tiles_n;
    GroupedItem g;
    g.e = lo;
    g.nt = local / mtiles;
    g.mt = t0 + (local - g.nt * mtiles);
    return g;
}

// LDS tiles hold rows of eight 16-byte chunks.  MI355X LDS serves a 16-byte
// read for 16 lanes per cycle (64 banks); the MFMA fragment reads touch 16
// consecutive rows at one logical chunk, so the physical chunk is the logical
// one XOR (row / 2) % 8: rows of equal parity then hit 8 distinct chunks.
__device__ __forceinline__ int lds_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Workgroups of `kernel` that are resident at once on the current device,
// rounded down to a multiple of 8 XCDs: a persistent grid must never exceed
// it, or its tail workgroups would start only after the first ones finish.
inline int resident_grid(const void* kernel, int threads, int cu_count) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int g = per_cu * cu_count;
    return g >= kXcds ? (g / kXcds) * kXcds : kXcds;
}

}  // namespace moe

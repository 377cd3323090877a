/*
 * moe_experts.h - C ABI of the routed-experts MoE layer for MI355X (gfx950).
 *
 * The layer (model card "DeepSeek-OCR-2 MoE experts", description and
 * "Usage"): given hidden states x [T,H], per-expert gate_up weights
 * [E,2F,H] and down weights [E,H,F], and the router's top_k_index [T,k]
 * (int32) and top_k_weights [T,k] (fp32), compute for every token t
 *
 *     out[t] = sum_j  w[t,j] * down[e] @ ( silu(g[0:F]) * g[F:2F] ),
 *              g = gate_up[e] @ x[t],  e = top_k_index[t,j],
 *
 * i.e. a per-expert token permutation, a grouped gate_up product, the SwiGLU
 * activation (rows [0,F) of gate_up are the gate, rows [F,2F) are "up"),
 * a grouped down product and the router-weighted combine.  Routing and shared
 * experts are outside the layer; top_k_weights already include any routed
 * scaling factor.  The fp8 variant follows mirage issue "Supporting
 * MegaKernel for DeepSeek Models", Layer Tensor Details: moe_w13_fp8_layer,
 * moe_silu_mul_layer, moe_w2_fp8_layer, moe_local_reduction (its
 * residual optional): E4M3 operands with one fp32 scale per row and 128-wide K block.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, dense row-major, and 16-byte
 *    aligned.  They are borrowed: the caller owns them and must keep them
 *    alive until the work enqueued on `stream` has completed.
 *  - bf16 is passed as uint16_t bit patterns, fp8 as uint8_t OCP E4M3FN codes
 *    (bias 7, max 448, 0x7F/0xFF are NaN).
 *  - Expert ids outside [0,E) drop their slot: it contributes nothing.
 *  - `out` is fully overwritten (never accumulated into).  The layer entry
 *    points take an optional `residual` [T,H] bf16 (NULL: none), added to
 *    the routing-weighted sum in fp32 before the single rounding of out
 *    (mirage issue "Supporting MegaKernel for DeepSeek Models",
 *    moe_local_reduction: out = sum_k in[:,k,:] * w[:,k] + residual);
 *    `out` may not alias `residual`.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *    default stream).  No call allocates memory, synchronises, or copies
 *    between host and device.  The library keeps no mutable global state
 *    apart from the optional stage-timing recorder (moe_profile_*, off by
 *    default); concurrent calls are safe when each has its own workspace.
 *  - Results are deterministic: the combine is a gather-reduce in slot order
 *    and no floating-point atomics are used anywhere.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  Argument errors
 *    are detected on the host before anything is enqueued.  T == 0 returns
 *    MOE_OK and enqueues nothing.
 */
#ifndef MOE_EXPERTS_H
#define MOE_EXPERTS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 9

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,       /* a required pointer is NULL                     */
    MOE_ERR_SHAPE = -2,      /* a dimension is out of the supported range       */
    MOE_ERR_ALIGN = -3,      /* a pointer is not 16-byte aligned                */
    MOE_ERR_WORKSPACE = -4,  /* workspace missing, too small or misaligned      */
    MOE_ERR_LAUNCH = -5,     /* the HIP runtime rejected a kernel launch        */
    MOE_ERR_DEVICE = -6,     /* the current device is not a gfx950 GPU          */
    MOE_ERR_SCRATCH = -7,    /* more scratch than MOE_SCRATCH_BYTES needed      */
};

enum moe_variant {
    MOE_VARIANT_PREFILL = 0, /* moe_experts_prefill                            */
    MOE_VARIANT_DECODE = 1,  /* moe_experts_decode                             */
    MOE_VARIANT_FP8 = 2,     /* moe_experts_fp8                                */
    MOE_VARIANT_PLAN = 3,    /* moe_routing_plan                               */
    MOE_VARIANT_FP8_BF16IN = 4, /* moe_experts_fp8_bf16in                      */
    MOE_VARIANT_MXFP4 = 5,   /* moe_experts_mxfp4                              */
};

/* Supported ranges (checked on every call; MOE_ERR_SHAPE otherwise):
 *   1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= E, T >= 0, T*k < 2^31,
 *   bf16 variants: H and F multiples of 64;  fp8 and mxfp4: H and F
 *   multiples of 128. */
#define MOE_MAX_EXPERTS 512

/* Version of this interface (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* moe_strerror(int status);

/*
 * Bytes of device workspace `variant` needs for these sizes, written to
 * *bytes.  The workspace is caller-allocated device memory, 256-byte aligned,
 * that the call uses as scratch (routing plan, intermediate activations and
 * per-slot expert outputs).  Its contents need no initialisation and are
 * undefined after the call.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE.
 */
int moe_workspace_size(int variant, int64_t T, int H, int F, int E, int k, size_t* bytes);

/*
 * Byte offsets, inside the workspace of `variant`, of its stages, for tests
 * and inspection:  offs[0] counts[E] int32, offs[1] offsets[E+1] int32,
 * offs[2] perm[T*k] int32, offs[3] inv[T*k] int32, offs[4] h (bf16 [T*k,F]
 * for prefill, fp8 codes [T*k,F] for fp8 and mxfp4), offs[5] h scales (fp32
 * [T*k,F/128] for fp8, E8M0 bytes [T*k,F/32] for mxfp4), offs[6] y (bf16
 * [T*k,H], expert order like h:
 * row m holds slot perm[m]).
 * Entries a variant does not use are SIZE_MAX.  The decode fast path
 * (T <= 4) builds no plan: its workspace holds the hand-off flags and h
 * (bf16 [T*k, F]), and every entry but the total is SIZE_MAX.
 */
int moe_workspace_layout(int variant, int64_t T, int H, int F, int E, int k, size_t offs[8]);

/*
 * Routing plan: the deterministic per-expert token permutation that the
 * grouped products of the model card's prefill op imply (the [E+1] int32
 * "masks" operand of moe_w13_fp8_layer plays the role of `offsets`).
 *   top_k_index [T,k] int32 (device)  ->
 *   counts[E]    number of valid slots per expert,
 *   offsets[E+1] exclusive prefix of counts; offsets[E] = valid slots,
 *   perm[T*k]    flat slot ids s = t*k+j grouped by expert, ascending s
 *                inside a group, -1 after offsets[E],
 *   inv[T*k]     position of slot s in perm, -1 for a dropped slot.
 * All outputs are device pointers; ws/ws_bytes as for MOE_VARIANT_PLAN.
 * The result is bit-exact and independent of launch configuration.
 */
int moe_routing_plan(const int32_t* top_k_index, int64_t T, int k, int E,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bf16 routed experts, grouped-GEMM form (the model card's prefill op and
 * its operand list in "Usage").
 *   hidden  [T,H]    bf16        gate_up [E,2F,H] bf16     down [E,H,F] bf16
 *   top_k_index [T,k] int32      top_k_weights [T,k] fp32
 *   out     [T,H]    bf16 (written)
 * Accumulation is fp32; the SwiGLU output h and the per-slot expert outputs
 * are rounded to bf16 in the workspace; the combine sums in fp32 in slot
 * order and rounds once (round to nearest even).
 */
int moe_experts_prefill(const uint16_t* hidden, const uint16_t* gate_up, const uint16_t* down,
                        const int32_t* top_k_index, const float* top_k_weights,
                        const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                        uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same layer as moe_experts_prefill (same operands, workspace
 * moe_workspace_size(MOE_VARIANT_PREFILL, ...), errors and results: out is
 * bit-for-bit that of moe_experts_prefill), with the grouped gate_up
 * product, the grouped down product and the combine in one persistent
 * launch after the routing plan (the single-kernel MoE idea of the DeepGEMM
 * "Mega MoE" news item, on one GPU).  Workgroups hand tiles to each other
 * through flags in the workspace: a down tile starts as soon as its rows of
 * h are stored, and the combine once every down tile is, so the tails of
 * the two products overlap.  The workgroups wait for each other, so they
 * must be resident together (the library sizes the grid from the device's
 * occupancy); a wait longer than 2 s gives NaN outputs.  The workspace needs
 * no initialisation: a generation word in it, advanced on the device by
 * every call, stamps the flags (calls must be ordered, as on one stream).
 * H and F multiples of 128; other shapes run the moe_experts_prefill
 * sequence.
 */
int moe_experts_prefill_fused(const uint16_t* hidden, const uint16_t* gate_up,
                              const uint16_t* down, const int32_t* top_k_index,
                              const float* top_k_weights, const uint16_t* residual, int64_t T,
                              int H, int F, int E, int k, uint16_t* out, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * bf16 routed experts, gather-GEMV form for a handful of tokens (the model
 * card's decode op: two persistent phases, no per-expert loop on the host,
 * no device-to-host synchronisation).  Same operands and results contract as
 * moe_experts_prefill.  For T <= 4 (T*k <= 32, H and F <= 2048, H <= 1536
 * when T > 1, and T*k*F <= 49152) the whole layer is one launch of one
 * workgroup per compute unit: gate/up rows of the selected experts produce
 * h, handed between workgroups through the workspace, then the down rows
 * produce out directly; every selected weight byte is read once.  h is
 * stored once per (expert, token) as bf16 of W * silu(gate . x) * (up . x),
 * W the token's summed routing weight on that expert (fp32 products); each
 * output element is a fixed-order fp32 sum over the token's experts, rounded
 * once (deterministic, independent of the grid).  The workgroups wait for
 * each other at the hand-off, so they must be resident together: the
 * library sizes the grid from the device's occupancy, and if other work
 * keeps the compute units busy for more than 100 ms the affected rows come
 * out NaN rather than wait longer.  The workspace needs no initialisation: a
 * generation word in it, advanced on the device by every call, stamps the
 * hand-off flags (calls must be ordered, as on one stream).  Larger calls
 * run the grouped-GEMM path.
 */
int moe_experts_decode(const uint16_t* hidden, const uint16_t* gate_up, const uint16_t* down,
                       const int32_t* top_k_index, const float* top_k_weights,
                       const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                       uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_experts_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The call allocates nothing: its
 * scratch memory is a static device array of MOE_SCRATCH_BYTES inside the
 * library, one per GPU, held from the first call on that GPU until the
 * process ends.  Every call on one GPU uses that GPU's array, so calls that
 * overlap in time on one GPU (concurrent streams, or several host threads)
 * race and must be ordered by the caller; calls on one stream are ordered.
 * Operands, results and limits are those of moe_experts_decode; a shape
 * whose moe_workspace_size(MOE_VARIANT_DECODE, ...) exceeds
 * MOE_SCRATCH_BYTES is rejected with MOE_ERR_SCRATCH before anything is
 * enqueued (the gather-GEMV form of every T <= 4 shape fits).
 */
#define MOE_SCRATCH_BYTES ((size_t)16 << 20)
int moe_experts_decode_noalloc(const uint16_t* hidden, const uint16_t* gate_up,
                               const uint16_t* down, const int32_t* top_k_index,
                               const float* top_k_weights, const uint16_t* residual, int64_t T,
                               int H, int F, int E, int k, uint16_t* out, hipStream_t stream);

/*
 * bf16 routed experts plus S shared experts fused into the same products
 * (DeepGEMM issue "GC MoE": routed experts with optional fused shared
 * experts; the model card "DeepSeek-OCR-2 MoE experts" keeps two shared
 * experts beside the routed ones).  Every token passes through each shared
 * expert with weight 1:
 *   out[t] = sum_j w[t,j] * E_idx[t,j](x[t]) + sum_s S_s(x[t]) (+ residual[t])
 * where each expert is down @ (silu(gate @ x) * (up @ x)).
 *   shared_gate_up [S,2F,H] bf16, shared_down [S,H,F] bf16: device, 16-byte
 *   aligned, the same F and layout as the routed experts; 1 <= S and
 *   E + S <= MOE_MAX_EXPERTS.  Other operands as moe_experts_prefill.
 * The call appends one weight-1 slot per shared expert to each token's
 * routing (in the workspace; routed ids outside [0, E) stay dropped) and runs
 * the prefill (or decode) sequence over E + S experts and k + S slots; the
 * shared slots come after the routed ones in the fixed summation order.
 * ws_bytes: moe_workspace_size_shared.  Errors as moe_experts_prefill, plus
 * MOE_ERR_NULL / MOE_ERR_ALIGN for the shared weights and MOE_ERR_SHAPE for
 * S out of range.
 */
int moe_experts_prefill_shared(const uint16_t* hidden, const uint16_t* gate_up,
                               const uint16_t* down, const uint16_t* shared_gate_up,
                               const uint16_t* shared_down, const int32_t* top_k_index,
                               const float* top_k_weights, const uint16_t* residual, int64_t T,
                               int H, int F, int E, int k, int S, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Decode form of moe_experts_prefill_shared (the gather-GEMV kernels when
 * T*(k+S) <= 32 and the moe_experts_decode size limits hold, else the
 * grouped path).  Same operands, workspace rule and errors. */
int moe_experts_decode_shared(const uint16_t* hidden, const uint16_t* gate_up,
                              const uint16_t* down, const uint16_t* shared_gate_up,
                              const uint16_t* shared_down, const int32_t* top_k_index,
                              const float* top_k_weights, const uint16_t* residual, int64_t T,
                              int H, int F, int E, int k, int S, uint16_t* out, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for the shared-expert entry points: variant
 * MOE_VARIANT_PREFILL (moe_experts_prefill_shared), MOE_VARIANT_DECODE
 * (moe_experts_decode_shared), MOE_VARIANT_FP8 (moe_experts_fp8_shared) or
 * MOE_VARIANT_MXFP4 (moe_experts_mxfp4_shared); MOE_ERR_SHAPE otherwise or
 * when the shapes are out of range. */
int moe_workspace_size_shared(int variant, int64_t T, int H, int F, int E, int k, int S,
                              size_t* bytes);

/*
 * FP8 block-scaled routed experts (mirage issue "Supporting MegaKernel for
 * DeepSeek Models": moe_w13_fp8_layer, moe_silu_mul_layer, moe_w2_fp8_layer,
 * moe_local_reduction).
 *   x        [T,H]        fp8   x_scale        [T,H/128]      fp32
 *   gate_up  [E,2F,H]     fp8   gate_up_scale  [E,2F,H/128]   fp32
 *   down     [E,H,F]      fp8   down_scale     [E,H,F/128]    fp32
 *   top_k_index [T,k] int32, top_k_weights [T,k] fp32, out [T,H] bf16.
 * The three scale tensors must be 16-byte aligned (the kernels read the
 * scales of four K blocks per load); other pointers as above.
 * value(code, block) = e4m3(code) * scale[row][col/128].  Products accumulate
 * in fp32, one 128-wide K block at a time, then scale by x_scale*w_scale.
 * The SwiGLU output is re-quantised per (slot row, 128 block) before the down
 * product: s = amax/448, code = RNE(clamp(h*(448/amax), +-448)); an all-zero
 * block gets s = 1 and zero codes.
 */
int moe_experts_fp8(const uint8_t* x, const float* x_scale,
                    const uint8_t* gate_up, const float* gate_up_scale,
                    const uint8_t* down, const float* down_scale,
                    const int32_t* top_k_index, const float* top_k_weights,
                    const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                    uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_experts_fp8 with the two grouped products and the combine in one
 * persistent launch after the routing plan, as moe_experts_prefill_fused
 * does for bf16 (same operands, workspace moe_workspace_size(MOE_VARIANT_FP8,
 * ...), errors and results: out is bit-for-bit that of moe_experts_fp8; the
 * same residency requirement, 2 s wait limit and generation word).  Used
 * for prefill shapes (more than 32 slots per expert on average) with H and F
 * multiples of 512; other calls run the moe_experts_fp8 sequence.
 */
int moe_experts_fp8_fused(const uint8_t* x, const float* x_scale,
                          const uint8_t* gate_up, const float* gate_up_scale,
                          const uint8_t* down, const float* down_scale,
                          const int32_t* top_k_index, const float* top_k_weights,
                          const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                          uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The FP8 layer with S fused shared experts (DeepGEMM issue "GC MoE":
 * routed experts with optional fused shared experts, FP8 shared weights;
 * mirage issue "Supporting MegaKernel for DeepSeek Models": the shared
 * expert is an FP8 block-scaled product of the same kind).  The shared
 * experts are stored like the routed ones: shared_gate_up [S,2F,H] E4M3 with
 * fp32 scales [S,2F,H/128], shared_down [S,H,F] E4M3 with fp32 scales
 * [S,H,F/128] (device; codes 16-byte aligned, scales 16-byte aligned), the
 * same F as the routed experts.  Every token passes through each with
 * weight 1, after its routed slots in the fixed summation order:
 *   out[t] = sum_j w[t,j] * E_idx[t,j](x[t]) + sum_s S_s(x[t]) (+ residual[t]).
 * The call appends the weight-1 slots to each token's routing in the
 * workspace and runs the moe_experts_fp8 sequence over E + S experts and
 * k + S slots.  1 <= S, E + S <= MOE_MAX_EXPERTS.  ws_bytes:
 * moe_workspace_size_shared(MOE_VARIANT_FP8, ...).  Errors as
 * moe_experts_fp8.
 */
int moe_experts_fp8_shared(const uint8_t* x, const float* x_scale, const uint8_t* gate_up,
                           const float* gate_up_scale, const uint8_t* down,
                           const float* down_scale, const uint8_t* shared_gate_up,
                           const float* shared_gate_up_scale, const uint8_t* shared_down,
                           const float* shared_down_scale, const int32_t* top_k_index,
                           const float* top_k_weights, const uint16_t* residual, int64_t T, int H,
                           int F, int E, int k, int S, uint16_t* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * The same FP8 layer fed with bf16 hidden states [T,H] (mirage issue
 * "Supporting MegaKernel for DeepSeek Models": bf16_to_fp8_quantize before
 * moe_w13_fp8_layer).  Each row is quantised per 128-wide block into the
 * workspace by the rule of moe_quantize_fp8_block128 (fp32 scale amax/448,
 * RNE codes; all-zero block: scale 1, codes 0), then moe_experts_fp8 runs on
 * those codes and scales.  Workspace: moe_workspace_size(MOE_VARIANT_FP8_BF16IN,
 * ...).  Other operands, results and errors as moe_experts_fp8.
 */
int moe_experts_fp8_bf16in(const uint16_t* hidden,
                           const uint8_t* gate_up, const float* gate_up_scale,
                           const uint8_t* down, const float* down_scale,
                           const int32_t* top_k_index, const float* top_k_weights,
                           const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                           uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Routed experts with MXFP4 weights and MXFP8 activations (DeepGEMM issue
 * "GC MoE": FP8 activations with packed FP4 routed weights; its FP8 x FP4
 * grouped GEMM kinds; mirage issue "Supporting MegaKernel for DeepSeek
 * Models": ue8m0 scales per 32 elements), read as the OCP Microscaling
 * formats.
 *   x        [T,H]      E4M3 codes         x_scale        [T,H/32]    E8M0
 *   gate_up  [E,2F,H/2] E2M1 pairs         gate_up_scale  [E,2F,H/32] E8M0
 *   down     [E,H,F/2]  E2M1 pairs         down_scale     [E,H,F/32]  E8M0
 *   top_k_index [T,k] int32, top_k_weights [T,k] fp32, residual/out [T,H] bf16.
 * E2M1 element 2i of a row is the low nibble of byte i; an E8M0 byte s scales
 * its 32 elements by 2^(s-127) (s = 255 is NaN).  Products accumulate in
 * fp32 with both scales applied by the matrix cores.  The SwiGLU output is
 * re-quantised to MXFP8 per (slot row, 32 block): shared exponent
 * e = floor(log2(amax)) - 8 clamped to [-127, 127], code =
 * RNE_e4m3(clamp(h / 2^e, +-448)), scale byte e + 127; an all-zero block
 * gets byte 0 and zero codes.  x, gate_up, down, residual and out 16-byte
 * aligned, the scale tensors 4-byte aligned.  Workspace:
 * moe_workspace_size(MOE_VARIANT_MXFP4, ...).  Errors as moe_experts_fp8.
 */
int moe_experts_mxfp4(const uint8_t* x, const uint8_t* x_scale,
                      const uint8_t* gate_up, const uint8_t* gate_up_scale,
                      const uint8_t* down, const uint8_t* down_scale,
                      const int32_t* top_k_index, const float* top_k_weights,
                      const uint16_t* residual, int64_t T, int H, int F, int E, int k,
                      uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_experts_mxfp4 in one persistent launch (the FP8 x FP4 single-kernel
 * layer): the routing plan, the two grouped MX products and the combine, as
 * moe_experts_prefill_fused does for bf16 (same operands, workspace
 * moe_workspace_size(MOE_VARIANT_MXFP4, ...), errors and results: out is
 * bit-for-bit that of moe_experts_mxfp4; the same residency requirement,
 * 2 s wait limit and generation word).  Used for prefill shapes (more than
 * 64 slots per expert on average, F a multiple of 256, H of 512); other
 * calls run the moe_experts_mxfp4 sequence.
 */
int moe_experts_mxfp4_fused(const uint8_t* x, const uint8_t* x_scale, const uint8_t* gate_up,
                            const uint8_t* gate_up_scale, const uint8_t* down,
                            const uint8_t* down_scale, const int32_t* top_k_index,
                            const float* top_k_weights, const uint16_t* residual, int64_t T, int H,
                            int F, int E, int k, uint16_t* out, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * The MXFP4 layer with S fused shared experts, stored like the routed ones:
 * shared_gate_up [S,2F,H/2] and shared_down [S,H,F/2] E2M1 pairs with E8M0
 * scales [S,2F,H/32] and [S,H,F/32] (codes 16-byte aligned, scales 4-byte
 * aligned), the same F; weight 1 for every token, summed after the routed
 * slots, as moe_experts_fp8_shared.  (The pages' GC MoE pairs FP4 routed
 * weights with FP8 shared weights; here the shared experts take the routed
 * experts' format, so that one grouped product serves both.)  ws_bytes:
 * moe_workspace_size_shared(MOE_VARIANT_MXFP4, ...).  Errors as
 * moe_experts_mxfp4.
 */
int moe_experts_mxfp4_shared(const uint8_t* x, const uint8_t* x_scale, const uint8_t* gate_up,
                             const uint8_t* gate_up_scale, const uint8_t* down,
                             const uint8_t* down_scale, const uint8_t* shared_gate_up,
                             const uint8_t* shared_gate_up_scale, const uint8_t* shared_down,
                             const uint8_t* shared_down_scale, const int32_t* top_k_index,
                             const float* top_k_weights, const uint16_t* residual, int64_t T,
                             int H, int F, int E, int k, int S, uint16_t* out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * Routers: router logits -> top_k_index [T,k] int32 and top_k_weights [T,k]
 * fp32 (device), the operands every layer entry point takes.
 *   MOE_ROUTE_SOFTMAX (model card "DeepSeek-OCR-2 MoE experts", description:
 *     fp32 softmax, greedy top-k scaled by routed_scaling_factor): the k
 *     largest logits (softmax is increasing, so the choice is made on the
 *     logits themselves), weight = softmax probability * routed_scaling_factor,
 *     not renormalised.  bias must be NULL; the group arguments are ignored.
 *   MOE_ROUTE_SIGMOID_GROUP (mirage issue "Supporting MegaKernel for DeepSeek
 *     Models", moe_topk_sigmoid_routing_layer: logits + bias, num_groups,
 *     topk_group, routed_scaling_factor): s = sigmoid(logit), choice score
 *     c = s + bias[e] (fp64); the E experts form num_groups consecutive
 *     groups, ranked by the sum of their group_top (1 or 2) largest c; the
 *     topk_group best groups are kept and the k largest c among their experts
 *     chosen; weights = chosen s / sum of chosen s * routed_scaling_factor.
 *     DeepSeek-V3 uses group_top = 2.
 * Ties go to the lower expert (group) id; chosen ids are written largest
 * score first; a NaN score ranks below every number.
 * logits [T,E] and bias [E] are fp32 (logits_bf16 = 0) or bf16 (1).
 * Ranges: 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, 32); sigmoid-group:
 * E % num_groups == 0, 1 <= topk_group <= num_groups <= 64, group_top 1 or 2
 * (2 needs groups of at least 2), k <= topk_group * E / num_groups.
 * Pointers 4-byte aligned (logits/bias 2-byte for bf16).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_DEVICE,
 * MOE_ERR_LAUNCH.
 */
#define MOE_ROUTE_SOFTMAX 0
#define MOE_ROUTE_SIGMOID_GROUP 1
int moe_route_topk(const void* logits, const void* bias, int logits_bf16, int mode, int64_t T,
                   int E, int k, int num_groups, int topk_group, int group_top,
                   float routed_scaling_factor, int32_t* top_k_index, float* top_k_weights,
                   hipStream_t stream);

/*
 * Router and routing plan together: the routing of moe_route_topk, then the
 * plan of moe_routing_plan over the ids it chose (counts[E], offsets[E+1] —
 * the MegaKernel layer's "masks" — perm[T*k], inv[T*k]).  Batches of up to
 * MOE_ROUTE_PLAN_FUSED_MAX_T tokens take one launch of one workgroup that
 * routes and then plans; larger ones take the router launch and the plan
 * launch.  Workspace: moe_workspace_size(MOE_VARIANT_PLAN, T, 0, 0, E, k).
 * Arguments and errors as moe_route_topk and moe_routing_plan.
 */
#define MOE_ROUTE_PLAN_FUSED_MAX_T 64
int moe_route_plan(const void* logits, const void* bias, int logits_bf16, int mode, int64_t T,
                   int E, int k, int num_groups, int topk_group, int group_top,
                   float routed_scaling_factor, int32_t* top_k_index, float* top_k_weights,
                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * bf16 decode from router logits: the router of moe_route_topk fused into
 * moe_experts_decode.  On the gather-GEMV form (the limits of
 * moe_experts_decode) every workgroup of the slice kernel routes the T <= 4
 * tokens itself, so the call is the same two launches as moe_experts_decode;
 * larger calls take a router launch first.  The chosen ids and weights are
 * written to top_k_index [T,k] / top_k_weights [T,k] (device, caller-owned),
 * bit-identical to moe_route_topk's.  Router arguments as moe_route_topk,
 * layer arguments and workspace (MOE_VARIANT_DECODE) as moe_experts_decode;
 * the output equals moe_experts_decode on those ids and weights.
 */
int moe_experts_decode_routed(const uint16_t* hidden, const void* logits, const void* bias,
                              int logits_bf16, int mode, int num_groups, int topk_group,
                              int group_top, float routed_scaling_factor, const uint16_t* gate_up,
                              const uint16_t* down, const uint16_t* residual, int64_t T, int H,
                              int F, int E, int k, uint16_t* out, int32_t* top_k_index,
                              float* top_k_weights, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Block-128 fp8 quantisation of `rows` rows of K values (mirage issue
 * "Supporting MegaKernel for DeepSeek Models", bf16_to_fp8_quantize, with the
 * fp32 scale that moe_w2_fp8_layer's input_scale carries).  `in` is fp32
 * (in_is_bf16 = 0) or bf16 (in_is_bf16 = 1) [rows,K]; codes [rows,K] fp8;
 * scales [rows,K/128] fp32.  Per block: s = amax/448,
 * code = RNE_e4m3(clamp(v*(448/amax), +-448)), all in fp32; an all-zero block
 * gets s = 1 and zero codes.  This is the same device routine the fp8 layer
 * uses on h, so it makes the layer's input operands from bf16 activations.
 * K must be a multiple of 128.
 */
int moe_quantize_fp8_block128(const void* in, int in_is_bf16, int64_t rows, int K,
                              uint8_t* codes, float* scales, hipStream_t stream);

/*
 * The same block-128 fp8 quantisation with power-of-two scales (mirage issue
 * "Supporting MegaKernel for DeepSeek Models", bf16_to_fp8_quantize: "FP8
 * E4M3 + scale ue8m0", block size 128).  The page states no rule; this one:
 * per block, e is the smallest integer with amax <= 448 * 2^e, clamped to
 * [-127, 127]; codes = RNE_e4m3(clamp(v * 2^-e, +-448)) (the multiplication
 * by 2^-e is exact, so the e4m3 rounding is the only one); the scale byte is
 * e + 127, value 2^e.  An all-zero block gets byte 127 and zero codes.
 * `in` fp32 or bf16 [rows,K] (4-byte aligned); codes [rows,K]; scales
 * [rows,K/128] bytes.  K must be a multiple of 128.  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_DEVICE, MOE_ERR_LAUNCH.
 */
int moe_quantize_fp8_block128_ue8m0(const void* in, int in_is_bf16, int64_t rows, int K,
                                    uint8_t* codes, uint8_t* scales, hipStream_t stream);

/*
 * Stage timing, for measurement (not needed for normal use).
 * moe_profile_begin(max_calls) switches the recorder on: each of the next
 * max_calls calls (moe_experts_prefill / _decode / _fp8 / _mxfp4 and the
 * routers, from any host thread) launches every kernel with a start/stop HIP event pair attached to
 * that kernel's own dispatch (hipExtLaunchKernelGGL), on the stream it runs
 * on, so each pair times exactly one kernel's execution.  Creating the
 * events is the only allocation and happens here.
 * moe_profile_end(max_calls, &n, ms, ids) waits for those events, switches the
 * recorder off and writes, for the first n <= max_calls recorded calls,
 * ms[c * MOE_PROFILE_MAX_STAGES + i] = milliseconds of the call's i-th kernel
 * and ids[...] = its MOE_STAGE_* (-1 and -1.0 past the call's last kernel).
 * ms and ids hold max_calls * MOE_PROFILE_MAX_STAGES entries (host memory).
 * Calls made while begin/end run on another thread race with them.
 * Errors: MOE_ERR_SHAPE (max_calls outside [1, MOE_PROFILE_MAX_CALLS]),
 * MOE_ERR_NULL, MOE_ERR_LAUNCH (event creation or query failed),
 * MOE_ERR_DEVICE.
 */
/*
 * Measurement helper (not part of the layer): one launch of a plain
 * streaming read of `bytes` bytes at `src` by `grid` workgroups of 512
 * threads (16-byte non-temporal loads, eight in flight per thread), the HBM
 * ceiling the layer's weight streams are compared with.  Nothing is written
 * except, never in practice, to `sink` (4 KB).  src and sink are device
 * pointers, 16-byte aligned; bytes a positive multiple of 16; 1 <= grid <=
 * 65535.  Timed by the stage recorder as MOE_STAGE_PROBE.
 * Errors: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_SHAPE, MOE_ERR_DEVICE,
 * MOE_ERR_LAUNCH.
 */
int moe_probe_stream_read(const void* src, size_t bytes, int grid, void* sink,
                          hipStream_t stream);

/*
 * Test hook: caps the persistent grids of the grouped products (and the
 * persistent decode kernel) at max_workgroups (rounded down to a multiple of
 * 8, at least 8), so that every workgroup runs many work items; 0 removes
 * the cap (the default: one resident grid per kernel).  Results do not
 * depend on the grid.  Process-wide; takes effect at the next launch.
 * Errors: MOE_ERR_SHAPE for a negative value.
 */
int moe_set_grid_cap(int max_workgroups);

#define MOE_PROFILE_MAX_STAGES 5
#define MOE_PROFILE_MAX_CALLS 4096
enum moe_stage {
    MOE_STAGE_PLAN = 0,          /* routing plan (grouped paths)             */
    MOE_STAGE_GATE_UP = 1,       /* grouped gate_up product + SwiGLU         */
    MOE_STAGE_DOWN = 2,          /* grouped down product                     */
    MOE_STAGE_COMBINE = 3,       /* router-weighted combine                  */
    MOE_STAGE_DECODE = 4,        /* decode form: the whole layer, one launch  */
    MOE_STAGE_QUANTIZE = 5,      /* input-side block-128 fp8 quantisation    */
    MOE_STAGE_SHARED_ROUTE = 6,  /* routing with the shared experts appended */
    MOE_STAGE_ROUTER = 7,        /* router (logits -> ids, weights)          */
    MOE_STAGE_ROUTE_PLAN = 8,    /* router and plan in one launch            */
    MOE_STAGE_PROBE = 9,         /* moe_probe_stream_read                    */
    MOE_STAGE_LAYER = 10,        /* gate_up, down and combine in one launch  */
};
int moe_profile_begin(int max_calls);
int moe_profile_end(int max_calls, int* n_calls, float* ms, int* stage_ids);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERTS_H */

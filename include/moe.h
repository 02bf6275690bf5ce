/*
 * moe.h - C ABI of the MI355X (gfx950) fused top-k Mixture-of-Experts layer.
 *
 * The layer, as the pages describe it: a router yields a weight
 * distribution over E experts, each token keeps its top-k experts, the
 * tokens are sorted by expert so every expert's rows are contiguous, one
 * grouped kernel multiplies each slice by its own expert's weights, and
 * the expert outputs are summed back in token order with the routing
 * weights (FusedMoE vs MegaMoE post, sections 2 and 3.1).  Each expert
 * product is A[M,K] x B[K,N] over the expert's routed token rows (MoE
 * kernel engineering post, Eq. 1); weights are stored as the K-contiguous
 * transpose B^T[N,K] that the Swap-AB formulation puts in the leading
 * operand (same post, Eq. 2).
 *
 * Conventions for every call:
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device and be 16-byte aligned.  The library never
 *    allocates, frees or keeps a pointer after a call returns, except the
 *    expert cache (moe_cache_*), which keeps the host and slot pointers it is
 *    created with and allocates host bookkeeping and HIP events.
 *  - Calls return without waiting for the device, except fused_moe_cached,
 *    which waits for its own routing (the miss path needs the ids).
 *  - Every call enqueues work on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream).  Device faults surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated on the host before any HIP call; a rejected
 *    call enqueues nothing.  M = 0 is a valid no-op.
 *  - Matrices are row-major.  Outputs are overwritten, never accumulated.
 *  - No C++ exception crosses this boundary.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                         */
    MOE_ERR_SHAPE = 2,       /* M<0, E<1, topk<1, topk>E, H or I not a multiple of 128, ... */
    MOE_ERR_UNSUPPORTED = 3, /* E>256, topk>16, dtype/kind combination, block_m      */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than fused_moe_workspace_size()   */
    MOE_ERR_ALIGNMENT = 5,   /* a pointer is not 16-byte aligned                    */
    MOE_ERR_HIP = 6,         /* a HIP launch failed                                 */
    MOE_ERR_SCRATCH = 7      /* fused_moe_noalloc: sizes need more than its scratch */
} moe_status;

typedef enum {
    MOE_F32 = 0,     /* IEEE binary32                                          */
    MOE_BF16 = 1,    /* bfloat16                                               */
    MOE_FP8_E4M3 = 2, /* OCP OFP8 E4M3 (bias 7, max 448, no inf) + float32 scale */
    MOE_W4A16 = 3     /* weights: 4-bit codes with a float32 scale per 128 k of a row;
                         activations and outputs bfloat16 (see moe_grouped_gemm) */
} moe_dtype;

typedef enum {
    MOE_GEMM_GATE_UP_SILU = 0, /* act[p] = silu(W1[e][0:I] x) * (W1[e][I:2I] x) */
    MOE_GEMM_DOWN = 1,         /* y[p]   = W2[e] act[p]                         */
    MOE_GEMM_DOWN_E4M3_ACT = 2 /* as DOWN, act given as e4m3 codes (moe_quant_act) */
} moe_gemm_kind;

/* The index system produced by moe_align (all device pointers, int32):
 *  sorted_ids[cap]        pair ids p = t*topk + j grouped by expert, stable in p;
 *                         every expert's run is padded to a multiple of block_m
 *                         with the sentinel P = M*topk, and rows past the padded
 *                         total hold P as well
 *  tile_expert[cap/block_m]  expert of each block_m-row tile, -1 past the total
 *  expert_counts[E]       pairs routed to each expert
 *  expert_offsets[E+1]    exclusive prefix sum of the padded counts; the last
 *                         entry is the padded total
 *  active_experts[min(E,P)]  experts with a non-zero count, ascending, then -1
 *  num_active[1]          number of experts with a non-zero count
 * where cap = moe_align_capacity(M, topk, E, block_m). */
typedef struct {
    int32_t* sorted_ids;
    int32_t* tile_expert;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* active_experts;
    int32_t* num_active;
} moe_align_bufs;

/* Router scores (FusedMoE vs MegaMoE post, section 2: the router yields a
 * score per expert for every token, from which the weight distribution and
 * the top-k are taken):
 *  logits[t][e] = sum_h x[t][h] * router_w[e][h], float32 accumulation.
 *  x         device [M][H] in x_dtype: MOE_F32, MOE_BF16, or MOE_FP8_E4M3 with
 *            x_scale -> its float32 per-tensor scale (x_scale must be NULL
 *            otherwise)
 *  router_w  device float32 [E][H] (K-contiguous, like the expert weights)
 *  logits    device float32 [M][E]
 * Every score is computed the same way (lane l of a wavefront sums, in
 * ascending h, the products at h = 256 i + 4 l + j, j = 0..3, and the 64
 * partials are combined by a butterfly), so the result does not depend on
 * the batch or on which entry point computes it.  H must be a multiple of 4.  Errors: NULL ->
 * MOE_ERR_NULL; M<0, H<1, E<1 -> MOE_ERR_SHAPE; bad dtype -> MOE_ERR_UNSUPPORTED. */
moe_status moe_router_logits(moe_dtype x_dtype, const void* x, const float* x_scale, const float* router_w,
                             int32_t M, int32_t H, int32_t E, float* logits, void* stream);

/* Top-k routing (FusedMoE vs MegaMoE post, section 2; section 3.1 step 1).
 *  logits        device, float32 [M][E], finite (non-finite values give
 *                unspecified ids, but every id written is in [0, E))
 *  topk_ids      device, int32 [M][topk]: slot j holds the j-th largest logit,
 *                ties broken by the lower expert index (+0 and -0 are equal)
 *  topk_weights  device, float32 [M][topk]: exp(l_j - l_max) divided by the
 *                sum over the selected experts (renormalize != 0) or over all
 *                E experts (renormalize == 0)
 * Errors: NULL -> MOE_ERR_NULL; M<0, E<1, topk<1, topk>E -> MOE_ERR_SHAPE;
 * E>256 or topk>16 -> MOE_ERR_UNSUPPORTED. */
moe_status moe_route(const float* logits, int32_t M, int32_t E, int32_t topk, int32_t renormalize,
                     int32_t* topk_ids, float* topk_weights, void* stream);

/* Rows of sorted_ids needed by moe_align: the smallest multiple of block_m
 * that is >= P + min(E, P) * (block_m - 1), P = M*topk.  Pure host function;
 * returns -1 for invalid arguments. */
int64_t moe_align_capacity(int32_t M, int32_t topk, int32_t E, int32_t block_m);

/* Token-to-expert alignment (FusedMoE vs MegaMoE post, section 3.1 steps 1-2):
 * per-expert counts, padded exclusive prefix sum, stable sort of the pairs
 * by expert, tile->expert map and the compacted active-expert list.  Output
 * is fully determined by topk_ids (no dependence on scheduling).
 *  topk_ids  device, int32 [M][topk], each in [0, E) (ids outside are skipped)
 *  out       device buffers sized as described at moe_align_bufs
 * block_m must be one of 1, 16, 32, 64, 128, 256 (else MOE_ERR_UNSUPPORTED). */
moe_status moe_align(const int32_t* topk_ids, int32_t M, int32_t topk, int32_t E, int32_t block_m,
                     moe_align_bufs out, void* stream);

/* Grouped expert GEMM over routed rows (section 3.1 step 3; Eq. 1 per
 * expert, with the weights in the leading operand at decode per Eq. 2).
 *  kind = MOE_GEMM_GATE_UP_SILU: a = x [M][K=H], w = W1 [E][N=2I][K] (gate rows
 *         0..I-1, up rows I..2I-1), c = act [P][I] in pair order.
 *  kind = MOE_GEMM_DOWN: a = act [P][K=I], w = W2 [E][N=H][K], c = y [P][N] in
 *         pair order.
 *  dtype: MOE_F32 (a, w, c float32), MOE_BF16 (a, w, c bfloat16),
 *         MOE_FP8_E4M3 (w e4m3 with w_scale[E] float32 per expert matrix;
 *         GATE_UP: a = x e4m3 with a_scale -> its float32 scale, c = act
 *         float32 (the intermediate stays in float32 until it is quantised),
 *         c_amax -> float32 that receives max|act| (zeroed by the call
 *         itself); DOWN: a = act float32, a_scale -> that amax, the act rows
 *         are quantised on load with one per-tensor scale s = amax/448: code
 *         = e4m3(act / s), IEEE float32 quotient, round to nearest even,
 *         saturating at +-448; c = y bfloat16).
 *         MOE_W4A16 (weight-only int4; FusedMoE vs MegaMoE post, sections
 *         6.2-6.3): a and c bfloat16 as for MOE_BF16; w = uint8 [E][N][K/2]
 *         codes, w_scale -> float32 [E][K/128][N] scales (group-major), and
 *         W[e][n][k] = (u - 8) * w_scale[e][k/128][n] for the 4-bit code u of
 *         (n, k): the codes of 8 consecutive k (k0 a multiple of 8) fill one
 *         little-endian 32-bit word, k0+2i at bits 4i..4i+3 and k0+2i+1 at
 *         bits 16+4i..16+4i+3; K must be a multiple of 256.  Served by the
 *         decode kernel at every batch size (a batch with many rows per
 *         expert streams the weights once per 32 of them).
 *  kind = MOE_GEMM_DOWN_E4M3_ACT (MOE_FP8_E4M3 only): as MOE_GEMM_DOWN, but a
 *         holds the e4m3 codes [P][K] that moe_quant_act wrote for the same
 *         amax, and a_scale -> that amax.  Same codes, same scales, same
 *         products as MOE_GEMM_DOWN; the rows are read at one byte per value
 *         (what the tile kernels want when many rows share an expert).
 *  a_scale, w_scale, c_amax must be NULL unless dtype is MOE_FP8_E4M3.
 *  al, block_m: the output of moe_align for the same topk_ids and block_m.
 *  Rows of a expert's run are read through al->sorted_ids; only the first
 *  expert_counts[e] rows of each run are written to c.
 * Errors as for the other calls; K and N must be multiples of 128 (K of 256
 * for MOE_FP8_E4M3). */
moe_status moe_grouped_gemm(moe_gemm_kind kind, moe_dtype dtype, const void* a, const float* a_scale,
                            const void* w, const float* w_scale, const moe_align_bufs* al, int32_t M,
                            int32_t topk, int32_t E, int32_t N, int32_t K, int32_t block_m, void* c,
                            float* c_amax, void* stream);

/* Per-tensor e4m3 quantisation of the float32 intermediate, the scaling the
 * fp8 down projection needs (MoE kernel engineering post, FP8 backend-routing
 * section: one scale per tensor): s = amax / 448 in float32, code = e4m3 of
 * act / s with an IEEE float32 quotient, round to nearest even, saturating
 * at +-448 (the codes the e4m3 DOWN call forms on load).
 *  act    device float32 [n]
 *  amax   device float32 [1], > 0 (as written by the fp8 GATE_UP GEMM)
 *  act_q  device uint8 [n], e4m3 codes
 * n must be a multiple of 16 (MOE_ERR_SHAPE otherwise); n = 0 is a no-op. */
moe_status moe_quant_act(const void* act, const float* amax, int64_t n, void* act_q, void* stream);

/* Weighted combine back into token order (section 3.1 step 4):
 *  out[t][h] = sum_{j=0..topk-1} topk_weights[t][j] * y[t*topk+j][h], j
 *  ascending, float32 accumulation.
 *  y_dtype: MOE_F32 or MOE_BF16; out_dtype: MOE_F32 or MOE_BF16.
 *  y device [M*topk][H]; topk_weights device [M][topk]; out device [M][H]. */
moe_status moe_combine(moe_dtype y_dtype, const void* y, const float* topk_weights, int32_t M,
                       int32_t topk, int32_t H, moe_dtype out_dtype, void* out, void* stream);

/* Bytes of device workspace fused_moe needs for these sizes (0 for M=0). */
size_t fused_moe_workspace_size(moe_dtype dtype, int32_t M, int32_t E, int32_t topk, int32_t H,
                                int32_t I);

/* The whole layer: route -> align -> GATE_UP GEMM -> DOWN GEMM -> combine, all
 * on `stream`, no host synchronisation.  For one token of a bf16, e4m3 or
 * W4A16 layer on the decode kernels the two GEMM launches route the token
 * themselves (the same top-k and weights, bit for bit) and no route / align
 * launch runs; topk_ids_out / topk_weights_out are then written by the
 * GATE_UP launch (e4m3: the intermediate's amax goes from the GATE_UP launch
 * to the DOWN launch as partial maxima in the workspace, the same value).
 *  x              device [M][H]: float32, bfloat16 (also for MOE_W4A16) or e4m3
 *                 (x_scale -> float32)
 *  router_logits  device float32 [M][E]
 *  w1, w2         device [E][2I][H] and [E][H][I] in dtype (fp8: w1_scale,
 *                 w2_scale device float32 [E]; MOE_W4A16: packed codes
 *                 [E][2I][H/2] and [E][H][I/2], w1_scale [E][H/128][2I],
 *                 w2_scale [E][I/128][H], as for moe_grouped_gemm)
 *  out            device [M][H]: float32 for MOE_F32, bfloat16 otherwise
 *  topk_ids_out, topk_weights_out  optional device [M][topk] copies of the
 *                 routing result (NULL to skip)
 *  H and I must be multiples of 128 (of 256 for MOE_FP8_E4M3 and MOE_W4A16).
 *  workspace      device, >= fused_moe_workspace_size(...) bytes, 256-byte
 *                 aligned; its contents on entry do not matter.
 * Kernel choice (not results beyond rounding order; read at each call):
 *  MOE_GEMM_PATH=decode|prefill forces the decode kernels or the tile
 *  kernels (64-row tiles); MOE_DOWN_COMBINE=1 lets a bf16 decode batch of
 *  about one token tile per expert run the down GEMM with the combine inside
 *  (the same bits as the separate combine, not faster on MI355X). */
moe_status fused_moe(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                     const void* w1, const float* w1_scale, const void* w2, const float* w2_scale,
                     int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I, int32_t renormalize,
                     void* out, int32_t* topk_ids_out, float* topk_weights_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* fused_moe from the hidden states: the router scores are computed on the
 * GPU first (router_w device float32 [E][H]; router_logits is then an OUTPUT,
 * device float32 [M][E], that receives them), and the layer routes on those
 * scores (the MoE kernel engineering post's introduction: routing, data
 * shuffling and expert compute as one batched GPU operation).  For a few
 * tokens and a small router (up to 16 tokens, 64 K router weights and 128 K
 * multiply-adds) scoring, top-k and alignment are one launch; otherwise
 * moe_router_logits runs first, and for one token whose GEMMs route it
 * themselves (as in fused_moe) it is the only launch before them.  The
 * scores are the same bits either way.
 * Workspace, arguments and errors as for fused_moe (fused_moe_workspace_size
 * gives the workspace). */
moe_status fused_moe_router(moe_dtype dtype, const void* x, const float* x_scale, const float* router_w,
                            float* router_logits, const void* w1, const float* w1_scale, const void* w2,
                            const float* w2_scale, int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I,
                            int32_t renormalize, void* out, int32_t* topk_ids_out, float* topk_weights_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind fused_moe_noalloc (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* fused_moe without a workspace argument, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as fused_moe, except that the workspace is a
 * file-scope device array of MOE_NOALLOC_SCRATCH_BYTES inside the library:
 *  - each GPU the library runs on holds its own copy until the process
 *    ends; its address is looked up (hipGetSymbolAddress) on the first call
 *    on each device and kept, so that call is not capturable;
 *  - sizes whose workspace (fused_moe_workspace_size) exceeds
 *    MOE_NOALLOC_SCRATCH_BYTES are rejected with MOE_ERR_SCRATCH before any
 *    HIP call (64 MiB covers the decode batches up to 64 tokens of every
 *    layer shape here);
 *  - the call allocates nothing and frees nothing;
 *  - every call on one GPU uses the same scratch, whose contents on entry do
 *    not matter: calls that overlap in time on one GPU (different streams,
 *    or different host threads without ordering) race and give undefined
 *    results. */
moe_status fused_moe_noalloc(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                             const void* w1, const float* w1_scale, const void* w2, const float* w2_scale,
                             int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I, int32_t renormalize,
                             void* out, int32_t* topk_ids_out, float* topk_weights_out, void* stream);

/* MOE_NOALLOC_SCRATCH_BYTES, as a call (for bindings that cannot read macros). */
size_t fused_moe_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------- expert streaming
 * The MoE inference post's second design (FusedMoE vs MegaMoE, sections
 * 4.1-4.3): all experts' weights stay in host memory, a GPU pool of
 * `capacity` slots holds the experts in use, missing experts are copied in
 * (least recently used slot first) on a copy stream that can run ahead of the
 * compute, and the layer itself is fused_moe over the slots.
 *
 * The weights of a set of experts, laid out as for fused_moe: experts one
 * after another, each expert's w1, w2 (and scales) contiguous. */
typedef struct {
    const void* w1;        /* [n][2I][H] (MOE_W4A16: packed codes [n][2I][H/2]) */
    const void* w2;        /* [n][H][I]  (MOE_W4A16: [n][H][I/2])               */
    const float* w1_scale; /* fp8: [n]; MOE_W4A16: [n][H/128][2I]; else NULL    */
    const float* w2_scale; /* fp8: [n]; MOE_W4A16: [n][I/128][H];  else NULL    */
} moe_expert_weights;

/* Opaque cache state (host bookkeeping and HIP events). */
typedef struct moe_expert_cache moe_expert_cache;

/* Creates a cache over the E experts of `host` (pinned host memory, e.g.
 * hipHostMalloc, with n = E; it must outlive the cache) and the device slot
 * pool `slots` (n = capacity, 16-byte aligned; the caller owns it and keeps it
 * for the cache's life).  copy_stream: the hipStream_t (as void*) the copies
 * run on; a stream of its own lets them overlap the compute.  The cache starts
 * empty.  Errors: NULL pointers -> MOE_ERR_NULL; capacity outside [1, E], H
 * or I not multiples of 128 (256 for fp8 and W4A16) -> MOE_ERR_SHAPE; E > 256,
 * unknown dtype, scales given for an unscaled dtype -> MOE_ERR_UNSUPPORTED;
 * misaligned slots -> MOE_ERR_ALIGNMENT; event creation -> MOE_ERR_HIP.
 * The cache allocates host memory for its bookkeeping and HIP events; none of
 * its calls is thread-safe. */
moe_status moe_cache_create(moe_dtype dtype, int32_t E, int32_t H, int32_t I, int32_t capacity,
                            moe_expert_weights host, moe_expert_weights slots, void* copy_stream,
                            moe_expert_cache** out);

/* Waits for the copies in flight and frees the cache (not the buffers). */
moe_status moe_cache_destroy(moe_expert_cache* cache);

/* Asynchronously copies the listed experts (host ids in [0, E), repeats
 * allowed) that are not resident into free or least recently used slots, on
 * the copy stream (the page's predicted-expert prefetch; the prediction is
 * the caller's).  A slot is overwritten only after the last layer call that
 * read it; later layer calls wait for these copies only if they read the
 * slots.  More distinct experts than slots -> MOE_ERR_UNSUPPORTED; an id out
 * of range -> MOE_ERR_SHAPE. */
moe_status moe_cache_prefetch(moe_expert_cache* cache, const int32_t* experts, int32_t n);

/* Counters since creation: distinct experts found resident by layer calls
 * (hits), copied by layer calls (misses), copied by prefetches, and host to
 * device bytes of all copies.  NULL outputs are skipped. */
moe_status moe_cache_stats(const moe_expert_cache* cache, int64_t* hits, int64_t* misses, int64_t* prefetched,
                           int64_t* h2d_bytes);

/* fused_moe over the cache: routes router_logits [M][E] over all E experts
 * on `stream`, waits for the routing on the host (the page's synchronous miss
 * path), copies the missing experts in, and runs alignment, both GEMMs and
 * the combine over the slots with expert ids renamed to slot ids.  out,
 * topk_ids_out and topk_weights_out are as for fused_moe (the ids are host
 * expert ids).  host_ids: host int32 [M*topk] (pinned for speed) the call
 * uses for the routed ids; leave it untouched until the stream has finished
 * the call.  workspace: fused_moe_workspace_size(dtype, M, capacity, topk, H,
 * I) bytes, 256-byte aligned.  Errors as for fused_moe (checked against E),
 * plus: topk > capacity, or a batch routed to more distinct experts than
 * slots -> MOE_ERR_UNSUPPORTED (the batch was routed, nothing else ran).
 * Layer calls of one cache form one chain: a call on another stream waits
 * for the previous call. */
moe_status fused_moe_cached(moe_expert_cache* cache, const void* x, const float* x_scale,
                            const float* router_logits, int32_t M, int32_t topk, int32_t renormalize, void* out,
                            int32_t* topk_ids_out, float* topk_weights_out, int32_t* host_ids, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */

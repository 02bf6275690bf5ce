// Internals of the fused layer shared by the C ABI (moe_abi.hip) and the
// expert cache (expert_cache.hip): the workspace layout and the two halves
// of the launch sequence.  Arguments are validated before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// The fused layer's workspace, carved 256-byte aligned from one buffer.
struct FusedLayout {
    int32_t block_m;
    int32_t ksplit;  // K split of the DOWN GEMM (partials summed by the combine)
    int64_t cap;
    size_t bytes;
    int32_t* ids;    // routed expert ids (when the caller keeps none)
    int32_t* remap;  // ids renamed to cache slots (expert cache)
    float* wts;
    moe_align_bufs al;
    void* act;
    void* y;
    bool q_on_load;  // fp8: the DOWN kernel quantises the float32 act on load
    bool dc;         // the DOWN kernel also combines (no y, no combine launch)
    void* act_q;     // fp8 otherwise: e4m3 codes of act
    float* ypart;
    float* amax;
    float* amax_parts;  // e4m3, one token: partial maxima of act ([topk][I/32]), see GemmCall
    int32_t amax_nparts;
};

// ws == nullptr: only the sizes (L.bytes).  E: the experts the weights hold.
FusedLayout fused_layout(char* ws, moe_dtype dtype, int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I);

bool misaligned(const void* p);
moe_status hip_status(hipError_t e);
moe_status check_router(int32_t M, int32_t E, int32_t topk);

// Argument checks of fused_moe (host only; router_logits may be an output).
moe_status check_fused(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                       const void* w1, const float* w1_scale, const void* w2, const float* w2_scale, int32_t M,
                       int32_t E, int32_t topk, int32_t H, int32_t I, const void* out, const int32_t* topk_ids_out,
                       const float* topk_weights_out);

// GATE_UP -> DOWN -> combine, once L.al aligns the pairs over the E experts
// that w1/w2 hold and wts holds the routing weights.
moe_status run_experts(moe_dtype dtype, const void* x, const float* x_scale, const void* w1, const float* w1_scale,
                       const void* w2, const float* w2_scale, int32_t M, int32_t E, int32_t topk, int32_t H,
                       int32_t I, void* out, const float* wts, const FusedLayout& L, hipStream_t s,
                       const float* route_logits = nullptr, int32_t renormalize = 1, int32_t* route_ids = nullptr);

}  // namespace moe

// Internal launchers behind the C ABI.  Arguments are validated by the
// caller (moe_abi.hip) before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Limits the ABI enforces (the kernels size LDS tables and unrolled loops by them).
constexpr int kMaxExperts = 256;
constexpr int kMaxTopk = 16;
constexpr int kMaxKsplit = 8;  // K split of the decode DOWN GEMM (float32 partials)

// Which grouped-GEMM kernel family serves a call.
enum class GemmPath { kAuto = 0, kDecode = 1, kPrefill = 2 };

hipError_t launch_route(const float* logits, int M, int E, int topk, int renormalize, int32_t* ids,
                        float* weights, hipStream_t s);

hipError_t launch_align(const int32_t* ids, int M, int topk, int E, int block_m, int64_t cap,
                        const moe_align_bufs& out, float* zero_f32, hipStream_t s);

// Both steps in one launch for M <= 16 (one wavefront routes each token).
bool route_align_fits(int M);
hipError_t launch_route_align(const float* logits, int M, int E, int topk, int renormalize, int32_t* ids,
                              float* weights, int block_m, int64_t cap, const moe_align_bufs& out,
                              float* zero_f32, hipStream_t s);

// Router scores logits[M][E] = x . wg^T (wg float32 [E][H]).
hipError_t launch_router_logits(moe_dtype xdt, const void* x, const float* x_scale, const float* wg, int M, int E,
                                int H, float* logits, hipStream_t s);

// Router + route + align in one launch, for a few tokens and a small router.
bool router_route_align_fits(int M, int E, int H);
hipError_t launch_router_route_align(moe_dtype xdt, const void* x, const float* x_scale, const float* wg, int H,
                                     float* logits_out, int M, int E, int topk, int renormalize, int32_t* ids,
                                     float* weights, int block_m, int64_t cap, const moe_align_bufs& out,
                                     float* zero_f32, hipStream_t s);

hipError_t launch_fill_zero_f32(float* p, int n, hipStream_t s);

struct GemmCall {
    moe_gemm_kind kind;
    moe_dtype dtype;
    const void* a;
    const float* a_scale;
    const void* w;
    const float* w_scale;
    moe_align_bufs al;
    int M, topk, E, N, K, block_m;
    void* c;
    float* c_amax;
    int ksplit = 1;         // decode DOWN: split of K across workgroups
    float* cpart = nullptr;  // with ksplit > 1: float32 partials [ksplit][P][N] instead of c
    bool act_q8 = false;     // fp8 DOWN: a holds e4m3 codes (quantised with amax/448), not the float32 act
    // self-routing (M = 1, bf16, e4m3 or W4A16 decode kernels): every
    // workgroup routes the token from its logits instead of reading the
    // alignment (al is then unused); route_ids / route_wts, when set, receive
    // its topk ids and weights (written by one workgroup)
    const float* route_logits = nullptr;
    int route_renorm = 1;
    int32_t* route_ids = nullptr;
    float* route_wts = nullptr;
    // e4m3 with self-routing: the intermediate's amax as partial maxima, one
    // float per 32 gate/up output columns of each slot ([slots][N/2/32]),
    // every one written by the GATE_UP launch (so nothing needs clearing)
    // and reduced by the DOWN launch (amax_nparts of them) instead of c_amax
    // / a_scale
    float* amax_parts = nullptr;
    int amax_nparts = 0;
};

// Kernel family chosen for a call (decode for few rows per expert, or when
// block_m has no prefill tile; MOE_GEMM_PATH=decode|prefill overrides).
GemmPath choose_gemm_path(const GemmCall& g);
int prefill_supported_block_m(int block_m);

hipError_t launch_grouped_gemm(const GemmCall& g, hipStream_t s);

// Decode DOWN GEMM with the combine inside (bf16, about one 16-row token tile
// per expert, at most 512 pairs, I a multiple of 256): out[M][H] directly,
// the same bits as the per-expert DOWN kernel followed by launch_combine.
// Used by the fused layer only with MOE_DOWN_COMBINE=1 (not faster here).
bool down_combine_fits(moe_dtype dtype, int M, int topk, int E, int H, int I, int block_m);
hipError_t launch_down_combine(const GemmCall& c, const float* topk_weights, void* out, hipStream_t s);

// K split the fused layer uses for the DOWN GEMM (1 when the decode kernel
// already has enough workgroups, or when the prefill kernel serves the call).
int down_ksplit(moe_dtype dtype, int M, int topk, int E, int N, int K, int block_m);

// Whether an e4m3 DOWN call of these sizes runs a kernel that reads the
// float32 intermediate and quantises it on load (decode kernel, one token
// tile); otherwise the fused layer quantises the intermediate once
// (launch_quant_act) and the DOWN kernel reads the codes.
bool fp8_down_quantises_on_load(int M, int topk, int E, int N, int K, int block_m);

// e4m3 codes of n float32 intermediate values (n a multiple of 16), scale amax/448.
hipError_t launch_quant_act(const void* act, const float* amax, void* q, size_t n, hipStream_t s);

hipError_t launch_combine_partials(const float* ypart, int ksplit, const float* w, int M, int topk, int H,
                                   moe_dtype out_dtype, void* out, hipStream_t s);

hipError_t launch_combine(moe_dtype y_dtype, const void* y, const float* w, int M, int topk, int H,
                          moe_dtype out_dtype, void* out, hipStream_t s);

}  // namespace moe

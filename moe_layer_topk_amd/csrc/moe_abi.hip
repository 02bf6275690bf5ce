// C ABI of the fused MoE layer: host-side validation (before any HIP call),
// workspace carving and the launch sequence route -> align -> GATE_UP GEMM
// -> DOWN GEMM -> combine (FusedMoE vs MegaMoE post, section 3.1).
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "moe_fused.h"
#include "moe_launch.h"

using namespace moe;

namespace moe {

constexpr int64_t kMaxPairs = 1 << 24;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_router(int32_t M, int32_t E, int32_t topk) {
    if (M < 0 || E < 1 || topk < 1 || topk > E) return MOE_ERR_SHAPE;
    if (E > kMaxExperts || topk > kMaxTopk) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)M * topk > kMaxPairs) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

bool valid_block_m(int32_t b) { return b == 1 || b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

bool known_dtype(moe_dtype d) { return d == MOE_F32 || d == MOE_BF16 || d == MOE_FP8_E4M3 || d == MOE_W4A16; }

// layer dtypes whose weights carry scales (fp8: one per expert matrix; W4A16: per group)
bool scaled_weights(moe_dtype d) { return d == MOE_FP8_E4M3 || d == MOE_W4A16; }

// bytes of an element of y: f32 for the f32 path, bf16 otherwise
size_t inter_bytes(moe_dtype d) { return d == MOE_F32 ? 4 : 2; }
// ... and of act: the e4m3 layer keeps it in float32 until it is quantised
size_t act_bytes(moe_dtype d) { return (d == MOE_BF16 || d == MOE_W4A16) ? 2 : 4; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int32_t fused_block_m(moe_dtype dtype, int32_t M, int32_t E, int32_t topk) {
    if (dtype == MOE_F32 || dtype == MOE_W4A16) return 16;  // decode kernels only
    const char* env = getenv("MOE_GEMM_PATH");
    if (env && strcmp(env, "prefill") == 0) return 64;
    if (env && strcmp(env, "decode") == 0) return 16;
    // Tile height from the pairs per expert (layer times, tile kernel against
    // the decode kernels).  bf16: the decode kernels up to 24 (Mixtral shape
    // at 24: 0.506 ms against 0.517 on 64-row tiles; 128 experts at 16 and
    // 24 are 4% faster and 12% slower there), 64-row tiles above that
    // (Mixtral shape at 32 and 40: 0.536 -> 0.529, 0.560 -> 0.543 ms; 128
    // experts at 32 and 40: 0.318 -> 0.276, 0.346 -> 0.280), 128-row tiles
    // above 48 (Mixtral shape at 64: 0.890 -> 0.593 ms, 0.695 on 64-row
    // tiles; 128 experts at 48 a tie between the two heights, at 64 0.468
    // -> 0.312).  e4m3 (products a quarter of bf16's cost per byte): 128-row
    // tiles above 32, else 64-row tiles from two tokens up (64-expert
    // layer: 2 tokens 0.268 -> 0.250 ms, 32 tokens 1.048 -> 1.011, 256
    // tokens 1.432 -> 1.196; one token a tie, left to the decode kernels)
    const int64_t per_expert = (int64_t)M * topk / E;
    if (dtype == MOE_FP8_E4M3) return per_expert > 32 ? 128 : (M >= 2 ? 64 : 16);
    return per_expert > 48 ? 128 : (per_expert > 24 ? 64 : 16);
}

struct Carve {
    char* base;
    size_t off;
    template <typename T>
    T* take(size_t n) {
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off = round_up(off + n * sizeof(T), 256);
        return p;
    }
};


FusedLayout fused_layout(char* ws, moe_dtype dtype, int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I) {
    FusedLayout L;
    const int64_t P = (int64_t)M * topk;
    L.block_m = fused_block_m(dtype, M, E, topk);
    L.cap = moe_align_capacity(M, topk, E, L.block_m);
    Carve c{ws, 0};
    L.ids = c.take<int32_t>(P);
    L.remap = c.take<int32_t>(P);
    L.wts = c.take<float>(P);
    L.al.sorted_ids = c.take<int32_t>(L.cap);
    L.al.tile_expert = c.take<int32_t>(L.cap / L.block_m);
    L.al.expert_counts = c.take<int32_t>(E);
    L.al.expert_offsets = c.take<int32_t>(E + 1);
    L.al.active_experts = c.take<int32_t>(P < E ? P : E);
    L.al.num_active = c.take<int32_t>(1);
    L.amax = c.take<float>(1);
    L.act = c.take<char>((size_t)P * I * act_bytes(dtype));
    L.dc = down_combine_fits(dtype, M, topk, E, H, I, L.block_m);
    L.y = L.dc ? nullptr : c.take<char>((size_t)P * H * inter_bytes(dtype));
    L.q_on_load = dtype == MOE_FP8_E4M3 && fp8_down_quantises_on_load(M, topk, E, H, I, L.block_m);
    L.act_q = (dtype == MOE_FP8_E4M3 && !L.q_on_load) ? c.take<char>((size_t)P * I) : nullptr;
    L.ksplit = L.dc ? 1 : down_ksplit(dtype, M, topk, E, H, I, L.block_m);
    L.ypart = L.ksplit > 1 ? c.take<float>((size_t)L.ksplit * P * H) : nullptr;
    // one e4m3 token (the GEMMs may route it themselves): the intermediate's
    // amax as partials, one per 32 gate/up output columns of each slot
    L.amax_nparts = (dtype == MOE_FP8_E4M3 && M == 1) ? (P < E ? (int32_t)P : E) * (I / 32) : 0;
    L.amax_parts = L.amax_nparts ? c.take<float>((size_t)L.amax_nparts) : nullptr;
    L.bytes = c.off;
    return L;
}

}  // namespace moe

extern "C" {

const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "invalid shape";
        case MOE_ERR_UNSUPPORTED: return "unsupported size, dtype or block_m";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_SCRATCH: return "sizes exceed the static scratch of fused_moe_noalloc";
    }
    return "unknown status";
}

moe_status moe_route(const float* logits, int32_t M, int32_t E, int32_t topk, int32_t renormalize,
                     int32_t* topk_ids, float* topk_weights, void* stream) {
    moe_status st = check_router(M, E, topk);
    if (st != MOE_OK) return st;
    if (M == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
    if (misaligned(logits) || misaligned(topk_ids) || misaligned(topk_weights)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_route(logits, M, E, topk, renormalize, topk_ids, topk_weights,
                                   static_cast<hipStream_t>(stream)));
}

int64_t moe_align_capacity(int32_t M, int32_t topk, int32_t E, int32_t block_m) {
    if (M < 0 || topk < 1 || E < 1 || block_m < 1) return -1;
    const int64_t P = (int64_t)M * topk;
    const int64_t act = P < E ? P : E;
    const int64_t rows = P + act * (block_m - 1);
    return (rows + block_m - 1) / block_m * block_m;
}

moe_status moe_align(const int32_t* topk_ids, int32_t M, int32_t topk, int32_t E, int32_t block_m,
                     moe_align_bufs out, void* stream) {
    moe_status st = check_router(M, E, topk);
    if (st != MOE_OK) return st;
    if (!valid_block_m(block_m)) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!topk_ids || !out.sorted_ids || !out.tile_expert || !out.expert_counts || !out.expert_offsets ||
        !out.active_experts || !out.num_active)
        return MOE_ERR_NULL;
    if (misaligned(topk_ids) || misaligned(out.sorted_ids) || misaligned(out.tile_expert) ||
        misaligned(out.expert_counts) || misaligned(out.expert_offsets) || misaligned(out.active_experts) ||
        misaligned(out.num_active))
        return MOE_ERR_ALIGNMENT;
    const int64_t cap = moe_align_capacity(M, topk, E, block_m);
    return hip_status(launch_align(topk_ids, M, topk, E, block_m, cap, out, nullptr,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm(moe_gemm_kind kind, moe_dtype dtype, const void* a, const float* a_scale,
                            const void* w, const float* w_scale, const moe_align_bufs* al, int32_t M,
                            int32_t topk, int32_t E, int32_t N, int32_t K, int32_t block_m, void* c,
                            float* c_amax, void* stream) {
    if (kind != MOE_GEMM_GATE_UP_SILU && kind != MOE_GEMM_DOWN && kind != MOE_GEMM_DOWN_E4M3_ACT)
        return MOE_ERR_UNSUPPORTED;
    if (!known_dtype(dtype)) return MOE_ERR_UNSUPPORTED;
    if (kind == MOE_GEMM_DOWN_E4M3_ACT && dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    const bool act_q8 = kind == MOE_GEMM_DOWN_E4M3_ACT;
    if (act_q8) kind = MOE_GEMM_DOWN;
    moe_status st = check_router(M, E, topk);
    if (st != MOE_OK) return st;
    if (N < 1 || K < 1 || N % 128 || K % 128) return MOE_ERR_SHAPE;
    if (kind == MOE_GEMM_GATE_UP_SILU && N % 256) return MOE_ERR_SHAPE;
    if (!valid_block_m(block_m)) return MOE_ERR_UNSUPPORTED;
    const bool fp8 = dtype == MOE_FP8_E4M3, w4 = dtype == MOE_W4A16;
    if ((fp8 || w4) && K % 256) return MOE_ERR_SHAPE;
    if (!fp8 && (a_scale || c_amax)) return MOE_ERR_UNSUPPORTED;
    if (!scaled_weights(dtype) && w_scale) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!a || !w || !al || !c || !al->sorted_ids || !al->tile_expert || !al->expert_counts ||
        !al->expert_offsets || !al->active_experts || !al->num_active)
        return MOE_ERR_NULL;
    if (fp8 && (!a_scale || !w_scale || (kind == MOE_GEMM_GATE_UP_SILU && !c_amax))) return MOE_ERR_NULL;
    if (w4 && !w_scale) return MOE_ERR_NULL;
    if (misaligned(a) || misaligned(w) || misaligned(c) || misaligned(w_scale)) return MOE_ERR_ALIGNMENT;
    GemmCall g{kind, dtype, a, a_scale, w, w_scale, *al, M, topk, E, N, K, block_m, c, c_amax, 1, nullptr, act_q8};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fp8 && kind == MOE_GEMM_GATE_UP_SILU) {
        hipError_t e = launch_fill_zero_f32(c_amax, 1, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return hip_status(launch_grouped_gemm(g, s));
}

moe_status moe_quant_act(const void* act, const float* amax, int64_t n, void* act_q, void* stream) {
    if (n < 0 || n % 16) return MOE_ERR_SHAPE;
    if (n == 0) return MOE_OK;
    if (!act || !amax || !act_q) return MOE_ERR_NULL;
    if (misaligned(act) || misaligned(act_q)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_quant_act(act, amax, act_q, (size_t)n, static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(moe_dtype y_dtype, const void* y, const float* topk_weights, int32_t M,
                       int32_t topk, int32_t H, moe_dtype out_dtype, void* out, void* stream) {
    if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
        return MOE_ERR_UNSUPPORTED;
    if (M < 0 || topk < 1 || H < 1 || H % 8) return MOE_ERR_SHAPE;
    if (topk > kMaxTopk) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!y || !topk_weights || !out) return MOE_ERR_NULL;
    if (misaligned(y) || misaligned(out)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_combine(y_dtype, y, topk_weights, M, topk, H, out_dtype, out,
                                     static_cast<hipStream_t>(stream)));
}

size_t fused_moe_workspace_size(moe_dtype dtype, int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I) {
    if (M <= 0 || check_router(M, E, topk) != MOE_OK || H < 1 || I < 1) return 0;
    return fused_layout(nullptr, dtype, M, E, topk, H, I).bytes;
}

}  // extern "C"

namespace moe {

// Argument checks shared by fused_moe and fused_moe_noalloc (host only).
moe_status check_fused(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                       const void* w1, const float* w1_scale, const void* w2, const float* w2_scale, int32_t M,
                       int32_t E, int32_t topk, int32_t H, int32_t I, const void* out, const int32_t* topk_ids_out,
                       const float* topk_weights_out) {
    if (!known_dtype(dtype)) return MOE_ERR_UNSUPPORTED;
    moe_status st = check_router(M, E, topk);
    if (st != MOE_OK) return st;
    if (H < 1 || I < 1 || H % 128 || I % 128) return MOE_ERR_SHAPE;
    const bool fp8 = dtype == MOE_FP8_E4M3, w4 = dtype == MOE_W4A16;
    if ((fp8 || w4) && (H % 256 || I % 256)) return MOE_ERR_SHAPE;
    if (!fp8 && x_scale) return MOE_ERR_UNSUPPORTED;
    if (!scaled_weights(dtype) && (w1_scale || w2_scale)) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!x || !router_logits || !w1 || !w2 || !out) return MOE_ERR_NULL;
    if (fp8 && !x_scale) return MOE_ERR_NULL;
    if (scaled_weights(dtype) && (!w1_scale || !w2_scale)) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(router_logits) || misaligned(w1) || misaligned(w2) || misaligned(out) ||
        misaligned(topk_ids_out) || misaligned(topk_weights_out) || misaligned(w1_scale) || misaligned(w2_scale))
        return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

// The expert half of the layer (GATE_UP -> DOWN -> combine) once L.al holds
// the alignment of the routed pairs over E experts (E: the experts whose
// weights w1/w2 hold, in that order) and wts the routing weights.
moe_status run_experts(moe_dtype dtype, const void* x, const float* x_scale, const void* w1, const float* w1_scale,
                       const void* w2, const float* w2_scale, int32_t M, int32_t E, int32_t topk, int32_t H,
                       int32_t I, void* out, const float* wts, const FusedLayout& L, hipStream_t s,
                       const float* route_logits, int32_t renormalize, int32_t* route_ids) {
    const bool fp8 = dtype == MOE_FP8_E4M3;
    const moe_dtype inter = dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
    GemmCall g1{MOE_GEMM_GATE_UP_SILU, dtype, x, x_scale, w1, w1_scale, L.al, M, topk, E, 2 * I, H,
                L.block_m, L.act, fp8 ? L.amax : nullptr};
    // route_logits: the GEMMs route the one token themselves; the gate/up
    // launch writes its ids and weights (which the combine reads)
    g1.route_logits = route_logits;
    g1.route_renorm = renormalize;
    g1.route_ids = route_ids;
    g1.route_wts = const_cast<float*>(wts);
    // e4m3 then passes the intermediate's amax through partials (nothing
    // clears c_amax without the align launch)
    float* parts = (fp8 && route_logits) ? L.amax_parts : nullptr;
    g1.amax_parts = parts;
    if (launch_grouped_gemm(g1, s) != hipSuccess) return MOE_ERR_HIP;
    // e4m3: the down kernel quantises the float32 intermediate as it loads it,
    // or (tile kernels) reads codes quantised once here
    const bool codes = fp8 && !L.q_on_load;
    if (codes && launch_quant_act(L.act, L.amax, L.act_q, (size_t)M * topk * I, s) != hipSuccess) return MOE_ERR_HIP;
    GemmCall g2{MOE_GEMM_DOWN, dtype, codes ? L.act_q : L.act, fp8 ? L.amax : nullptr, w2, w2_scale, L.al, M, topk, E,
                H, I, L.block_m, L.y, nullptr, L.ksplit, L.ypart, codes};
    g2.route_logits = route_logits;
    g2.route_renorm = renormalize;
    g2.amax_parts = parts;
    g2.amax_nparts = parts ? L.amax_nparts : 0;
    if (L.dc) return hip_status(launch_down_combine(g2, wts, out, s));  // y stays on chip
    if (launch_grouped_gemm(g2, s) != hipSuccess) return MOE_ERR_HIP;
    if (L.ksplit > 1) return hip_status(launch_combine_partials(L.ypart, L.ksplit, wts, M, topk, H, inter, out, s));
    return hip_status(launch_combine(inter, L.y, wts, M, topk, H, inter, out, s));
}

// One token of a bf16, e4m3 or int4 layer whose GEMMs both run the decode
// kernels (the kernels that can route a token themselves) and whose down
// GEMM is not the fused down + combine kernel (it reads the alignment); an
// e4m3 down kernel must quantise the float32 intermediate on load.
static bool self_route_fits(moe_dtype dtype, int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I,
                            const FusedLayout& L) {
    const bool fp8 = dtype == MOE_FP8_E4M3 && L.q_on_load && L.amax_parts;
    if (M != 1 || L.dc || !(dtype == MOE_BF16 || dtype == MOE_W4A16 || fp8)) return false;
    const GemmCall g1{MOE_GEMM_GATE_UP_SILU, dtype, nullptr, nullptr, nullptr, nullptr, {}, M, topk, E, 2 * I, H,
                      L.block_m, nullptr, nullptr};
    const GemmCall g2{MOE_GEMM_DOWN, dtype, nullptr, nullptr, nullptr, nullptr, {}, M, topk, E, H, I,
                      L.block_m, nullptr, nullptr};
    return choose_gemm_path(g1) == GemmPath::kDecode && choose_gemm_path(g2) == GemmPath::kDecode;
}

// The launch sequence over a carved workspace (arguments already checked, M > 0).
// router_w non-null: router_logits is an output the layer first fills with
// x . router_w^T (in the same launch as route + align when that fits).
moe_status run_fused(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                     const void* w1, const float* w1_scale, const void* w2, const float* w2_scale, int32_t M,
                     int32_t E, int32_t topk, int32_t H, int32_t I, int32_t renormalize, void* out,
                     int32_t* topk_ids_out, float* topk_weights_out, const FusedLayout& L, hipStream_t s,
                     const float* router_w = nullptr) {
    const bool fp8 = dtype == MOE_FP8_E4M3;
    int32_t* ids = topk_ids_out ? topk_ids_out : L.ids;
    float* wts = topk_weights_out ? topk_weights_out : L.wts;
    float* logits = const_cast<float*>(router_logits);
    const moe_dtype xdt = dtype == MOE_W4A16 ? MOE_BF16 : dtype;  // the activations' storage
    if (self_route_fits(dtype, M, E, topk, H, I, L)) {
        // one token on the decode kernels: they route it themselves, so the
        // layer needs no route / align launch (the launch and its dependent
        // loads are most of the non-GEMM time at one token); from hidden
        // states, the router scores come first
        if (router_w && launch_router_logits(xdt, x, x_scale, router_w, M, E, H, logits, s) != hipSuccess)
            return MOE_ERR_HIP;
        return run_experts(dtype, x, x_scale, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, out, wts, L, s,
                           router_logits, renormalize, ids);
    }
    if (router_w && router_route_align_fits(M, E, H)) {
        // router scores, top-k and alignment in one launch
        if (launch_router_route_align(xdt, x, x_scale, router_w, H, logits, M, E, topk, renormalize, ids, wts,
                                      L.block_m, L.cap, L.al, fp8 ? L.amax : nullptr, s) != hipSuccess)
            return MOE_ERR_HIP;
    } else {
        if (router_w && launch_router_logits(xdt, x, x_scale, router_w, M, E, H, logits, s) != hipSuccess)
            return MOE_ERR_HIP;
        if (route_align_fits(M)) {
            if (launch_route_align(logits, M, E, topk, renormalize, ids, wts, L.block_m, L.cap, L.al,
                                   fp8 ? L.amax : nullptr, s) != hipSuccess)
                return MOE_ERR_HIP;
        } else {
            if (launch_route(logits, M, E, topk, renormalize, ids, wts, s) != hipSuccess) return MOE_ERR_HIP;
            if (launch_align(ids, M, topk, E, L.block_m, L.cap, L.al, fp8 ? L.amax : nullptr, s) != hipSuccess)
                return MOE_ERR_HIP;
        }
    }
    return run_experts(dtype, x, x_scale, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, out, wts, L, s);
}

}  // namespace moe

namespace {

// ------------------------------------------------------ static scratch
//
// The workspace of fused_moe_noalloc: a file-scope device array, one copy
// per GPU for the life of the process.  Host code never uses the array's
// name as an address (on the host it only names the symbol); its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// The current device's scratch address, or nullptr (with *err set) if the
// lookup fails.
void* scratch_for_current_device(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        scratch_dev[dev] = p;
    }
    return scratch_dev[dev];
}

}  // namespace

extern "C" {

moe_status fused_moe(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                     const void* w1, const float* w1_scale, const void* w2, const float* w2_scale,
                     int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I, int32_t renormalize,
                     void* out, int32_t* topk_ids_out, float* topk_weights_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
    moe_status st = check_fused(dtype, x, x_scale, router_logits, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, out,
                                topk_ids_out, topk_weights_out);
    if (st != MOE_OK || M == 0) return st;
    if (!workspace) return MOE_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MOE_ERR_ALIGNMENT;
    FusedLayout L = fused_layout(static_cast<char*>(workspace), dtype, M, E, topk, H, I);
    if (workspace_bytes < L.bytes) return MOE_ERR_WORKSPACE;
    return run_fused(dtype, x, x_scale, router_logits, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, renormalize, out,
                     topk_ids_out, topk_weights_out, L, static_cast<hipStream_t>(stream));
}

moe_status moe_router_logits(moe_dtype x_dtype, const void* x, const float* x_scale, const float* router_w,
                             int32_t M, int32_t H, int32_t E, float* logits, void* stream) {
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16 && x_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    if (M < 0 || H < 1 || E < 1 || H % 4) return MOE_ERR_SHAPE;
    if ((x_dtype == MOE_FP8_E4M3) != (x_scale != nullptr)) return x_scale ? MOE_ERR_UNSUPPORTED : MOE_ERR_NULL;
    if (M == 0) return MOE_OK;
    if (!x || !router_w || !logits) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(router_w) || misaligned(logits)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_router_logits(x_dtype, x, x_scale, router_w, M, E, H, logits,
                                           static_cast<hipStream_t>(stream)));
}

moe_status fused_moe_router(moe_dtype dtype, const void* x, const float* x_scale, const float* router_w,
                            float* router_logits, const void* w1, const float* w1_scale, const void* w2,
                            const float* w2_scale, int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I,
                            int32_t renormalize, void* out, int32_t* topk_ids_out, float* topk_weights_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
    moe_status st = check_fused(dtype, x, x_scale, router_logits, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, out,
                                topk_ids_out, topk_weights_out);
    if (st != MOE_OK || M == 0) return st;
    if (!router_w || !workspace) return MOE_ERR_NULL;
    if (misaligned(router_w)) return MOE_ERR_ALIGNMENT;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MOE_ERR_ALIGNMENT;
    FusedLayout L = fused_layout(static_cast<char*>(workspace), dtype, M, E, topk, H, I);
    if (workspace_bytes < L.bytes) return MOE_ERR_WORKSPACE;
    return run_fused(dtype, x, x_scale, router_logits, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, renormalize, out,
                     topk_ids_out, topk_weights_out, L, static_cast<hipStream_t>(stream), router_w);
}

size_t fused_moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status fused_moe_noalloc(moe_dtype dtype, const void* x, const float* x_scale, const float* router_logits,
                             const void* w1, const float* w1_scale, const void* w2, const float* w2_scale,
                             int32_t M, int32_t E, int32_t topk, int32_t H, int32_t I, int32_t renormalize,
                             void* out, int32_t* topk_ids_out, float* topk_weights_out, void* stream) {
    moe_status st = check_fused(dtype, x, x_scale, router_logits, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, out,
                                topk_ids_out, topk_weights_out);
    if (st != MOE_OK || M == 0) return st;
    // sizes first (host only), then the one-time address lookup
    if (fused_layout(nullptr, dtype, M, E, topk, H, I).bytes > kScratchBytes) return MOE_ERR_SCRATCH;
    hipError_t err = hipSuccess;
    void* ws = scratch_for_current_device(&err);
    if (!ws) return MOE_ERR_HIP;
    FusedLayout L = fused_layout(static_cast<char*>(ws), dtype, M, E, topk, H, I);
    return run_fused(dtype, x, x_scale, router_logits, w1, w1_scale, w2, w2_scale, M, E, topk, H, I, renormalize, out,
                     topk_ids_out, topk_weights_out, L, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// Expert streaming (FusedMoE vs MegaMoE post, sections 4.1-4.3): every
// expert's weights stay in host memory, a fixed number of GPU slots hold the
// experts in use, and the layer runs over the slots.
//
// A layer call routes on the GPU, brings the routed ids to the host (the
// synchronous miss path: the host must know which experts the batch needs),
// copies each missing expert into a free or least recently used slot on the
// cache's copy stream, and runs alignment, the grouped GEMMs and the combine
// with the expert ids renamed to slot ids: the slots are an ordinary set of
// E' = capacity experts, so the kernels are the fused layer's own, and each
// pair's products do not depend on which slot holds its expert.
//
// Ordering: a copy into a slot waits for the end of the last layer call that
// read the slot (an event on the compute stream); a layer call's GEMMs wait
// for the newest copy into a slot they read (an event on the copy stream).
// Prefetching issues copies ahead of a call on the same copy stream, so they
// overlap the compute of calls that read other slots.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <utility>
#include <vector>

#include "moe_fused.h"
#include "moe_launch.h"

using namespace moe;

// Copies and layer calls are ordered through two rings of events.  Copy
// batch b records copy_ev[b % kRing] on the copy stream after its copies; layer
// call n records call_ev[n % kRing] on its stream at its end.  A slot keeps the
// numbers of the last batch that filled it and of the last call that read it.
// An event of the ring re-recorded for a later batch (call) marks a later point
// of the same in-order stream, so waiting on it still waits long enough.  Layer
// calls form one chain: a call on another stream than the previous call's first
// waits for the previous call.
constexpr int kRing = 16;

struct moe_expert_cache {
    moe_dtype dtype;
    int32_t E, C, H, I;
    moe_expert_weights host;   // all E experts, one after another
    moe_expert_weights slots;  // C slots, same layout
    size_t bytes[4];           // per expert: w1, w2, w1_scale, w2_scale
    hipStream_t copy;
    std::vector<int32_t> slot_of;     // [E] -> slot or -1
    std::vector<int32_t> expert_in;   // [C] -> expert or -1
    std::vector<uint64_t> last_use;   // [C] clock of the last request that wanted the slot (LRU)
    std::vector<int64_t> slot_batch;  // [C] last copy batch that filled the slot, -1: none
    std::vector<int64_t> slot_call;   // [C] last layer call that read the slot, -1: none
    uint64_t clock = 0;
    int64_t nbatch = 0, ncall = 0;
    hipEvent_t copy_ev[kRing] = {};
    hipEvent_t call_ev[kRing] = {};
    hipStream_t last_stream = nullptr;
    int64_t hits = 0, misses = 0, prefetched = 0, h2d_bytes = 0;
};

namespace {

// bytes of one expert's w1, w2, w1_scale, w2_scale
void part_bytes(moe_dtype d, int64_t H, int64_t I, size_t b[4]) {
    if (d == MOE_W4A16) {  // 4-bit codes, one float scale per 128 along K
        b[0] = (size_t)(2 * I * H / 2);
        b[1] = (size_t)(H * I / 2);
        b[2] = (size_t)(H / 128 * 2 * I * 4);
        b[3] = (size_t)(I / 128 * H * 4);
        return;
    }
    const size_t eb = d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1;
    b[0] = (size_t)(2 * I * H) * eb;
    b[1] = (size_t)(H * I) * eb;
    b[2] = b[3] = d == MOE_FP8_E4M3 ? 4 : 0;  // one scale per expert matrix
}

const void* part(const moe_expert_weights& w, int i) {
    return i == 0 ? w.w1 : i == 1 ? w.w2 : i == 2 ? static_cast<const void*>(w.w1_scale)
                                                  : static_cast<const void*>(w.w2_scale);
}

// Slot for a new expert: an empty one, else the least recently used one not
// kept by the current request.
int32_t victim(const moe_expert_cache* c, const std::vector<char>& keep) {
    int32_t best = -1;
    for (int32_t s = 0; s < c->C; ++s) {
        if (keep[s]) continue;
        if (c->expert_in[s] < 0) return s;
        if (best < 0 || c->last_use[s] < c->last_use[best]) best = s;
    }
    return best;
}

// Make the distinct experts `need` (|need| <= C) resident and mark their slots
// used at a new clock.  Missing experts go to victim slots in one copy batch
// on the copy stream, after the last layer call that read any of those slots.
// Counts hits and misses when `count`; *copies += experts copied.
moe_status make_resident(moe_expert_cache* c, const std::vector<int32_t>& need, bool count, int64_t* copies) {
    std::vector<char> keep(c->C, 0);
    ++c->clock;
    for (int32_t e : need)
        if (c->slot_of[e] >= 0) {
            keep[c->slot_of[e]] = 1;
            c->last_use[c->slot_of[e]] = c->clock;
            if (count) ++c->hits;
        }
    std::vector<std::pair<int32_t, int32_t>> fills;  // (expert, slot)
    int64_t after_call = -1;
    for (int32_t e : need) {
        if (c->slot_of[e] >= 0) continue;
        const int32_t s = victim(c, keep);
        if (s < 0) return MOE_ERR_UNSUPPORTED;  // unreachable while |need| <= C
        keep[s] = 1;
        fills.push_back({e, s});
        after_call = std::max(after_call, c->slot_call[s]);
    }
    if (fills.empty()) return MOE_OK;
    if (after_call >= 0 && hipStreamWaitEvent(c->copy, c->call_ev[after_call % kRing], 0) != hipSuccess)
        return MOE_ERR_HIP;
    for (auto [e, s] : fills) {
        for (int i = 0; i < 4; ++i) {
            if (!c->bytes[i]) continue;
            const char* src = static_cast<const char*>(part(c->host, i)) + (size_t)e * c->bytes[i];
            char* dst = const_cast<char*>(static_cast<const char*>(part(c->slots, i))) + (size_t)s * c->bytes[i];
            if (hipMemcpyAsync(dst, src, c->bytes[i], hipMemcpyHostToDevice, c->copy) != hipSuccess)
                return MOE_ERR_HIP;
            c->h2d_bytes += (int64_t)c->bytes[i];
        }
        if (c->expert_in[s] >= 0) c->slot_of[c->expert_in[s]] = -1;
        c->expert_in[s] = e;
        c->slot_of[e] = s;
        c->last_use[s] = c->clock;
        c->slot_batch[s] = c->nbatch;
        if (count) ++c->misses;
        if (copies) ++*copies;
    }
    if (hipEventRecord(c->copy_ev[c->nbatch % kRing], c->copy) != hipSuccess) return MOE_ERR_HIP;
    ++c->nbatch;
    return MOE_OK;
}

void destroy_events(moe_expert_cache* c) {
    for (int i = 0; i < kRing; ++i) {
        if (c->copy_ev[i]) (void)hipEventDestroy(c->copy_ev[i]);
        if (c->call_ev[i]) (void)hipEventDestroy(c->call_ev[i]);
    }
}

}  // namespace

extern "C" {

moe_status moe_cache_create(moe_dtype dtype, int32_t E, int32_t H, int32_t I, int32_t capacity,
                            moe_expert_weights host, moe_expert_weights slots, void* copy_stream,
                            moe_expert_cache** out) {
    if (!out) return MOE_ERR_NULL;
    *out = nullptr;
    if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_FP8_E4M3 && dtype != MOE_W4A16)
        return MOE_ERR_UNSUPPORTED;
    if (E < 1 || capacity < 1 || capacity > E || H < 1 || I < 1 || H % 128 || I % 128) return MOE_ERR_SHAPE;
    if ((dtype == MOE_FP8_E4M3 || dtype == MOE_W4A16) && (H % 256 || I % 256)) return MOE_ERR_SHAPE;
    if (E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    const bool scaled = dtype == MOE_FP8_E4M3 || dtype == MOE_W4A16;
    if (!host.w1 || !host.w2 || !slots.w1 || !slots.w2) return MOE_ERR_NULL;
    if (scaled && (!host.w1_scale || !host.w2_scale || !slots.w1_scale || !slots.w2_scale)) return MOE_ERR_NULL;
    if (!scaled && (host.w1_scale || host.w2_scale || slots.w1_scale || slots.w2_scale)) return MOE_ERR_UNSUPPORTED;
    if (misaligned(slots.w1) || misaligned(slots.w2) || misaligned(slots.w1_scale) || misaligned(slots.w2_scale))
        return MOE_ERR_ALIGNMENT;
    moe_expert_cache* c = new (std::nothrow) moe_expert_cache;
    if (!c) return MOE_ERR_UNSUPPORTED;
    c->dtype = dtype;
    c->E = E;
    c->C = capacity;
    c->H = H;
    c->I = I;
    c->host = host;
    c->slots = slots;
    part_bytes(dtype, H, I, c->bytes);
    c->copy = static_cast<hipStream_t>(copy_stream);
    c->slot_of.assign(E, -1);
    c->expert_in.assign(capacity, -1);
    c->last_use.assign(capacity, 0);
    c->slot_batch.assign(capacity, -1);
    c->slot_call.assign(capacity, -1);
    for (int i = 0; i < kRing; ++i)
        if (hipEventCreateWithFlags(&c->copy_ev[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&c->call_ev[i], hipEventDisableTiming) != hipSuccess) {
            destroy_events(c);
            delete c;
            return MOE_ERR_HIP;
        }
    *out = c;
    return MOE_OK;
}

moe_status moe_cache_destroy(moe_expert_cache* c) {
    if (!c) return MOE_OK;
    // copies still in flight read the caller's host buffers: let them finish
    moe_status st = MOE_OK;
    if (c->nbatch > 0 && hipEventSynchronize(c->copy_ev[(c->nbatch - 1) % kRing]) != hipSuccess) st = MOE_ERR_HIP;
    destroy_events(c);
    delete c;
    return st;
}

moe_status moe_cache_prefetch(moe_expert_cache* c, const int32_t* experts, int32_t n) {
    if (!c || (n > 0 && !experts)) return MOE_ERR_NULL;
    if (n < 0) return MOE_ERR_SHAPE;
    std::vector<int32_t> need;
    for (int32_t i = 0; i < n; ++i) {
        if (experts[i] < 0 || experts[i] >= c->E) return MOE_ERR_SHAPE;
        need.push_back(experts[i]);
    }
    std::sort(need.begin(), need.end());
    need.erase(std::unique(need.begin(), need.end()), need.end());
    if ((int32_t)need.size() > c->C) return MOE_ERR_UNSUPPORTED;
    int64_t copies = 0;
    moe_status st = make_resident(c, need, false, &copies);
    c->prefetched += copies;
    return st;
}

moe_status moe_cache_stats(const moe_expert_cache* c, int64_t* hits, int64_t* misses, int64_t* prefetched,
                           int64_t* h2d_bytes) {
    if (!c) return MOE_ERR_NULL;
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (prefetched) *prefetched = c->prefetched;
    if (h2d_bytes) *h2d_bytes = c->h2d_bytes;
    return MOE_OK;
}

moe_status fused_moe_cached(moe_expert_cache* c, const void* x, const float* x_scale, const float* router_logits,
                            int32_t M, int32_t topk, int32_t renormalize, void* out, int32_t* topk_ids_out,
                            float* topk_weights_out, int32_t* host_ids, void* workspace, size_t workspace_bytes,
                            void* stream) {
    if (!c) return MOE_ERR_NULL;
    const int32_t E = c->E, C = c->C, H = c->H, I = c->I;
    if (topk > C) return MOE_ERR_UNSUPPORTED;
    // the slot arrays take the weights' place: the same checks as fused_moe over them
    moe_status st = check_fused(c->dtype, x, x_scale, router_logits, c->slots.w1, c->slots.w1_scale, c->slots.w2,
                                c->slots.w2_scale, M, E, topk, H, I, out, topk_ids_out, topk_weights_out);
    if (st != MOE_OK || M == 0) return st;
    if (!host_ids || !workspace) return MOE_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MOE_ERR_ALIGNMENT;
    FusedLayout L = fused_layout(static_cast<char*>(workspace), c->dtype, M, C, topk, H, I);
    if (workspace_bytes < L.bytes) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t P = (int64_t)M * topk;
    int32_t* ids = topk_ids_out ? topk_ids_out : L.ids;
    float* wts = topk_weights_out ? topk_weights_out : L.wts;

    // calls form one chain across streams (the event rings rely on it)
    if (c->ncall > 0 && s != c->last_stream &&
        hipStreamWaitEvent(s, c->call_ev[(c->ncall - 1) % kRing], 0) != hipSuccess)
        return MOE_ERR_HIP;
    // route over the E experts, then the ids to the host
    if (launch_route(router_logits, M, E, topk, renormalize, ids, wts, s) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpyAsync(host_ids, ids, (size_t)P * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return MOE_ERR_HIP;
    std::vector<int32_t> need(host_ids, host_ids + P);
    for (int32_t e : need)
        if (e < 0 || e >= E) return MOE_ERR_HIP;  // not a routing result (the route kernel writes [0, E))
    std::sort(need.begin(), need.end());
    need.erase(std::unique(need.begin(), need.end()), need.end());
    if ((int32_t)need.size() > C) return MOE_ERR_UNSUPPORTED;  // more experts than slots in one batch
    st = make_resident(c, need, true, nullptr);
    if (st != MOE_OK) return st;
    // the GEMMs wait for the newest copy batch that filled a slot they read
    int64_t after_batch = -1;
    for (int32_t e : need) after_batch = std::max(after_batch, c->slot_batch[c->slot_of[e]]);
    if (after_batch >= 0 && hipStreamWaitEvent(s, c->copy_ev[after_batch % kRing], 0) != hipSuccess)
        return MOE_ERR_HIP;

    // expert ids renamed to slots; the layer runs over the C slots
    for (int64_t p = 0; p < P; ++p) host_ids[p] = c->slot_of[host_ids[p]];
    if (hipMemcpyAsync(L.remap, host_ids, (size_t)P * 4, hipMemcpyHostToDevice, s) != hipSuccess) return MOE_ERR_HIP;
    if (launch_align(L.remap, M, topk, C, L.block_m, L.cap, L.al, c->dtype == MOE_FP8_E4M3 ? L.amax : nullptr, s) !=
        hipSuccess)
        return MOE_ERR_HIP;
    st = run_experts(c->dtype, x, x_scale, c->slots.w1, c->slots.w1_scale, c->slots.w2, c->slots.w2_scale, M, C, topk,
                     H, I, out, wts, L, s);
    if (st != MOE_OK) return st;
    for (int32_t e : need) c->slot_call[c->slot_of[e]] = c->ncall;
    if (hipEventRecord(c->call_ev[c->ncall % kRing], s) != hipSuccess) return MOE_ERR_HIP;
    ++c->ncall;
    c->last_stream = s;
    return MOE_OK;
}

}  // extern "C"

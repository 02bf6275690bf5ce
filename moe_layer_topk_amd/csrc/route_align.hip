// Top-k routing and token-to-expert alignment (FusedMoE vs MegaMoE post,
// section 2 and section 3.1 steps 1-2).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// ------------------------------------------------------------------ route
//
// One wavefront per token.  Lane l holds logits l, l+64, l+128, l+192.
// topk rounds of a wave-wide argmax on (value desc, index asc); the winner
// is marked taken.  Values are compared as order-preserving 32-bit keys
// (IEEE order; -0 is mapped to +0 first, so +0 and -0 tie); the wave maximum
// of the keys comes from a DPP reduction (VALU lane moves, no LDS permute),
// and the lowest expert index holding it from ballots over the four logit
// slots in index order.  Weights are exp(l - l_max) over the chosen (or
// all) logits.

__device__ __forceinline__ unsigned order_key(float v) {
    const unsigned b = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Maximum of x over the wavefront, in every lane.  Quad swaps, half-row and
// row mirrors leave every lane of a 16-lane row with the row maximum; two row
// broadcasts carry it to lane 63.
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
    x = max(x, (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x = max(x, (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x = max(x, (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
    x = max(x, (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
    x = max(x, (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
    x = max(x, (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (unsigned)__builtin_amdgcn_readlane((int)x, 63);
}

// Routes token `t` with the calling wavefront; lane j < topk ends up holding
// slot j (returned through *sel_out / *w_out for lanes < topk).
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int topk, int renormalize,
                                            int* sel_out, float* w_out) {
    const int lane = __lane_id();
    unsigned key[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int e = lane + 64 * q;
        live[q] = e < E;
        key[q] = live[q] ? order_key(row[e]) : 0u;  // finite values have keys > 0
    }
    float lmax = 0.0f, den = 0.0f;
    float sel_v = 0.0f;
    int sel_i = 0;
    for (int j = 0; j < topk; ++j) {
        unsigned best = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (live[q]) best = max(best, key[q]);
        const unsigned kmax = wave_max_u32(best);
        // lowest index holding kmax: slots in index order, lowest lane first
        int bi = 0;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
            const uint64_t m = __ballot(live[q] && key[q] == kmax);
            if (m) bi = 64 * q + (int)__builtin_ctzll(m);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q == bi) live[q] = false;
        const float bv = key_value(kmax);
        if (j == 0) lmax = bv;
        if (lane == j) {
            sel_v = bv;
            sel_i = bi;
        }
    }
    float ex = (lane < topk) ? __expf(sel_v - lmax) : 0.0f;
    if (renormalize) {
        den = ex;
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int e = lane + 64 * q;
            if (e < E) den += __expf(row[e] - lmax);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    *sel_out = sel_i;
    *w_out = ex / den;
}

__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, int M, int E,
                                                    int topk, int renormalize,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= M) return;
    int sel;
    float w;
    route_token(logits + (size_t)t * E, E, topk, renormalize, &sel, &w);
    if (lane < topk) {
        ids[(size_t)t * topk + lane] = sel;
        weights[(size_t)t * topk + lane] = w;
    }
}

hipError_t launch_route(const float* logits, int M, int E, int topk, int renormalize, int32_t* ids,
                        float* weights, hipStream_t s) {
    if (M == 0) return hipSuccess;
    dim3 grid((M + 3) / 4);
    hipLaunchKernelGGL(route_kernel, grid, dim3(256), 0, s, logits, M, E, topk, renormalize, ids, weights);
    return hipGetLastError();
}

// ------------------------------------------------------------------ align
//
// min(ceil(P / 1024), 64) workgroups of 1024 threads, no inter-workgroup
// traffic.  Counting sort with a stable scatter; workgroup b scatters the
// pairs [b C, b C + C) (C = 1024 up to 64 K pairs):
//  1. Every workgroup histograms all P expert ids, and separately the ids
//     before its own chunk, in per-wavefront LDS counters (summed after),
//     so it knows each expert's count and how many of the expert's pairs
//     precede its chunk.  (P ids are read by every workgroup: a few KB
//     to 64 KB from L2, cheaper than a second launch.)
//  2. Padded exclusive scan over experts (one wavefront, shuffles).
//     Workgroup 0 writes the counts, offsets and the active-expert list.
//  3. Sentinels and the tile map for this workgroup's share of the rows,
//     tile experts by binary search over the offsets.
//  4. Stable scatter of the chunk: inside a wavefront, lanes with the same
//     expert are found with eight ballots (one per bit of the id) and ranked
//     by popcount below the lane; per-wavefront counts are prefix-summed
//     across the 16 wavefronts through LDS.
//  Every write position is a function of topk_ids alone.

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxE = kMaxExperts;
constexpr int kAlignMaxBlocks = 64;

__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = __lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

template <typename GetId>
__device__ __forceinline__ void align_core(GetId get_id, int P, int E, int block_m, int cap, int blk, int nblk,
                                           int chunk,
                                           int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert,
                                           int32_t* __restrict__ counts_out, int32_t* __restrict__ offsets_out,
                                           int32_t* __restrict__ active, int32_t* __restrict__ num_active) {
    __shared__ int cnt[kMaxE];
    __shared__ int before[kMaxE];
    __shared__ int off[kMaxE + 1];
    __shared__ int cursor[kMaxE];
    __shared__ int wcnt[kAlignWaves][kMaxE];
    __shared__ int wbef[kAlignWaves][kMaxE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int chunk0 = blk * chunk;
    for (int i = tid; i < kAlignWaves * kMaxE; i += kAlignThreads) {
        (&wcnt[0][0])[i] = 0;
        (&wbef[0][0])[i] = 0;
    }
    __syncthreads();
    for (int p = tid; p < P; p += kAlignThreads) {
        const int e = get_id(p);
        if ((unsigned)e < (unsigned)E) {
            atomicAdd(&wcnt[wave][e], 1);
            if (p < chunk0) atomicAdd(&wbef[wave][e], 1);
        }
    }
    __syncthreads();
    for (int e = tid; e < kMaxE; e += kAlignThreads) {
        int c = 0, b = 0;
#pragma unroll
        for (int w = 0; w < kAlignWaves; ++w) {
            c += wcnt[w][e];
            b += wbef[w][e];
        }
        cnt[e] = c;
        before[e] = b;
    }
    __syncthreads();

    if (wave == 0) {
        // lane handles experts 4*lane .. 4*lane+3
        int c[4], pc[4], act[4];
        int s = 0, a = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int e = 4 * lane + q;
            c[q] = (e < E) ? cnt[e] : 0;
            pc[q] = (c[q] + block_m - 1) / block_m * block_m;
            act[q] = c[q] > 0;
            s += pc[q];
            a += act[q];
        }
        int incl = wave_incl_scan(s);
        int aincl = wave_incl_scan(a);
        int run = incl - s, arun = aincl - a;
        int nact_total = __shfl(aincl, 63, 64);
        int amax = P < E ? P : E;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int e = 4 * lane + q;
            if (e < E) {
                off[e] = run;
                cursor[e] = run + before[e];
                if (blk == 0) {
                    offsets_out[e] = run;
                    counts_out[e] = c[q];
                    if (act[q]) active[arun] = e;
                }
            }
            run += pc[q];
            arun += act[q];
        }
        if (lane == 63) {
            off[E] = run;  // E <= 256 so 4*64 covers every expert
            if (blk == 0) {
                offsets_out[E] = run;
                *num_active = nact_total;
            }
        }
        if (blk == 0)
            for (int i = nact_total + lane; i < amax; i += 64) active[i] = -1;
    }
    __syncthreads();

    const int total = off[E];
    // sentinels and tile map for rows [r0, r1): every row that is not a real
    // row of a run gets P; tiles are block_m-aligned so each tile belongs to
    // exactly one workgroup's row range
    const int tiles = cap / block_m;
    const int r0 = (int)((long)tiles * blk / nblk) * block_m, r1 = (int)((long)tiles * (blk + 1) / nblk) * block_m;
    for (int r = r0 + tid; r < r1; r += kAlignThreads) {
        int e = -1;
        if (r < total) {
            int lo = 0, hi = E - 1;  // last e with off[e] <= r
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= r) lo = mid; else hi = mid - 1;
            }
            e = lo;
            if (r - off[e] >= cnt[e]) sorted[r] = P;
        } else {
            sorted[r] = P;
        }
        if (r % block_m == 0) tile_expert[r / block_m] = e;
    }

    // stable scatter of this workgroup's pairs, 1024 at a time; the
    // per-expert cursor carries over between sub-chunks
    const int chunk1 = min(P, chunk0 + chunk);
    for (int base = chunk0; base < chunk1; base += kAlignThreads) {
        for (int i = tid; i < kAlignWaves * kMaxE; i += kAlignThreads) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int p = base + tid;
        const int e = (p < chunk1) ? get_id(p) : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            uint64_t bb = __ballot(valid && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? bb : ~bb;
        }
        const int rank = __popcll(same & lanemask_lt());
        if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
        __syncthreads();
        if (valid) {
            int pos = cursor[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            sorted[pos] = p;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kAlignThreads) {
            int sum = 0;
            for (int w = 0; w < kAlignWaves; ++w) sum += wcnt[w][x];
            cursor[x] += sum;
        }
        __syncthreads();
    }
}

// ----------------------------------------------------- align, one workgroup
//
// Up to 1024 pairs (thread p owns pair p): the same outputs as align_core
// in four barriers and no LDS atomics.
//  1. ids to LDS (or routed here: wavefront w routes token w).
//  2. Within a wavefront, lanes holding the same expert are found with eight
//     ballots and ranked by popcount; the lowest lane records the count in
//     wcnt[wave][e].
//  3. Wavefront 0 totals each expert over the wavefronts, scans the padded
//     counts and writes counts, offsets and the active-expert list.
//  4. Pair p goes to offsets[e] + (pairs of e in earlier wavefronts) + rank.
//     Each tile's expert is found once (binary search over the offsets);
//     every row that is not a real row of its tile's expert gets sentinel P.

constexpr int kSmallMaxPairs = kAlignThreads;
constexpr int kSmallMaxTiles = kAlignThreads;  // cap/block_m <= min(E,P) + P/block_m <= 1024 (see moe_align_capacity)

template <bool ROUTE>
__global__ void __launch_bounds__(kAlignThreads) align_small_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ids_in, int M, int E, int topk, int renormalize,
    int32_t* __restrict__ ids_out, float* __restrict__ weights_out, int block_m, int cap,
    int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ active, int32_t* __restrict__ num_active,
    float* __restrict__ zero_f32) {
    __shared__ int ids_s[kSmallMaxPairs];
    __shared__ int wcnt[kAlignWaves][kMaxE];
    __shared__ int off_s[kMaxE + 1];
    __shared__ int cnt_s[kMaxE];
    __shared__ int tile_s[kSmallMaxTiles];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = M * topk;
    if (tid == 0 && zero_f32) *zero_f32 = 0.0f;
    for (int i = tid; i < kAlignWaves * kMaxE; i += kAlignThreads) (&wcnt[0][0])[i] = 0;
    if constexpr (ROUTE) {
        if (wave < M) {
            int sel;
            float w;
            route_token(logits + (size_t)wave * E, E, topk, renormalize, &sel, &w);
            if (lane < topk) {
                ids_out[(size_t)wave * topk + lane] = sel;
                weights_out[(size_t)wave * topk + lane] = w;
                ids_s[wave * topk + lane] = sel;
            }
        }
    } else {
        if (tid < P) ids_s[tid] = ids_in[tid];
    }
    __syncthreads();

    const int e = (tid < P) ? ids_s[tid] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint64_t bb = __ballot(valid && ((e >> b) & 1));
        same &= ((e >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(same & lanemask_lt());
    if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
    __syncthreads();

    if (wave == 0) {
        // lane handles experts 4*lane .. 4*lane+3
        int c[4], pc[4], act[4];
        int s = 0, a = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ex = 4 * lane + q;
            c[q] = 0;
            if (ex < E)
#pragma unroll
                for (int w = 0; w < kAlignWaves; ++w) c[q] += wcnt[w][ex];
            pc[q] = (c[q] + block_m - 1) / block_m * block_m;
            act[q] = c[q] > 0;
            s += pc[q];
            a += act[q];
        }
        const int incl = wave_incl_scan(s);
        const int aincl = wave_incl_scan(a);
        int run = incl - s, arun = aincl - a;
        const int nact_total = __shfl(aincl, 63, 64);
        const int amax = P < E ? P : E;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ex = 4 * lane + q;
            if (ex < E) {
                off_s[ex] = run;
                cnt_s[ex] = c[q];
                offsets_out[ex] = run;
                counts_out[ex] = c[q];
                if (act[q]) active[arun] = ex;
            }
            run += pc[q];
            arun += act[q];
        }
        if (lane == 63) {
            off_s[E] = run;
            offsets_out[E] = run;
            *num_active = nact_total;
        }
        for (int i = nact_total + lane; i < amax; i += 64) active[i] = -1;
    }
    __syncthreads();

    if (valid) {
        int pos = off_s[e] + rank;
        for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
        sorted[pos] = tid;
    }
    const int total = off_s[E];
    const int ntiles = cap / block_m;
    for (int t = tid; t < ntiles; t += kAlignThreads) {
        const int r = t * block_m;
        int ex = -1;
        if (r < total) {
            int lo = 0, hi = E - 1;  // last expert with off_s <= r
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off_s[mid] <= r) lo = mid; else hi = mid - 1;
            }
            ex = lo;
        }
        tile_s[t] = ex;
        tile_expert[t] = ex;
    }
    __syncthreads();
    for (int r = tid; r < cap; r += kAlignThreads) {
        const int ex = tile_s[r / block_m];
        if (ex < 0 || r - off_s[ex] >= cnt_s[ex]) sorted[r] = P;
    }
}

__global__ void __launch_bounds__(kAlignThreads) align_kernel(
    const int32_t* __restrict__ ids, int P, int E, int block_m, int cap, int32_t* __restrict__ sorted,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ active, int32_t* __restrict__ num_active,
    float* __restrict__ zero_f32, int chunk) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && zero_f32) *zero_f32 = 0.0f;
    align_core([&](int p) { return ids[p]; }, P, E, block_m, cap, blockIdx.x, gridDim.x, chunk, sorted, tile_expert,
               counts_out, offsets_out, active, num_active);
}

hipError_t launch_align(const int32_t* ids, int M, int topk, int E, int block_m, int64_t cap,
                        const moe_align_bufs& out, float* zero_f32, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int P = M * topk;
    if (P <= kSmallMaxPairs) {
        hipLaunchKernelGGL((align_small_kernel<false>), dim3(1), dim3(kAlignThreads), 0, s, nullptr, ids, M, E, topk,
                           1, nullptr, nullptr, block_m, (int)cap, out.sorted_ids, out.tile_expert,
                           out.expert_counts, out.expert_offsets, out.active_experts, out.num_active, zero_f32);
        return hipGetLastError();
    }
    // every workgroup reads all P ids, so their number is capped: past 64 K
    // pairs a workgroup scatters several 1024-pair sub-chunks
    const int units = (P + kAlignThreads - 1) / kAlignThreads;
    const int nblk = units < kAlignMaxBlocks ? units : kAlignMaxBlocks;
    const int chunk = (units + nblk - 1) / nblk * kAlignThreads;
    hipLaunchKernelGGL(align_kernel, dim3(nblk), dim3(kAlignThreads), 0, s, ids, P, E, block_m, (int)cap,
                       out.sorted_ids, out.tile_expert, out.expert_counts, out.expert_offsets, out.active_experts,
                       out.num_active, zero_f32, chunk);
    return hipGetLastError();
}

// Small batches (M <= 16): one launch for both steps.  Wavefront w routes
// token w (route_token, as route_kernel does), the ids go to LDS and to the
// outputs, and after a barrier the workgroup aligns them (align_small_kernel
// with ROUTE).  Saves a launch and the dependency gap between the two, which
// dominate at a few tokens.
constexpr int kRouteAlignMaxM = kAlignWaves;

bool route_align_fits(int M) { return M > 0 && M <= kRouteAlignMaxM; }

hipError_t launch_route_align(const float* logits, int M, int E, int topk, int renormalize, int32_t* ids,
                              float* weights, int block_m, int64_t cap, const moe_align_bufs& out,
                              float* zero_f32, hipStream_t s) {
    if (!route_align_fits(M) || M * topk > kSmallMaxPairs) return hipErrorInvalidValue;
    hipLaunchKernelGGL((align_small_kernel<true>), dim3(1), dim3(kAlignThreads), 0, s, logits, nullptr, M, E, topk,
                       renormalize, ids, weights, block_m, (int)cap, out.sorted_ids, out.tile_expert,
                       out.expert_counts, out.expert_offsets, out.active_experts, out.num_active, zero_f32);
    return hipGetLastError();
}

__global__ void fill_zero_f32_kernel(float* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

hipError_t launch_fill_zero_f32(float* p, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace moe

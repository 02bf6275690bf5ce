// Top-k routing and token-to-expert alignment (FusedMoE vs MegaMoE post,
// section 2 and section 3.1 steps 1-2).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// ------------------------------------------------------------------ route
//
// One wavefront per token (route_token, shared with the decode GEMMs that
// route a single token themselves).

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

constexpr int kAlignWavesR = 16;      // wavefronts of the one-workgroup route + align launch
constexpr int kRouteRouterMaxM = 16;  // tokens it scores with the router itself

// ----------------------------------------------------------------- router
//
// logits[t][e] = sum_h x[t][h] * wg[e][h] (FusedMoE vs MegaMoE post,
// section 2: the router scores every expert for every token), wg float32
// [E][H], x float32, bfloat16 or e4m3 times its per-tensor scale.

// Four consecutive activations x[i..i+3] as float32 (e4m3: their values
// times the scale); i is a multiple of 4 and rows are 16-byte aligned.
template <int XDT>
__device__ __forceinline__ float4 router_x4(const void* x, size_t i, float sx) {
    if constexpr (XDT == MOE_F32) {
        return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
    } else if constexpr (XDT == MOE_BF16) {
        const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + i);
        return float4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                      __uint_as_float(v.y & 0xffff0000u)};
    } else {
        // OCP e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits, no inf
        const uint32_t w = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(x) + i);
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t c = (w >> (8 * j)) & 0xffu, ef = (c >> 3) & 15, m = c & 7;
            float v;
            if (ef == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
            else if (ef == 0) v = (float)m * (1.0f / 512.0f);
            else v = __uint_as_float(((ef + 120u) << 23) | (m << 20));
            r[j] = ((c & 0x80u) ? -v : v) * sx;
        }
        return float4{r[0], r[1], r[2], r[3]};
    }
}

// The scores of a block of TT tokens x TE experts by one wavefront.  Every
// score is defined the same way wherever it is computed: lane l sums, in
// ascending h, the products at h = 256 i + 4 l + j (j = 0..3), and the 64
// lane partials are combined by a butterfly (offsets 32, 16, ..., 1; every
// lane ends with the same sum).  So the one-workgroup front end and the
// many-token kernel give the same bits.
template <int XDT, int TT, int TE, int UH = 4>
__device__ __forceinline__ void router_block(const void* __restrict__ x, float sx, const float* __restrict__ wg,
                                             int M, int E, int H, int t0, int e0, float (&acc)[TT][TE]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < TE; ++e) acc[t][e] = 0.0f;
    // rows past M (E) read the last row: every load is unconditional, so a
    // chunk's loads are all issued before its first product; those sums are
    // never stored.  Lanes past H (H an odd multiple of 128) add nothing.
    const char* xr[TT];
    const float* wr[TE];
#pragma unroll
    for (int t = 0; t < TT; ++t) xr[t] = reinterpret_cast<const char*>(x) + (size_t)min(t0 + t, M - 1) * H * (XDT == MOE_F32 ? 4 : XDT == MOE_BF16 ? 2 : 1);
#pragma unroll
    for (int e = 0; e < TE; ++e) wr[e] = wg + (size_t)min(e0 + e, E - 1) * H;
    const int nit = (H + 255) / 256;
    for (int i0 = 0; i0 < nit; i0 += UH) {
        float4 w4[UH][TE], x4[UH][TT];
#pragma unroll
        for (int u = 0; u < UH; ++u) {
            const int h = min(256 * (i0 + u) + 4 * lane, H - 4);
#pragma unroll
            for (int e = 0; e < TE; ++e) w4[u][e] = *reinterpret_cast<const float4*>(wr[e] + h);
#pragma unroll
            for (int t = 0; t < TT; ++t) x4[u][t] = router_x4<XDT>(xr[t], (size_t)h, sx);
        }
#pragma unroll
        for (int u = 0; u < UH; ++u) {
            // steps past the row (the last chunk's tail, or this lane's last
            // step when H is an odd multiple of 128) add nothing; no branch,
            // so the chunk's loads stay ahead of its products
            const bool live = 256 * (i0 + u) + 4 * lane < H;
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int e = 0; e < TE; ++e) {
                    float a = acc[t][e];
                    a = __builtin_fmaf(x4[u][t].x, w4[u][e].x, a);
                    a = __builtin_fmaf(x4[u][t].y, w4[u][e].y, a);
                    a = __builtin_fmaf(x4[u][t].z, w4[u][e].z, a);
                    a = __builtin_fmaf(x4[u][t].w, w4[u][e].w, a);
                    acc[t][e] = live ? a : acc[t][e];
                }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < TE; ++e) {
            float v = acc[t][e];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[t][e] = v;
        }
}

// One wavefront per block of TT tokens x TE experts, four per workgroup, no
// LDS and no barrier.  The block shape only spreads the work: for a few
// tokens one token and one expert per wavefront (as many wavefronts as
// scores, each a chain of H/256 steps whose loads are issued UH at a time);
// for many, 8 tokens by 1 expert while that makes fewer than 1024 blocks,
// else 8 by 4 (each row of x and of the router read a quarter as often).
template <int XDT, int TT, int TE>
__global__ void __launch_bounds__(256) router_logits_kernel(const void* __restrict__ x, const float* __restrict__ x_scale,
                                                            const float* __restrict__ wg, int M, int E, int H,
                                                            float* __restrict__ logits) {
    const int eblocks = (E + TE - 1) / TE;
    const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= ((M + TT - 1) / TT) * eblocks) return;
    const int t0 = (blk / eblocks) * TT, e0 = (blk % eblocks) * TE;
    const float sx = x_scale ? x_scale[0] : 1.0f;
    float acc[TT][TE];
    // loads in flight per chunk: all 16 steps of a 4096-wide row for one score
    router_block<XDT, TT, TE, TT == 1 ? 16 : (TE == 1 ? 4 : 2)>(x, sx, wg, M, E, H, t0, e0, acc);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < TE; ++e)
            if (lane == t * TE + e && t0 + t < M && e0 + e < E) logits[(size_t)(t0 + t) * E + e0 + e] = acc[t][e];
}

template <int XDT, int TT, int TE>
static hipError_t launch_router_tt(const void* x, const float* x_scale, const float* wg, int M, int E, int H,
                                   float* logits, hipStream_t s) {
    const long blocks = (long)((M + TT - 1) / TT) * ((E + TE - 1) / TE);
    hipLaunchKernelGGL((router_logits_kernel<XDT, TT, TE>), dim3((unsigned)((blocks + 3) / 4)), dim3(256), 0, s, x,
                       x_scale, wg, M, E, H, logits);
    return hipGetLastError();
}

template <int XDT>
static hipError_t launch_router_x(const void* x, const float* x_scale, const float* wg, int M, int E, int H,
                                  float* logits, hipStream_t s) {
    if ((long)M * E <= 4096) return launch_router_tt<XDT, 1, 1>(x, x_scale, wg, M, E, H, logits, s);
    if ((long)((M + 7) / 8) * E < 1024) return launch_router_tt<XDT, 8, 1>(x, x_scale, wg, M, E, H, logits, s);
    return launch_router_tt<XDT, 8, 4>(x, x_scale, wg, M, E, H, logits, s);
}

hipError_t launch_router_logits(moe_dtype xdt, const void* x, const float* x_scale, const float* wg, int M, int E,
                                int H, float* logits, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (xdt == MOE_F32) return launch_router_x<MOE_F32>(x, x_scale, wg, M, E, H, logits, s);
    if (xdt == MOE_BF16) return launch_router_x<MOE_BF16>(x, x_scale, wg, M, E, H, logits, s);
    return launch_router_x<MOE_FP8_E4M3>(x, x_scale, wg, M, E, H, logits, s);
}

// A few tokens, inside the one-workgroup route + align launch: the 16
// wavefronts take (4-token, 1-expert) blocks round robin (small blocks and a
// short unroll: a 1024-thread workgroup has 128 registers per lane).
template <int XDT>
__device__ __forceinline__ void router_phase(const void* __restrict__ x, const float* __restrict__ x_scale,
                                             const float* __restrict__ wg, int M, int E, int H, float* logits_s,
                                             float* __restrict__ logits_out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float sx = x_scale ? x_scale[0] : 1.0f;
    constexpr int TT = 4;
    const int blocks = ((M + TT - 1) / TT) * E;
    for (int blk = wave; blk < blocks; blk += kAlignWavesR) {
        const int t0 = (blk / E) * TT, e0 = blk % E;
        float acc[TT][1];
        router_block<XDT, TT, 1, 2>(x, sx, wg, M, E, H, t0, e0, acc);
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (lane == t && t0 + t < M) {
                logits_s[(t0 + t) * E + e0] = acc[t][0];
                if (logits_out) logits_out[(size_t)(t0 + t) * E + e0] = acc[t][0];
            }
    }
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
static_assert(kAlignWaves == kAlignWavesR, "router phase wavefronts");
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

// Router inputs of the MODE 2 launch (scores computed in the kernel).
struct RouterIn {
    const void* x;
    const float* x_scale;
    const float* wg;
    int H;
    float* logits_out;  // nullable
};

// MODE 0: ids given; 1: logits given (wavefront w routes token w); 2: router
// weights given (the workgroup scores the tokens first, router_phase).
template <int MODE, int XDT = MOE_BF16>
__global__ void __launch_bounds__(kAlignThreads) align_small_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ids_in, int M, int E, int topk, int renormalize,
    int32_t* __restrict__ ids_out, float* __restrict__ weights_out, int block_m, int cap,
    int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ active, int32_t* __restrict__ num_active,
    float* __restrict__ zero_f32, RouterIn rin) {
    __shared__ int ids_s[kSmallMaxPairs];
    __shared__ int wcnt[kAlignWaves][kMaxE];
    __shared__ int off_s[kMaxE + 1];
    __shared__ int cnt_s[kMaxE];
    __shared__ int tile_s[kSmallMaxTiles];
    __shared__ float logits_s[MODE == 2 ? kRouteRouterMaxM * kMaxE : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = M * topk;
    if (tid == 0 && zero_f32) *zero_f32 = 0.0f;
    for (int i = tid; i < kAlignWaves * kMaxE; i += kAlignThreads) (&wcnt[0][0])[i] = 0;
    if constexpr (MODE == 2) {
        router_phase<XDT>(rin.x, rin.x_scale, rin.wg, M, E, rin.H, logits_s, rin.logits_out);
        __syncthreads();
    }
    if constexpr (MODE >= 1) {
        if (wave < M) {
            int sel;
            float w;
            const float* row = (MODE == 2) ? logits_s + wave * E : logits + (size_t)wave * E;
            route_token(row, E, topk, renormalize, &sel, &w);
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
        hipLaunchKernelGGL((align_small_kernel<0>), dim3(1), dim3(kAlignThreads), 0, s, nullptr, ids, M, E, topk,
                           1, nullptr, nullptr, block_m, (int)cap, out.sorted_ids, out.tile_expert,
                           out.expert_counts, out.expert_offsets, out.active_experts, out.num_active, zero_f32,
                           RouterIn{});
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
    hipLaunchKernelGGL((align_small_kernel<1>), dim3(1), dim3(kAlignThreads), 0, s, logits, nullptr, M, E, topk,
                       renormalize, ids, weights, block_m, (int)cap, out.sorted_ids, out.tile_expert,
                       out.expert_counts, out.expert_offsets, out.active_experts, out.num_active, zero_f32,
                       RouterIn{});
    return hipGetLastError();
}

// Router + route + align in one launch: a few tokens and a router matrix
// small enough for one workgroup to stream.
bool router_route_align_fits(int M, int E, int H) {
    // the workgroup streams the router matrix once per 8-token block: at most
    // 64 K weights and 128 K multiply-adds in all
    return route_align_fits(M) && M <= kRouteRouterMaxM && (long)E * H <= 65536 && (long)M * E * H <= 131072 &&
           H % 4 == 0;
}

hipError_t launch_router_route_align(moe_dtype xdt, const void* x, const float* x_scale, const float* wg, int H,
                                     float* logits_out, int M, int E, int topk, int renormalize, int32_t* ids,
                                     float* weights, int block_m, int64_t cap, const moe_align_bufs& out,
                                     float* zero_f32, hipStream_t s) {
    if (!router_route_align_fits(M, E, H) || M * topk > kSmallMaxPairs) return hipErrorInvalidValue;
    const RouterIn rin{x, x_scale, wg, H, logits_out};
#define MOE_RRA(XDT)                                                                                              \
    hipLaunchKernelGGL((align_small_kernel<2, XDT>), dim3(1), dim3(kAlignThreads), 0, s, nullptr, nullptr, M, E,   \
                       topk, renormalize, ids, weights, block_m, (int)cap, out.sorted_ids, out.tile_expert,         \
                       out.expert_counts, out.expert_offsets, out.active_experts, out.num_active, zero_f32, rin)
    if (xdt == MOE_F32) MOE_RRA(MOE_F32);
    else if (xdt == MOE_BF16) MOE_RRA(MOE_BF16);
    else MOE_RRA(MOE_FP8_E4M3);
#undef MOE_RRA
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

// Grouped expert GEMMs over routed rows (FusedMoE vs MegaMoE post, section
// 3.1 step 3: one kernel multiplies every expert's sorted slice by that
// expert's weights).  Two kernel families:
//
//  decode   - few rows per expert.  Weight rows sit on the MFMA row
//             operand (16 rows) and the expert's tokens on the 16-wide
//             column operand, so C^T[N,M] = B^T[N,K] A^T[K,M] (MoE kernel
//             engineering post, Eq. 2, the Swap-AB formulation).  Each
//             workgroup owns 64 weight rows of one active expert and
//             streams them from HBM exactly once per pass over the expert's
//             tokens; its four wavefronts split K and reduce through LDS.
//  prefill  - many rows per expert.  Tokens on the row operand, weights on
//             the column operand (Eq. 1), BM x 128 output tiles staged
//             through LDS, one tile of block_m sorted rows per workgroup row.
//
// The decode family has two kernels: bf16 and e4m3 operands stream through
// a wavefront-private LDS ring filled by direct-to-LDS copies of whole cache
// lines (gemm_decode_ring_kernel); f32 calls, and an e4m3 down projection
// that quantises a bf16 intermediate on load, use the register-operand
// kernel (gemm_decode_kernel).  Within one MFMA the pairing of k indices
// between the two operands is the same for A and B, so any permutation of K
// applied identically to both operands leaves the dot product unchanged; the
// loaders use that to give each lane contiguous bytes of a row.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// ------------------------------------------------------------- operands

template <int DT>
struct Opnd;

template <>
struct Opnd<MOE_BF16> {
    using chunk = uint4;  // 8 bf16
    static constexpr int kElemBytes = 2;
    __device__ static __forceinline__ f32x4 mfma(const chunk& a, const chunk& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <>
struct Opnd<MOE_F32> {
    using chunk = uint4;  // 4 float32
    static constexpr int kElemBytes = 4;
};

template <>
struct Opnd<MOE_FP8_E4M3> {
    using chunk = uint2;  // 8 e4m3
    static constexpr int kElemBytes = 1;
    __device__ static __forceinline__ f32x4 mfma(const chunk& a, const chunk& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                          __builtin_bit_cast(long, b), c, 0, 0, 0);
    }
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 16x16 tile over 128 e4m3 products per lane group: gfx950's f8f6f4 MFMA
// (4x the K of v_mfma_f32_16x16x32_fp8_fp8 per instruction, about 3x its
// throughput).  Each operand is 32 bytes per lane given as two 16-byte
// halves; the same byte positions of A and B meet in the same product, so
// any K order works as long as both operands are loaded alike.  Scale
// operands 0 select the unscaled form.
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(const uint4& a0, const uint4& a1, const uint4& b0,
                                                   const uint4& b1, f32x4 c) {
    const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Per-tensor e4m3 quantiser of the float32 intermediate: code = e4m3 of the
// IEEE float32 quotient a / s (round to nearest even, saturated at +-448),
// s = amax / 448.  The quotient is formed from r = 1/s (one IEEE division
// per thread) and two remainder corrections by fused multiply-add: with r
// correctly rounded, the first correction leaves the quotient within one
// ulp and the second returns the correctly rounded quotient (Markstein's
// theorem), provided nothing under- or overflows.  A scale below the normal
// range is brought into it by multiplying s and every a by 2^64 (exact, and
// the quotient is unchanged; s <= FLT_MAX/448 keeps r normal at the top);
// quotients small enough to lose exactness in the corrections (below
// 2^-100) quantise to zero either way.  The corrections turn a -0 quotient
// into +0, so the sign is taken from a (s > 0): a zero quotient keeps the
// sign an IEEE division gives it.  Everything here is uniform across the
// wavefront except a, so the per-value path has no branch.
struct ActQuant {
    float pre, s, r;
    __device__ __forceinline__ explicit ActQuant(float scale) {
        const bool sub = scale < 1.17549435e-38f;
        pre = sub ? 18446744073709551616.0f : 1.0f;  // 2^64
        s = scale * pre;
        r = 1.0f / s;
    }
    __device__ __forceinline__ float quot(float a0) const {
        const float a = a0 * pre;
        float q = a * r;
        float e = __builtin_fmaf(-q, s, a);
        q = __builtin_fmaf(e, r, q);
        e = __builtin_fmaf(-q, s, a);
        return __builtin_copysignf(__builtin_fmaf(e, r, q), a);
    }
    __device__ __forceinline__ float sat(float a) const { return __builtin_amdgcn_fmed3f(quot(a), -448.0f, 448.0f); }
    // 16 float32 values (four 16-byte chunks) -> 16 e4m3 codes
    __device__ __forceinline__ uint4 codes16(const uint4& v0, const uint4& v1, const uint4& v2,
                                             const uint4& v3) const {
        return uint4{pack4(v0), pack4(v1), pack4(v2), pack4(v3)};
    }
    __device__ __forceinline__ uint32_t pack4(const uint4& v) const {
        return pack_fp8x4(sat(__uint_as_float(v.x)), sat(__uint_as_float(v.y)), sat(__uint_as_float(v.z)),
                          sat(__uint_as_float(v.w)));
    }
};

__device__ __forceinline__ float act_scale_from_amax(const float* amax) {
    float a = *amax;
    return a > 0.0f ? a / 448.0f : 1.0f;
}

struct GemmArgs {
    const void* a;
    const float* a_scale;
    const void* w;
    const float* w_scale;
    const int32_t* sorted;
    const int32_t* tile_expert;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* active;
    const int32_t* num_active;
    int topk, N, K, P;
    void* c;
    float* c_amax;
    int ksplit;    // decode DOWN only: K ranges handled by blockIdx.z
    float* cpart;  // non-null: DOWN writes float32 partials [ksplit][P][N] here instead of c
    int act_q8;    // fp8 DOWN: a holds e4m3 codes already quantised with amax/448
    // one token routed by every workgroup of a decode kernel itself (the
    // alignment buffers are then not read); NULL: the alignment gives the rows
    const float* route_logits;  // [route_E] logits of the token
    int route_E, route_renorm;
    int32_t* route_ids;  // non-null: workgroup 0 writes the token's topk ids and weights
    float* route_wts;
    // e4m3 self-routing: GATE_UP writes the intermediate's amax as partial
    // maxima here (G floats per workgroup at slot * gridDim.x * G +
    // blockIdx.x * G: its maximum, then zeros), DOWN reduces amax_nparts of
    // them instead of reading a_scale
    float* amax_parts;
    int amax_nparts;
};

// The rows of active-expert slot `slot` of a decode kernel: the expert, its
// pair-row count and where their pair ids start in `sorted`.  With
// self-routing (one token) every wavefront routes the token as the route
// kernel does; the slot's expert is the slot-th smallest of the selected
// (distinct) ids and its one pair id the slot j it was selected in, and
// workgroup 0 writes the token's ids and weights.  False for a slot past the
// active experts.
struct SlotRows {
    int e, cnt, base, p1;
};
__device__ __forceinline__ bool slot_rows(const GemmArgs& g, int slot, SlotRows& r) {
    if (g.route_logits) {
        int sel;
        float w;
        route_token(g.route_logits, g.route_E, g.topk, g.route_renorm, &sel, &w);
        const int lane = __lane_id();
        int rank = 0;
        for (int i = 0; i < g.topk; ++i) rank += (__shfl(sel, i, 64) < sel) ? 1 : 0;
        const uint64_t m = __ballot(lane < g.topk && rank == slot);
        if (m == 0) return false;
        const int j = (int)__builtin_ctzll(m);
        r.e = __builtin_amdgcn_readfirstlane(__shfl(sel, j, 64));
        r.cnt = 1;
        r.base = 0;
        r.p1 = j;  // pair id t * topk + j of token 0
        if (g.route_ids && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && (int)threadIdx.x < g.topk) {
            g.route_ids[threadIdx.x] = sel;
            g.route_wts[threadIdx.x] = w;
        }
        return true;
    }
    if (slot >= *g.num_active) return false;
    r.e = g.active[slot];
    r.cnt = g.counts[r.e];
    r.base = g.offsets[r.e];
    r.p1 = 0;
    return true;
}

__device__ __forceinline__ void amax_publish(float m, float* dst) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (__lane_id() == 0 && m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(m));
}

// The workgroup's maximum of m (four wavefronts) into dst[0] and zeros into
// dst[1..n): plain stores, so the partials need no clearing between calls.
// lds: four floats no wavefront reads or writes any more (every wavefront of
// the workgroup calls this).
__device__ __forceinline__ void amax_parts_publish(float m, float* dst, int n, float* lds) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const int wave = threadIdx.x >> 6;
    if (__lane_id() == 0) lds[wave] = m;
    __syncthreads();
    if ((int)threadIdx.x < n) dst[threadIdx.x] = threadIdx.x == 0 ? fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3])) : 0.0f;
}

// The intermediate's e4m3 scale amax/448 from n partial maxima (every
// thread of the workgroup calls this; lds: four floats, free until the
// closing barrier).
__device__ __forceinline__ float act_scale_from_parts(const float* parts, int n, float* lds) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, parts[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (__lane_id() == 0) lds[threadIdx.x >> 6] = m;
    __syncthreads();
    const float a = fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
    __syncthreads();
    return a > 0.0f ? a / 448.0f : 1.0f;
}

// ----------------------------------------------------------------- decode
//
// Work split: blockIdx.y is an active-expert slot, blockIdx.x a block of
// weight rows of that expert (G groups of four 16-row tiles; for GATE_UP a
// group is 16+16 gate rows and the matching 16+16 up rows).  A step is 256
// bytes of every row of one group; the four wavefronts take steps
// round-robin along K and reduce their partial sums through LDS at the end.
// Each lane issues 16-byte loads at byte 64u + 16g of the step span (g = lane
// group, u = 0..3), so one load instruction reads 64 contiguous bytes of each
// of 16 rows; the K order this induces is applied to the token operand too.
// The next step's loads are issued before the current step's MFMAs
// (register double buffer, pinned by scheduling barriers) so a wavefront
// always has a full step of weights in flight.

constexpr int kDecThreads = 256;
constexpr int kDecSpan = 256;  // bytes of each row per step

// AQ: the DOWN operand is already e4m3 (quantised once by quant_act_kernel);
// otherwise an e4m3 DOWN reads the float32 intermediate and quantises it on load
template <int KIND, int DT, bool AQ>
struct DecodeTokens {
    static constexpr bool kF32Act = KIND == MOE_GEMM_DOWN && DT == MOE_FP8_E4M3 && !AQ;
    // one 16-byte MFMA operand chunk of the token rows for load u of a step
    __device__ static __forceinline__ uint4 load(const char* brow, size_t step_off, int u, const ActQuant& q) {
        if constexpr (kF32Act) {
            // act is float32: 16 elements = 64 bytes, quantised on load
            const uint4* p = reinterpret_cast<const uint4*>(brow + 4 * (step_off + u * 64));
            return q.codes16(p[0], p[1], p[2], p[3]);
        } else {
            return *reinterpret_cast<const uint4*>(brow + step_off + u * 64);
        }
    }
};

template <int DT>
__device__ __forceinline__ f32x4 mfma_chunk(const uint4& a, const uint4& b, f32x4 c) {
    if constexpr (DT == MOE_BF16) {
        return Opnd<MOE_BF16>::mfma(a, b, c);
    } else if constexpr (DT == MOE_F32) {
        // 16x16x4 f32: one float per lane and operand; float i of the lane's
        // chunk goes to the i-th MFMA for A and B alike
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    } else {
        c = Opnd<MOE_FP8_E4M3>::mfma(uint2{a.x, a.y}, uint2{b.x, b.y}, c);
        return Opnd<MOE_FP8_E4M3>::mfma(uint2{a.z, a.w}, uint2{b.z, b.w}, c);
    }
}

template <int KIND, int DT, int NT, int G, bool AQ>
__global__ void __launch_bounds__(kDecThreads) gemm_decode_kernel(GemmArgs g) {
    using Tok = DecodeTokens<KIND, DT, AQ>;
    constexpr int kElem = Opnd<DT>::kElemBytes;
    constexpr int T = 4;  // 16-row tiles per group

    const int slot = blockIdx.y;
    if (slot >= *g.num_active) return;
    const int e = g.active[slot];
    const int cnt = g.counts[e];
    const int base = g.offsets[e];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15;  // row within a tile / token column
    const int lg = lane >> 4;  // lane group
    const int K = g.K, N = g.N;
    const int I = N / 2;
    const size_t rowb = (size_t)K * kElem;
    const int nks_all = (int)(rowb / kDecSpan);  // steps along K per group
    // split-K: this workgroup covers steps [ks0, ks0 + nks) of every group
    const int ks0 = (int)((long)blockIdx.z * nks_all / g.ksplit);
    const int nks = (int)((long)(blockIdx.z + 1) * nks_all / g.ksplit) - ks0;
    const int total = G * nks;

    const int n0 = (KIND == MOE_GEMM_GATE_UP_SILU) ? blockIdx.x * 32 * G : blockIdx.x * 64 * G;
    const char* wbase = reinterpret_cast<const char*>(g.w) + (size_t)e * N * rowb + lg * 16;
    // byte offset of this lane's row of tile t in group 0 (groups add gstride rows)
    size_t arow[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        int row;
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU)
            row = (t < 2) ? n0 + 16 * t + lr : I + n0 + 16 * (t - 2) + lr;
        else
            row = n0 + 16 * t + lr;
        arow[t] = (size_t)row * rowb;
    }
    const size_t gstride = (size_t)((KIND == MOE_GEMM_GATE_UP_SILU) ? 32 : 64) * rowb;

    float scale = 1.0f, qs = 1.0f;
    if constexpr (DT == MOE_FP8_E4M3) {
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
            scale = g.a_scale[0] * g.w_scale[e];
        } else {
            qs = act_scale_from_amax(g.a_scale);
            scale = qs * g.w_scale[e];
        }
    }
    const ActQuant quant(qs);
    // token-row byte stride and the lane's offset inside a step
    const size_t brow_bytes = Tok::kF32Act ? (size_t)K * 4 : rowb;
    const int blane = lg * 16;  // in operand bytes (float32 act: in elements, scaled x4 inside the loader)

    extern __shared__ f32x4 red[];  // [4 waves][G*T tiles][NT][64 lanes]
    float amax = 0.0f;

    for (int pass = 0; pass < cnt; pass += NT * 16) {
        const int ntiles = min(NT, (cnt - pass + 15) / 16);
        const char* brow[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int r = min(pass + c * 16 + lr, cnt - 1);
            const int p = g.sorted[base + r];
            const int src = (KIND == MOE_GEMM_GATE_UP_SILU) ? p / g.topk : p;
            brow[c] = reinterpret_cast<const char*>(g.a) + (size_t)src * brow_bytes +
                      (Tok::kF32Act ? 4 * blane : blane);
        }

        f32x4 acc[G][T][NT];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < NT; ++c) acc[gi][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 a0[T][4], b0[NT][4], a1[T][4], b1[NT][4];
        auto load = [&](uint4 (&a)[T][4], uint4 (&b)[NT][4], int s) {
            const int gi = s / nks, ks = ks0 + s % nks;
            const char* wg = wbase + gi * gstride + (size_t)ks * kDecSpan;
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u) a[t][u] = *reinterpret_cast<const uint4*>(wg + arow[t] + u * 64);
            const size_t soff = (size_t)ks * kDecSpan;
#pragma unroll
            for (int c = 0; c < NT; ++c)
                if (c < ntiles)
#pragma unroll
                    for (int u = 0; u < 4; ++u) b[c][u] = Tok::load(brow[c], soff, u, quant);
        };

        int s = wave;
        if (s < total) load(a0, b0, s);
        for (; s < total; s += 4) {
            const bool nx = s + 4 < total;
            if (nx) load(a1, b1, s + 4);
            __builtin_amdgcn_sched_barrier(0);
            const int gi = s / nks;
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                if (gg != gi) continue;
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    if (c < ntiles) {
                        if constexpr (DT == MOE_FP8_E4M3) {
                            // a step's 256 bytes per row: two f8f6f4 MFMAs
#pragma unroll
                            for (int h = 0; h < 2; ++h)
#pragma unroll
                                for (int t = 0; t < T; ++t)
                                    acc[gg][t][c] = mfma_f8_16x16x128(a0[t][2 * h], a0[t][2 * h + 1], b0[c][2 * h],
                                                                      b0[c][2 * h + 1], acc[gg][t][c]);
                        } else {
#pragma unroll
                            for (int u = 0; u < 4; ++u)
#pragma unroll
                                for (int t = 0; t < T; ++t)
                                    acc[gg][t][c] = mfma_chunk<DT>(a0[t][u], b0[c][u], acc[gg][t][c]);
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (nx) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int u = 0; u < 4; ++u) a0[t][u] = a1[t][u];
#pragma unroll
                for (int c = 0; c < NT; ++c)
#pragma unroll
                    for (int u = 0; u < 4; ++u) b0[c][u] = b1[c][u];
            }
        }

        // K-split reduction across the four wavefronts
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < NT; ++c) red[((wave * G * T + gi * T + t) * NT + c) * 64 + lane] = acc[gi][t][c];
        __syncthreads();

        constexpr int kPer = (KIND == MOE_GEMM_GATE_UP_SILU) ? 2 : 4;  // output tiles per group
        const int units = G * kPer * ntiles;
        for (int u = wave; u < units; u += 4) {
            const int c = u / (G * kPer);
            const int gq = u % (G * kPer);
            const int gi = gq / kPer, q = gq % kPer;
            const int r = pass + c * 16 + lr;
            if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
                f32x4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    gs += red[((w * G * T + gi * T + q) * NT + c) * 64 + lane];
                    us += red[((w * G * T + gi * T + q + 2) * NT + c) * 64 + lane];
                }
                if (r < cnt && DT == MOE_F32) {
                    const int p = g.sorted[base + r];
                    f32x4 o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = silu(gs[v]) * us[v];
                    const int n = n0 + gi * 32 + 16 * q + 4 * lg;
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.c) + (size_t)p * I + n) = o;
                } else if (r < cnt && DT == MOE_FP8_E4M3) {
                    // the e4m3 layer keeps its intermediate in float32 until it is quantised
                    const int p = g.sorted[base + r];
                    f32x4 o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        o[v] = silu(gs[v] * scale) * (us[v] * scale);
                        amax = fmaxf(amax, fabsf(o[v]));
                    }
                    const int n = n0 + gi * 32 + 16 * q + 4 * lg;
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.c) + (size_t)p * I + n) = o;
                } else if (r < cnt) {
                    const int p = g.sorted[base + r];
                    float o[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = silu(gs[v] * scale) * (us[v] * scale);
                    uint2 pk;
                    pk.x = pack_bf2(o[0], o[1]);
                    pk.y = pack_bf2(o[2], o[3]);
                    const int n = n0 + gi * 32 + 16 * q + 4 * lg;
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.c) + (size_t)p * I + n) = pk;
                }
            } else {
                f32x4 ys = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) ys += red[((w * G * T + gi * T + q) * NT + c) * 64 + lane];
                if (r < cnt && DT == MOE_F32) {
                    const int p = g.sorted[base + r];
                    const int n = n0 + gi * 64 + 16 * q + 4 * lg;
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.c) + (size_t)p * N + n) = ys;
                } else if (r < cnt && g.cpart) {
                    const int p = g.sorted[base + r];
                    const int n = n0 + gi * 64 + 16 * q + 4 * lg;
                    *reinterpret_cast<f32x4*>(g.cpart + ((size_t)blockIdx.z * g.P + p) * N + n) = ys * scale;
                } else if (r < cnt) {
                    const int p = g.sorted[base + r];
                    const int n = n0 + gi * 64 + 16 * q + 4 * lg;
                    uint2 pk;
                    pk.x = pack_bf2(ys[0] * scale, ys[1] * scale);
                    pk.y = pack_bf2(ys[2] * scale, ys[3] * scale);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.c) + (size_t)p * N + n) = pk;
                }
            }
        }
        __syncthreads();
    }
    if constexpr (DT == MOE_FP8_E4M3 && KIND == MOE_GEMM_GATE_UP_SILU) amax_publish(amax, g.c_amax);
}

// ---------------------------------------------------------------- prefill

constexpr int kPreThreads = 256;
constexpr int kPreBN = 128;  // weight rows per workgroup
constexpr int kPreBK = 64;   // K elements per stage (bf16; e4m3 stages 128 elements, the same bytes)

template <int KIND, int DT, int BM>
__global__ void __launch_bounds__(kPreThreads) gemm_prefill_kernel(GemmArgs g) {
    using O = Opnd<DT>;
    using chunk = typename O::chunk;
    constexpr int kElem = O::kElemBytes;
    constexpr int kBK = (DT == MOE_FP8_E4M3) ? 2 * kPreBK : kPreBK;  // K elements per stage
    constexpr int kRowBytes = kBK * kElem;           // bytes of one staged row
    constexpr int kLdsStride = kRowBytes + 16;       // padded LDS row
    constexpr int kChunksPerRow = kRowBytes / 16;    // 16-byte global chunks per row
    constexpr int kAChunks = BM * kChunksPerRow / kPreThreads;
    constexpr int kBChunks = kPreBN * kChunksPerRow / kPreThreads;
    constexpr int kWM = BM / 2;       // rows per wavefront
    constexpr int kTM = kWM / 16;     // 16-row tiles per wavefront

    const int tile = blockIdx.y;
    const int e = g.tile_expert[tile];
    if (e < 0) return;

    __shared__ __attribute__((aligned(16))) char As[BM * kLdsStride];
    __shared__ __attribute__((aligned(16))) char Bs[kPreBN * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    const int K = g.K, N = g.N, I = N / 2;
    const int P = g.P;

    float qs = 1.0f, scale = 1.0f;
    if constexpr (DT == MOE_FP8_E4M3) {
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
            scale = g.a_scale[0] * g.w_scale[e];
        } else {
            qs = act_scale_from_amax(g.a_scale);
            scale = qs * g.w_scale[e];
        }
    }

    // global sources of the chunks this thread stages
    const int n0 = (KIND == MOE_GEMM_GATE_UP_SILU) ? blockIdx.x * 64 : blockIdx.x * 128;
    const char* asrc[kAChunks];
    const char* bsrc[kBChunks];
    int adst[kAChunks], bdst[kBChunks];
    // an e4m3 DOWN reads the float32 intermediate and quantises it on load
    const bool a_is_f32_act = (KIND == MOE_GEMM_DOWN && DT == MOE_FP8_E4M3) && !g.act_q8;
    const ActQuant quant(qs);
#pragma unroll
    for (int q = 0; q < kAChunks; ++q) {
        int id = tid + q * kPreThreads;
        int r = id / kChunksPerRow, cc = id % kChunksPerRow;
        int p = g.sorted[tile * BM + r];
        adst[q] = r * kLdsStride + cc * 16;
        if (p >= P) {
            asrc[q] = nullptr;
        } else if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
            asrc[q] = reinterpret_cast<const char*>(g.a) + (size_t)(p / g.topk) * K * kElem + cc * 16;
        } else if (a_is_f32_act) {
            asrc[q] = reinterpret_cast<const char*>(g.a) + (size_t)p * K * 4 + cc * 64;
        } else {
            asrc[q] = reinterpret_cast<const char*>(g.a) + (size_t)p * K * kElem + cc * 16;
        }
    }
    const char* wbase = reinterpret_cast<const char*>(g.w) + (size_t)e * N * K * kElem;
#pragma unroll
    for (int q = 0; q < kBChunks; ++q) {
        int id = tid + q * kPreThreads;
        int j = id / kChunksPerRow, cc = id % kChunksPerRow;
        int row = (KIND == MOE_GEMM_GATE_UP_SILU) ? ((j < 64) ? n0 + j : I + n0 + j - 64) : n0 + j;
        bsrc[q] = wbase + (size_t)row * K * kElem + cc * 16;
        bdst[q] = j * kLdsStride + cc * 16;
    }

    uint4 ra[kAChunks], rb[kBChunks];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < kAChunks; ++q) {
            if (!asrc[q]) {
                ra[q] = uint4{0, 0, 0, 0};
            } else if (a_is_f32_act) {
                const uint4* s = reinterpret_cast<const uint4*>(asrc[q] + (size_t)k0 * 4);
                ra[q] = quant.codes16(s[0], s[1], s[2], s[3]);
            } else {
                ra[q] = *reinterpret_cast<const uint4*>(asrc[q] + (size_t)k0 * kElem);
            }
        }
#pragma unroll
        for (int q = 0; q < kBChunks; ++q) rb[q] = *reinterpret_cast<const uint4*>(bsrc[q] + (size_t)k0 * kElem);
    };
    auto sstore = [&]() {
#pragma unroll
        for (int q = 0; q < kAChunks; ++q) *reinterpret_cast<uint4*>(As + adst[q]) = ra[q];
#pragma unroll
        for (int q = 0; q < kBChunks; ++q) *reinterpret_cast<uint4*>(Bs + bdst[q]) = rb[q];
    };

    f32x4 acc[kTM][4];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS rows of this wavefront's column tiles
    int bcol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU)
            bcol[j] = (j < 2) ? wn * 32 + 16 * j : 64 + wn * 32 + 16 * (j - 2);
        else
            bcol[j] = wn * 64 + 16 * j;
    }

    const int nk = K / kBK;
    gload(0);
    sstore();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload((kt + 1) * kBK);
        if constexpr (DT == MOE_FP8_E4M3) {
            // the stage's 128 bytes per row: lane group lg takes bytes [32 lg, 32 lg + 32)
            const int koff = lg * 32;
            uint4 af[kTM][2], bf[4][2];
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    af[i][hh] = *reinterpret_cast<const uint4*>(As + (wm * kWM + 16 * i + lr) * kLdsStride + koff +
                                                                16 * hh);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    bf[j][hh] = *reinterpret_cast<const uint4*>(Bs + (bcol[j] + lr) * kLdsStride + koff + 16 * hh);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma_f8_16x16x128(af[i][0], af[i][1], bf[j][0], bf[j][1], acc[i][j]);
        } else {
#pragma unroll
            for (int ks = 0; ks < kBK / 32; ++ks) {
                const int koff = (ks * 32 + lg * 8) * kElem;
                chunk af[kTM], bf[4];
#pragma unroll
                for (int i = 0; i < kTM; ++i)
                    af[i] = *reinterpret_cast<const chunk*>(As + (wm * kWM + 16 * i + lr) * kLdsStride + koff);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bf[j] = *reinterpret_cast<const chunk*>(Bs + (bcol[j] + lr) * kLdsStride + koff);
#pragma unroll
                for (int i = 0; i < kTM; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = O::mfma(af[i], bf[j], acc[i][j]);
            }
        }
        __syncthreads();
        if (kt + 1 < nk) {
            sstore();
            __syncthreads();
        }
    }

    // epilogue: lane holds C[token row 4*lg+v][weight col lr] of each tile
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = wm * kWM + 16 * i + 4 * lg + v;
            const int p = g.sorted[tile * BM + r];
            if (p >= P) continue;
            if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float gv = acc[i][j][v] * scale, uv = acc[i][j + 2][v] * scale;
                    const float o = silu(gv) * uv;
                    const int n = n0 + wn * 32 + 16 * j + lr;
                    if constexpr (DT == MOE_FP8_E4M3) {
                        // float32 intermediate until it is quantised
                        amax = fmaxf(amax, fabsf(o));
                        reinterpret_cast<float*>(g.c)[(size_t)p * I + n] = o;
                    } else {
                        reinterpret_cast<uint16_t*>(g.c)[(size_t)p * I + n] = f2bf(o);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 64 + 16 * j + lr;
                    reinterpret_cast<uint16_t*>(g.c)[(size_t)p * N + n] = f2bf(acc[i][j][v] * scale);
                }
            }
        }
    }
    if constexpr (DT == MOE_FP8_E4M3 && KIND == MOE_GEMM_GATE_UP_SILU) amax_publish(amax, g.c_amax);
}

// ------------------------------------------------------- prefill (bf16)
//
// Many rows per expert.  Block tile BM sorted rows x BN weight rows x BK, four
// wavefronts in a 2x2 grid, each computing (BM/2) x (BN/2) with
// v_mfma_f32_32x32x16_bf16 (tokens on the row operand, weights on the
// column operand: Eq. 1).  Operands reach LDS with direct-to-LDS 16-byte
// loads (no register staging) into an ST-stage ring, so ST-1 K stages are in
// flight while one is multiplied; one barrier per stage.  The 16-byte chunks
// of each LDS row are XOR-swizzled so that the fragment reads of 16
// consecutive rows at one logical chunk fall into distinct bank groups of
// the 64 x 4-byte banks; the swizzle is applied by the choice of each lane's
// source chunk.  Tile order: a flat index over (weight-tile group, row tile,
// weight tile in group), cut into eight contiguous ranges, one per XCD
// (workgroups are dealt to XCDs round robin), so the row tiles sharing a
// weight tile run on one XCD, the weight tile is fetched from HBM once into
// that XCD's L2, and each token tile is reused by the group's weight tiles.

constexpr int kP2Xcds = 8;

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: the wave's 64
// lanes fill 1 KB at the wave-uniform LDS byte address in M0 (a 32-bit LDS
// address, so a ring's stage addresses are plain scalar adds).  Issued
// through inline asm so the compiler does not treat every later LDS read as
// dependent on the copy (it would wait for all copies in flight, prefetched
// stages included); the kernels order their rings themselves with explicit
// vmcnt waits and barriers.  "memory" keeps LDS reads and writes of the
// kernel in program order around it.
__device__ __forceinline__ void lds_dma16_at(const void* src, unsigned lds_addr) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

// The same copy with the non-temporal hint: for data read once (decode
// weights), so the stream does not displace reused lines (token rows) from
// L2; on MI355X it also streams faster (weights of the Mixtral-shaped gate/up
// projection through the decode ring: 5.83 TB/s plain, 6.59 TB/s with nt).
__device__ __forceinline__ void lds_dma16_nt_at(const void* src, unsigned lds_addr) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(m0) : "memory", "m0");
}

// Buffer-addressed copies into LDS: a raw (stride 0) buffer resource over
// [base, base + bytes) plus a 32-bit per-lane offset (VGPR) and a wave-uniform
// one (SGPR).  Reads past `bytes` return zeros instead of touching memory.
// The tile kernel's copies take this form rather than 64-bit flat addresses:
// one VGPR per source instead of two, and on MI355X it measured 1-3% faster
// for bf16 prefill (same bytes, less address work per 16-byte copy).  Callers
// keep every offset below 2^32 (the host checks the operand sizes).
typedef int v4i_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i_rsrc buf_rsrc(const void* base, unsigned bytes) {
    const unsigned long long b = (unsigned long long)base;
    v4i_rsrc r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(b & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}
__device__ __forceinline__ void lds_dma16_buf(v4i_rsrc rsrc, unsigned voff, unsigned soff, unsigned lds_addr) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    const unsigned so = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc), "s"(m0), "s"(so)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma16_buf_nt(v4i_rsrc rsrc, unsigned voff, unsigned soff, unsigned lds_addr) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    const unsigned so = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(m0), "s"(so)
                 : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr_of(const void* p) {
    return (unsigned)(uintptr_t)(const lds_void*)p;
}

// wait until at most n vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int L>
__device__ __forceinline__ void wait_vm_runtime(int stages_outstanding) {
    switch (stages_outstanding) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<L>(); break;
        case 2: wait_vm<2 * L < 64 ? 2 * L : 63>(); break;
        default: wait_vm<3 * L < 64 ? 3 * L : 63>(); break;
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int BM_, int BN_, int BK_, int ST_, int WM_ = 2, int WN_ = 2>
struct P2Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, ST = ST_;
    static constexpr int WM = WM_, WN = WN_, Waves = WM * WN, Threads = 64 * Waves;
    static constexpr int RowBytes = BK * 2;
    static constexpr int Chunks = BK / 8;                // 16-byte chunks per LDS row
    static constexpr int RowsPerLoad = 64 / Chunks;      // rows one 1 KB load instruction fills
    static constexpr int ABytes = BM * RowBytes, BBytes = BN * RowBytes;
    static constexpr int StageBytes = ABytes + BBytes;
    static constexpr int IdsOffset = ST * StageBytes;
    static constexpr int LdsBytes = IdsOffset + BM * 4;
    static constexpr int ALoads = BM / RowsPerLoad / Waves;  // per wave per stage
    static constexpr int BLoads = BN / RowsPerLoad / Waves;
    static constexpr int L = ALoads + BLoads;
    static constexpr int WTM = BM / WM, WTN = BN / WN;       // wave tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;       // 32x32 MFMA tiles per wave
    // physical chunk of logical chunk c in row r: rows in groups of 16/Chunks
    // share a bank window of 256 bytes
    __device__ static __forceinline__ int swz(int c, int r) { return c ^ ((r / (16 / Chunks)) % Chunks); }
    static_assert(ALoads * RowsPerLoad * Waves == BM && BLoads * RowsPerLoad * Waves == BN, "load split");
    static_assert(TN % 2 == 0, "gate/up pairing needs an even number of column tiles");
    static_assert(LdsBytes <= 160 * 1024, "LDS");
};

// 32x32 MFMA on one K substep of the LDS ring.  bf16: 16 K values, one
// 16-byte chunk per lane; e4m3: 64 K values, two chunks per lane, gfx950's
// f8f6f4 MFMA with its scale operands at 0 (unscaled form).
template <int DT>
struct P2Mfma {
    static constexpr int kChunks = (DT == MOE_FP8_E4M3) ? 2 : 1;  // 16-byte chunks per lane per substep
    __device__ static __forceinline__ f32x16 run(const uint4 (&a)[kChunks], const uint4 (&b)[kChunks], f32x16 c) {
        if constexpr (DT == MOE_FP8_E4M3) {
            const i32x8 av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                              (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
            const i32x8 bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                              (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
            return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[0]),
                                                           __builtin_bit_cast(bf16x8_t, b[0]), c, 0, 0, 0);
        }
    }
};

// One wavefront per SIMD (the LDS ring fills the CU): registers are not
// rationed for occupancy.  A stage holds C::RowBytes bytes of every row
// (64 bf16 or 128 e4m3 values of K).
// NTW: weight tiles are copied with the non-temporal hint (chosen at launch
// when each weight tile feeds about one row tile, so L2 reuse of the weights
// is small; measured on the e4m3 512-token layer: 5% faster, on the layers
// whose experts hold more rows, where weight tiles are reused, 7-10% slower).
template <int KIND, int DT, class C, bool NTW>
__global__ void __launch_bounds__(C::Threads) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_prefill2_kernel(GemmArgs g, int m_tiles, int n_tiles, int group_n) {
    using Mf = P2Mfma<DT>;
    constexpr int kElem = (DT == MOE_FP8_E4M3) ? 1 : 2;
    constexpr int kKStage = C::RowBytes / kElem;            // K values per stage
    constexpr int kSub = C::RowBytes / (16 * Mf::kChunks * 2);  // MFMA K substeps per stage
    extern __shared__ __attribute__((aligned(1024))) char p2_lds[];
    const int nb = m_tiles * n_tiles;
    const int per = (nb + kP2Xcds - 1) / kP2Xcds;
    const int t = (blockIdx.x % kP2Xcds) * per + blockIdx.x / kP2Xcds;
    if (t >= nb) return;
    // flat order: groups of group_n weight tiles; inside a group the row
    // tiles advance slowest, so the blocks an XCD runs together cover a few
    // row tiles x a few weight tiles and both operands are reused from L2
    const int ng = t / (group_n * m_tiles);
    const int gw = min(group_n, n_tiles - ng * group_n);
    const int rem = t - ng * group_n * m_tiles;
    const int mtile = rem / gw, ntile = ng * group_n + rem % gw;
    const int e = g.tile_expert[mtile];
    if (e < 0) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to M0
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int K = g.K, N = g.N, I = N / 2, P = g.P;
    const size_t rowb = (size_t)K * kElem;
    int* ids_s = reinterpret_cast<int*>(p2_lds + C::IdsOffset);
    for (int i = tid; i < C::BM; i += C::Threads) ids_s[i] = g.sorted[mtile * C::BM + i];

    // ---- per-lane sources of this wave's load instructions.  Lane l fills
    // physical chunk l % Chunks of row l / Chunks of the instruction's rows,
    // so it loads the logical chunk the swizzle (an involution in c) maps there.
    const int lrow = lane / C::Chunks, lphys = lane % C::Chunks;
    unsigned asrc[C::ALoads];
#pragma unroll
    for (int j = 0; j < C::ALoads; ++j) {
        const int r = (wave * C::ALoads + j) * C::RowsPerLoad + lrow;
        int p = g.sorted[mtile * C::BM + r];
        if (p >= P) p = g.sorted[mtile * C::BM];  // padding row: any valid row (its output is dropped)
        const int src = (KIND == MOE_GEMM_GATE_UP_SILU) ? p / g.topk : p;
        asrc[j] = (unsigned)((size_t)src * rowb + C::swz(lphys, r) * 16);
    }
    // A: the tokens (GATE_UP, P / topk rows) or the intermediate (DOWN, P rows)
    const size_t arows = (KIND == MOE_GEMM_GATE_UP_SILU) ? (size_t)(P / g.topk) : (size_t)P;
    const v4i_rsrc arsrc = buf_rsrc(g.a, (unsigned)(arows * rowb));
    const char* wbase = reinterpret_cast<const char*>(g.w) + (size_t)e * N * rowb;
    const v4i_rsrc brsrc = buf_rsrc(wbase, (unsigned)((size_t)N * rowb));  // this expert's N weight rows
    const int n0 = (KIND == MOE_GEMM_GATE_UP_SILU) ? ntile * (C::BN / 2) : ntile * C::BN;
    unsigned bsrc[C::BLoads];
#pragma unroll
    for (int j = 0; j < C::BLoads; ++j) {
        const int r = (wave * C::BLoads + j) * C::RowsPerLoad + lrow;  // B row in the tile
        int row;
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU)
            row = (r < C::BN / 2) ? n0 + r : I + n0 + (r - C::BN / 2);
        else
            row = n0 + r;
        bsrc[j] = (unsigned)((size_t)row * rowb + C::swz(lphys, r) * 16);
    }

    // copy instructions [j0, j1) of stage kt (A rows first, then B rows)
    const unsigned lds0 = lds_addr_of(p2_lds);
    auto issue_part = [&](int kt, int j0, int j1) {
        const unsigned st = lds0 + (unsigned)((kt % C::ST) * C::StageBytes);
        const size_t koff = (size_t)kt * C::RowBytes;
#pragma unroll
        for (int j = 0; j < C::L; ++j) {
            if (j < j0 || j >= j1) continue;
            if (j < C::ALoads)
                lds_dma16_buf(arsrc, asrc[j], (unsigned)koff, st + (wave * C::ALoads + j) * C::RowsPerLoad * C::RowBytes);
            else if constexpr (NTW)
                lds_dma16_buf_nt(brsrc, bsrc[j - C::ALoads], (unsigned)koff,
                                 st + C::ABytes + (wave * C::BLoads + (j - C::ALoads)) * C::RowsPerLoad * C::RowBytes);
            else
                lds_dma16_buf(brsrc, bsrc[j - C::ALoads], (unsigned)koff,
                              st + C::ABytes + (wave * C::BLoads + (j - C::ALoads)) * C::RowsPerLoad * C::RowBytes);
        }
    };
    auto issue = [&](int kt) { issue_part(kt, 0, C::L); };

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // fragment rows (LDS row index) of this wave
    int arow[C::TM], brow[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) arow[i] = wm * C::WTM + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        // GATE_UP: a wave's columns are WTN/2 gate rows and the matching up rows
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU)
            brow[j] = (j < C::TN / 2) ? wn * (C::WTN / 2) + 32 * j + (lane & 31)
                                      : C::BN / 2 + wn * (C::WTN / 2) + 32 * (j - C::TN / 2) + (lane & 31);
        else
            brow[j] = wn * C::WTN + 32 * j + (lane & 31);
    }
    const int khalf = lane >> 5;  // which half of a K substep this lane holds
    // the tile's real rows are a prefix (an expert's last tile is padded):
    // 32-row MFMA tiles past them are skipped, fragment reads included.  The
    // copies still stream the whole weight tile, which is what a mostly empty
    // tile waits on: measured 1.4% on the e4m3 layer at 512 tokens (half of
    // each tile padding), neutral on the 128-expert layer at 2048 tokens
    const int nreal = min(C::BM, g.offsets[e] + g.counts[e] - mtile * C::BM);
    const int live_tm = __builtin_amdgcn_readfirstlane(min(C::TM, max(0, (nreal - wm * C::WTM + 31) / 32)));

    float scale = 1.0f;
    if constexpr (DT == MOE_FP8_E4M3) {
        // per-tensor scales: x (GATE_UP) or the intermediate's amax/448 (DOWN)
        scale = ((KIND == MOE_GEMM_GATE_UP_SILU) ? g.a_scale[0] : act_scale_from_amax(g.a_scale)) * g.w_scale[e];
    }

    const int nk = K / kKStage;
#pragma unroll
    for (int s0 = 0; s0 < C::ST - 1; ++s0)
        if (s0 < nk) issue(s0);
    // one stage; PF: the copies of stage kt + ST - 1 are issued during it (every
    // stage but the last ST - 1, which run as a separate tail so that the main
    // loop carries no per-copy condition)
    auto stage = [&](int kt, auto pf_tag, auto lt_tag) {
        constexpr bool pf = decltype(pf_tag)::value;
        constexpr int LT = decltype(lt_tag)::value;  // live 32-row MFMA tiles of this wave
        if constexpr (pf) {
            wait_vm<(C::ST - 2) * C::L < 64 ? (C::ST - 2) * C::L : 63>();  // stage kt landed; ST - 2 later ones in flight
        } else {
            wait_vm_runtime<C::L>(min(C::ST - 2, nk - 1 - kt));
        }
        __syncthreads();
        // the copies of stage kt + ST - 1 (into the buffer every wave finished
        // reading before this barrier) are spread over the K substeps, between
        // MFMA groups, so the wave never stalls on a burst of copies while its
        // matrix core idles
        const char* st = p2_lds + (kt % C::ST) * C::StageBytes;
        const char* sa = st;
        const char* sb = st + C::ABytes;
        // fragments double buffered across the K substeps: the reads for
        // substep ks+1 are interleaved with the MFMAs of substep ks.  A lane
        // takes logical chunks (ks * 2 + khalf) * kChunks + h of its row; the
        // same chunks of A and B rows meet in the same products
        uint4 af[2][C::TM][Mf::kChunks], bfr[2][C::TN][Mf::kChunks];
        auto read_frags = [&](int buf, int ks) {
#pragma unroll
            for (int h = 0; h < Mf::kChunks; ++h) {
                const int c = (ks * 2 + khalf) * Mf::kChunks + h;  // logical 16-byte chunk
#pragma unroll
                for (int i = 0; i < LT; ++i)
                    af[buf][i][h] = *reinterpret_cast<const uint4*>(sa + arow[i] * C::RowBytes + (C::swz(c, arow[i]) << 4));
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    bfr[buf][j][h] = *reinterpret_cast<const uint4*>(sb + brow[j] * C::RowBytes + (C::swz(c, brow[j]) << 4));
            }
        };
        read_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < kSub; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < kSub) read_frags(cur ^ 1, ks + 1);
            // this substep's share of the copies, one after every kGap MFMAs:
            // a copy is issued while the matrix core works on the MFMA before it
            constexpr int kPer = (C::L + kSub - 1) / kSub;
            constexpr int kGap = (C::TM * C::TN) / kPer > 0 ? (C::TM * C::TN) / kPer : 1;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < C::TM * C::TN; ++q) {
                const int i = q / C::TN, j = q % C::TN;
                if (i < LT) acc[i][j] = Mf::run(af[cur][i], bfr[cur][j], acc[i][j]);
                if ((q + 1) % kGap == 0) {
                    const int jj = ks * kPer + (q + 1) / kGap - 1;
                    if (pf && (q + 1) / kGap <= kPer && jj < C::L) {
                        __builtin_amdgcn_sched_barrier(0);
                        issue_part(kt + C::ST - 1, jj, jj + 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            // a substep with fewer MFMAs than copies issues the rest here
            constexpr int kInLoop = (C::TM * C::TN) / kGap < kPer ? (C::TM * C::TN) / kGap : kPer;
            if (pf && kInLoop < kPer) {
                __builtin_amdgcn_sched_barrier(0);
                issue_part(kt + C::ST - 1, ks * kPer + kInLoop, min(C::L, (ks + 1) * kPer));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nmain = nk - (C::ST - 1) > 0 ? nk - (C::ST - 1) : 0;
    auto kloop = [&](auto lt_tag) {
        for (int kt = 0; kt < nmain; ++kt) stage(kt, std::true_type{}, lt_tag);
        for (int kt = nmain; kt < nk; ++kt) stage(kt, std::false_type{}, lt_tag);
    };
    // one branch per tile: the loop of a wave with all its rows real has no
    // per-MFMA condition
    static_assert(C::TM <= 2, "live tile counts 0, 1 and TM only");
    if (live_tm == C::TM) {
        kloop(std::integral_constant<int, C::TM>{});
    } else if constexpr (C::TM > 1) {
        if (live_tm == 1) kloop(std::integral_constant<int, 1>{});
        else kloop(std::integral_constant<int, 0>{});
    } else {
        kloop(std::integral_constant<int, 0>{});
    }

    // ---- epilogue: lane holds C[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 tile
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm * C::WTM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int p = ids_s[r];
            if (p >= P) continue;
            if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
#pragma unroll
                for (int j = 0; j < C::TN / 2; ++j) {
                    float gv = acc[i][j][v], uv = acc[i][j + C::TN / 2][v];
                    if constexpr (DT == MOE_FP8_E4M3) {
                        gv *= scale;
                        uv *= scale;
                    }
                    const int n = n0 + wn * (C::WTN / 2) + 32 * j + (lane & 31);
                    const float o = silu(gv) * uv;
                    if constexpr (DT == MOE_FP8_E4M3) {
                        // float32 intermediate until it is quantised
                        amax = fmaxf(amax, fabsf(o));
                        reinterpret_cast<float*>(g.c)[(size_t)p * I + n] = o;
                    } else {
                        reinterpret_cast<uint16_t*>(g.c)[(size_t)p * I + n] = f2bf(o);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int n = n0 + wn * C::WTN + 32 * j + (lane & 31);
                    const float y = (DT == MOE_FP8_E4M3) ? acc[i][j][v] * scale : acc[i][j][v];
                    reinterpret_cast<uint16_t*>(g.c)[(size_t)p * N + n] = f2bf(y);
                }
            }
        }
    }
    if constexpr (DT == MOE_FP8_E4M3 && KIND == MOE_GEMM_GATE_UP_SILU) amax_publish(amax, g.c_amax);
}

// block shapes of the LDS-ring prefill kernel: 128-row tiles, and 64-row
// tiles (the fused layer takes them for bf16 batches of 25-48 pairs per
// expert and for e4m3 batches of two tokens up to 32 pairs per expert)
using PrefillCfg = P2Cfg<128, 256, 64, 3>;
using PrefillCfg64 = P2Cfg<64, 256, 64, 3>;
static_assert(PrefillCfg::BN == PrefillCfg64::BN, "one weight-tile width");

template <int KIND, int DT, class C, bool NTW>
static hipError_t launch_prefill2_nt(const GemmArgs& a, int64_t cap, int E, hipStream_t s) {
    const int m_tiles = (int)(cap / C::BM);
    const int n_tiles = (KIND == MOE_GEMM_GATE_UP_SILU) ? (a.N / 2) / (C::BN / 2) : a.N / C::BN;
    const int nb = m_tiles * n_tiles;
    const int grid = (nb + kP2Xcds - 1) / kP2Xcds * kP2Xcds;
    // LDS above the default dynamic limit must be requested once per kernel
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_prefill2_kernel<KIND, DT, C, NTW>), hipFuncAttributeMaxDynamicSharedMemorySize,
        C::LdsBytes);
    if (attr != hipSuccess) return attr;
    // weight tiles per group.  DOWN: one (the row tiles of a weight tile run
    // back to back; measured down GEMM times, one tile against the rule
    // below: Mixtral 4096 tokens 1043 -> 1015 us, e4m3 512 tokens 480 -> 429,
    // 128 experts at 2048 tokens 148 -> 126).  GATE_UP: one as well when an
    // expert averages at most 64 pairs (one row tile each: e4m3 512 tokens
    // 894 -> 852 us); otherwise all of them when there are few (each token
    // tile is then fetched once per XCD), else 2 (Mixtral 4096 tokens: 2
    // against 1, 3, 4, 8, 16: 1954 against 2024, 1974, 2020, 2100, 2330 us;
    // 128 experts at 2048 tokens: all six 244 us, one 257)
    const bool one = KIND == MOE_GEMM_DOWN || (long)a.P <= 64L * E;
    const int group_n = one ? 1 : (n_tiles <= 8 ? n_tiles : 2);
    hipLaunchKernelGGL((gemm_prefill2_kernel<KIND, DT, C, NTW>), dim3(grid), dim3(C::Threads), C::LdsBytes, s, a, m_tiles,
                       n_tiles, group_n);
    return hipGetLastError();
}

// pairs per expert (P / E) at most 64: each weight tile feeds about one row
// tile, and the weights go non-temporal (e4m3 512 tokens, P / E = 64: 1.48
// against 1.40 ms cached); with more, an expert's second row tile re-reads
// its weight tiles from L2 (128 experts at 2048 tokens, P / E = 128: cached
// 0.426 against 0.457 ms non-temporal)
template <int KIND, int DT, class C>
static hipError_t launch_prefill2(const GemmArgs& a, int64_t cap, int E, hipStream_t s) {
    if ((long)a.P <= 64L * E) return launch_prefill2_nt<KIND, DT, C, true>(a, cap, E, s);
    return launch_prefill2_nt<KIND, DT, C, false>(a, cap, E, s);
}

// ------------------------------------------------------ decode (LDS ring)
//
// The decode work split above (blockIdx.y = active-expert slot, blockIdx.x =
// G groups of 64 weight rows, blockIdx.z = K split; the four wavefronts take
// K steps round robin and reduce through LDS at the end), with every operand
// brought to the MFMAs through a wavefront-private ring of KD LDS stages
// filled by direct-to-LDS copies.  One copy instruction moves 128 contiguous
// bytes (a whole cache line) of each of 8 rows, where a register load in the
// MFMA lane layout can only read 64 bytes of each of 16 rows; on MI355X the
// whole-line pattern streams the weights about 14% faster, and the weight
// copies carry the non-temporal hint (read once; another 13%), the token
// copies not (they are re-read by every row group).  A stage holds 128
// bytes of the group's 64 weight rows and of the pass's 16*NT token rows.
// No other wavefront touches a ring, so the main loop has no barrier: each
// wave waits on its own copies with vmcnt.
//
// TQ (e4m3 down projection over the float32 intermediate, one token tile):
// the token rows do not go through the ring.  Each lane loads the float32
// values of its MFMA operand (two 64-byte pieces of its token row per step)
// into registers two steps ahead and quantises them to e4m3 codes just
// before the step's MFMAs, so the intermediate is read once per row group
// at four bytes per value and never written back as codes.  The loads of
// step j+2 are issued after the wait that retires step j's weight copies,
// which keeps that wait exact: the weight copies of step j+1 are the only
// younger vector-memory operations, and the compiler's own wait before the
// token registers of step j asks for no more than that one.

constexpr int kRingSB = 128;  // bytes of every row per step

template <int NT, int G, int KD, bool TQ = false>
struct DecRing {
    static constexpr int WInstr = 64 * kRingSB / 1024;                   // copy instructions for the weight rows
    static constexpr int TInstr = TQ ? 0 : NT * 16 * kRingSB / 1024;     // ... and for the token rows
    static constexpr int Instr = WInstr + TInstr;
    static constexpr int TokOff = 64 * kRingSB;                          // token rows follow the weight rows
    static constexpr int Stage = (64 + (TQ ? 0 : 16 * NT)) * kRingSB;
    static constexpr int Ring = 4 * KD * Stage;
    static constexpr int Red = 4 * G * 4 * NT * 64 * 16;     // [4 waves][G*4 tiles][NT][64 lanes] f32x4
    static constexpr int Lds = Ring > Red ? Ring : Red;
    static_assert(Lds <= 160 * 1024, "LDS");
    static_assert((KD - 1) * Instr < 64, "vmcnt range");
};

// Physical 16-byte chunk of logical chunk c in ring row r.  Rows are 128
// bytes, so rows 2q and 2q+1 share a 256-byte bank window; XOR with q mod 8
// puts 16 consecutive rows read at one logical chunk into 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int ring_swz(int c, int r) { return c ^ ((r >> 1) & 7); }

// vmcnt wait that is also a compiler memory barrier (LDS reads of the
// stage may not move above it)
template <int N>
__device__ __forceinline__ void ring_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int KIND, int DT, int NT, int G, int KD, bool TQ>
__global__ void __launch_bounds__(kDecThreads) gemm_decode_ring_kernel(GemmArgs g) {
    using R = DecRing<NT, G, KD, TQ>;
    static_assert(!TQ || (NT == 1 && KIND == MOE_GEMM_DOWN && DT == MOE_FP8_E4M3), "TQ: e4m3 DOWN, one token tile");
    constexpr int kElem = Opnd<DT>::kElemBytes;
    constexpr int T = 4;  // 16-row tiles per group
    extern __shared__ __attribute__((aligned(1024))) char ring_lds[];

    const int slot = blockIdx.y;
    SlotRows sr;
    if (!slot_rows(g, slot, sr)) return;
    const int e = sr.e;
    const int cnt = sr.cnt;
    // pair id of the expert's row r
    auto pair_id = [&](int r) { return g.route_logits ? sr.p1 : g.sorted[sr.base + r]; };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int drow = lane >> 3, dpc = lane & 7;  // copy lane: row drow of 8, physical chunk dpc
    const int K = g.K, N = g.N, I = N / 2;
    const size_t rowb = (size_t)K * kElem;
    const int nks_all = (int)(rowb / kRingSB);
    const int ks0 = (int)((long)blockIdx.z * nks_all / g.ksplit);
    const int nks = (int)((long)(blockIdx.z + 1) * nks_all / g.ksplit) - ks0;
    const int total = G * nks;
    const int nw = total > wave ? (total - wave + 3) / 4 : 0;  // this wave's steps: s = wave + 4j

    const int n0 = (KIND == MOE_GEMM_GATE_UP_SILU) ? blockIdx.x * 32 * G : blockIdx.x * 64 * G;
    const size_t gstride = (size_t)((KIND == MOE_GEMM_GATE_UP_SILU) ? 32 : 64) * rowb;
    // source offsets of this lane's weight copies: instruction i fills group
    // rows 8i..8i+7 (gate rows then up rows for GATE_UP)
    const char* wexp = reinterpret_cast<const char*>(g.w) + (size_t)e * N * rowb;
    size_t woff[R::WInstr];
#pragma unroll
    for (int i = 0; i < R::WInstr; ++i) {
        const int ri = 8 * i + drow;
        int row;
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU)
            row = (ri < 32) ? n0 + ri : I + n0 + ri - 32;
        else
            row = n0 + ri;
        woff[i] = (size_t)row * rowb + ring_swz(dpc, ri) * 16;
    }

    float scale = 1.0f, qs = 1.0f;
    if constexpr (DT == MOE_FP8_E4M3) {
        if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
            scale = g.a_scale[0] * g.w_scale[e];
        } else {
            // (the ring's LDS is not in use before the first copies below)
            qs = g.amax_parts ? act_scale_from_parts(g.amax_parts, g.amax_nparts, reinterpret_cast<float*>(ring_lds))
                              : act_scale_from_amax(g.a_scale);
            scale = qs * g.w_scale[e];
        }
    }
    const ActQuant quant(qs);

    char* ring = ring_lds + wave * (KD * R::Stage);
    const unsigned ring_lds0 = lds_addr_of(ring);
    f32x4* red = reinterpret_cast<f32x4*>(ring_lds);  // after the main loop only
    float amax = 0.0f;

    for (int pass = 0; pass < cnt; pass += NT * 16) {
        const int ntiles = min(NT, (cnt - pass + 15) / 16);
        // token-row sources of this lane's copies (rows past the expert's
        // count repeat its last row; their products are not used)
        size_t toff[NT][2];
        const char* trow = nullptr;  // TQ: this lane's float32 token row, at its lane group's 64 bytes
        if constexpr (TQ) {
            const int p = pair_id(min(pass + lr, cnt - 1));
            trow = reinterpret_cast<const char*>(g.a) + (size_t)p * K * 4 + 64 * lg;
        } else {
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rr = 16 * c + 8 * h + drow;
                    const int r = min(pass + rr, cnt - 1);
                    const int p = pair_id(r);
                    const int src = (KIND == MOE_GEMM_GATE_UP_SILU) ? p / g.topk : p;
                    toff[c][h] = (size_t)src * rowb + ring_swz(dpc, rr) * 16;
                }
        }

        // the copies of step j: the weight rows, then the token rows of the
        // pass's LT live tiles
        auto issue = [&](int j, auto lt_tag) __attribute__((always_inline)) {
            const int s = wave + 4 * j;
            const int gi = s / nks, ks = ks0 + s % nks;
            const unsigned st = ring_lds0 + (unsigned)((j % KD) * R::Stage);
            // this wave's earlier LDS reads of the slot have completed
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const char* wsrc = wexp + gi * gstride + (size_t)ks * kRingSB;
#pragma unroll
            for (int i = 0; i < R::WInstr; ++i) lds_dma16_nt_at(wsrc + woff[i], st + i * 1024);
            if constexpr (!TQ) {
                const char* tsrc = reinterpret_cast<const char*>(g.a) + (size_t)ks * kRingSB;
#pragma unroll
                for (int c = 0; c < decltype(lt_tag)::value; ++c)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        lds_dma16_at(tsrc + toff[c][h], st + R::TokOff + (2 * c + h) * 1024);
            }
        };
        // TQ: the float32 operand values of step j (elements 16 lg.. and 64 + 16 lg.. of the
        // step's 128, i.e. logical chunks lg and lg + 4 of the weight rows)
        auto tload = [&](uint4 (&b)[8], int j) {
            const int ks = ks0 + (wave + 4 * j) % nks;
            const uint4* src = reinterpret_cast<const uint4*>(trow + (size_t)ks * (4 * kRingSB));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                b[u] = src[u];
                b[4 + u] = src[16 + u];
            }
        };

        f32x4 acc[G][T][NT];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < NT; ++c) acc[gi][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 tb[TQ ? 2 : 1][TQ ? 8 : 1];
        if constexpr (TQ) {
            // token values of steps 0 and 1 before the first weight copies (a
            // wave with fewer steps loads step 0 again: any step index >= 0
            // names an in-bounds K step of this workgroup's range)
            tload(tb[0], 0);
            tload(tb[1], nw > 1 ? 1 : 0);
        }
        // one step of the ring; TQ: tbuf holds step j's token values and is
        // refilled with step j + 2's (two buffers in fixed roles, so no
        // register copy makes the compiler wait on the loads just issued)
        auto step = [&](int j, uint4 (&tbuf)[TQ ? 8 : 1], auto lt_tag) __attribute__((always_inline)) {
            constexpr int LT = decltype(lt_tag)::value;
            constexpr int kInstr = R::WInstr + (TQ ? 0 : LT * 16 * kRingSB / 1024);  // copies per step
            if (j + KD - 1 < nw) {
                issue(j + KD - 1, lt_tag);
                ring_wait_vm<(KD - 1) * kInstr>();
            } else {
                ring_wait_vm<0>();
            }
            // TQ: every vector-memory operation older than the weight copies
            // just issued has completed, the token loads of step j included
            uint4 tq0 = {0, 0, 0, 0}, tq1 = {0, 0, 0, 0};
            if constexpr (TQ) {
                tq0 = quant.codes16(tbuf[0], tbuf[1], tbuf[2], tbuf[3]);
                tq1 = quant.codes16(tbuf[4], tbuf[5], tbuf[6], tbuf[7]);
                // unconditional (the last steps reload step nw-1, unused): a
                // conditional refill would merge two register states and the
                // copies that merge needs would wait on these very loads
                tload(tbuf, min(j + 2, nw - 1));
            }
            const char* st = ring + (j % KD) * R::Stage;
            const int gi = (wave + 4 * j) / nks;
            const int sw = (lr >> 1) & 7;  // ring_swz of rows 16t + lr
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                if (gg != gi) continue;
                if constexpr (DT == MOE_FP8_E4M3) {
                    // one f8f6f4 MFMA per tile pair covers the 128-byte step;
                    // a lane group supplies logical chunks lg and lg + 4
                    uint4 a0[T], a1[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        const char* rp = st + (16 * t + lr) * kRingSB;
                        a0[t] = *reinterpret_cast<const uint4*>(rp + ((lg ^ sw) << 4));
                        a1[t] = *reinterpret_cast<const uint4*>(rp + (((lg + 4) ^ sw) << 4));
                    }
                    if constexpr (TQ) {
#pragma unroll
                        for (int t = 0; t < T; ++t) acc[gg][t][0] = mfma_f8_16x16x128(a0[t], a1[t], tq0, tq1, acc[gg][t][0]);
                    } else {
#pragma unroll
                        for (int c = 0; c < LT; ++c) {
                            const char* bp = st + R::TokOff + (16 * c + lr) * kRingSB;
                            const uint4 b0 = *reinterpret_cast<const uint4*>(bp + ((lg ^ sw) << 4));
                            const uint4 b1 = *reinterpret_cast<const uint4*>(bp + (((lg + 4) ^ sw) << 4));
#pragma unroll
                            for (int t = 0; t < T; ++t)
                                acc[gg][t][c] = mfma_f8_16x16x128(a0[t], a1[t], b0, b1, acc[gg][t][c]);
                        }
                    }
                } else {
                    // bf16: two 32-wide K chunks per step, logical chunk 4u + lg
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int pc = ((4 * u + lg) ^ sw) << 4;
                        uint4 a[T];
#pragma unroll
                        for (int t = 0; t < T; ++t)
                            a[t] = *reinterpret_cast<const uint4*>(st + (16 * t + lr) * kRingSB + pc);
#pragma unroll
                        for (int c = 0; c < LT; ++c) {
                            const uint4 b = *reinterpret_cast<const uint4*>(st + R::TokOff + (16 * c + lr) * kRingSB + pc);
#pragma unroll
                            for (int t = 0; t < T; ++t) acc[gg][t][c] = Opnd<MOE_BF16>::mfma(a[t], b, acc[gg][t][c]);
                        }
                    }
                }
            }
        };
        // LT token tiles copied and multiplied, fixed per pass: ntiles rounded
        // up to 1, 2 or NT (the rows of a tile past the count repeat the
        // last row; their products are not used), so a pass whose rows fit
        // fewer tiles than NT copies fewer token rows, and the loop carries
        // no per-tile branch
        auto steps = [&](auto lt_tag) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < KD - 1; ++j)
                if (j < nw) issue(j, lt_tag);
            if constexpr (TQ) {
                int j = 0;
                for (; j + 1 < nw; j += 2) {
                    step(j, tb[0], lt_tag);
                    step(j + 1, tb[1], lt_tag);
                }
                if (j < nw) step(j, tb[0], lt_tag);
            } else {
                for (int j = 0; j < nw; ++j) step(j, tb[0], lt_tag);
            }
        };
        if constexpr (NT == 1) {
            steps(std::integral_constant<int, 1>{});
        } else {
            if (ntiles == 1)
                steps(std::integral_constant<int, 1>{});
            else if (NT > 2 && ntiles == 2)
                steps(std::integral_constant<int, (NT > 2 ? 2 : NT)>{});
            else
                steps(std::integral_constant<int, NT>{});
        }

        // every wave is done with its ring: the reduction area aliases it
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < NT; ++c) red[((wave * G * T + gi * T + t) * NT + c) * 64 + lane] = acc[gi][t][c];
        __syncthreads();

        constexpr int kPer = (KIND == MOE_GEMM_GATE_UP_SILU) ? 2 : 4;  // output tiles per group
        const int units = G * kPer * ntiles;
        for (int u = wave; u < units; u += 4) {
            const int c = u / (G * kPer);
            const int gq = u % (G * kPer);
            const int gi = gq / kPer, q = gq % kPer;
            const int r = pass + c * 16 + lr;
            if (r >= cnt) continue;
            const int p = pair_id(r);
            if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
                f32x4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    gs += red[((w * G * T + gi * T + q) * NT + c) * 64 + lane];
                    us += red[((w * G * T + gi * T + q + 2) * NT + c) * 64 + lane];
                }
                f32x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = silu(gs[v] * scale) * (us[v] * scale);
                const int n = n0 + gi * 32 + 16 * q + 4 * lg;
                if constexpr (DT == MOE_FP8_E4M3) {
                    // the e4m3 layer keeps its intermediate in float32 until it is quantised
#pragma unroll
                    for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(o[v]));
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.c) + (size_t)p * I + n) = o;
                } else {
                    uint2 pk;
                    pk.x = pack_bf2(o[0], o[1]);
                    pk.y = pack_bf2(o[2], o[3]);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.c) + (size_t)p * I + n) = pk;
                }
            } else {
                f32x4 ys = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) ys += red[((w * G * T + gi * T + q) * NT + c) * 64 + lane];
                const int n = n0 + gi * 64 + 16 * q + 4 * lg;
                if (g.cpart) {
                    *reinterpret_cast<f32x4*>(g.cpart + ((size_t)blockIdx.z * g.P + p) * N + n) = ys * scale;
                } else {
                    uint2 pk;
                    pk.x = pack_bf2(ys[0] * scale, ys[1] * scale);
                    pk.y = pack_bf2(ys[2] * scale, ys[3] * scale);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.c) + (size_t)p * N + n) = pk;
                }
            }
        }
        // the next pass refills the rings over the reduction area
        __syncthreads();
    }
    if constexpr (DT == MOE_FP8_E4M3 && KIND == MOE_GEMM_GATE_UP_SILU) {
        // (every copy has landed and every wavefront has passed the pass's
        // closing barrier: the LDS is free)
        if (g.amax_parts)
            amax_parts_publish(amax, g.amax_parts + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * G, G,
                               reinterpret_cast<float*>(ring_lds));
        else
            amax_publish(amax, g.c_amax);
    }
}

template <int KIND, int DT, int NT, int G, int KD, bool TQ = false>
static hipError_t launch_decode_ring(const GemmArgs& a, int nslots, hipStream_t s) {
    using R = DecRing<NT, G, KD, TQ>;
    const int rows = (KIND == MOE_GEMM_GATE_UP_SILU) ? 32 * G : 64 * G;  // output columns per workgroup
    const int ncols = (KIND == MOE_GEMM_GATE_UP_SILU) ? a.N / 2 : a.N;
    // LDS above the default dynamic limit must be requested once per kernel
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_decode_ring_kernel<KIND, DT, NT, G, KD, TQ>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, R::Lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemm_decode_ring_kernel<KIND, DT, NT, G, KD, TQ>), dim3(ncols / rows, nslots, a.ksplit),
                       dim3(kDecThreads), R::Lds, s, a);
    return hipGetLastError();
}

// -------------------------------- decode DOWN with the combine (few tokens)
//
// The kernel writes the final token-ordered rows itself (FusedMoE vs MegaMoE
// post, section 3.1 step 4), so y never goes to memory and the separate
// combine launch disappears.  Work split: blockIdx.x owns RB output columns
// of H and runs every active expert's K steps over those weight rows; a
// pair's y therefore stays inside one workgroup, and the combine over a
// token's k pairs needs no other workgroup.  With RB = 16 (8) rows per
// workgroup the grid has H/16 (H/8) workgroups, 256 for the layer shapes
// here, as many as the per-expert decode grid it replaces.
//
// Unit u is an 8-row token tile of one expert (normally the expert's only
// one); a unit has nks steps of 128 bytes of every row, brought in through
// wavefront-private LDS rings as in the per-expert ring kernel.  With few
// units the four waves take each unit's steps round robin (step ks to wave
// ks mod 4) and meet at a barrier per unit, where wave u mod 4 adds the four
// partial sums in wave order; with many, each wave runs whole units and keeps
// the sums of the four residues ks mod 4 apart, adding them in the same
// order.  Both are the per-expert kernel's products and sums in its order
// (same lane layout, nks a multiple of 4), so y has the same bits; y is
// rounded to bf16 into an LDS row per pair and the closing combine runs
// fmaf over j ascending from 0, as the combine kernel does.

static int decode_token_tiles(int M, int topk, int E);

constexpr int kDcMaxPairs = 512;   // y rows kept in LDS
constexpr int kDcMaxUnits = 320;   // >= 256 experts + 512 pairs / 8
constexpr int kDcTok = 8;          // token rows per unit

template <int RB, int KD>
struct DcLayout {
    static constexpr int WInstr = RB * kRingSB / 1024;       // weight copies per step
    static constexpr int TInstr = kDcTok * kRingSB / 1024;   // token copies per step
    static constexpr int Instr = WInstr + TInstr;
    static constexpr int TokOff = RB * kRingSB;
    static constexpr int Stage = (RB + kDcTok) * kRingSB;
    static constexpr int Ring = 4 * KD * Stage;
    static constexpr int RedOff = Ring;                              // [2][4 waves][64] f32x4
    static constexpr int YOff = RedOff + 2 * 4 * 64 * 16;            // [kDcMaxPairs][RB] bf16
    static constexpr int UnitOff = YOff + kDcMaxPairs * RB * 2;      // [kDcMaxUnits] int4 {e, rows, first sorted row}
    static constexpr int PidOff = UnitOff + kDcMaxUnits * 16;        // [kDcMaxUnits][kDcTok] pair ids
    static constexpr int Lds = PidOff + kDcMaxUnits * kDcTok * 4;
    static_assert(Lds <= 160 * 1024, "LDS");
    static_assert((KD - 1) * Instr < 64, "vmcnt range");
};

template <int RB, int KD>
__global__ void __launch_bounds__(kDecThreads) gemm_down_combine_kernel(GemmArgs g, const float* __restrict__ cw,
                                                                        uint16_t* __restrict__ out, int M) {
    using L = DcLayout<RB, KD>;
    extern __shared__ __attribute__((aligned(1024))) char dc_lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int drow = lane >> 3, dpc = lane & 7;
    const int K = g.K, N = g.N;
    const size_t rowb = (size_t)K * 2;
    const int nks = (int)(rowb / kRingSB);  // a multiple of 4 (checked by the launcher)
    const int n0 = blockIdx.x * RB;

    int4* units = reinterpret_cast<int4*>(dc_lds + L::UnitOff);
    int* pids = reinterpret_cast<int*>(dc_lds + L::PidOff);
    f32x4* red = reinterpret_cast<f32x4*>(dc_lds + L::RedOff);
    uint16_t* ybuf = reinterpret_cast<uint16_t*>(dc_lds + L::YOff);
    int* scan = reinterpret_cast<int*>(dc_lds);  // [4] wave totals, before the rings are used

    // units: thread i takes active slot i; an exclusive scan of the tiles per
    // slot places its units (slot order, then tile order)
    const int na = *g.num_active;
    int e = 0, cnt = 0, tiles = 0;
    if (tid < na) {
        e = g.active[tid];
        cnt = g.counts[e];
        tiles = (cnt + kDcTok - 1) / kDcTok;
    }
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += scan[w];
    const int U = scan[0] + scan[1] + scan[2] + scan[3];
    __syncthreads();
    const int first = before + incl - tiles;
    for (int q = 0; q < tiles; ++q)
        units[first + q] = make_int4(e, min(kDcTok, cnt - kDcTok * q), g.offsets[e] + kDcTok * q, 0);
    __syncthreads();
    // the tiles' pair ids (rows past a tile's count repeat its last pair)
    for (int i = tid; i < U * kDcTok; i += kDecThreads) {
        const int4 un = units[i / kDcTok];
        pids[i] = g.sorted[un.z + min(i % kDcTok, un.y - 1)];
    }
    __syncthreads();

    // Two orders of the same sums.  Few units (split): the four waves take
    // each unit's K steps round robin and meet at a barrier per unit.  Many
    // units: wave w runs units w, w+4, ... alone, keeping the partial sums of
    // the four K residues apart (acc[r] = what wave r holds in the split
    // order) and adding them in the same order, with no barrier until the end.
    const bool split = U < 8;
    const int jpu = nks / 4;
    const int mine = split ? U : (U > wave ? (U - wave + 3) / 4 : 0);
    const int nsteps = split ? U * jpu : mine * nks;
    auto unit_of = [&](int j, int& u, int& ks) {
        if (split) {
            u = j / jpu;
            ks = wave + 4 * (j - u * jpu);
        } else {
            const int i = j / nks;
            u = wave + 4 * i;
            ks = j - i * nks;
        }
    };

    size_t woff[L::WInstr];
#pragma unroll
    for (int i = 0; i < L::WInstr; ++i) {
        const int ri = 8 * i + drow;
        woff[i] = (size_t)(n0 + ri) * rowb + ring_swz(dpc, ri) * 16;
    }
    const char* wall = reinterpret_cast<const char*>(g.w);
    const char* aall = reinterpret_cast<const char*>(g.a);
    char* ring = dc_lds + wave * (KD * L::Stage);
    const unsigned ring_lds0 = lds_addr_of(ring);

    auto issue = [&](int j) {
        int u, ks;
        unit_of(j, u, ks);
        const int ue = units[u].x;
        const int p = pids[u * kDcTok + drow];
        const unsigned st = ring_lds0 + (unsigned)((j % KD) * L::Stage);
        // this wave's earlier LDS reads of the slot (and of the tables) have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const char* wsrc = wall + (size_t)ue * N * rowb + (size_t)ks * kRingSB;
#pragma unroll
        for (int i = 0; i < L::WInstr; ++i) lds_dma16_nt_at(wsrc + woff[i], st + i * 1024);
        lds_dma16_at(aall + (size_t)ks * kRingSB + (size_t)p * rowb + ring_swz(dpc, drow) * 16, st + L::TokOff);
    };
    // one step: wait for stage j, two MFMAs into acc
    const int ar = (RB == 16) ? lr : (lr & 7);  // weight row of this lane's MFMA row (RB 8: rows 8-15 repeat 0-7)
    const int br = lr & 7;                      // token row (columns 8-15 repeat 0-7)
    const int swa = (ar >> 1) & 7, swb = (br >> 1) & 7;
    auto step = [&](int j, f32x4& acc) {
        if (j + KD - 1 < nsteps) {
            issue(j + KD - 1);
            ring_wait_vm<(KD - 1) * L::Instr>();
        } else {
            ring_wait_vm<0>();
        }
        const char* st = ring + (j % KD) * L::Stage;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint4 a = *reinterpret_cast<const uint4*>(st + ar * kRingSB + (((4 * u + lg) ^ swa) << 4));
            const uint4 b = *reinterpret_cast<const uint4*>(st + L::TokOff + br * kRingSB + (((4 * u + lg) ^ swb) << 4));
            acc = Opnd<MOE_BF16>::mfma(a, b, acc);
        }
    };
    // y of unit u (this lane's 4 rows of column lr) into the pair rows of LDS
    auto store_y = [&](int u, const f32x4& ys) {
        if (lr < units[u].y && (RB == 16 || lg < 2)) {
            uint2 pk;
            pk.x = pack_bf2(ys[0], ys[1]);
            pk.y = pack_bf2(ys[2], ys[3]);
            *reinterpret_cast<uint2*>(ybuf + pids[u * kDcTok + lr] * RB + 4 * lg) = pk;
        }
    };

    // vmcnt(0) as a builtin the compiler sees: the table loads above are then
    // complete on every path into the loop, so it adds no wait of its own
    // there (it would drain the copies in flight every iteration)
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int j = 0; j < KD - 1; ++j)
        if (j < nsteps) issue(j);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if (split) {
        f32x4 acc = zero;
        for (int j = 0; j < nsteps; ++j) {
            step(j, acc);
            if ((j + 1) % jpu == 0) {
                // end of unit u: the four partial sums, added in wave order by wave u mod 4
                const int u = j / jpu;
                f32x4* r = red + (u & 1) * 4 * 64;
                r[wave * 64 + lane] = acc;
                acc = zero;
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (wave == (u & 3)) {
                    f32x4 ys = zero;
#pragma unroll
                    for (int w = 0; w < 4; ++w) ys += r[w * 64 + lane];
                    store_y(u, ys);
                }
            }
        }
    } else {
        f32x4 acc0 = zero, acc1 = zero, acc2 = zero, acc3 = zero;
        for (int j = 0; j < nsteps; j += 4) {  // nks, and so nsteps, is a multiple of 4
            step(j, acc0);
            step(j + 1, acc1);
            step(j + 2, acc2);
            step(j + 3, acc3);
            if ((j + 4) % nks == 0) {
                f32x4 ys = zero;
                ys += acc0;
                ys += acc1;
                ys += acc2;
                ys += acc3;
                store_y(wave + 4 * (j / nks), ys);
                acc0 = acc1 = acc2 = acc3 = zero;
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // out[t] = sum_j w[t,j] y[t*k+j], j ascending, 8 columns per thread
    for (int i = tid; i < M * (RB / 8); i += kDecThreads) {
        const int t = i / (RB / 8), h = 8 * (i % (RB / 8));
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < g.topk; ++j) {
            const float wj = cw[(size_t)t * g.topk + j];
            const uint4 v = *reinterpret_cast<const uint4*>(ybuf + (t * g.topk + j) * RB + h);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[2 * c] = fmaf(wj, __uint_as_float(q[c] << 16), o[2 * c]);
                o[2 * c + 1] = fmaf(wj, __uint_as_float(q[c] & 0xffff0000u), o[2 * c + 1]);
            }
        }
        uint4 pk;
        pk.x = pack_bf2(o[0], o[1]);
        pk.y = pack_bf2(o[2], o[3]);
        pk.z = pack_bf2(o[4], o[5]);
        pk.w = pack_bf2(o[6], o[7]);
        *reinterpret_cast<uint4*>(out + (size_t)t * N + n0 + h) = pk;
    }
}

template <int RB, int KD>
static hipError_t launch_down_combine_rb(const GemmArgs& a, const float* w, void* out, int M, hipStream_t s) {
    using L = DcLayout<RB, KD>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_down_combine_kernel<RB, KD>), hipFuncAttributeMaxDynamicSharedMemorySize,
        L::Lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemm_down_combine_kernel<RB, KD>), dim3(a.N / RB), dim3(kDecThreads), L::Lds, s, a, w,
                       static_cast<uint16_t*>(out), M);
    return hipGetLastError();
}

// Opt-in (MOE_DOWN_COMBINE=1): measured on MI355X it does not beat the
// per-expert kernel plus the combine launch (Mixtral-shaped layer at 1 and 4
// tokens: 1% and 0.5% slower; 128-expert layer at 1, 8 and 16 tokens: 4%,
// 13% and 9% slower).  The launch it saves overlaps the previous kernel's
// tail, while the column-block order re-reads each unit's token rows for
// every block of 8 or 16 weight rows instead of every 64 to 256.
bool down_combine_fits(moe_dtype dtype, int M, int topk, int E, int H, int I, int block_m) {
    if (dtype != MOE_BF16 || M < 1 || block_m != 16) return false;
    const char* env = getenv("MOE_DOWN_COMBINE");
    if (!env || strcmp(env, "1") != 0) return false;
    GemmCall probe{MOE_GEMM_DOWN, dtype, nullptr, nullptr, nullptr, nullptr, {}, M, topk, E, H, I, block_m,
                   nullptr, nullptr};
    if (choose_gemm_path(probe) != GemmPath::kDecode) return false;
    // one 16-row token tile per expert expected (the per-expert kernel's one-tile case)
    if (decode_token_tiles(M, topk, E) != 1) return false;
    return (long)M * topk <= kDcMaxPairs && I % 256 == 0 && H % 16 == 0;
}

hipError_t launch_down_combine(const GemmCall& c, const float* topk_weights, void* out, hipStream_t s) {
    GemmArgs a{c.a, c.a_scale, c.w, c.w_scale, c.al.sorted_ids, c.al.tile_expert, c.al.expert_counts,
               c.al.expert_offsets, c.al.active_experts, c.al.num_active, c.topk, c.N, c.K, c.M * c.topk,
               nullptr, nullptr, 1, nullptr, 0};
    // 256 workgroups where H allows: 16 rows each from H = 4096 up, else 8
    if (c.N >= 4096) return launch_down_combine_rb<16, 8>(a, topk_weights, out, c.M, s);
    return launch_down_combine_rb<8, 12>(a, topk_weights, out, c.M, s);
}

// ------------------------------------------- decode, int4 weights (W4A16)
//
// Weight-only int4 (FusedMoE vs MegaMoE post, sections 6.2-6.3: INT4 weights
// cut the memory the expert GEMMs stream).  W[n][k] = (u - 8) * s[k/128][n]:
// 4-bit codes u packed so that the 32-bit word of 8 consecutive k holds
// k0+2i at bits 4i and k0+2i+1 at bits 16+4i, and one float32 scale per
// 128-wide group of k of a row, stored group-major.  Activations are bf16.
//
// The decode work split of the ring kernel (blockIdx.y active-expert slot,
// blockIdx.x G groups of 64 weight rows, blockIdx.z K split; the four
// wavefronts take steps round robin and reduce through LDS at the end).  A
// step is 128 bytes of every weight row (256 k, two scale groups); the codes
// stream through a wavefront-private LDS ring of direct-to-LDS copies (as
// in the ring kernel, non-temporal), one more copy per stage brings the
// step's group scales of the 64 rows.  The token values of a step (bf16)
// come through registers, two buffers in fixed roles.  Step j begins with
// a wait for every vector-memory operation of the wave (a wait the compiler
// sees, so it adds none of its own before the token values are used: it
// cannot count the copies, which are asm, and any wait it placed later
// would also retire the next step's loads); what is in flight then is
// exactly step j's scales, codes and token values, issued at the start of
// step j - 1.  It then issues step j + 1's (the scales and codes into step
// j - 1's slot, whose reads are done, the token values into step j - 1's
// buffer), which load during step j's products.
//
// Products on the bf16 MFMA without converting codes to values: OR-ing a
// code into 0x4300 gives the bf16 128 + u exactly, so one AND-OR turns a
// word of codes into two bf16 operand words, and for a group g
//   sum_k W[n][k] x[k] = s[g][n] * (sum_k (128 + u_k) x_k - 136 * sum_k x_k),
// the token sums coming from an MFMA with an all-ones operand.  Each MFMA
// covers 32 k of one group (lane group lg: k = 128 g + 32 lg + 8 q + j), so
// every group's products are accumulated apart (starting from -136 * sum x)
// and scaled per row.

// Two codes of a word (bits 0-3 and 16-19 of w) as two bf16 words 128 + u:
// (w & 0x000F000F) | 0x43004300, one v_and_or_b32 when both constants sit in
// registers the compiler cannot see through (w4_opaque).  Written in C, not
// asm, so that the compiler knows the result is a vector ALU write and keeps
// the wait states an MFMA reading it needs.
__device__ __forceinline__ uint32_t w4_bf16x2(uint32_t w, uint32_t mask, uint32_t magic) {
    return (w & mask) | magic;
}

// a constant held in a vector register and hidden from constant folding: a
// folded mask and magic become two literal-operand instructions, since the
// fused AND-OR (VOP3) takes no literal on this target
__device__ __forceinline__ uint32_t w4_opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int KIND, int NT, int G, int KD>
__global__ void __launch_bounds__(kDecThreads, 2) gemm_decode_w4_kernel(GemmArgs g) {
    constexpr int T = 4;                      // 16-row tiles per group of 64 rows
    constexpr int kWInstr = 64 * kRingSB / 1024;
    constexpr int kScaleOff = 64 * kRingSB;   // [2 groups][64 rows] float32 after the codes
    constexpr int kStage = 64 * kRingSB + 1024;
    static_assert(KD == 2, "the scale copy of step j+2 goes to step j's slot");
    static_assert(NT == 1 || NT == 2, "live token tiles are NT or 1");
    extern __shared__ __attribute__((aligned(1024))) char w4_lds[];

    const int slot = blockIdx.y;
    SlotRows sr;
    if (!slot_rows(g, slot, sr)) return;
    const int e = sr.e;
    const int cnt = sr.cnt;
    // pair id of the expert's row r
    auto pair_id = [&](int r) { return g.route_logits ? sr.p1 : g.sorted[sr.base + r]; };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int drow = lane >> 3, dpc = lane & 7;
    const int K = g.K, N = g.N, I = N / 2;
    const size_t rowb = (size_t)K / 2;  // packed codes per row
    const int nks_all = (int)(rowb / kRingSB);
    const int ks0 = (int)((long)blockIdx.z * nks_all / g.ksplit);
    const int nks = (int)((long)(blockIdx.z + 1) * nks_all / g.ksplit) - ks0;
    const int total = G * nks;
    const int nw = total > wave ? (total - wave + 3) / 4 : 0;
    // step s of the workgroup: row group s / nks, K step s % nks (with one
    // group, s itself: no division in the loop).  A wave with no steps
    // still loads token values once (step index 0, so s = wave may be past
    // the workgroup's steps): with one group that s maps to step 0, which
    // every workgroup has, so the load stays inside the token rows
    auto step_group = [&](int s) { return G == 1 ? 0 : s / nks; };
    auto step_ks = [&](int s) { return G == 1 ? (s < nks ? s : 0) : s % nks; };

    const int n0 = (KIND == MOE_GEMM_GATE_UP_SILU) ? blockIdx.x * 32 * G : blockIdx.x * 64 * G;
    const int grows = (KIND == MOE_GEMM_GATE_UP_SILU) ? 32 : 64;  // row offset between this block's groups
    const char* wexp = reinterpret_cast<const char*>(g.w) + (size_t)e * N * rowb;
    // 32-bit offsets inside one expert's matrix (N * K / 2 bytes < 4 GiB,
    // checked by the launcher): registers are what bounds this kernel
    uint32_t woff[kWInstr];
#pragma unroll
    for (int i = 0; i < kWInstr; ++i) {
        const int ri = 8 * i + drow;
        const int row = (KIND == MOE_GEMM_GATE_UP_SILU) ? ((ri < 32) ? n0 + ri : I + n0 + ri - 32) : n0 + ri;
        woff[i] = (uint32_t)row * (uint32_t)rowb + (uint32_t)ring_swz(dpc, ri) * 16u;
    }
    // the scale copy: lane l (mod 32) brings 4 scales of group (l / 16) of the
    // step, rows 4 (l % 16).. of the 64 (gate rows then up rows for GATE_UP),
    // to LDS bytes 16 l: the [group][row] layout the MFMA epilogues read
    const float* sexp = g.w_scale + (size_t)e * (K / 128) * N;
    const int sl = lane & 31, skg = sl >> 4, sq = sl & 15;
    const int srow = (KIND == MOE_GEMM_GATE_UP_SILU) ? ((sq < 8) ? n0 + 4 * sq : I + n0 + 4 * (sq - 8)) : n0 + 4 * sq;

    char* ring = w4_lds + wave * (KD * kStage);
    const unsigned ring_lds0 = lds_addr_of(ring);
    f32x4* red = reinterpret_cast<f32x4*>(w4_lds);  // after the main loop only
    const uint4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
    // the AND-OR constants in registers
    const uint32_t nib_mask = w4_opaque(0x000F000Fu);
    const uint32_t bf_magic = w4_opaque(0x43004300u);

    for (int pass = 0; pass < cnt; pass += NT * 16) {
        const int ntiles = min(NT, (cnt - pass + 15) / 16);
        // this lane's token rows (rows past the count repeat the last one) at
        // its lane group's 32 values of each 128-value group
        const char* trow[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int p = pair_id(min(pass + 16 * c + lr, cnt - 1));
            const int src = (KIND == MOE_GEMM_GATE_UP_SILU) ? p / g.topk : p;
            trow[c] = reinterpret_cast<const char*>(g.a) + (size_t)src * K * 2 + 64 * lg;
        }
        // the codes of step j (8 copies)
        auto issue = [&](int j) __attribute__((always_inline)) {
            const int s = wave + 4 * j;
            const int gi = step_group(s), ks = ks0 + step_ks(s);
            const unsigned st = ring_lds0 + (unsigned)((j % KD) * kStage);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const char* wsrc = wexp + (size_t)gi * grows * rowb + (size_t)ks * kRingSB;
#pragma unroll
            for (int i = 0; i < kWInstr; ++i) lds_dma16_nt_at(wsrc + woff[i], st + i * 1024);
        };
        // the group scales of step j (one copy)
        auto issue_scales = [&](int j) __attribute__((always_inline)) {
            const int s = wave + 4 * j;
            const int gi = step_group(s), ks = ks0 + step_ks(s);
            const unsigned st = ring_lds0 + (unsigned)((j % KD) * kStage);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_dma16_at(sexp + (size_t)(2 * ks + skg) * N + srow + gi * grows, st + kScaleOff);
        };
        // the bf16 token values of step j for LT live tiles: 8 x 16 bytes per
        // tile (values 128 kg + 32 lg + 8 q .. + 7 of the step, kg = 0..1,
        // q = 0..3)
        auto tload = [&](uint4 (&b)[NT][8], int j, auto lt_tag) __attribute__((always_inline)) {
            const int ks = ks0 + step_ks(wave + 4 * j);
#pragma unroll
            for (int c = 0; c < decltype(lt_tag)::value; ++c) {
                const char* src = trow[c] + (size_t)ks * (2 * 2 * kRingSB);
#pragma unroll
                for (int kg = 0; kg < 2; ++kg)
#pragma unroll
                    for (int q = 0; q < 4; ++q) b[c][4 * kg + q] = *reinterpret_cast<const uint4*>(src + 256 * kg + 16 * q);
            }
        };

        f32x4 acc[G][T][NT];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < NT; ++c) acc[gi][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 tb0[NT][8], tb1[NT][8];
        // tb holds step j's token values, tn is refilled with step j + 1's
        // (unconditionally: the last step reloads step nw-1, unused, since a
        // conditional refill would merge two register states and the copies
        // that merge needs would wait on these very loads)
        auto step = [&](int j, uint4 (&tb)[NT][8], uint4 (&tn)[NT][8], auto lt_tag) __attribute__((always_inline)) {
            wait_vm<0>();
            if (j + 1 < nw) {
                issue_scales(j + 1);
                issue(j + 1);
            }
            tload(tn, min(j + 1, nw - 1), lt_tag);
            const char* st = ring + (j % KD) * kStage;
            const float* sc = reinterpret_cast<const float*>(st + kScaleOff);
            const int gi = step_group(wave + 4 * j);
            const int sw = (lr >> 1) & 7;
            // the compiler can overlap one tile's AND-ORs with the MFMAs of
            // another and interleave the LT tiles' MFMA chains (each MFMA's
            // accumulator comes from the one before)
            auto body = [&](auto lt_tag) __attribute__((always_inline)) {
                constexpr int LT = decltype(lt_tag)::value;
#pragma unroll
                for (int gg = 0; gg < G; ++gg) {
                    if (gg != gi) continue;
#pragma unroll
                    for (int kg = 0; kg < 2; ++kg) {
                        f32x4 xs[LT];
#pragma unroll
                        for (int c = 0; c < LT; ++c) xs[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int q = 0; q < 4; ++q)
#pragma unroll
                            for (int c = 0; c < LT; ++c) xs[c] = Opnd<MOE_BF16>::mfma(ones, tb[c][4 * kg + q], xs[c]);
#pragma unroll
                        for (int c = 0; c < LT; ++c) xs[c] *= -136.0f;  // the row products start from -136 * sum x
#pragma unroll
                        for (int t = 0; t < T; ++t) {
                            const uint4 wq =
                                *reinterpret_cast<const uint4*>(st + (16 * t + lr) * kRingSB + (((4 * kg + lg) ^ sw) << 4));
                            const f32x4 s4 = *reinterpret_cast<const f32x4*>(sc + kg * 64 + 16 * t + 4 * lg);
                            const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
                            uint4 av[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const uint32_t w = wd[q];
                                av[q] = uint4{w4_bf16x2(w, nib_mask, bf_magic), w4_bf16x2(w >> 4, nib_mask, bf_magic),
                                              w4_bf16x2(w >> 8, nib_mask, bf_magic), w4_bf16x2(w >> 12, nib_mask, bf_magic)};
                            }
                            f32x4 a[LT];
#pragma unroll
                            for (int c = 0; c < LT; ++c) a[c] = xs[c];
#pragma unroll
                            for (int q = 0; q < 4; ++q)
#pragma unroll
                                for (int c = 0; c < LT; ++c) a[c] = Opnd<MOE_BF16>::mfma(av[q], tb[c][4 * kg + q], a[c]);
#pragma unroll
                            for (int c = 0; c < LT; ++c)
#pragma unroll
                                for (int v = 0; v < 4; ++v)
                                    acc[gg][t][c][v] = __builtin_fmaf(s4[v], a[c][v], acc[gg][t][c][v]);
                        }
                    }
                }
            };
            body(lt_tag);
        };
        // LT live token tiles, fixed per pass: a pass whose rows fit in fewer
        // tiles than NT loads and multiplies only those, and its loop carries
        // no per-tile branch
        auto steps = [&](auto lt_tag) __attribute__((always_inline)) {
            // step 0's token values first: their addresses wait on the row-id
            // loads, and a wait placed after the copies would retire those too
            tload(tb0, 0, lt_tag);
            if (0 < nw) {
                issue_scales(0);
                issue(0);
            }
            int j = 0;
            for (; j + 1 < nw; j += 2) {
                step(j, tb0, tb1, lt_tag);
                step(j + 1, tb1, tb0, lt_tag);
            }
            if (j < nw) step(j, tb0, tb1, lt_tag);
        };
        if constexpr (NT > 1) {
            if (ntiles == NT)
                steps(std::integral_constant<int, NT>{});
            else
                steps(std::integral_constant<int, 1>{});
        } else {
            steps(std::integral_constant<int, 1>{});
        }

        // every wave is done with its ring: the reduction area aliases it
        __syncthreads();
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < NT; ++c) red[((wave * G * T + gi * T + t) * NT + c) * 64 + lane] = acc[gi][t][c];
        __syncthreads();

        constexpr int kPer = (KIND == MOE_GEMM_GATE_UP_SILU) ? 2 : 4;  // output tiles per group
        const int units = G * kPer * ntiles;
        for (int u = wave; u < units; u += 4) {
            const int c = u / (G * kPer);
            const int gq = u % (G * kPer);
            const int gi = gq / kPer, q = gq % kPer;
            const int r = pass + c * 16 + lr;
            if (r >= cnt) continue;
            const int p = pair_id(r);
            if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
                f32x4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    gs += red[((w * G * T + gi * T + q) * NT + c) * 64 + lane];
                    us += red[((w * G * T + gi * T + q + 2) * NT + c) * 64 + lane];
                }
                float o[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = silu(gs[v]) * us[v];
                uint2 pk;
                pk.x = pack_bf2(o[0], o[1]);
                pk.y = pack_bf2(o[2], o[3]);
                const int n = n0 + gi * 32 + 16 * q + 4 * lg;
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.c) + (size_t)p * I + n) = pk;
            } else {
                f32x4 ys = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < 4; ++w) ys += red[((w * G * T + gi * T + q) * NT + c) * 64 + lane];
                const int n = n0 + gi * 64 + 16 * q + 4 * lg;
                if (g.cpart) {
                    *reinterpret_cast<f32x4*>(g.cpart + ((size_t)blockIdx.z * g.P + p) * N + n) = ys;
                } else {
                    uint2 pk;
                    pk.x = pack_bf2(ys[0], ys[1]);
                    pk.y = pack_bf2(ys[2], ys[3]);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.c) + (size_t)p * N + n) = pk;
                }
            }
        }
        // the next pass refills the rings over the reduction area
        __syncthreads();
    }
}

template <int KIND, int NT, int G>
static hipError_t launch_decode_w4_g(const GemmArgs& a, int nslots, hipStream_t s) {
    constexpr int KD = 2;
    constexpr int kRing = 4 * KD * (64 * kRingSB + 1024);
    constexpr int kRed = 4 * G * 4 * NT * 64 * 16;
    constexpr int kLds = kRing > kRed ? kRing : kRed;
    static_assert(kLds <= 160 * 1024, "LDS");
    const int rows = (KIND == MOE_GEMM_GATE_UP_SILU) ? 32 * G : 64 * G;
    const int ncols = (KIND == MOE_GEMM_GATE_UP_SILU) ? a.N / 2 : a.N;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_decode_w4_kernel<KIND, NT, G, KD>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemm_decode_w4_kernel<KIND, NT, G, KD>), dim3(ncols / rows, nslots, a.ksplit),
                       dim3(kDecThreads), kLds, s, a);
    return hipGetLastError();
}

template <int KIND, int NT>
static hipError_t launch_decode_w4_nt(const GemmArgs& a, int nslots, hipStream_t s) {
    // The int4 kernel is bound by its ALU work and one workgroup per CU leaves
    // one wavefront per SIMD: with one token tile the gate/up GEMM takes the
    // most row groups (4, 2, 1) that still give about 400 workgroups, the
    // down GEMM two groups from 512 workgroups (measured on the Mixtral and
    // 128-expert int4 layers against four and two fixed groups: 128 experts
    // at one token 32.1 -> 25.0 us, Mixtral at one token 56.3 -> 50.7, at 8
    // tokens 156.9 -> 147.2).  With two token tiles, one group (registers).
    const int ncols = (KIND == MOE_GEMM_GATE_UP_SILU) ? a.N / 2 : a.N;
    if constexpr (NT == 1) {
        if (a.ksplit == 1) {
            if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
                if (ncols % 128 == 0 && (long)(ncols / 128) * nslots >= 400)
                    return launch_decode_w4_g<KIND, NT, 4>(a, nslots, s);
                if (ncols % 64 == 0 && (long)(ncols / 64) * nslots >= 400)
                    return launch_decode_w4_g<KIND, NT, 2>(a, nslots, s);
            } else {
                if (ncols % 128 == 0 && (long)(ncols / 128) * nslots >= 512)
                    return launch_decode_w4_g<KIND, NT, 2>(a, nslots, s);
            }
        }
    }
    return launch_decode_w4_g<KIND, NT, 1>(a, nslots, s);
}

// ------------------------------------------------------------------- f32
//
// Plain fp32 path: one thread per (sorted row, output column), dot products
// straight from global memory.

template <int KIND>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g, int block_m, int cap) {
    const int n = blockIdx.y * 64 + (threadIdx.x & 63);
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= cap) return;
    const int e = g.tile_expert[r / block_m];
    if (e < 0) return;
    const int p = g.sorted[r];
    if (p >= g.P) return;
    const int K = g.K, N = g.N;
    const float* w = reinterpret_cast<const float*>(g.w) + (size_t)e * N * K;
    if constexpr (KIND == MOE_GEMM_GATE_UP_SILU) {
        const int I = N / 2;
        if (n >= I) return;
        const float* x = reinterpret_cast<const float*>(g.a) + (size_t)(p / g.topk) * K;
        float gs = 0.f, us = 0.f;
        for (int k = 0; k < K; ++k) {
            gs = fmaf(w[(size_t)n * K + k], x[k], gs);
            us = fmaf(w[(size_t)(I + n) * K + k], x[k], us);
        }
        reinterpret_cast<float*>(g.c)[(size_t)p * I + n] = gs / (1.0f + expf(-gs)) * us;
    } else {
        if (n >= N) return;
        const float* a = reinterpret_cast<const float*>(g.a) + (size_t)p * K;
        float s = 0.f;
        for (int k = 0; k < K; ++k) s = fmaf(w[(size_t)n * K + k], a[k], s);
        reinterpret_cast<float*>(g.c)[(size_t)p * N + n] = s;
    }
}

// --------------------------------------------------------------- dispatch

int prefill_supported_block_m(int block_m) { return block_m == 64 || block_m == 128; }

int down_ksplit(moe_dtype dtype, int M, int topk, int E, int N, int K, int block_m) {
    if (dtype == MOE_F32 || M == 0) return 1;
    GemmCall probe{MOE_GEMM_DOWN, dtype, nullptr, nullptr, nullptr, nullptr, {}, M, topk, E, N, K, block_m,
                   nullptr, nullptr};
    if (choose_gemm_path(probe) != GemmPath::kDecode) return 1;
    const long P = (long)M * topk;
    const long slots = P < E ? P : E;
    const long wgs = (long)(N / 64) * slots;  // one row group per workgroup
    // the LDS ring holds one or two workgroups per CU, so a split pays only
    // until one round of 256 workgroups is filled (measured: the Mixtral
    // layer at one token runs 6% faster in 2 splits than in 6, the
    // 128-expert one 10% faster unsplit than in 2)
    if (wgs >= 256) return 1;
    // 256-byte steps of a weight row
    const long rowb = dtype == MOE_BF16 ? 2L * K : dtype == MOE_W4A16 ? K / 2 : (long)K;
    const int steps = (int)(rowb / kDecSpan);
    int ks = (int)((256 + wgs - 1) / wgs);
    if (ks > kMaxKsplit) ks = kMaxKsplit;
    // at least three 256-byte steps per split
    if (ks > steps / 3) ks = steps / 3;
    return ks < 1 ? 1 : ks;
}

GemmPath choose_gemm_path(const GemmCall& g) {
    if (g.dtype == MOE_W4A16) return GemmPath::kDecode;  // the int4 kernel is a decode kernel
    const char* env = getenv("MOE_GEMM_PATH");
    const bool pre_ok = prefill_supported_block_m(g.block_m);
    if (env && strcmp(env, "decode") == 0) return GemmPath::kDecode;
    if (env && strcmp(env, "prefill") == 0 && pre_ok) return GemmPath::kPrefill;
    const long P = (long)g.M * g.topk;
    const long per_expert = P / g.E;
    // the tile kernel (weights read once per row tile) above 24 pairs per
    // expert for bf16; e4m3 products cost a quarter of bf16's per byte on the
    // f8f6f4 MFMA, so e4m3 takes it on 64-row tiles at any batch (what the
    // fused e4m3 layer asks for from two tokens up) and on 128-row tiles
    // above 32 pairs per expert
    if (g.dtype == MOE_FP8_E4M3 && g.block_m == 64 && pre_ok) return GemmPath::kPrefill;
    const long min_rows = (g.dtype == MOE_FP8_E4M3) ? 32 : 24;
    return (per_expert > min_rows && pre_ok) ? GemmPath::kPrefill : GemmPath::kDecode;
}

template <int KIND, int DT, int NT, int G, bool AQ>
static hipError_t launch_decode_ntga(const GemmArgs& a, int nslots, hipStream_t s) {
    // operands whose rows the MFMAs read as stored go through the LDS ring
    // kernel, and so does an e4m3 DOWN over the float32 intermediate with one
    // token tile (its token values through registers, quantised on load);
    // f32 calls and an e4m3 DOWN with more token tiles take the register kernel
    constexpr bool kF32Act = KIND == MOE_GEMM_DOWN && DT == MOE_FP8_E4M3 && !AQ;
    constexpr bool kRing = DT != MOE_F32 && (!kF32Act || NT == 1);
    // (two stages per ring: measured as fast as three on every decode
    // workload, and it leaves LDS for a second workgroup at one token tile)
    if constexpr (kRing) {
        return launch_decode_ring<KIND, DT, NT, G, 2, kF32Act>(a, nslots, s);
    } else {
        const int rows = (KIND == MOE_GEMM_GATE_UP_SILU) ? 32 * G : 64 * G;  // output columns per workgroup
        const int ncols = (KIND == MOE_GEMM_GATE_UP_SILU) ? a.N / 2 : a.N;
        constexpr size_t kLds = sizeof(f32x4) * 4 * G * 4 * NT * 64;  // the cross-wavefront reduction
        static_assert(kLds <= 160 * 1024, "LDS");
        // LDS above the default dynamic limit must be requested once per kernel
        static const hipError_t attr =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_decode_kernel<KIND, DT, NT, G, AQ>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((gemm_decode_kernel<KIND, DT, NT, G, AQ>), dim3(ncols / rows, nslots, a.ksplit),
                           dim3(kDecThreads), kLds, s, a);
        return hipGetLastError();
    }
}

template <int KIND, int DT, int NT, int G>
static hipError_t launch_decode_ntg(const GemmArgs& a, int nslots, hipStream_t s) {
    if constexpr (KIND == MOE_GEMM_DOWN && DT == MOE_FP8_E4M3) {
        if (a.act_q8) return launch_decode_ntga<KIND, DT, NT, G, true>(a, nslots, s);
    }
    return launch_decode_ntga<KIND, DT, NT, G, false>(a, nslots, s);
}

// Fraction of the workgroup slots of whole dispatch rounds that `wgs`
// workgroups of `lds` bytes each keep busy (LDS decides how many share a CU).
static double round_fill(double wgs, int lds) {
    const double slots = 256.0 * (160 * 1024 / lds);
    const double rounds = __builtin_ceil(wgs / slots);
    return rounds > 0 ? wgs / (rounds * slots) : 1.0;
}

template <int KIND, int DT, int NT>
static hipError_t launch_decode_nt(const GemmArgs& a, int nslots, long active_est, double active_exp,
                                   hipStream_t s) {
    // Two row groups per workgroup (twice the weight rows per token load):
    // measured on the Mixtral, 128-expert and e4m3 decode layers, the bf16
    // down GEMM gains from 256 workgroups up (Mixtral shape at 8 to 64 tokens:
    // 3-4% over one group), the gate/up GEMM only for bf16 with two token
    // tiles and at least 512 workgroups; the e4m3 down GEMM with one token
    // tile (token values quantised in registers) is as fast or faster with
    // one (64-expert layer at 8 tokens: 246 -> 233 us).  With one token
    // tile the bf16 gate/up GEMM takes two when a weight row is at least
    // 8 KB (Mixtral shape at 2 tokens 3.5% faster for the layer, at 4-8
    // tokens 0.4-0.6%; the 128-expert layer's 4 KB rows measured 1-2%
    // slower with two)
    const int ncols = (KIND == MOE_GEMM_GATE_UP_SILU) ? a.N / 2 : a.N;
    const int rows2 = (KIND == MOE_GEMM_GATE_UP_SILU) ? 64 : 128;
    const bool two = (KIND == MOE_GEMM_DOWN)
                         ? (NT < 4 && !(DT == MOE_FP8_E4M3 && NT == 1) && (long)(ncols / rows2) * active_est >= 256)
                         : (DT == MOE_BF16 && ((NT == 2 && (long)(ncols / rows2) * active_est >= 512) ||
                                               (NT == 1 && 2L * a.K >= 8192)));
    if constexpr (KIND == MOE_GEMM_GATE_UP_SILU && NT < 4) {
        // four row groups per workgroup for the gate/up GEMM: always for
        // e4m3 (a row holds half the bytes of a bf16 one, so one group is few
        // copy steps; measured 1-4% faster on the 64-expert layer at 1, 8
        // and 32 tokens), and for bf16 when the one-group grid is at most
        // 1024 workgroups and the four-group one, over the experts expected
        // to be active, still covers most CUs, so the launch fits in one
        // round (Mixtral shape at one token: 896 -> 224 workgroups, 7%
        // faster; with larger grids four groups measured 2-3% slower, and
        // the 128-expert layer at 4 tokens, about 175 four-group
        // workgroups, 5% slower than with one)
        const long g1 = (long)(ncols / 32) * active_est;
        const double g4_exp = (ncols / 128) * active_exp;
        if (ncols % 128 == 0 && a.ksplit == 1 &&
            (DT == MOE_FP8_E4M3 || (DT == MOE_BF16 && g1 <= 1024 && g4_exp >= 224.0)))
            return launch_decode_ntg<KIND, DT, NT, 4>(a, nslots, s);
    }
    if constexpr (KIND == MOE_GEMM_DOWN) {
        // a short K (at most eight 256-byte steps, two per wavefront) leaves
        // each workgroup little to stream against its fixed costs: four row
        // groups, unless two fill the chip's dispatch rounds better.  The
        // active experts are estimated for uniform top-k routing.  128-expert
        // layer, K = 768: at 256 tokens (all experts active, 1024 four-group
        // workgroups, whole rounds) four groups are fastest; at 16 tokens
        // (about 82 active: 659 four-group workgroups on 512 slots) two are
        // 4% faster for the layer (down GEMM 55 -> 49 us)
        const long steps = (long)a.K * Opnd<DT>::kElemBytes / kDecSpan;
        if constexpr (NT < 4) {
            if (steps <= 8 && a.ksplit == 1 && ncols % 256 == 0 && (long)(ncols / 256) * active_est >= 256) {
                const double fill4 = round_fill((ncols / 256) * active_exp, DecRing<NT, 4, 2, false>::Lds);
                const double fill2 = round_fill((ncols / 128) * active_exp, DecRing<NT, 2, 2, false>::Lds);
                if (fill2 > fill4 + 0.05) return launch_decode_ntg<KIND, DT, NT, 2>(a, nslots, s);
                return launch_decode_ntg<KIND, DT, NT, 4>(a, nslots, s);
            }
        }
    }
    if (two && a.ksplit == 1 && ncols % rows2 == 0) return launch_decode_ntg<KIND, DT, NT, 2>(a, nslots, s);
    return launch_decode_ntg<KIND, DT, NT, 1>(a, nslots, s);
}

// Token tiles of 16 rows per pass of the decode kernels: a high quantile of
// the rows per expert under uniform routing.
static int decode_token_tiles(int M, int topk, int E) {
    const double avg = (double)M * topk / E;
    const double hi = avg + 3.0 * __builtin_sqrt(avg) + 1.0;
    return hi <= 16.0 ? 1 : hi <= 32.0 ? 2 : 4;
}

template <int KIND, int DT>
static hipError_t launch_decode(const GemmArgs& a, int M, int topk, int E, hipStream_t s) {
    const long P = (long)M * topk;
    const int nslots = (int)(P < E ? P : E);
    const long active_est = nslots;
    const int nt = decode_token_tiles(M, topk, E);
    // expected distinct experts among M tokens' top-k picks under uniform routing
    const double active_exp = E * (1.0 - __builtin_pow(1.0 - (double)topk / E, (double)M));
    if (nt == 1) return launch_decode_nt<KIND, DT, 1>(a, nslots, active_est, active_exp, s);
    if (nt == 2) return launch_decode_nt<KIND, DT, 2>(a, nslots, active_est, active_exp, s);
    return launch_decode_nt<KIND, DT, 4>(a, nslots, active_est, active_exp, s);
}

bool fp8_down_quantises_on_load(int M, int topk, int E, int N, int K, int block_m) {
    GemmCall probe{MOE_GEMM_DOWN, MOE_FP8_E4M3, nullptr, nullptr, nullptr, nullptr, {}, M, topk, E, N, K, block_m,
                   nullptr, nullptr};
    return choose_gemm_path(probe) == GemmPath::kDecode && decode_token_tiles(M, topk, E) == 1;
}

template <int KIND, int DT>
static hipError_t launch_prefill(const GemmArgs& a, int block_m, int64_t cap, hipStream_t s) {
    const int nblk = (KIND == MOE_GEMM_GATE_UP_SILU) ? (a.N / 2) / 64 : a.N / 128;
    const int ntiles = (int)(cap / block_m);
    if (block_m == 64)
        hipLaunchKernelGGL((gemm_prefill_kernel<KIND, DT, 64>), dim3(nblk, ntiles), dim3(kPreThreads), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_prefill_kernel<KIND, DT, 128>), dim3(nblk, ntiles), dim3(kPreThreads), 0, s, a);
    return hipGetLastError();
}

template <int KIND>
static hipError_t launch_decode_w4(const GemmArgs& a, int M, int topk, int E, hipStream_t s) {
    const long P = (long)M * topk;
    const int nslots = (int)(P < E ? P : E);
    // one or two 16-row token tiles per pass (more rows per expert: more passes)
    if (decode_token_tiles(M, topk, E) == 1) return launch_decode_w4_nt<KIND, 1>(a, nslots, s);
    return launch_decode_w4_nt<KIND, 2>(a, nslots, s);
}

template <int KIND>
static hipError_t launch_kind(const GemmCall& c, const GemmArgs& a, int64_t cap, hipStream_t s) {
    if (c.dtype == MOE_W4A16) return launch_decode_w4<KIND>(a, c.M, c.topk, c.E, s);
    if (c.dtype == MOE_F32 && choose_gemm_path(c) == GemmPath::kDecode)
        return launch_decode<KIND, MOE_F32>(a, c.M, c.topk, c.E, s);
    if (c.dtype == MOE_F32) {
        const int ncols = (KIND == MOE_GEMM_GATE_UP_SILU) ? c.N / 2 : c.N;
        dim3 grid((unsigned)((cap + 3) / 4), (ncols + 63) / 64);
        hipLaunchKernelGGL((gemm_f32_kernel<KIND>), grid, dim3(256), 0, s, a, c.block_m, (int)cap);
        return hipGetLastError();
    }
    const GemmPath path = choose_gemm_path(c);
    const int n2 = (KIND == MOE_GEMM_GATE_UP_SILU) ? (c.N / 2) % (PrefillCfg::BN / 2) : c.N % PrefillCfg::BN;
    // the LDS-ring tile kernel addresses its operands with 32-bit offsets:
    // A (M token rows for GATE_UP, M * topk intermediate rows for DOWN) and
    // one expert's N weight rows must each stay below 4 GiB, else the
    // register-staged tile kernel (64-bit addresses) runs
    const uint64_t rowb = (uint64_t)c.K * (c.dtype == MOE_BF16 ? 2 : 1);
    const uint64_t arows = (uint64_t)c.M * (KIND == MOE_GEMM_GATE_UP_SILU ? 1 : c.topk);
    const bool off32 = arows * rowb <= 0xffffffffull && (uint64_t)c.N * rowb <= 0xffffffffull;
    const bool ring = path == GemmPath::kPrefill && (c.block_m == PrefillCfg::BM || c.block_m == PrefillCfg64::BM) &&
                      n2 == 0 && off32;
    if (c.dtype == MOE_BF16) {
        if (ring && c.block_m == PrefillCfg::BM) return launch_prefill2<KIND, MOE_BF16, PrefillCfg>(a, cap, c.E, s);
        if (ring) return launch_prefill2<KIND, MOE_BF16, PrefillCfg64>(a, cap, c.E, s);
        if (path == GemmPath::kPrefill) return launch_prefill<KIND, MOE_BF16>(a, c.block_m, cap, s);
        return launch_decode<KIND, MOE_BF16>(a, c.M, c.topk, c.E, s);
    }
    // the ring kernel reads e4m3 rows only: a bf16 intermediate (DOWN without
    // act_q8) is quantised on load by the register-staged kernels
    if (ring && (KIND == MOE_GEMM_GATE_UP_SILU || c.act_q8)) {
        if (c.block_m == PrefillCfg::BM) return launch_prefill2<KIND, MOE_FP8_E4M3, PrefillCfg>(a, cap, c.E, s);
        return launch_prefill2<KIND, MOE_FP8_E4M3, PrefillCfg64>(a, cap, c.E, s);
    }
    if (path == GemmPath::kPrefill) return launch_prefill<KIND, MOE_FP8_E4M3>(a, c.block_m, cap, s);
    return launch_decode<KIND, MOE_FP8_E4M3>(a, c.M, c.topk, c.E, s);
}

hipError_t launch_grouped_gemm(const GemmCall& c, hipStream_t s) {
    if (c.M == 0) return hipSuccess;
    // self-routing is implemented by the bf16, e4m3 and int4 decode kernels
    // only, for one token; any other kernel would read an alignment nobody
    // wrote.  e4m3 also takes its intermediate's amax through partials (the
    // DOWN launch quantises the float32 intermediate on load; a launch over
    // codes would need the separately quantised ones)
    const bool fp8_ok = c.dtype == MOE_FP8_E4M3 && c.amax_parts && !c.act_q8;
    if (c.route_logits && (c.M != 1 || !(c.dtype == MOE_BF16 || c.dtype == MOE_W4A16 || fp8_ok) ||
                           choose_gemm_path(c) != GemmPath::kDecode))
        return hipErrorInvalidValue;
    if (c.amax_parts && !(c.route_logits && c.dtype == MOE_FP8_E4M3)) return hipErrorInvalidValue;
    GemmArgs a{};
    a.a = c.a;
    a.a_scale = c.a_scale;
    a.w = c.w;
    a.w_scale = c.w_scale;
    a.sorted = c.al.sorted_ids;
    a.tile_expert = c.al.tile_expert;
    a.counts = c.al.expert_counts;
    a.offsets = c.al.expert_offsets;
    a.active = c.al.active_experts;
    a.num_active = c.al.num_active;
    a.topk = c.topk;
    a.N = c.N;
    a.K = c.K;
    a.P = c.M * c.topk;
    a.c = c.c;
    a.c_amax = c.c_amax;
    a.ksplit = c.ksplit;
    a.cpart = c.cpart;
    a.act_q8 = c.act_q8 ? 1 : 0;
    a.route_logits = c.route_logits;
    a.route_E = c.E;
    a.route_renorm = c.route_renorm;
    a.route_ids = c.route_ids;
    a.route_wts = c.route_wts;
    a.amax_parts = c.amax_parts;
    a.amax_nparts = c.amax_nparts;
    const int64_t cap = moe_align_capacity(c.M, c.topk, c.E, c.block_m);
    if (c.kind == MOE_GEMM_GATE_UP_SILU) return launch_kind<MOE_GEMM_GATE_UP_SILU>(c, a, cap, s);
    return launch_kind<MOE_GEMM_DOWN>(c, a, cap, s);
}

}  // namespace moe

namespace moe {

// ------------------------------------------------------- fp8 intermediate
//
// e4m3 codes of the float32 intermediate, s = amax/448 (ActQuant), for the
// down projections that read codes (tile kernels with many rows per expert,
// where every weight tile would otherwise re-read and re-quantise the
// four-byte rows).
__global__ void __launch_bounds__(256) quant_act_kernel(const float* __restrict__ act,
                                                        const float* __restrict__ amax, uint8_t* __restrict__ q,
                                                        size_t n4) {
    const ActQuant quant(act_scale_from_amax(amax));
    // each lane converts 4 consecutive values per round: a wavefront reads
    // 1 KB and writes 256 contiguous bytes per instruction
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(act) + i);
        reinterpret_cast<uint32_t*>(q)[i] = quant.pack4(uint4{v.x, v.y, v.z, v.w});
    }
}

hipError_t launch_quant_act(const void* act, const float* amax, void* q, size_t n, hipStream_t s) {
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    const size_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                       static_cast<const float*>(act), amax, static_cast<uint8_t*>(q), n4);
    return hipGetLastError();
}

}  // namespace moe

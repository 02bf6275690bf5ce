// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// OCP e4m3 codes of four floats (round to nearest even; |v| <= 448 assumed).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (__lane_id() == 0) ? 0ull : (~0ull >> (64 - __lane_id()));
}

// ------------------------------------------------------- top-k of one token
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

}  // namespace moe

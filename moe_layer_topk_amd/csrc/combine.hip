// Weighted combine back into token order (FusedMoE vs MegaMoE post, section
// 3.1 step 4): out[t] = sum_j w[t,j] * y[t*k+j], j ascending, fp32 sums.
// Each thread owns 8 consecutive hidden elements of one token, so a token's
// k expert rows are read as contiguous 16-byte (bf16) or 32-byte (f32)
// vectors and the result is written once.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

template <int YDT, int ODT>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ w, int topk, int H,
                                                      void* __restrict__ out) {
    const int t = blockIdx.x;
    const int h = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (h >= H) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (YDT == MOE_BF16) {
        // all k rows' loads are issued before the first use (one memory
        // latency per thread, not k); the sum still runs j ascending
        uint4 v[kMaxTopk];
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j)
            if (j < topk)
                v[j] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) +
                                                       ((size_t)t * topk + j) * H + h);
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j) {
            if (j < topk) {
                const float wj = w[(size_t)t * topk + j];
                const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(wj, __uint_as_float(q[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(wj, __uint_as_float(q[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
        }
    } else
    for (int j = 0; j < topk; ++j) {
        const float wj = w[(size_t)t * topk + j];
        const size_t row = (size_t)t * topk + j;
        if (YDT == MOE_BF16) {
            const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) + row * H + h);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(wj, __uint_as_float(q[i] << 16), acc[2 * i]);
                acc[2 * i + 1] = fmaf(wj, __uint_as_float(q[i] & 0xffff0000u), acc[2 * i + 1]);
            }
        } else {
            const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + row * H + h);
            const float4 a = p[0], b = p[1];
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
        }
    }
    if (ODT == MOE_BF16) {
        uint4 o;
        o.x = pack_bf2(acc[0], acc[1]);
        o.y = pack_bf2(acc[2], acc[3]);
        o.z = pack_bf2(acc[4], acc[5]);
        o.w = pack_bf2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + h) = o;
    } else {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)t * H + h);
        p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

hipError_t launch_combine(moe_dtype y_dtype, const void* y, const float* w, int M, int topk, int H,
                          moe_dtype out_dtype, void* out, hipStream_t s) {
    if (M == 0) return hipSuccess;
    dim3 grid(M, (H / 8 + 255) / 256);
    if (y_dtype == MOE_BF16 && out_dtype == MOE_BF16)
        hipLaunchKernelGGL((combine_kernel<MOE_BF16, MOE_BF16>), grid, dim3(256), 0, s, y, w, topk, H, out);
    else if (y_dtype == MOE_BF16)
        hipLaunchKernelGGL((combine_kernel<MOE_BF16, MOE_F32>), grid, dim3(256), 0, s, y, w, topk, H, out);
    else if (out_dtype == MOE_BF16)
        hipLaunchKernelGGL((combine_kernel<MOE_F32, MOE_BF16>), grid, dim3(256), 0, s, y, w, topk, H, out);
    else
        hipLaunchKernelGGL((combine_kernel<MOE_F32, MOE_F32>), grid, dim3(256), 0, s, y, w, topk, H, out);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Split-K variant: the down projection left ksplit float32 partial rows per
// pair; y[p] = sum over z ascending, then out[t] = sum_j w[t,j] y[t*k+j] with
// j ascending, so the result does not depend on scheduling.
template <int ODT>
__global__ void __launch_bounds__(256) combine_partials_kernel(const float* __restrict__ ypart, int ksplit,
                                                               size_t zstride, const float* __restrict__ w,
                                                               int topk, int H, void* __restrict__ out) {
    const int t = blockIdx.x;
    const int h = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (h >= H) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
        const float wj = w[(size_t)t * topk + j];
        const float* row = ypart + ((size_t)t * topk + j) * H + h;
        // the ksplit partial loads of a row are issued together, then summed z ascending
        float4 a[kMaxKsplit], b[kMaxKsplit];
#pragma unroll
        for (int z = 0; z < kMaxKsplit; ++z) {
            if (z < ksplit) {
                const float4* p = reinterpret_cast<const float4*>(row + z * zstride);
                a[z] = p[0];
                b[z] = p[1];
            }
        }
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int z = 0; z < kMaxKsplit; ++z) {
            if (z < ksplit) {
                y[0] += a[z].x; y[1] += a[z].y; y[2] += a[z].z; y[3] += a[z].w;
                y[4] += b[z].x; y[5] += b[z].y; y[6] += b[z].z; y[7] += b[z].w;
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, y[i], acc[i]);
    }
    if (ODT == MOE_BF16) {
        uint4 o;
        o.x = pack_bf2(acc[0], acc[1]);
        o.y = pack_bf2(acc[2], acc[3]);
        o.z = pack_bf2(acc[4], acc[5]);
        o.w = pack_bf2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + h) = o;
    } else {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)t * H + h);
        p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

hipError_t launch_combine_partials(const float* ypart, int ksplit, const float* w, int M, int topk, int H,
                                   moe_dtype out_dtype, void* out, hipStream_t s) {
    if (M == 0) return hipSuccess;
    dim3 grid(M, (H / 8 + 255) / 256);
    const size_t zstride = (size_t)M * topk * H;
    if (out_dtype == MOE_BF16)
        hipLaunchKernelGGL((combine_partials_kernel<MOE_BF16>), grid, dim3(256), 0, s, ypart, ksplit, zstride, w,
                           topk, H, out);
    else
        hipLaunchKernelGGL((combine_partials_kernel<MOE_F32>), grid, dim3(256), 0, s, ypart, ksplit, zstride, w,
                           topk, H, out);
    return hipGetLastError();
}

}  // namespace moe

// pack.hpp -- absmean ternary weight quantization and 4-per-byte packing.
//
// gamma = mean|W| ("absmean": "微软AI大模型炸场" s.1; whole-tensor mean in
// "BitNet b1.58 深度解析" s.2.2). The binary64 sum of |W| is the pairwise tree over the
// row-major array zero-padded to a power of two. The GPU evaluates exactly that tree:
//   stage A   each 256-thread block sums one aligned 4096-element subtree: a thread
//             reduces 16 consecutive elements as a 4-level tree, then the 256 thread
//             sums are combined in lane order (xor-butterfly inside each wave, then
//             (w0 + w1) + (w2 + w3)); fp addition is commutative, so a butterfly
//             step equals the tree node of the two siblings.
//   stage B   the same 4096-to-1 reduction on the binary64 partials, repeated until
//             one value is left. Missing elements and partials are +0.0, and x + 0.0
//             equals x, so padding to any larger power of two changes nothing.
// Codes q = clip(round_half_even(W / gamma), -1, 1) use an fp32 division
// ("BitNet b1.58 深度解析" s.2.2); packing: byte j of row n holds codes 4j..4j+3, code
// 4j+i as the field q + 1 in bits 2i..2i+1 ("微软AI大模型炸场" s.3, several ternary
// values per 8-bit integer; "BitNet b1.58 深度解析" s.2.1, 2-bit codes, one state unused).
#pragma once

#include "device_common.hpp"

namespace bl {

constexpr int kSumChunk = 4096;  // elements per block in the |W| tree

// 16 values -> pairwise tree of depth 4.
__device__ __forceinline__ double tree16(const double d[16])
{
    double a[8], b[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        a[i] = d[2 * i] + d[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        b[i] = a[2 * i] + a[2 * i + 1];
    return (b[0] + b[1]) + (b[2] + b[3]);
}

// Combine the 256 per-thread subtree sums of a block in lane order.
__device__ __forceinline__ double block_tree256(double s)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        s += __shfl_xor(s, m);
    __shared__ double wsum[4];
    if ((threadIdx.x & (kWave - 1)) == 0)
        wsum[threadIdx.x / kWave] = s;
    __syncthreads();
    return (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// Stage A: |W| (fp32) -> one binary64 partial per 4096 elements.
__global__ __launch_bounds__(256) void abs_sum_f32_kernel(const float* __restrict__ w, int64_t n,
                                                          double* __restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * kSumChunk + (int64_t)threadIdx.x * 16;
    double d[16];
    if (base + 16 <= n) {
        const float4* p = reinterpret_cast<const float4*>(w + base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = p[i];
            d[4 * i + 0] = fabs((double)v.x);
            d[4 * i + 1] = fabs((double)v.y);
            d[4 * i + 2] = fabs((double)v.z);
            d[4 * i + 3] = fabs((double)v.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            d[i] = (base + i < n) ? fabs((double)w[base + i]) : 0.0;
    }
    const double s = block_tree256(tree16(d));
    if (threadIdx.x == 0)
        out[blockIdx.x] = s;
}

// Stage B: binary64 partials -> one partial per 4096 of them.
__global__ __launch_bounds__(256) void sum_f64_kernel(const double* __restrict__ in, int64_t n,
                                                      double* __restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * kSumChunk + (int64_t)threadIdx.x * 16;
    double d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        d[i] = (base + i < n) ? in[base + i] : 0.0;
    const double s = block_tree256(tree16(d));
    if (threadIdx.x == 0)
        out[blockIdx.x] = s;
}

__device__ __forceinline__ float gamma_from_sum(double S, int64_t n)
{
    float g = (float)(S / (double)n);
    return g < kFloor ? kFloor : g;
}

__device__ __forceinline__ uint32_t weight_field(float w, float gamma)
{
    float r = __builtin_rintf(w / gamma);
    r = r > 1.0f ? 1.0f : r;
    r = r < -1.0f ? -1.0f : r;
    return (uint32_t)((int)r + 1);
}

// Quantize + pack. Thread i produces packed bytes 4i..4i+3 (weights 16i..16i+15); the
// flat row-major order makes the packing independent of the row length because K % 4
// == 0 keeps every byte inside one row.
__global__ __launch_bounds__(256) void quant_pack_kernel(const float* __restrict__ w, int64_t n,
                                                         const double* __restrict__ sum, float* __restrict__ gamma_out,
                                                         uint8_t* __restrict__ packed)
{
    const float gamma = gamma_from_sum(*sum, n);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *gamma_out = gamma;
    const int64_t nbytes = n >> 2;
    const int64_t nwords = (nbytes + 3) >> 2;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * 256) {
        const int64_t e0 = i * 16;
        if (e0 + 16 <= n) {
            const float4* p = reinterpret_cast<const float4*>(w + e0);
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float4 v = p[b];
                const uint32_t byte = weight_field(v.x, gamma) | (weight_field(v.y, gamma) << 2) |
                                      (weight_field(v.z, gamma) << 4) | (weight_field(v.w, gamma) << 6);
                word |= byte << (8 * b);
            }
            reinterpret_cast<uint32_t*>(packed)[i] = word;
        } else {
            for (int64_t byte_i = i * 4; byte_i < nbytes; ++byte_i) {
                uint32_t byte = 0;
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    byte |= weight_field(w[byte_i * 4 + f], gamma) << (2 * f);
                packed[byte_i] = (uint8_t)byte;
            }
        }
    }
}

}  // namespace bl

// quant.hpp -- per-token absmax int8 activation quantization (optionally with the
// squared-ReLU or gated squared-ReLU + RMSNorm subln input), one 256-thread block per
// token.
//
// Absmax per token with scale 127/max(|x|, 1e-8), round, clamp to [-128, 127]:
// "BitNet b1.58 深度解析" s.2.2 and, for the per-token granularity, "微软AI大模型炸场"
// s.1 and "20亿参数仅0.4GB" s.2. The subln input folds the RMSNorm factor into the
// stored scale (the factor cancels inside absmax), so the codes are order-free.
#pragma once

#include "device_common.hpp"

namespace bl {

struct QuantArgs {
    const float* X;      // [M][K], or [M][2K] = [gate | up] when act == 2
    const float* gain;
    int8_t* Xq;
    float* scale;
    int64_t M;
    int K;
    float eps;
    int act;             // 0 identity, 1 squared ReLU, 2 gated squared ReLU
};

// Pass 1: block statistics of the token. Pass 2: codes, four per 32-bit store; the
// row is re-read (it is L2-resident after pass 1).
__global__ __launch_bounds__(256) void quantize_act_kernel(QuantArgs a)
{
    int calls = 0;  // statistics calls so far: their LDS slots alternate
    for (int64_t t = blockIdx.x; t < a.M; t += gridDim.x) {
        const int64_t stride = a.act == 2 ? 2 * (int64_t)a.K : (int64_t)a.K;
        const float* u = a.X + t * stride;
        const float* up = a.act == 2 ? u + a.K : nullptr;
        const bool norm = a.gain != nullptr;
        const RowStats st = row_stats<0, true>(u, a.K, a.gain, a.act, norm, up, calls++ & 1);
        float sp, s;
        token_scales(st, a.K, norm, a.eps, sp, s);
        if (threadIdx.x == 0)
            a.scale[t] = s;
        uint32_t* out = reinterpret_cast<uint32_t*>(a.Xq + t * (int64_t)a.K);
        const int G = a.K >> 2;
#pragma unroll 4
        for (int g = threadIdx.x; g < G; g += 256) {
            const float4 x = reinterpret_cast<const float4*>(u)[g];
            float4 gv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            float4 uv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            if (a.gain)
                gv = reinterpret_cast<const float4*>(a.gain)[g];
            if (up)
                uv = reinterpret_cast<const float4*>(up)[g];
            const float xa[4] = {x.x, x.y, x.z, x.w};
            const float ga[4] = {gv.x, gv.y, gv.z, gv.w};
            const float ub[4] = {uv.x, uv.y, uv.z, uv.w};
            uint32_t word = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float v = act_v(xa[c], ub[c], a.act);
                const float w = a.gain ? v * ga[c] : v;
                word |= (uint32_t)(act_code(w, sp) & 0xff) << (8 * c);
            }
            out[g] = word;
        }
    }
}

}  // namespace bl

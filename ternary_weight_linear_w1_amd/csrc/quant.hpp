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

// Pass 1: block statistics of the token. Pass 2: codes; the row is read again (it is
// L2-resident after pass 1). Both passes keep kQuantUnits units of 16 elements per thread
// in flight and visit the units in the order of the fused GEMV prologue, so the two entry
// points give the same bits.
constexpr int kQuantUnits = 4;

__global__ __launch_bounds__(256) void quantize_act_kernel(QuantArgs a)
{
    int calls = 0;  // statistics calls so far: their LDS slots alternate
    const int units = (a.K + 15) >> 4;
    const bool wide = (a.K & 15) == 0;   // whole units: one 16-byte store each
    with_mode(a.act, a.gain != nullptr, [&](auto md) {
        using MD = decltype(md);
        constexpr int NB = kQuantUnits;
        for (int64_t t = blockIdx.x; t < a.M; t += gridDim.x) {
            const RowRes rr = row_res(a.X, t, a.K, MD::kAct, a.gain);
            const RowStats st = row_stats_units<MD, NB>(rr, units, calls++ & 1);
            float sp, s;
            token_scales(st, a.K, MD::kNorm, a.eps, sp, s);
            if (threadIdx.x == 0)
                a.scale[t] = s;
            // the store range ends at the row end: codes of groups past it are dropped
            const __amdgpu_buffer_rsrc_t out =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.Xq + t * (int64_t)a.K), (short)0, a.K, kRowFlags);
            for (int u = threadIdx.x; u < units; u += NB * 256) {
                UnitRaw in[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    unit_load<MD>(rr, u + 256 * b, in[b]);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float w[16], m = 0.0f;
                    double q = 0.0;
                    unit_visit<MD>(in[b], w, m, q);
                    const uint4 c = unit_codes(w, sp);
                    const int ub = u + 256 * b;
                    if (wide) {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c), out, 16 * ub, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b32((int)c.x, out, 16 * ub, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b32((int)c.y, out, 16 * ub + 4, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b32((int)c.z, out, 16 * ub + 8, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b32((int)c.w, out, 16 * ub + 12, 0, 0);
                    }
                }
            }
        }
    });
}

}  // namespace bl

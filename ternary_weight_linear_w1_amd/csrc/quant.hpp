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

// Pass 1: block statistics of the token. Pass 2: codes, sixteen per thread and step; the
// row is read again (it is L2-resident after pass 1). Both passes visit the units in the
// order of the fused GEMV prologue, so the two entry points give the same bits.
__global__ __launch_bounds__(256) void quantize_act_kernel(QuantArgs a)
{
    int calls = 0;  // statistics calls so far: their LDS slots alternate
    const int units = (a.K + 15) >> 4;
    const bool wide = (a.K & 15) == 0;   // whole units: one 16-byte store each
    with_mode(a.act, a.gain != nullptr, [&](auto md) {
        using MD = decltype(md);
        for (int64_t t = blockIdx.x; t < a.M; t += gridDim.x) {
            const RowRes rr = row_res(a.X, t, a.K, MD::kAct, a.gain);
            const RowStats st = row_stats_units<MD>(rr, units, calls++ & 1);
            float sp, s;
            token_scales(st, a.K, MD::kNorm, a.eps, sp, s);
            if (threadIdx.x == 0)
                a.scale[t] = s;
            // the store range ends at the row end: codes of groups past it are dropped
            const __amdgpu_buffer_rsrc_t out =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.Xq + t * (int64_t)a.K), (short)0, a.K, kRowFlags);
            for (int u = threadIdx.x; u < units; u += 512) {
                UnitRaw in0, in1;
                unit_load<MD>(rr, u, in0);
                unit_load<MD>(rr, u + 256, in1);
                float w0[16], w1[16], m = 0.0f;
                double q = 0.0;
                unit_visit<MD>(in0, w0, m, q);
                unit_visit<MD>(in1, w1, m, q);
                const uint4 c0 = unit_codes(w0, sp), c1 = unit_codes(w1, sp);
                if (wide) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c0), out, 16 * u, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c1), out, 16 * (u + 256), 0, 0);
                } else {
                    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32((int)cw[e], out, 16 * (u + 256 * (e >> 2)) + 4 * (e & 3),
                                                              0, 0);
                }
            }
        }
    });
}

}  // namespace bl

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

// Per token: the first UK units per thread are loaded at once and their w values stay in
// registers from the statistics to the codes, so a row of up to UK * 4096 elements is read
// once; longer rows visit the rest (two units at a time with UK = 8) and read it again
// for the codes.
// Units are visited in the order of the fused GEMV prologue (per thread t: t, t + 256, ...),
// so the two entry points give the same bits. UK is chosen from K at launch: few registers
// (many blocks per CU) for short rows.
template <int UK>
__global__ __launch_bounds__(256) void quantize_act_kernel(QuantArgs a)
{
    int calls = 0;  // statistics calls so far: their LDS slots alternate
    const int tid = threadIdx.x;
    const int units = (a.K + 15) >> 4;
    const bool wide = (a.K & 15) == 0;   // whole units: one 16-byte store each
    with_mode(a.act, a.gain != nullptr, [&](auto md) {
        using MD = decltype(md);
        for (int64_t t = blockIdx.x; t < a.M; t += gridDim.x) {
            const RowRes rr = row_res(a.X, t, a.K, MD::kAct, a.gain);
            float w[UK][16];
            float mx = 0.0f;
            double ss = 0.0;
            {
                UnitRaw in[UK];
#pragma unroll
                for (int i = 0; i < UK; ++i)
                    unit_load<MD>(rr, tid + 256 * i, in[i]);   // past the row: zeros
#pragma unroll
                for (int i = 0; i < UK; ++i)
                    unit_visit<MD>(in[i], w[i], mx, ss);
            }
            if constexpr (UK >= 8) {
#pragma unroll 1
                for (int u = tid + 256 * UK; u < units; u += 512) {
                    UnitRaw in0, in1;
                    unit_load<MD>(rr, u, in0);
                    unit_load<MD>(rr, u + 256, in1);
                    float tmp[16];
                    unit_visit<MD>(in0, tmp, mx, ss);
                    unit_visit<MD>(in1, tmp, mx, ss);
                }
            } else {   // rows up to UK units per thread are launched with this UK
#pragma unroll 1
                for (int u = tid + 256 * UK; u < units; u += 256) {
                    UnitRaw in;
                    unit_load<MD>(rr, u, in);
                    float tmp[16];
                    unit_visit<MD>(in, tmp, mx, ss);
                }
            }
            const RowStats st = block_stats(mx, ss, MD::kNorm, calls++ & 1);
            float sp, s;
            token_scales(st, a.K, MD::kNorm, a.eps, sp, s);
            if (tid == 0)
                a.scale[t] = s;
            // the store range ends at the row end: codes of groups past it are dropped
            const __amdgpu_buffer_rsrc_t out =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.Xq + t * (int64_t)a.K), (short)0, a.K, kRowFlags);
            auto store = [&](int u, const float (&wv)[16]) {
                const uint4 c = unit_codes(wv, sp);
                if (wide) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c), out, 16 * u, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32((int)c.x, out, 16 * u, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32((int)c.y, out, 16 * u + 4, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32((int)c.z, out, 16 * u + 8, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32((int)c.w, out, 16 * u + 12, 0, 0);
                }
            };
#pragma unroll
            for (int i = 0; i < UK; ++i)
                if (tid + 256 * i < units)
                    store(tid + 256 * i, w[i]);
#pragma unroll 1
            for (int u = tid + 256 * UK; u < units; u += 256) {
                UnitRaw in;
                unit_load<MD>(rr, u, in);
                float wv[16], m2 = 0.0f;
                double s2 = 0.0;
                unit_visit<MD>(in, wv, m2, s2);
                store(u, wv);
            }
        }
    });
}

}  // namespace bl

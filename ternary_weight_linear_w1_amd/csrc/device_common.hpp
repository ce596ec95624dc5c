// device_common.hpp -- small device helpers shared by the BitLinear kernels (gfx950).
//
// Wave64 throughout. Every reduction here is either order-free (max, integer sums) or
// follows a fixed tree that depends only on the problem size, never on timing, so
// repeated calls and the fused/unfused entry points give identical bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kFloor = 1e-8f;  // floor of max|x| and of gamma
constexpr int kWave = 64;

// int8 code of one activation: clip(round_half_even(v * s), -128, 127). One fp32
// multiply, v_rndne_f32, then a clamp.
__device__ __forceinline__ int act_code(float v, float s)
{
    float r = __builtin_rintf(v * s);
    r = r > 127.0f ? 127.0f : r;
    r = r < -128.0f ? -128.0f : r;
    return (int)r;
}

// Elementwise activation of the subln input: act 0 = identity, 1 = squared ReLU,
// 2 = squared ReLU of the gate times the up value (gated FFN; `up` is the matching
// element of the second half of the row).
__device__ __forceinline__ float pre_v(float u, int act)
{
    if (act) {
        float p = u > 0.0f ? u : 0.0f;
        return p * p;
    }
    return u;
}

__device__ __forceinline__ float act_v(float u, float up, int act)
{
    float v = pre_v(u, act);
    if (act == 2)
        v = v * up;
    return v;
}

// Byte-transpose of four dwords: out[f] byte j = in[j] byte f. Eight v_perm_b32; a
// selector byte s picks byte s of the second operand (s < 4) or byte s-4 of the first.
__device__ __forceinline__ void transpose_bytes(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3,
                                                uint32_t out[4])
{
    const uint32_t p0 = __builtin_amdgcn_perm(e1, e0, 0x05010400u);  // e0.0 e1.0 e0.1 e1.1
    const uint32_t p1 = __builtin_amdgcn_perm(e1, e0, 0x07030602u);  // e0.2 e1.2 e0.3 e1.3
    const uint32_t p2 = __builtin_amdgcn_perm(e3, e2, 0x05010400u);  // e2.0 e3.0 e2.1 e3.1
    const uint32_t p3 = __builtin_amdgcn_perm(e3, e2, 0x07030602u);  // e2.2 e3.2 e2.3 e3.3
    out[0] = __builtin_amdgcn_perm(p2, p0, 0x05040100u);             // e0.0 e1.0 e2.0 e3.0
    out[1] = __builtin_amdgcn_perm(p2, p0, 0x07060302u);             // e0.1 e1.1 e2.1 e3.1
    out[2] = __builtin_amdgcn_perm(p3, p1, 0x05040100u);             // e0.2 e1.2 e2.2 e3.2
    out[3] = __builtin_amdgcn_perm(p3, p1, 0x07060302u);             // e0.3 e1.3 e2.3 e3.3
}

// ------------------------------------------------------------------------------------
// Wave reductions through DPP (row-local lane exchange, no LDS traffic). Each step adds
// a lane's value to its partner's; partners hold the same two operands, so after a step
// both hold the same bits (addition is commutative). Rows of 16 lanes are combined
// through readlane in the fixed order (r0 + r1) + (r2 + r3).

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
    v = v + dpp_f64<0xB1>(v);
    v = v + dpp_f64<0x4E>(v);
    v = v + dpp_f64<0x141>(v);
    v = v + dpp_f64<0x140>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ------------------------------------------------------------------------------------
// Per-token statistics of the (activation + gain) input, shared by the standalone
// quantizer and the fused GEMV prologue so that both produce the same bits. Blocks of
// 256 threads.
//
//   m     = max_k |w_k|,  w_k = act_v(u_k, up_k) * gain_k   (order-free)
//   sumsq = sum_k v_k^2 in binary64: thread t adds the float4 groups g = t, t+256, ...
//           in increasing order (components in order); the 256 thread sums are combined
//           by the fixed DPP/readlane tree of wave_sum_f64 per wave, then as
//           (w0 + w1) + (w2 + w3) over the four waves. The order depends only on K.
// The w values of the first KEEP groups of each thread (g = tid + 256 i, i < KEEP) are
// returned in `wk` so the caller can quantize them without re-reading.
// Must be called by all 256 threads of the block. `slot` (0 or 1) picks the LDS scratch;
// consecutive calls alternate it, so no barrier is needed after the call (a slot is
// written again only after every thread has passed the next call's barrier, which
// follows its reads of the slot).
// ------------------------------------------------------------------------------------
struct RowStats {
    float m;
    double sumsq;
};

// Loads of the first KEEP float4 groups of each thread (g = tid + 256 q), issued early
// so that they are not queued behind other loads; groups past the row give x = 0, g = 1.
template <int KEEP>
__device__ __forceinline__ void row_load(const float* __restrict__ u, int K, const float* __restrict__ gain,
                                         const float* __restrict__ up, float4 (&xa)[KEEP], float4 (&gb)[KEEP])
{
    const int G = K >> 2;
#pragma unroll
    for (int q = 0; q < KEEP; ++q) {
        const int g = (int)threadIdx.x + q * 256;
        xa[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        gb[q] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if (g < G) {
            xa[q] = reinterpret_cast<const float4*>(u)[g];
            const float* second = up ? up : gain;
            if (second)
                gb[q] = reinterpret_cast<const float4*>(second)[g];
        }
    }
}

// Statistics from values preloaded by row_load (KEEP > 0) or read here. WIDE keeps eight
// loads per thread in flight over the groups it reads itself (for long rows in the
// standalone quantizer; the summation order is unchanged, only registers grow).
template <int KEEP, bool WIDE = false>
__device__ RowStats row_stats_pre(const float* __restrict__ u, int K, const float* __restrict__ gain, int act,
                                  bool want_sumsq, const float* __restrict__ up,
                                  const float4 (&xa)[KEEP > 0 ? KEEP : 1], const float4 (&gb)[KEEP > 0 ? KEEP : 1],
                                  float4* wk, int slot)
{
    const int tid = threadIdx.x;
    const int G = K >> 2;
    double s = 0.0;
    float mx = 0.0f;
    auto visit = [&](float4 a, float4 gv, float4 uv) -> float4 {
        const float va[4] = {a.x, a.y, a.z, a.w};
        const float ga[4] = {gv.x, gv.y, gv.z, gv.w};
        const float ub[4] = {uv.x, uv.y, uv.z, uv.w};
        float wa[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float v = act_v(va[c], ub[c], act);
            if (want_sumsq)
                s += (double)v * (double)v;
            wa[c] = gain ? v * ga[c] : v;
            mx = fmaxf(mx, fabsf(wa[c]));
        }
        return make_float4(wa[0], wa[1], wa[2], wa[3]);
    };
    int g = tid;
    if constexpr (KEEP > 0) {
#pragma unroll
        for (int q = 0; q < KEEP; ++q) {
            if (g + q * 256 < G) {
                // gb holds the up values when gated (the gain, a small shared vector, is
                // then read here), else the gain
                float4 gv = gb[q];
                float4 uv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                if (up) {
                    uv = gb[q];
                    gv = gain ? reinterpret_cast<const float4*>(gain)[g + q * 256]
                              : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                }
                wk[q] = visit(xa[q], gv, uv);
            }
        }
        g += KEEP * 256;
    }
    // groups past the kept ones (WIDE: eight loads in flight per thread, visited in order,
    // which is the same summation order as one group at a time)
    for (; WIDE && g + 7 * 256 < G; g += 8 * 256) {
        float4 a[8], gv[8], uv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            a[q] = reinterpret_cast<const float4*>(u)[g + q * 256];
            gv[q] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            uv[q] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            if (gain)
                gv[q] = reinterpret_cast<const float4*>(gain)[g + q * 256];
            if (up)
                uv[q] = reinterpret_cast<const float4*>(up)[g + q * 256];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            visit(a[q], gv[q], uv[q]);
    }
    for (; g < G; g += 256) {
        const float4 a = reinterpret_cast<const float4*>(u)[g];
        float4 gv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        float4 uv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if (gain)
            gv = reinterpret_cast<const float4*>(gain)[g];
        if (up)
            uv = reinterpret_cast<const float4*>(up)[g];
        visit(a, gv, uv);
    }
    __shared__ float redm[2][4];
    __shared__ double red[2][4];
    const int wv = tid / kWave;
    mx = wave_max(mx);
    if (want_sumsq)
        s = wave_sum_f64(s);
    if ((tid & (kWave - 1)) == 0) {
        redm[slot][wv] = mx;
        red[slot][wv] = s;
    }
    __syncthreads();
    const float m = fmaxf(fmaxf(redm[slot][0], redm[slot][1]), fmaxf(redm[slot][2], redm[slot][3]));
    double total = 0.0;
    if (want_sumsq)
        total = (red[slot][0] + red[slot][1]) + (red[slot][2] + red[slot][3]);
    return RowStats{m, total};
}

template <int KEEP = 0, bool WIDE = false>
__device__ RowStats row_stats(const float* __restrict__ u, int K, const float* __restrict__ gain, int act,
                              bool want_sumsq, const float* __restrict__ up, int slot, float4* wk = nullptr)
{
    float4 xa[KEEP > 0 ? KEEP : 1], gb[KEEP > 0 ? KEEP : 1];
    if constexpr (KEEP > 0)
        row_load<KEEP>(u, K, gain, up, xa, gb);
    return row_stats_pre<KEEP, WIDE>(u, K, gain, act, want_sumsq, up, xa, gb, wk, slot);
}

__device__ __forceinline__ void token_scales(const RowStats& st, int K, bool norm, float eps, float& sp, float& s)
{
    const float m = st.m < kFloor ? kFloor : st.m;
    sp = 127.0f / m;
    if (norm) {
        const double ms = st.sumsq / (double)K;
        s = (float)((double)sp * sqrt(ms + (double)eps));
    } else {
        s = sp;
    }
}

}  // namespace bl

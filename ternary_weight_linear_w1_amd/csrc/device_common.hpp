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
// Per-token prologue: statistics and codes of the (activation + gain) input, shared by
// the standalone quantizer and the fused GEMV prologues so that both produce the same
// bits. Blocks of 256 threads.
//
// A unit is 16 consecutive elements of a row (four float4 groups); thread t owns units
// t, t + 256, t + 512, ... . Rows are read through buffer loads whose range ends at the
// row end, so groups past it read as zero: a zero input adds nothing to the maximum or
// the sum of squares and gets code 0, and loops may run past the row without checks.
//
//   v_k   = x_k, max(x_k, 0)^2, or max(x_k, 0)^2 * up_k     (act 0, 1, 2)
//   w_k   = v_k * gain_k (RMSNorm input) or v_k
//   m     = max_k |w_k|                                       (order-free)
//   sumsq = sum_k v_k^2 in binary64 (v_k^2 is exact there): each thread adds its units in
//           increasing order, elements in order; the 256 thread sums are combined by the
//           fixed DPP/readlane tree of wave_sum_f64 per wave, then as (w0 + w1) + (w2 + w3)
//           over the four waves. The order depends only on K.
//
// The activation kind and the norm are template parameters of the arithmetic (no
// per-element selects); with_mode() turns the runtime values into them once.
// ------------------------------------------------------------------------------------
struct RowStats {
    float m;
    double sumsq;
};

constexpr int kRowFlags = 0x00020000;  // buffer descriptor word 3 (gfx9)

// Buffer ranges of one token: x (the gate half when gated), y = up (gated) or gain (norm),
// z = gain when gated and normed. An operand that is not used has an empty range.
struct RowRes {
    __amdgpu_buffer_rsrc_t x, y, z;
};

__device__ __forceinline__ RowRes row_res(const float* X, int64_t tok, int K, int act, const float* gain)
{
    const float* x = X + tok * (act == 2 ? 2 * (int64_t)K : (int64_t)K);
    const float* y = act == 2 ? x + K : gain;
    const float* z = act == 2 ? gain : nullptr;
    RowRes r;
    r.x = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, 4 * K, kRowFlags);
    r.y = __builtin_amdgcn_make_buffer_rsrc((void*)(y ? y : x), (short)0, y ? 4 * K : 0, kRowFlags);
    r.z = __builtin_amdgcn_make_buffer_rsrc((void*)(z ? z : x), (short)0, z ? 4 * K : 0, kRowFlags);
    return r;
}

struct UnitRaw {
    float4 x[4], y[4], z[4];
};

__device__ __forceinline__ float4 load_f4(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float f4_get(const float4& v, int c)
{
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

template <int ACT, bool NORM>
struct Mode {
    static constexpr int kAct = ACT;
    static constexpr bool kNorm = NORM;
    static constexpr bool kY = ACT == 2 || NORM;     // up or gain in y
    static constexpr bool kZ = ACT == 2 && NORM;     // gain in z
};

// f(Mode<act, norm>{}) for the runtime activation kind (0, 1, 2) and norm flag.
template <typename F>
__device__ __forceinline__ void with_mode(int act, bool norm, F&& f)
{
    if (act == 0) {
        if (norm) f(Mode<0, true>{}); else f(Mode<0, false>{});
    } else if (act == 1) {
        if (norm) f(Mode<1, true>{}); else f(Mode<1, false>{});
    } else {
        if (norm) f(Mode<2, true>{}); else f(Mode<2, false>{});
    }
}

// Loads of unit u (elements 16u .. 16u + 15).
template <class MD>
__device__ __forceinline__ void unit_load(const RowRes& rr, int u, UnitRaw& in)
{
    const int off = u << 6;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        in.x[q] = load_f4(rr.x, off + 16 * q);
        if constexpr (MD::kY)
            in.y[q] = load_f4(rr.y, off + 16 * q);
        if constexpr (MD::kZ)
            in.z[q] = load_f4(rr.z, off + 16 * q);
    }
}

// x and y with y chosen at run time (a uniform branch), for loads that are issued before
// the mode-specialised code is entered; z (gated and normed) is left to unit_load_z.
__device__ __forceinline__ void unit_load_xy(const RowRes& rr, int u, bool ly, UnitRaw& in)
{
    const int off = u << 6;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        in.x[q] = load_f4(rr.x, off + 16 * q);
    if (ly) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            in.y[q] = load_f4(rr.y, off + 16 * q);
    }
}

__device__ __forceinline__ void unit_load_z(const RowRes& rr, int u, float4 (&z)[4])
{
    const int off = u << 6;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        z[q] = load_f4(rr.z, off + 16 * q);
}

// w of the 16 elements of a unit, folded into the running max |w| and sum of v^2.
template <class MD>
__device__ __forceinline__ void unit_visit(const float4 (&x)[4], const float4 (&y)[4], const float4 (&z)[4],
                                           float (&w)[16], float& mx, double& ss)
{
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float v = f4_get(x[e >> 2], e & 3);
        if constexpr (MD::kAct >= 1) {
            const float p = v > 0.0f ? v : 0.0f;
            v = p * p;
        }
        if constexpr (MD::kAct == 2)
            v = v * f4_get(y[e >> 2], e & 3);
        float wv = v;
        if constexpr (MD::kNorm) {
            ss = __builtin_fma((double)v, (double)v, ss);   // = ss + v*v: the product is exact
            wv = v * f4_get((MD::kAct == 2 ? z : y)[e >> 2], e & 3);
        }
        w[e] = wv;
        mx = fmaxf(mx, fabsf(wv));
    }
}

template <class MD>
__device__ __forceinline__ void unit_visit(const UnitRaw& in, float (&w)[16], float& mx, double& ss)
{
    unit_visit<MD>(in.x, in.y, in.z, w, mx, ss);
}

// Block maximum and binary64 sum (fixed tree). Must be called by all 256 threads. `slot`
// (0 or 1) picks the LDS scratch; consecutive calls alternate it, so no barrier is needed
// after the call (a slot is written again only after every thread has passed the next
// call's barrier, which follows its reads of the slot).
__device__ __forceinline__ RowStats block_stats(float mx, double ss, bool want_sumsq, int slot)
{
    __shared__ float redm[2][4];
    __shared__ double red[2][4];
    const int tid = threadIdx.x;
    const int wv = tid / kWave;
    mx = wave_max(mx);
    if (want_sumsq)
        ss = wave_sum_f64(ss);
    if ((tid & (kWave - 1)) == 0) {
        redm[slot][wv] = mx;
        red[slot][wv] = ss;
    }
    __syncthreads();
    const float m = fmaxf(fmaxf(redm[slot][0], redm[slot][1]), fmaxf(redm[slot][2], redm[slot][3]));
    double total = 0.0;
    if (want_sumsq)
        total = (red[slot][0] + red[slot][1]) + (red[slot][2] + red[slot][3]);
    return RowStats{m, total};
}

// block_stats for MT tokens at once (one barrier); each token's sum in the same order.
// Its LDS scratch is rewritten only after the caller's next block-wide barrier.
template <int MT>
__device__ __forceinline__ void block_stats_multi(const float (&mx)[MT], const double (&ss)[MT], bool want_sumsq,
                                                  RowStats (&st)[MT])
{
    __shared__ float redm[MT][4];
    __shared__ double red[MT][4];
    const int tid = threadIdx.x;
    const int wv = tid / kWave;
    float m[MT];
    double q[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        m[t] = wave_max(mx[t]);
        q[t] = want_sumsq ? wave_sum_f64(ss[t]) : 0.0;
    }
    if ((tid & (kWave - 1)) == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            redm[t][wv] = m[t];
            red[t][wv] = q[t];
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        st[t].m = fmaxf(fmaxf(redm[t][0], redm[t][1]), fmaxf(redm[t][2], redm[t][3]));
        st[t].sumsq = want_sumsq ? (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]) : 0.0;
    }
}

// Buffer ranges that read nothing (every load gives zeros).
__device__ __forceinline__ RowRes row_res_empty(const float* any)
{
    RowRes r;
    r.x = __builtin_amdgcn_make_buffer_rsrc((void*)any, (short)0, 0, kRowFlags);
    r.y = r.x;
    r.z = r.x;
    return r;
}

// Statistics of a whole row: units t, t + 256, ... read NB at a time (the per-thread
// order of the sum is unchanged; units past the row read zeros and change nothing).
template <class MD, int NB = 2>
__device__ __forceinline__ RowStats row_stats_units(const RowRes& rr, int nunits, int slot)
{
    float mx = 0.0f;
    double ss = 0.0;
    for (int u = threadIdx.x; u < nunits; u += NB * 256) {
        UnitRaw in[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            unit_load<MD>(rr, u + 256 * b, in[b]);
        float w[16];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            unit_visit<MD>(in[b], w, mx, ss);
    }
    return block_stats(mx, ss, MD::kNorm, slot);
}

// Four int32 values (their low bytes) as the bytes 0..3 of a dword.
__device__ __forceinline__ uint32_t pack_bytes(int c0, int c1, int c2, int c3)
{
    return __builtin_amdgcn_perm((uint32_t)c1, (uint32_t)c0, 0x0c0c0400u) |
           __builtin_amdgcn_perm((uint32_t)c3, (uint32_t)c2, 0x04000c0cu);
}

// Codes round_half_even(w * sp) of a unit. sp = 127 / m' with m' >= max |w| over the row,
// so |w * sp| <= 127 (1 + 2^-24)^2 < 127.5 and the clip to [-128, 127] can never act.
// Natural order: dword q holds codes 4q .. 4q + 3 (bytes in order).
__device__ __forceinline__ uint4 unit_codes(const float (&w)[16], float sp)
{
    int c[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
        c[e] = (int)__builtin_rintf(w[e] * sp);
    return make_uint4(pack_bytes(c[0], c[1], c[2], c[3]), pack_bytes(c[4], c[5], c[6], c[7]),
                      pack_bytes(c[8], c[9], c[10], c[11]), pack_bytes(c[12], c[13], c[14], c[15]));
}

// Transposed order: dword f holds codes f, 4 + f, 8 + f, 12 + f, the order in which the
// GEMV unpacks a dword of packed weights (field f of its four bytes).
__device__ __forceinline__ uint4 unit_codes_t(const float (&w)[16], float sp)
{
    int c[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
        c[e] = (int)__builtin_rintf(w[e] * sp);
    return make_uint4(pack_bytes(c[0], c[4], c[8], c[12]), pack_bytes(c[1], c[5], c[9], c[13]),
                      pack_bytes(c[2], c[6], c[10], c[14]), pack_bytes(c[3], c[7], c[11], c[15]));
}

// Sum over the 64 lanes of a wave (integer: exact in any order); every lane gets it.
__device__ __forceinline__ int wave_sum_i32(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
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

// attention.hpp -- decode attention at real context length (gfx950, wave64).
//
// One new token per sequence attends over its key/value cache: scaled dot-product
// attention ("BitNet b1.58 深度解析" s.2.4 block diagram) with rotary position embedding
// ("微软AI大模型炸场" s.2, 特殊设计), grouped-query heads (query head h reads KV head
// h / (H / KVH)), head dimension 128, bf16 cache [M][KVH][C][128].
//
// The work is HBM-bound (every cached key and value is read once per step, for all the
// query heads of its group), so the kernels are built for streaming, not for MFMA:
//
//   attn_chunk_kernel   one block per (span of 64-position sub-chunks, group of GB query
//                       heads of one KV head, sequence). Each wave builds the 64 rotation
//                       angles of pos (lane i owns pair (i, i + 64): pos * theta^(-2i/128)
//                       in binary64, cos and sin rounded once to binary32) while its first
//                       key/value loads are in flight, and rotates the block's queries,
//                       pre-scaled by log2(e)/sqrt(128). The block holding position pos
//                       rotates the new key (binary32, no fused multiply-add: its bf16
//                       rounding is a decision), appends it and the value, both rounded to
//                       bf16, and uses them from registers. A row of 16 lanes holds one
//                       cached position (8 dims of 16 bytes per lane, so a wave reads 4
//                       consecutive rows = 1 KB contiguous); a sub-chunk's keys are all
//                       requested before its values. Scores are reduced across the row with
//                       DPP, the block maximum through LDS, and the block writes its partial
//                       softmax state (max m, sum l, unnormalised sum acc of weighted
//                       values) per head to the workspace.
//   attn_combine_kernel one block per (head, sequence) merges the chunk partials:
//                       out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, eight chunk
//                       groups of 32 lanes (float4 each), each with a running maximum, then
//                       a fixed-order merge of the groups.
//
// Scores are kept in base 2, so weights are exp2 of differences. Every reduction follows
// a fixed order, so results do not depend on timing.
#pragma once

#include "device_common.hpp"
#include <type_traits>

namespace bl {

constexpr int kAttnD = 128;      // head dimension
constexpr int kAttnChunk = 64;   // positions per block: 4 waves x 4 rows x 4 iterations
constexpr int kAttnIter = 4;

struct AttnArgs {
    const float* qkv;     // [M][(H + 2 KVH) * 128]: query heads, key heads, value heads
    uint16_t* kc;         // bf16 [M][KVH][C][128]
    uint16_t* vc;         // bf16 [M][KVH][C][128]
    const int* pos;       // [M]
    float* out;           // [M][H * 128]
    float* part_acc;      // [M][H][S][128]
    float* part_ml;       // [M][H][S][2]: block max (base 2), block sum
    int H, KVH, C, S;     // S = ceil(C / 64): partial slots per (sequence, head)
    int cpb;              // 64-position sub-chunks per chunk block
    double theta;         // rotary base
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// Round a finite binary32 value to bfloat16, nearest with ties to even.
__device__ __forceinline__ uint32_t f32_to_bf16(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float row_sum16(float v)
{
    v = v + dpp_f32<0xB1>(v);
    v = v + dpp_f32<0x4E>(v);
    v = v + dpp_f32<0x141>(v);
    v = v + dpp_f32<0x140>(v);
    return v;
}

__device__ __forceinline__ float lane_f(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

constexpr float kQScale = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)

// One block per (span of `cpb` 64-position sub-chunks, group of GB query heads of one KV
// head, sequence). Per sub-chunk: request its keys and values, score them, take the
// block maximum (LDS, one barrier), rescale the running sums to the new maximum and add
// the sub-chunk's weighted values. Every row of the block uses the same running maximum,
// so the final sum over rows needs no rescaling.
//
// Two forms. LOOP = false (one sub-chunk per block, cpb == 1): no running state, each
// head's sums go straight to LDS. LOOP = true (cpb >= 1, at most 4 query heads per block
// so that the running state stays in registers): the running sums are rescaled per
// sub-chunk, and the next sub-chunk's keys and values are requested before the current
// one is scored, so two sub-chunks' loads are in flight.
template <int GB, bool LOOP>
__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnArgs a)
{
    __shared__ float2 rot[4][64];                  // per-wave (cos, sin) of the 64 pair angles
    __shared__ float wmax[2][4][GB];               // per-wave sub-chunk maxima, by parity
    __shared__ float4 red[4 * 4][GB][kAttnD / 4];  // per-row partial acc
    __shared__ float redl[4 * 4][GB];

    const int c = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
    const int G = a.H / a.KVH, per = G / GB;
    const int kh = gi / per, h0 = kh * G + (gi - kh * per) * GB;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane >> 4, t = lane & 15;
    const int d0 = 8 * t;                          // this lane's 8 dims
    const int dp = (d0 + kAttnD / 2) & (kAttnD - 1);  // the rotation partner's 8 dims

    // Query values first: they do not depend on pos, and loads complete in order, so they
    // must not queue behind the keys and values.
    float q[GB][8], yv[GB][8];
    const float* qrow = a.qkv + (size_t)b * (a.H + 2 * a.KVH) * kAttnD;
#pragma unroll
    for (int hh = 0; hh < GB; ++hh) {
        const float4* x = reinterpret_cast<const float4*>(qrow + (h0 + hh) * kAttnD + d0);
        const float4 x0 = x[0], x1 = x[1];
        q[hh][0] = x0.x; q[hh][1] = x0.y; q[hh][2] = x0.z; q[hh][3] = x0.w;
        q[hh][4] = x1.x; q[hh][5] = x1.y; q[hh][6] = x1.z; q[hh][7] = x1.w;
        const float4* y = reinterpret_cast<const float4*>(qrow + (h0 + hh) * kAttnD + dp);
        const float4 y0 = y[0], y1 = y[1];
        yv[hh][0] = y0.x; yv[hh][1] = y0.y; yv[hh][2] = y0.z; yv[hh][3] = y0.w;
        yv[hh][4] = y1.x; yv[hh][5] = y1.y; yv[hh][6] = y1.z; yv[hh][7] = y1.w;
    }

    const int p = a.pos[b];
    const int sc0 = c * a.cpb;                     // first sub-chunk of this block
    if (p < 0 || p >= a.C || sc0 * kAttnChunk > p)
        return;
    const int sc1 = min(sc0 + a.cpb, p / kAttnChunk + 1);
    // slot p is not read: the new key and value come from registers
    const int jlast = p - 1;
    const size_t row0 = ((size_t)b * a.KVH + kh) * (size_t)a.C;

    // all keys of a sub-chunk first, then its values: scoring waits only for the keys
    uint4 kb[LOOP ? 2 : 1][kAttnIter], vb[LOOP ? 2 : 1][kAttnIter];
    int jb[LOOP ? 2 : 1][kAttnIter];
    // Rows past the block's last cached one load row max(jmax, 0) instead: in bounds, and
    // no branch around a load, so that the compiler can keep the next sub-chunk's loads in
    // flight while it waits for the current one's. Every use of a row selects on j <= p.
    const int jmax = min(jlast, sc1 * kAttnChunk - 1);
    auto issue = [&](int sc, auto BF) {
        constexpr int bf = decltype(BF)::value;
        int jl[kAttnIter];
#pragma unroll
        for (int it = 0; it < kAttnIter; ++it) {
            const int j = sc * kAttnChunk + (it * 4 + w) * 4 + r;
            jb[bf][it] = j;
            jl[it] = j <= jmax ? j : max(jmax, 0);
            kb[bf][it] = *(const uint4*)(a.kc + (row0 + jl[it]) * kAttnD + d0);
        }
#pragma unroll
        for (int it = 0; it < kAttnIter; ++it)
            vb[bf][it] = *(const uint4*)(a.vc + (row0 + jl[it]) * kAttnD + d0);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, LOOP ? 1 : 0>;
    issue(sc0, B0{});

    // Rotated, pre-scaled queries of the block's heads (this lane's 8 dims).
    uint4 kn = make_uint4(0, 0, 0, 0), vn = make_uint4(0, 0, 0, 0);
    const bool own = p / kAttnChunk < sc1;         // this block holds position p
    {
        const double ang = (double)p * pow(a.theta, -(2.0 * lane) / (double)kAttnD);
        double sd, cd;
        sincos(ang, &sd, &cd);
        rot[w][lane] = make_float2((float)cd, (float)sd);
        // the table is private to the wave: a wave-scope release/acquire orders it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float cs[8], sn[8];
        const float4* tp = reinterpret_cast<const float4*>(&rot[w][d0 & 63]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float4 v = tp[e];
            cs[2 * e] = v.x; sn[2 * e] = v.y; cs[2 * e + 1] = v.z; sn[2 * e + 1] = v.w;
        }
        const bool hi = t >= 8;   // second half of the head: x2*c + x1*s
#pragma unroll
        for (int hh = 0; hh < GB; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float rv = hi ? q[hh][e] * cs[e] + yv[hh][e] * sn[e] : q[hh][e] * cs[e] - yv[hh][e] * sn[e];
                q[hh][e] = rv * kQScale;
            }
        // the new key: every product and sum rounded (its bf16 rounding is a decision)
        if (own) {
            const float* krow = qrow + (a.H + kh) * kAttnD;
            const float* vrow = qrow + (a.H + a.KVH + kh) * kAttnD;
            uint32_t kbits[8], vbits[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = krow[d0 + e], y = krow[dp + e];
                const float rv = hi ? __fadd_rn(__fmul_rn(x, cs[e]), __fmul_rn(y, sn[e]))
                                    : __fsub_rn(__fmul_rn(x, cs[e]), __fmul_rn(y, sn[e]));
                kbits[e] = f32_to_bf16(rv);
                vbits[e] = f32_to_bf16(vrow[d0 + e]);
            }
            kn = make_uint4(kbits[0] | kbits[1] << 16, kbits[2] | kbits[3] << 16, kbits[4] | kbits[5] << 16,
                            kbits[6] | kbits[7] << 16);
            vn = make_uint4(vbits[0] | vbits[1] << 16, vbits[2] | vbits[3] << 16, vbits[4] | vbits[5] << 16,
                            vbits[6] | vbits[7] << 16);
            if (gi - kh * per == 0 && w == 0 && r == 0) {   // append once per KV head
                *(uint4*)(a.kc + (row0 + p) * kAttnD + d0) = kn;
                *(uint4*)(a.vc + (row0 + p) * kAttnD + d0) = vn;
            }
        }
    }

    float mrun[GB], lrun[GB], acc[GB][8];
#pragma unroll
    for (int hh = 0; hh < GB; ++hh) {
        mrun[hh] = -__builtin_huge_valf();
        lrun[hh] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;
    }
    const int row = w * 4 + r;
    auto step = [&](int sc, auto BF) {
        constexpr int bf = decltype(BF)::value;
        uint4 (&kr)[kAttnIter] = kb[bf];
        uint4 (&vr)[kAttnIter] = vb[bf];
        const int (&jj)[kAttnIter] = jb[bf];
        if (own) {
#pragma unroll
            for (int it = 0; it < kAttnIter; ++it)
                if (jj[it] == p) {
                    kr[it] = kn;
                    vr[it] = vn;
                }
        }
        // scores (base 2) of the lane's row positions, reduced across the row
        float s[kAttnIter][GB];
#pragma unroll
        for (int it = 0; it < kAttnIter; ++it) {
            const uint32_t kw[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = bf16_to_f32(kw[e] & 0xFFFFu);
                kf[2 * e + 1] = bf16_to_f32(kw[e] >> 16);
            }
#pragma unroll
            for (int hh = 0; hh < GB; ++hh) {
                float d = q[hh][0] * kf[0];
#pragma unroll
                for (int e = 1; e < 8; ++e)
                    d = __builtin_fmaf(q[hh][e], kf[e], d);
                d = row_sum16(d);
                s[it][hh] = jj[it] <= p ? d : -__builtin_huge_valf();
            }
        }
        // sub-chunk maximum per head: the lane's positions, the wave's 4 rows, 4 waves
        const int par = (sc - sc0) & 1;
#pragma unroll
        for (int hh = 0; hh < GB; ++hh) {
            float m = s[0][hh];
#pragma unroll
            for (int it = 1; it < kAttnIter; ++it)
                m = fmaxf(m, s[it][hh]);
            m = fmaxf(fmaxf(lane_f(m, 0), lane_f(m, 16)), fmaxf(lane_f(m, 32), lane_f(m, 48)));
            if (lane == 0)
                wmax[par][w][hh] = m;
        }
        __syncthreads();
        // rescale the running sums to the new maximum, then add this sub-chunk's weights
#pragma unroll
        for (int hh = 0; hh < GB; ++hh) {
            const float msub = fmaxf(fmaxf(wmax[par][0][hh], wmax[par][1][hh]), fmaxf(wmax[par][2][hh], wmax[par][3][hh]));
            const float mnew = LOOP ? fmaxf(mrun[hh], msub) : msub;
            if constexpr (LOOP) {
                const float scale = exp2f(mrun[hh] - mnew);    // 0 on the first sub-chunk
                lrun[hh] *= scale;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[hh][e] *= scale;
            }
            mrun[hh] = mnew;
            // without LOOP the head's sums go straight to LDS (no state across heads)
            float a8[8], l = LOOP ? lrun[hh] : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a8[e] = LOOP ? acc[hh][e] : 0.0f;
#pragma unroll
            for (int it = 0; it < kAttnIter; ++it) {
                const float pw = exp2f(s[it][hh] - mnew);   // 0 for masked positions
                l += pw;
                // a masked row adds pw * 0 = 0 (selected, not branched around, so that
                // every path waits for its load)
                const bool live = jj[it] <= p;
                const uint32_t vw[4] = {live ? vr[it].x : 0u, live ? vr[it].y : 0u, live ? vr[it].z : 0u,
                                        live ? vr[it].w : 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a8[2 * e] = __builtin_fmaf(pw, bf16_to_f32(vw[e] & 0xFFFFu), a8[2 * e]);
                    a8[2 * e + 1] = __builtin_fmaf(pw, bf16_to_f32(vw[e] >> 16), a8[2 * e + 1]);
                }
            }
            if constexpr (LOOP) {
                lrun[hh] = l;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[hh][e] = a8[e];
            } else {
                red[row][hh][2 * t] = make_float4(a8[0], a8[1], a8[2], a8[3]);
                red[row][hh][2 * t + 1] = make_float4(a8[4], a8[5], a8[6], a8[7]);
                if (t == 0)
                    redl[row][hh] = l;
            }
        }
    };
    if constexpr (LOOP) {
        // the loads are unconditional (past sc1 they re-read row jmax), so every path to a
        // step has the same loads in flight
        for (int sc = sc0;; sc += 2) {
            issue(sc + 1, B1{});
            step(sc, B0{});
            if (sc + 1 >= sc1)
                break;
            issue(sc + 2, B0{});
            step(sc + 1, B1{});
            if (sc + 2 >= sc1)
                break;
        }
    } else {
        step(sc0, B0{});                         // cpb == 1
    }

    // Sum the 16 rows in order and write the block's partial state per head.
    if constexpr (LOOP) {
#pragma unroll
        for (int hh = 0; hh < GB; ++hh) {
            red[row][hh][2 * t] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
            red[row][hh][2 * t + 1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
            if (t == 0)
                redl[row][hh] = lrun[hh];
        }
    }
    __syncthreads();
    for (int o = tid; o < GB * kAttnD; o += 256) {
        const int hh = o / kAttnD, d = o - hh * kAttnD;
        const float* rp = reinterpret_cast<const float*>(&red[0][hh][0]) + d;
        float sum = 0.0f;
#pragma unroll
        for (int q16 = 0; q16 < 16; ++q16)
            sum += rp[(size_t)q16 * GB * kAttnD];
        const size_t rec = ((size_t)b * a.H + h0 + hh) * a.S + c;
        a.part_acc[rec * kAttnD + d] = sum;
        if (d == 0) {
            float l = 0.0f;
#pragma unroll
            for (int q16 = 0; q16 < 16; ++q16)
                l += redl[q16][hh];
            // every thread holds the same running maximum; pick it without dynamic indexing
            float m = mrun[0];
#pragma unroll
            for (int x = 1; x < GB; ++x)
                m = hh == x ? mrun[x] : m;
            a.part_ml[rec * 2] = m;
            a.part_ml[rec * 2 + 1] = l;
        }
    }
}

// One block per (head, sequence): thread (g, q) with g = tid / 32 (chunk group) and
// q = tid % 32 (dims 4q .. 4q+3) merges chunks g, g + 8, g + 16, ... with a running maximum
// of its own; the 8 groups are merged at the end in a fixed order. The first batch of
// records is requested together with pos (its addresses do not depend on it; records past
// the live ones are dropped by selection once pos is known), so a context of up to
// 64 * 8 * kCombUnroll positions per chunk block needs one memory round trip.
constexpr int kCombUnroll = 8;

__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a)
{
    __shared__ float4 red[8][kAttnD / 4];
    __shared__ float2 redml[8];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, g = tid >> 5, q = tid & 31;
    const int p = a.pos[b];
    const size_t rec0 = ((size_t)b * a.H + h) * a.S;
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml + rec0 * 2);
    const float4* pa = reinterpret_cast<const float4*>(a.part_acc + rec0 * kAttnD) + q;
    const int nrec = (a.S + a.cpb - 1) / a.cpb;    // records a chunk launch can write
    float4 v[kCombUnroll];
    float2 mlv[kCombUnroll];
    auto load = [&](int c0, int lim) {
#pragma unroll
        for (int u = 0; u < kCombUnroll; ++u) {
            const int c = c0 + 8 * u;
            v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            mlv[u] = make_float2(0.0f, 0.0f);
            if (c < lim) {
                v[u] = pa[(size_t)c * (kAttnD / 4)];
                mlv[u] = ml[c];
            }
        }
    };
    load(g, nrec);
    float* o = a.out + ((size_t)b * a.H + h) * kAttnD;
    if (p < 0 || p >= a.C) {
        if (tid < kAttnD)
            o[tid] = __builtin_nanf("");
        return;
    }
    const int n = p / (kAttnChunk * a.cpb) + 1;   // live chunk blocks
    float m = -__builtin_huge_valf(), l = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    // fold one batch in: a live record's maximum is finite (its first position is scored)
    auto fold = [&](int c0) {
        float mb = -__builtin_huge_valf();
#pragma unroll
        for (int u = 0; u < kCombUnroll; ++u)
            mb = c0 + 8 * u < n ? fmaxf(mb, mlv[u].x) : mb;
        if (c0 >= n)
            return;
        const float mnew = fmaxf(m, mb);
        const float sc = exp2f(m - mnew);          // 0 on the group's first batch
        l *= sc;
        acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
#pragma unroll
        for (int u = 0; u < kCombUnroll; ++u) {
            if (c0 + 8 * u < n) {
                const float wgt = exp2f(mlv[u].x - mnew);
                l = __builtin_fmaf(wgt, mlv[u].y, l);
                acc.x = __builtin_fmaf(wgt, v[u].x, acc.x);
                acc.y = __builtin_fmaf(wgt, v[u].y, acc.y);
                acc.z = __builtin_fmaf(wgt, v[u].z, acc.z);
                acc.w = __builtin_fmaf(wgt, v[u].w, acc.w);
            }
        }
        m = mnew;
    };
    fold(g);
    for (int c0 = g + 8 * kCombUnroll; c0 < n; c0 += 8 * kCombUnroll) {
        load(c0, n);
        fold(c0);
    }
    red[g][q] = acc;
    if (q == 0)
        redml[g] = make_float2(m, l);
    __syncthreads();
    if (tid < kAttnD) {
        // group 0 holds chunk 0, so the maximum is finite; empty groups weigh exp2(-inf) = 0
        float mx = redml[0].x;
#pragma unroll
        for (int gg = 1; gg < 8; ++gg)
            mx = fmaxf(mx, redml[gg].x);
        const float* rp = reinterpret_cast<const float*>(&red[0][0]) + tid;
        float sum = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) {
            const float wgt = exp2f(redml[gg].x - mx);
            sum = __builtin_fmaf(wgt, rp[gg * kAttnD], sum);
            lsum = __builtin_fmaf(wgt, redml[gg].y, lsum);
        }
        o[tid] = sum / lsum;
    }
}

}  // namespace bl

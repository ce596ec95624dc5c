// gemv.hpp -- W1.58A8 product for few tokens (decode): packed ternary rows streamed from
// HBM with 128-bit non-temporal loads, unpacked in registers and multiplied with
// v_dot4 (int8 x int8 -> int32), then rescaled to fp32.
//
// The product y = (W_q x_q) * gamma / s ("BitNet b1.58 深度解析" s.2.3) is exact in
// int32 before the rescale. The pages' GPU recipe ("微软AI大模型炸场" s.3: pack ternary
// values into bytes in HBM, load on chip, unpack, compute) is kept in spirit; on gfx950
// the packed weight bytes go straight from HBM into VGPRs and never touch LDS; only the
// activation codes of the token tile are staged in LDS, once per block.
//
// Unpack. A 16-byte chunk of a packed row holds codes k0 .. k0+63 (k0 = 64c). Dword d of
// the chunk holds bytes 4d..4d+3, byte jj holds codes k0 + 16d + 4jj + f in bits 2f.
// (dword >> 2f) & 0x03030303 would yield the four fields f of the four bytes, i.e. offset
// codes q + 1 in {0, 1, 2} for k0 + 16d + 4jj + f, jj = 0..3; the product masks them in
// place instead (scaled by 4^f, one accumulator per scale). The activations are held in
// the same order (a byte-transpose of each 16-byte group, done once per block), and
// sum_k (q+1) x - sum_k x = sum_k q x removes the offset exactly.
//
// Work split. A row is shared by L lanes (L = 8 .. 256); lane j owns chunks j, j+L, ...
// (at most 4/MT of them) and keeps their activation codes for MT tokens in VGPRs for
// the whole kernel. Each lane works on R rows per pass (256/L * R rows per block); the
// next pass's weights are loaded while the current pass is computed.
#pragma once

#include "device_common.hpp"

namespace bl {

struct FwdArgs {
    const int8_t* Xq;      // pre-quantized activations [M][K] (unfused)
    const float* xscale;   // [M] (unfused)
    const float* X;        // fp32 activations [M][K], [M][2K] when act == 2 (fused)
    const float* gain;     // [K] or null (fused)
    float eps;             // (fused)
    int act;               // activation (fused): 0 identity, 1 squared ReLU, 2 gated
    const uint8_t* W;      // packed [N][K/4]
    const float* gamma;    // [1]
    float* Y;              // [M][N]; with `residual` read and overwritten by Y + product
    int32_t* acc;          // [M][N] or null
    int64_t M;
    int64_t N;
    int K;
    int residual;          // 1: Y[t][n] = fl32(Y[t][n] + y[t][n])
};

constexpr int kBufFlags = 0x00020000;  // buffer descriptor word 3 (gfx9)
constexpr int kOob = 0x7ffffff0;       // an offset past every buffer: loads give 0, stores drop

__device__ __forceinline__ int64_t x_stride(const FwdArgs& a)
{
    return a.act == 2 ? 2 * (int64_t)a.K : (int64_t)a.K;
}

// Units of 16 elements per thread in the fused prologue (thread t owns units t, t + 256,
// ...): the longest row a tile shape serves has L * CPL chunks of four units.
template <int L, int CPL>
constexpr int units_per_thread()
{
    return (L * CPL * 4 + 255) / 256;
}

// Units per thread whose loads are issued before the weight loads (token 0): at most 2,
// and 1 when the tile has more rows per lane or more tokens (their weight and code
// registers would otherwise leave room for one wave per SIMD).
template <int L, int MT, int CPL, int R>
constexpr int preloaded_units()
{
    constexpr int need = units_per_thread<L, CPL>();
    constexpr int cap = R == 1 && MT == 1 ? 2 : 1;
    return need < cap ? need : cap;
}

// Units per thread whose w values stay in registers from the statistics to the codes:
// up to 8 (128 registers) with one row per lane and one token per tile (with more than 2
// these shapes take more than 256 registers and run one block per CU; a row of up to
// 32768 elements is then read once), else the preloaded ones. Units past them are read
// again for their codes.
template <int L, int MT, int CPL, int R>
constexpr int kept_units()
{
    constexpr int need = units_per_thread<L, CPL>();
    return R == 1 && MT == 1 ? (need < 8 ? need : 8) : preloaded_units<L, MT, CPL, R>();
}

// Multi-token tiles of the fused prologue stage the w values of units 1 .. NS per thread
// in LDS (16 KB per unit index and token, after the codes), within a budget that leaves
// room for the blocks per CU these tiles run with (one for four tokens, two for two);
// units past them are read again for their codes.
template <int L, int MT, int CPL>
constexpr int staged_units()
{
    constexpr int need = units_per_thread<L, CPL>() - 1;
    constexpr int budget = (MT >= 4 ? 150 : 78) * 1024 - MT * L * CPL * 64;
    constexpr int fit = budget > 0 ? budget / (MT * 16384) : 0;
    return MT == 1 ? 0 : (need < fit ? need : fit);
}

// Dynamic LDS bytes of a fused or staged launch: the codes, then the staged w values.
template <int L, int MT, int CPL>
constexpr size_t fused_lds_bytes(int K)
{
    const int nU = (K / 16 + 255) / 256;
    const int ns = staged_units<L, MT, CPL>() < nU - 1 ? staged_units<L, MT, CPL>() : nU - 1;
    return (size_t)MT * K + (size_t)(ns > 0 ? ns : 0) * MT * 16384;
}

// Early loads of token 0 of a tile for the pre-quantized product: the int8 codes and the
// scales, issued before the weight loads so that they are not queued behind them.
constexpr int kPreUnits = 2;  // 16-byte int8 units per thread preloaded (K <= 8192)
template <int MT>
struct Pre {
    uint4 q[kPreUnits];
    float xs[MT];          // per-token scales of the tile
};

template <bool STAGE, int MT>
__device__ __forceinline__ void stage_preload(const FwdArgs& a, int64_t tok, Pre<MT>& p)
{
    if constexpr (STAGE) {
        const uint4* src = reinterpret_cast<const uint4*>(a.Xq + tok * (int64_t)a.K);
        const int units = a.K >> 4;
#pragma unroll
        for (int i = 0; i < kPreUnits; ++i) {
            const int u = (int)threadIdx.x + 256 * i;
            p.q[i] = u < units ? src[u] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    // scales through vector loads (tokens past M read 0), so that no scalar-load wait
    // sits in front of the weight loads
    const int64_t left = a.M - tok;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.xscale + tok), (short)0, (int)(4 * (left < MT ? left : MT)), kBufFlags);
#pragma unroll
    for (int t = 0; t < MT; ++t)
        p.xs[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * t, 0, 0));
}

// Pre-quantized codes of the tile's tokens to LDS (natural order, K/16 slots per token;
// tokens past M get zeros).
template <int MT>
__device__ __forceinline__ void stage_codes(const FwdArgs& a, int64_t t0, int mt, uint4* __restrict__ lds,
                                            float (&s)[MT], const Pre<MT>& pre)
{
    constexpr int NT = 256;
    const int tid = threadIdx.x;
    const int units = a.K >> 4;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        s[t] = 1.0f;
        uint4* dst = lds + (size_t)t * units;
        if (t >= mt) {
            for (int u = tid; u < units; u += NT)
                dst[u] = make_uint4(0u, 0u, 0u, 0u);
            continue;
        }
        s[t] = pre.xs[t];
        const uint4* src = reinterpret_cast<const uint4*>(a.Xq + (t0 + t) * (int64_t)a.K);
        int u = tid;
        if (t == 0) {
#pragma unroll
            for (int i = 0; i < kPreUnits; ++i, u += NT)
                if (u < units)
                    dst[u] = pre.q[i];
        }
        for (; u < units; u += NT)
            dst[u] = src[u];
    }
}

// Fused prologue of the tile's tokens, specialised by mode MD: statistics, token scales
// s, and the codes in LDS in the order the product consumes them (slot u holds unit u
// transposed, K/16 slots per token), plus each wave's sum of the codes in csum (the row
// sum of the codes is their total). Token 0's first UP units come preloaded in `pre`;
// the w values of the first NK units per thread stay in registers, further units are
// read again for their codes.
template <int MT, int UP, int NK, int NS, class MD>
__device__ __forceinline__ void fused_stage(const FwdArgs& a, int64_t t0, int mt, uint4* __restrict__ lds,
                                            float (&s)[MT], int (&csum)[MT][4], const UnitRaw (&pre)[UP])
{
    static_assert(UP >= 1 && NK >= UP, "kept units include the preloaded ones");
    constexpr int NT = 256;
    const int tid = threadIdx.x;
    const int units = a.K >> 4;
    if constexpr (MT > 1) {
        // All tokens of the tile together, unit index by unit index: the gain is read once
        // for every token, each token's w of unit 0 stays in registers, units 1 .. ns go to
        // thread-private LDS slots and later ones are read again for their codes; one
        // barrier reduces every token's statistics. Tokens past M read nothing (zero codes,
        // dropped outputs).
        static_assert(UP == 1, "multi-token tiles preload one unit of token 0");
        RowRes rr[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t)
            rr[t] = t < mt ? row_res(a.X, t0 + t, a.K, MD::kAct, a.gain) : row_res_empty(a.X);
        const int nU = (units + NT - 1) / NT;
        const int ns = NS < nU - 1 ? NS : nU - 1;
        float4* stage = reinterpret_cast<float4*>(lds + (size_t)MT * units);
        float w0[MT][16];
        float mx[MT];
        double ss[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            mx[t] = 0.0f;
            ss[t] = 0.0;
        }
        // unit i of every token: loads (token 0's unit 0 preloaded), then visit(t, w)
        auto unit = [&](int i, auto&& visit) {
            const int off = (tid + NT * i) << 6;
            float4 g[4], xs[MT][4], ups[MT][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (MD::kNorm) {
                    if constexpr (MD::kAct == 2)
                        g[q] = load_f4(rr[0].z, off + 16 * q);
                    else
                        g[q] = i == 0 ? pre[0].y[q] : load_f4(rr[0].y, off + 16 * q);
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    xs[t][q] = i == 0 && t == 0 ? pre[0].x[q] : load_f4(rr[t].x, off + 16 * q);
                    if constexpr (MD::kAct == 2)
                        ups[t][q] = i == 0 && t == 0 ? pre[0].y[q] : load_f4(rr[t].y, off + 16 * q);
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                float wv[16];
                if constexpr (MD::kAct == 2)
                    unit_visit<MD>(xs[t], ups[t], g, wv, mx[t], ss[t]);
                else
                    unit_visit<MD>(xs[t], g, g, wv, mx[t], ss[t]);
                visit(t, wv);
            }
        };
        unit(0, [&](int t, const float (&wv)[16]) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                w0[t][e] = wv[e];
        });
#pragma unroll 1
        for (int i = 1; i < nU; ++i)
            unit(i, [&](int t, const float (&wv)[16]) {
                if (i <= ns) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        stage[(((i - 1) * MT + t) * 4 + q) * NT + tid] =
                            make_float4(wv[4 * q], wv[4 * q + 1], wv[4 * q + 2], wv[4 * q + 3]);
                }
            });
        RowStats st[MT];
        block_stats_multi<MT>(mx, ss, MD::kNorm, st);
        float sp[MT];
        int cs[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float sv;
            token_scales(st[t], a.K, MD::kNorm, a.eps, sp[t], sv);
            s[t] = t < mt ? sv : 1.0f;
            cs[t] = 0;
        }
        auto put = [&](int t, int u, const float (&wv)[16]) {
            const uint4 c = unit_codes_t(wv, sp[t]);
            lds[(size_t)t * units + u] = c;
            cs[t] = __builtin_amdgcn_sdot4((int)c.x, 0x01010101, cs[t], false);
            cs[t] = __builtin_amdgcn_sdot4((int)c.y, 0x01010101, cs[t], false);
            cs[t] = __builtin_amdgcn_sdot4((int)c.z, 0x01010101, cs[t], false);
            cs[t] = __builtin_amdgcn_sdot4((int)c.w, 0x01010101, cs[t], false);
        };
        if (tid < units) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
                put(t, tid, w0[t]);
        }
#pragma unroll 1
        for (int i = 1; i <= ns; ++i) {
            const int u = tid + NT * i;
            if (u < units) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    float wv[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 v = stage[(((i - 1) * MT + t) * 4 + q) * NT + tid];
                        wv[4 * q] = v.x;
                        wv[4 * q + 1] = v.y;
                        wv[4 * q + 2] = v.z;
                        wv[4 * q + 3] = v.w;
                    }
                    put(t, u, wv);
                }
            }
        }
        // units past the staged ones: statistics are done, read them again for the codes
#pragma unroll 1
        for (int i = ns + 1; i < nU; ++i) {
            const int u = tid + NT * i;
            unit(i, [&](int t, const float (&wv)[16]) {
                if (u < units)
                    put(t, u, wv);
            });
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int v = wave_sum_i32(cs[t]);
            if ((tid & (kWave - 1)) == 0)
                csum[t][tid / kWave] = v;
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        s[t] = 1.0f;
        uint4* dst = lds + (size_t)t * units;
        if (t >= mt) {
            for (int u = tid; u < units; u += NT)
                dst[u] = make_uint4(0u, 0u, 0u, 0u);
            if ((tid & (kWave - 1)) == 0)
                csum[t][tid / kWave] = 0;
            continue;
        }
        const RowRes rr = row_res(a.X, t0 + t, a.K, MD::kAct, a.gain);
        float w[NK][16];
        float mx = 0.0f;
        double ss = 0.0;
        // first UP units (preloaded for token 0)
        if (t == 0) {
            if constexpr (MD::kZ) {
                // the gain of the gated input is read here (not preloaded: registers)
                float4 z[UP][4];
#pragma unroll
                for (int i = 0; i < UP; ++i)
                    unit_load_z(rr, tid + NT * i, z[i]);
#pragma unroll
                for (int i = 0; i < UP; ++i)
                    unit_visit<MD>(pre[i].x, pre[i].y, z[i], w[i], mx, ss);
            } else {
#pragma unroll
                for (int i = 0; i < UP; ++i)
                    unit_visit<MD>(pre[i], w[i], mx, ss);
            }
        } else {
            UnitRaw in[UP];
#pragma unroll
            for (int i = 0; i < UP; ++i)
                unit_load<MD>(rr, tid + NT * i, in[i]);
#pragma unroll
            for (int i = 0; i < UP; ++i)
                unit_visit<MD>(in[i], w[i], mx, ss);
        }
        // further kept units, two loads in flight (units past the row read zeros)
#pragma unroll
        for (int i = UP; i < NK; i += 2) {
            UnitRaw in0, in1;
            unit_load<MD>(rr, tid + NT * i, in0);
            if (i + 1 < NK)
                unit_load<MD>(rr, tid + NT * (i + 1), in1);
            unit_visit<MD>(in0, w[i], mx, ss);
            if (i + 1 < NK)
                unit_visit<MD>(in1, w[i + 1 < NK ? i + 1 : i], mx, ss);
        }
        // units past the kept ones (only tiles with several rows per lane or tokens)
#pragma unroll 1
        for (int u = tid + NT * NK; u < units; u += NT) {
            UnitRaw in;
            unit_load<MD>(rr, u, in);
            float tmp[16];
            unit_visit<MD>(in, tmp, mx, ss);
        }
        const RowStats st = block_stats(mx, ss, MD::kNorm, t & 1);
        float sp;
        token_scales(st, a.K, MD::kNorm, a.eps, sp, s[t]);
        int cs = 0;
        auto put = [&](int u, const float (&wv)[16]) {
            const uint4 c = unit_codes_t(wv, sp);
            dst[u] = c;
            cs = __builtin_amdgcn_sdot4((int)c.x, 0x01010101, cs, false);
            cs = __builtin_amdgcn_sdot4((int)c.y, 0x01010101, cs, false);
            cs = __builtin_amdgcn_sdot4((int)c.z, 0x01010101, cs, false);
            cs = __builtin_amdgcn_sdot4((int)c.w, 0x01010101, cs, false);
        };
#pragma unroll
        for (int i = 0; i < NK; ++i)
            if (tid + NT * i < units)
                put(tid + NT * i, w[i]);
#pragma unroll 1
        for (int u = tid + NT * NK; u < units; u += NT) {
            UnitRaw in;
            unit_load<MD>(rr, u, in);
            float wv[16], m2 = 0.0f;
            double s2 = 0.0;
            unit_visit<MD>(in, wv, m2, s2);
            put(u, wv);
        }
        cs = wave_sum_i32(cs);
        if ((tid & (kWave - 1)) == 0)
            csum[t][tid / kWave] = cs;
    }
}

// Sum over aligned groups of L lanes (every lane of the group gets the sum). Within a
// row of 16 lanes: DPP quad permutes and the (half) row mirror; across rows: shuffles.
template <int L>
__device__ __forceinline__ int group_sum(int v)
{
    if constexpr (L >= 2)
        v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    if constexpr (L >= 4)
        v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    if constexpr (L >= 8)
        v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    if constexpr (L >= 16)
        v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    if constexpr (L >= 32)
        v += __shfl_xor(v, 16);
    if constexpr (L >= 64)
        v += __shfl_xor(v, 32);
    return v;
}


// L lanes per row, MT tokens per tile, CPL chunks per lane (16*CPL*MT VGPRs of
// activation codes, CPL*MT <= 8), R rows per lane per pass: R*CPL 16-byte weight loads
// are in flight per lane, and the next pass is requested before the current one is
// computed. Weights are read and outputs written with raw buffer instructions whose
// descriptor is rebased per pass; lanes without a valid chunk or row use an offset past
// the end (hardware zero-fill / dropped store), so the loop has no branches and the
// outstanding-load counts stay exact. With RES the old outputs of a pass are loaded
// just before its weights (in-order completion: waiting for the weights covers them)
// and the product is added to them. Pre-quantized codes are staged once per block in
// LDS when many row groups share them (L < 64); with L >= 64 (at most four row groups)
// each lane loads its own chunks into registers ahead of its weights, which skips the
// staging and its barriers.
template <int L, int MT, int CPL, int R, bool FUSED, bool RES, int S = 2>
__global__ __launch_bounds__(256) void gemv_k64_kernel(FwdArgs a)
{
    static_assert(S >= 2 && S <= 8, "passes in flight");
    constexpr int NT = 256;
    static_assert(CPL * MT <= 8, "activation codes must fit in 128 VGPRs");
    constexpr int RG = NT / L;             // row groups per block
    constexpr int RPP = RG * R;            // rows per pass
    constexpr int WPR = L > 64 ? L / 64 : 1;
    extern __shared__ uint4 lds_codes[];
    __shared__ int32_t xred[RG][WPR][R][MT];
    __shared__ int csum[MT][4];   // per-wave code sums of the fused prologue
    const int tid = threadIdx.x;
    const int j = tid % L;
    const int slot = tid / L;
    const int KC = a.K >> 6;
    const int KB = a.K >> 2;
    const int64_t N = a.N;
    const int64_t ntiles = (a.M + MT - 1) / MT;

    int woff[R][CPL];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = j + i * L;
            woff[r][i] = c < KC ? (slot + r * RG) * KB + c * 16 : kOob;
        }
    auto load_pass = [&](int64_t rb, u32x4 (&w)[R][CPL], float (&yo)[R][MT], __amdgpu_buffer_rsrc_t ry, int mt) {
        if constexpr (RES) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = rb + slot + (int64_t)r * RG;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const bool mine = j == 0 && row < N && t < mt;
                    yo[r][t] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(ry, mine ? (int)((t * N + row) * 4) : kOob, 0, 0));
                }
            }
        }
        const int64_t rows = rb < N ? ((N - rb) < RPP ? (N - rb) : RPP) : 0;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (rb < N ? rb : 0) * KB), (short)0, (int)(rows * KB), kBufFlags);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                w[r][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, woff[r][i], 0, 2));
    };

    // The grid has at most as many rows of blocks as there are token tiles, so every block
    // has a first tile (no entry check: the argument loads can all be issued at once).
    int64_t tile = blockIdx.y;
    do {
        const int64_t t0 = tile * MT;
        const int mt = (int)((a.M - t0) < MT ? (a.M - t0) : MT);
        const int64_t pstride = (int64_t)gridDim.x * RPP;
        int64_t rb = (int64_t)blockIdx.x * RPP;

        // Outputs of this token tile: y (and acc when requested; otherwise a zero-size
        // buffer that drops every store).
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.Y + t0 * N), (short)0, (int)(mt * N * 4), kBufFlags);
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            a.acc ? (void*)(a.acc + t0 * N) : (void*)a.Y, (short)0, a.acc ? (int)(mt * N * 4) : 0, kBufFlags);

        // Activations of token 0 first, then the first two passes of weights, then the
        // prologue arithmetic while the weights are in flight.
        constexpr bool DIRECT = !FUSED && L >= 64;
        constexpr int UP = preloaded_units<L, MT, CPL, R>();
        constexpr int NK = kept_units<L, MT, CPL, R>();
        Pre<MT> pre;
        UnitRaw pu[UP];
        if constexpr (FUSED) {
            const RowRes rr = row_res(a.X, t0, a.K, a.act, a.gain);
#pragma unroll
            for (int i = 0; i < UP; ++i)
                unit_load_xy(rr, tid + NT * i, a.act == 2 || a.gain != nullptr, pu[i]);
        } else {
            stage_preload<!DIRECT>(a, t0, pre);
        }
        uint32_t act[MT][CPL][16];
        if constexpr (DIRECT) {
            // tokens past M and chunks past K read as zero
            const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(a.Xq + t0 * (int64_t)a.K), (short)0, (int)(mt * a.K), kBufFlags);
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = j + i * L;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const u32x4 v = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rx, c < KC ? t * a.K + c * 64 + 16 * d : kOob, 0, 0));
                        act[t][i][4 * d + 0] = v.x;
                        act[t][i][4 * d + 1] = v.y;
                        act[t][i][4 * d + 2] = v.z;
                        act[t][i][4 * d + 3] = v.w;
                    }
                }
        }
        // gamma through a vector load as well, ahead of the weights
        const float gamma = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       __builtin_amdgcn_make_buffer_rsrc((void*)a.gamma, (short)0, 4, kBufFlags), 0, 0, 0));
        u32x4 wbuf[S][R][CPL];
        float ybuf[S][R][MT];
#pragma unroll
        for (int p = 0; p < S; ++p)
            load_pass(rb + p * pstride, wbuf[p], ybuf[p], ry, mt);

        float s[MT];
        if constexpr (DIRECT) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
                s[t] = t < mt ? pre.xs[t] : 1.0f;
        } else {
            __syncthreads();  // LDS of the previous tile is no longer read
            if constexpr (FUSED)
                with_mode(a.act, a.gain != nullptr, [&](auto md) {
                    fused_stage<MT, UP, NK, staged_units<L, MT, CPL>(), decltype(md)>(a, t0, mt, lds_codes, s,
                                                                                      csum, pu);
                });
            else
                stage_codes<MT>(a, t0, mt, lds_codes, s, pre);
            __syncthreads();
        }

        // Codes of the lane's chunks for every token, in the unpack order, and the part
        // of sum_k x_k the lane removes from its offset-code sum.
        int32_t xs[MT];
        float csc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const uint4* src = lds_codes + (size_t)t * (a.K >> 4);
            int32_t sum = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = j + i * L;
                if constexpr (FUSED) {
                    // already transposed; chunks past the row meet zero weights, so any
                    // in-range codes serve (the row sum comes from the prologue)
                    const int cc = c < KC ? c : KC - 1;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint4 v = src[4 * cc + d];
                        act[t][i][4 * d + 0] = v.x;
                        act[t][i][4 * d + 1] = v.y;
                        act[t][i][4 * d + 2] = v.z;
                        act[t][i][4 * d + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint4 v = make_uint4(0u, 0u, 0u, 0u);
                        if constexpr (DIRECT)
                            v = make_uint4(act[t][i][4 * d + 0], act[t][i][4 * d + 1], act[t][i][4 * d + 2],
                                           act[t][i][4 * d + 3]);
                        else if (c < KC)
                            v = src[4 * c + d];
                        uint32_t o[4];
                        transpose_bytes(v.x, v.y, v.z, v.w, o);
                        act[t][i][4 * d + 0] = o[0];
                        act[t][i][4 * d + 1] = o[1];
                        act[t][i][4 * d + 2] = o[2];
                        act[t][i][4 * d + 3] = o[3];
                    }
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        sum = __builtin_amdgcn_sdot4((int)act[t][i][q], 0x01010101, sum, false);
                }
            }
            if constexpr (FUSED)
                sum = j == 0 ? (csum[t][0] + csum[t][1]) + (csum[t][2] + csum[t][3]) : 0;
            xs[t] = sum;
            csc[t] = gamma / s[t];
        }

        auto compute_pass = [&](int64_t pb, const u32x4 (&w)[R][CPL], const float (&yo)[R][MT]) {
            int32_t accv[R][MT];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // Field f of the four bytes of a dword is masked in place, not shifted down:
                // w & 0x03030303, w & 0x0C0C0C0C and w & 0x30303030 are the offset codes of
                // fields 0, 1, 2 times 1, 4 and 16, and (w >> 2) & 0x30303030 those of field 3
                // times 16 (5 operations per dword instead of 7; every byte stays in 0..32, a
                // non-negative int8). Each scale has its own accumulators, so the sum is
                // part0 + part1 / 4 + (part2 + part3) / 16 with exact divisions (each part is
                // a multiple of its scale; |part| <= 127 * 32 * K / 4 < 2^31 for K <= 132104).
                // One accumulator per field for one or two tokens keeps the dot4 chains short;
                // with more tokens the tokens themselves are independent chains and fields 2
                // and 3 share one.
                constexpr int NA = MT >= 4 ? 3 : 4;
                int32_t part[MT][NA];
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int f = 0; f < NA; ++f)
                        part[t][f] = 0;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const uint32_t wd[4] = {w[r][i].x, w[r][i].y, w[r][i].z, w[r][i].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t u[4] = {wd[d] & 0x03030303u, wd[d] & 0x0C0C0C0Cu, wd[d] & 0x30303030u,
                                               (wd[d] >> 2) & 0x30303030u};
#pragma unroll
                        for (int f = 0; f < 4; ++f) {
                            const int a = f < NA ? f : NA - 1;
#pragma unroll
                            for (int t = 0; t < MT; ++t)
                                part[t][a] = __builtin_amdgcn_sdot4((int)u[f], (int)act[t][i][4 * d + f], part[t][a], false);
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < MT; ++t)
                {
                    int32_t hi = part[t][2];
                    if constexpr (NA == 4)
                        hi += part[t][3];
                    const int32_t sum = part[t][0] + (part[t][1] >> 2) + (hi >> 4);
                    accv[r][t] = group_sum<(L < 64 ? L : 64)>(sum - xs[t]);
                }
            }
            if constexpr (L > 64) {
                if ((tid & 63) == 0) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int t = 0; t < MT; ++t)
                            xred[slot][j / 64][r][t] = accv[r][t];
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        int32_t v = 0;
#pragma unroll
                        for (int wv = 0; wv < WPR; ++wv)
                            v += xred[slot][wv][r][t];
                        accv[r][t] = v;
                    }
                __syncthreads();
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = pb + slot + (int64_t)r * RG;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const bool mine = j == 0 && row < N && t < mt;
                    const int off = mine ? (int)((t * N + row) * 4) : kOob;
                    float yv = (float)accv[r][t] * csc[t];
                    if constexpr (RES)
                        yv = yo[r][t] + yv;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, yv), ry, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(accv[r][t], ra, off, 0, 0);
                }
            }
        };

        // S named buffers in turn (no register copy at the loop edge), so each wait for
        // weight data sits right before its use; S passes are in flight.
        if constexpr (S == 2) {
            for (; rb < N; rb += 2 * pstride) {
                compute_pass(rb, wbuf[0], ybuf[0]);
                load_pass(rb + 2 * pstride, wbuf[0], ybuf[0], ry, mt);
                if (rb + pstride >= N)
                    break;
                compute_pass(rb + pstride, wbuf[1], ybuf[1]);
                load_pass(rb + 3 * pstride, wbuf[1], ybuf[1], ry, mt);
            }
        } else
        for (; rb < N; rb += S * pstride) {
            bool done = false;
#pragma unroll
            for (int p = 0; p < S; ++p) {
                if (!done) {
                    if (p > 0 && rb + p * pstride >= N) {
                        done = true;
                    } else {
                        compute_pass(rb + p * pstride, wbuf[p], ybuf[p]);
                        load_pass(rb + (p + S) * pstride, wbuf[p], ybuf[p], ry, mt);
                    }
                }
            }
            if (done)
                break;
        }
        tile += gridDim.y;
    } while (tile < ntiles);
}

// One token, fused input, rows of L * CPL chunks (the 100B down projection: L = 64,
// CPL = 7; the K = 8192 matrices: L = 32, CPL = 4): 512 threads in two roles. A wave's loads complete in order, so in the 256-thread kernel
// the prologue's row loads wait behind the weight passes requested before them. Here
// waves 0-3 run the fused prologue exactly as that kernel does (the same canonical threads
// and order, so the same codes, scale and outputs) with no weight loads of their own in
// flight, while waves 4-7 request their first S passes once the prologue's statistics are
// in (requesting them at the start slows the prologue's row loads, which share the CU's
// memory pipeline, by more than it gains) and meet the prologue at its two barriers.
// Block b owns passes p = 0, 1, ... of RG = 256 / L rows each (rows b*RG + p*stride ..;
// within each role, lanes of group (tid mod 256) / L share a row); of its n passes the
// streaming waves compute the first n - n/4 and the prologue waves the rest, each wave
// with S weight buffers in turn.
template <int L, int CPL, int S, bool RES, int ACT, bool NORM>
__global__ __launch_bounds__(512) void gemv_split_kernel(FwdArgs a)
{
    constexpr int NT = 256, RG = NT / L;
    static_assert(L == 32 || L == 64, "a row within one wave");
    constexpr int UP = preloaded_units<L, 1, CPL, 1>();
    constexpr int NK = kept_units<L, 1, CPL, 1>();
    using MD = Mode<ACT, NORM>;
    extern __shared__ uint4 lds_codes[];
    __shared__ int csum[1][4];
    __shared__ float s_tok;
    // the wave index through readfirstlane: the compiler then knows the pass ranges below
    // are wave-uniform and keeps the weight descriptors in scalar registers
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), j = tid % L;
    const int slot = (tid % NT) / L;
    const bool pro = wave < 4;
    const int KC = a.K >> 6, KB = a.K >> 2;
    const int64_t N = a.N;
    const int64_t pstride = (int64_t)gridDim.x * RG;
    const int64_t rb0 = (int64_t)blockIdx.x * RG;
    const int n = rb0 < N ? (int)((N - rb0 + pstride - 1) / pstride) : 0;   // this block's passes
    const int ps = n - n / 4;                                               // streaming waves' share

    int woff[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = j + i * L;
        woff[i] = c < KC ? slot * KB + c * 16 : kOob;
    }
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void*)a.Y, (short)0, (int)(N * 4), kBufFlags);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        a.acc ? (void*)a.acc : (void*)a.Y, (short)0, a.acc ? (int)(N * 4) : 0, kBufFlags);
    // pass p of this block, or nothing (a zero-size range: loads give 0, stores drop) when
    // p lies outside [p0, p1); the loads are unconditional so that no branch surrounds them
    auto load_pass = [&](int p, int p0, int p1, u32x4 (&w)[CPL], float& yo) {
        const int64_t rb = p >= p0 && p < p1 ? rb0 + p * pstride : N;
        if constexpr (RES) {
            const int64_t row = rb + slot;
            yo = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(ry, j == 0 && row < N ? (int)(row * 4) : kOob, 0, 0));
        }
        const int64_t rows = rb < N ? ((N - rb) < RG ? (N - rb) : RG) : 0;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (rb < N ? rb : 0) * KB), (short)0, (int)(rows * KB), kBufFlags);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, woff[i], 0, 2));
    };

    UnitRaw pu[UP];
    if (pro) {
        const RowRes rr = row_res(a.X, 0, a.K, ACT, a.gain);
#pragma unroll
        for (int i = 0; i < UP; ++i)
            unit_load_xy(rr, tid + NT * i, MD::kY, pu[i]);
    }
    const float gamma = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(
                   __builtin_amdgcn_make_buffer_rsrc((void*)a.gamma, (short)0, 4, kBufFlags), 0, 0, 0));
    u32x4 wbuf[S][CPL];
    float ybuf[S];
    if (pro) {
        float s[1];
        fused_stage<1, UP, NK, 0, MD>(a, 0, 1, lds_codes, s, csum, pu);
        if (tid == 0)
            s_tok = s[0];
    } else {
        __syncthreads();   // the prologue's statistics barrier
#pragma unroll
        for (int i = 0; i < S; ++i)
            load_pass(i, 0, ps, wbuf[i], ybuf[i]);
    }
    __syncthreads();       // codes, code sums and the token scale are in LDS
    const int p0 = pro ? ps : 0, p1 = pro ? n : ps;
    if (pro) {
#pragma unroll
        for (int i = 0; i < S; ++i)
            load_pass(p0 + i, p0, p1, wbuf[i], ybuf[i]);
    }

    uint32_t act[CPL][16];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = j + i * L;
        const int cc = c < KC ? c : KC - 1;   // chunks past the row meet zero weights
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint4 v = lds_codes[4 * cc + d];
            act[i][4 * d + 0] = v.x;
            act[i][4 * d + 1] = v.y;
            act[i][4 * d + 2] = v.z;
            act[i][4 * d + 3] = v.w;
        }
    }
    const int32_t xs = j == 0 ? (csum[0][0] + csum[0][1]) + (csum[0][2] + csum[0][3]) : 0;
    const float csc = gamma / s_tok;

    // the same arithmetic as the 256-thread kernel's pass (fields masked in place, one
    // accumulator per field)
    auto compute_pass = [&](int p, const u32x4 (&w)[CPL], float yo) {
        int32_t part[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t wd[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t u[4] = {wd[d] & 0x03030303u, wd[d] & 0x0C0C0C0Cu, wd[d] & 0x30303030u,
                                       (wd[d] >> 2) & 0x30303030u};
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    part[f] = __builtin_amdgcn_sdot4((int)u[f], (int)act[i][4 * d + f], part[f], false);
            }
        }
        const int32_t sum = part[0] + (part[1] >> 2) + ((part[2] + part[3]) >> 4);
        const int32_t accv = group_sum<L>(sum - xs);
        const int64_t row = rb0 + p * pstride + slot;
        const int off = j == 0 && row < N ? (int)(row * 4) : kOob;
        float yv = (float)accv * csc;
        if constexpr (RES)
            yv = yo + yv;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, yv), ry, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(accv, ra, off, 0, 0);
    };
    for (int p = p0; p < p1; p += S) {
#pragma unroll
        for (int i = 0; i < S; ++i) {
            if (p + i < p1)
                compute_pass(p + i, wbuf[i], ybuf[i]);
            load_pass(p + i + S, p0, p1, wbuf[i], ybuf[i]);
        }
    }
}

// Any K % 4 == 0 and any alignment of the packed rows: byte loads, one wave per row,
// four tokens per tile. Used for shapes the 16-byte chunked kernel does not cover.
template <bool FUSED>
__global__ __launch_bounds__(256) void gemv_generic_kernel(FwdArgs a)
{
    constexpr int MT = 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t KB = a.K >> 2;
    const int64_t ntiles = (a.M + MT - 1) / MT;
    const float gamma = *a.gamma;
    const bool norm = a.gain != nullptr;
    int calls = 0;  // statistics calls so far: their LDS slots alternate
    for (int64_t tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        const int64_t t0 = tile * MT;
        const int mt = (int)((a.M - t0) < MT ? (a.M - t0) : MT);
        float sp[MT], csc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float s = 1.0f;
            sp[t] = 1.0f;
            if (t < mt) {
                if constexpr (FUSED) {
                    const RowRes rr = row_res(a.X, t0 + t, a.K, a.act, a.gain);
                    const int slot = calls++ & 1;
                    RowStats st;
                    with_mode(a.act, norm, [&](auto md) {
                        st = row_stats_units<decltype(md)>(rr, (a.K + 15) >> 4, slot);
                    });
                    token_scales(st, a.K, norm, a.eps, sp[t], s);
                } else {
                    s = a.xscale[t0 + t];
                }
            }
            csc[t] = gamma / s;
        }
        for (int64_t rb = (int64_t)blockIdx.x * 4; rb < a.N; rb += (int64_t)gridDim.x * 4) {
            const int64_t row = rb + wave;
            int32_t accv[MT] = {0, 0, 0, 0};
            if (row < a.N) {
                for (int64_t b = lane; b < KB; b += 64) {
                    const uint32_t byte = a.W[row * KB + b];
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const int q = (int)((byte >> (2 * f)) & 3u) - 1;
                        const int64_t k = 4 * b + f;
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            if (t < mt) {
                                int xv;
                                if constexpr (FUSED) {
                                    const float* xr = a.X + (t0 + t) * x_stride(a);
                                    const float v = act_v(xr[k], a.act == 2 ? xr[a.K + k] : 1.0f, a.act);
                                    xv = act_code(norm ? v * a.gain[k] : v, sp[t]);
                                } else {
                                    xv = a.Xq[(t0 + t) * (int64_t)a.K + k];
                                }
                                accv[t] += q * xv;
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1)
                    accv[t] += __shfl_xor(accv[t], m);
            if (lane == 0 && row < a.N) {
                for (int t = 0; t < mt; ++t) {
                    const int64_t o = (t0 + t) * a.N + row;
                    const float yv = (float)accv[t] * csc[t];
                    a.Y[o] = a.residual ? a.Y[o] + yv : yv;
                    if (a.acc)
                        a.acc[o] = accv[t];
                }
            }
        }
    }
}

}  // namespace bl

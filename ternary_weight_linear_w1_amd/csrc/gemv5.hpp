// gemv5.hpp -- W1.58A8 product on weights packed five ternary codes per byte (1.6 bits
// per weight): 20% fewer bytes to stream than the 2-bit fields.
//
// Format: byte j of a row is the base-3 numeral sum_i (q[5j+i] + 1) 3^i of codes
// 5j..5j+4; rows are whole 16-byte chunks of 80 codes ("微软AI大模型炸场" s.3: several
// trits in one 8-bit integer; "BitNet b1.58 深度解析" s.2.1: the 2-bit field wastes a
// state). The product is the same exact integer sum as with 2-bit fields.
//
// Decoding: a 243-entry table in LDS maps a byte to its five offset codes q + 1 (8
// bytes: codes 0..3 in the low dword, code 4 in byte 0 of the high dword). Per packed
// byte: a bit-field extract, an 8-byte LDS read, and one dot4 against the four
// activations of codes 0..3; the fifth codes of the four bytes of a packed dword are
// gathered into one dword (v_perm) for one more dot4. The activations of a chunk are
// rearranged once per token tile to match: for byte b, the dword of activations
// 5b..5b+3 (v_alignbyte) and, per packed dword, the dword of activations 5b+4.
// The offset is removed exactly as in the 2-bit path: sum (q+1) x - sum x.
#pragma once

#include "gemv.hpp"

namespace bl {

struct Fwd5Args {
    const int8_t* Xq;      // [M][K]
    const float* xscale;   // [M]
    const uint8_t* W;      // [N][RB] packed five codes per byte
    const float* gamma;    // [1]
    float* Y;              // [M][N]
    int32_t* acc;          // [M][N] or null
    int64_t M;
    int64_t N;
    int K;                 // multiple of 16
    int RB;                // row bytes, 16 * ceil(K / 80)
};

constexpr int kTrit5Values = 243;   // byte values the packer writes; the table has 256 entries

// L lanes per row (a row's 16-byte chunks are dealt to its lanes, CPL each), MT tokens
// per tile, one row per lane per pass, the next pass loaded while one is computed.
template <int L, int MT, int CPL>
__global__ __launch_bounds__(256) void gemv5_kernel(Fwd5Args a)
{
    constexpr int RG = 256 / L;            // rows per pass
    constexpr int WPR = L > 64 ? L / 64 : 1;
    static_assert(MT * CPL <= 8, "activation registers");
    extern __shared__ uint4 lds5[];        // staged codes: MT rows of K bytes
    __shared__ uint2 lut[256];
    __shared__ int32_t red5[RG][WPR][MT];
    const int tid = threadIdx.x;
    const int j = tid % L;
    const int slot = tid / L;
    const int KC = a.RB >> 4;              // chunks per row
    const int64_t N = a.N;
    const int64_t ntiles = (a.M + MT - 1) / MT;
    constexpr int kFlags = kBufFlags;
    constexpr int kPast = kOob;

    // byte value -> offset codes (digit i = code 5j+i plus one); values above 242 never
    // occur in packed data and map to zeros
    {
        unsigned v = tid, lo = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (v % 3u) << (8 * i);
            v /= 3u;
        }
        lut[tid] = tid < kTrit5Values ? make_uint2(lo, v) : make_uint2(0u, 0u);
    }

    int woff[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = j + i * L;
        woff[i] = c < KC ? slot * a.RB + c * 16 : kPast;
    }
    auto load_pass = [&](int64_t rb, u32x4 (&w)[CPL]) {
        const int64_t rows = rb < N ? ((N - rb) < RG ? (N - rb) : RG) : 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.W + (rb < N ? rb : 0) * (int64_t)a.RB), (short)0, (int)(rows * a.RB), kFlags);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, woff[i], 0, 2));
    };

    const float gamma = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(__builtin_amdgcn_make_buffer_rsrc((void*)a.gamma, (short)0, 4, kFlags),
                                                    0, 0, 0));
    int64_t tile = blockIdx.y;   // the grid has no more rows of blocks than token tiles
    do {
        const int64_t t0 = tile * MT;
        const int mt = (int)((a.M - t0) < MT ? (a.M - t0) : MT);
        const int64_t pstride = (int64_t)gridDim.x * RG;
        int64_t rb = (int64_t)blockIdx.x * RG;
        u32x4 cur[CPL], nxt[CPL];
        load_pass(rb, cur);
        load_pass(rb + pstride, nxt);

        // Stage the tile's codes (zeros for tokens past M and codes past K).
        __syncthreads();
        const int units = a.K >> 4;
        const int cunits = KC * 5;         // 16-byte units covered by the row's chunks
        for (int t = 0; t < MT; ++t) {
            const uint4* src = reinterpret_cast<const uint4*>(a.Xq + (t0 + t) * (int64_t)a.K);
            for (int u = tid; u < cunits; u += 256)
                lds5[t * cunits + u] = (t < mt && u < units) ? src[u] : make_uint4(0u, 0u, 0u, 0u);
        }
        float csc[MT];
        const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.xscale + t0), (short)0, 4 * mt, kFlags);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const float s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsx, 4 * t, 0, 0));
            csc[t] = t < mt ? gamma / s : 0.0f;
        }
        __syncthreads();

        // Activations per chunk: slot dword b (codes 5b..5b+3 of the chunk) and, per
        // packed dword d, the dword of codes 5b+4 for b = 4d..4d+3.
        uint32_t sl[MT][CPL][16], p4[MT][CPL][4];
        int32_t xs[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            int32_t sum = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = j + i * L;
                uint32_t A[21];
#pragma unroll
                for (int u = 0; u < 5; ++u) {
                    uint4 v = make_uint4(0u, 0u, 0u, 0u);
                    if (c < KC)
                        v = lds5[t * cunits + 5 * c + u];
                    A[4 * u + 0] = v.x;
                    A[4 * u + 1] = v.y;
                    A[4 * u + 2] = v.z;
                    A[4 * u + 3] = v.w;
                }
                A[20] = 0u;
#pragma unroll
                for (int q = 0; q < 20; ++q)
                    sum = __builtin_amdgcn_sdot4((int)A[q], 0x01010101, sum, false);
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    const int o = 5 * b;   // byte offset of the group in the chunk
                    sl[t][i][b] = __builtin_amdgcn_alignbyte(A[o / 4 + 1], A[o / 4], o % 4);
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // codes 20d+4, 20d+9, 20d+14, 20d+19: byte 0 of A[5d+1], byte 1 of
                    // A[5d+2], byte 2 of A[5d+3], byte 3 of A[5d+4]
                    const uint32_t lo = __builtin_amdgcn_perm(A[5 * d + 2], A[5 * d + 1], 0x0c0c0500u);
                    const uint32_t hi = __builtin_amdgcn_perm(A[5 * d + 4], A[5 * d + 3], 0x07020c0cu);
                    p4[t][i][d] = lo | hi;
                }
            }
            xs[t] = sum;
        }

        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.Y + t0 * N), (short)0, (int)(mt * N * 4), kFlags);
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            a.acc ? (void*)(a.acc + t0 * N) : (void*)a.Y, (short)0, a.acc ? (int)(mt * N * 4) : 0, kFlags);

        auto compute_pass = [&](int64_t pb, const u32x4 (&w)[CPL]) {
            int32_t part[MT][2];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                part[t][0] = part[t][1] = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t wd[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint2 e[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        e[jj] = lut[(wd[d] >> (8 * jj)) & 0xffu];
                    const uint32_t f4 = __builtin_amdgcn_perm(e[1].y, e[0].y, 0x0c0c0400u) |
                                        __builtin_amdgcn_perm(e[3].y, e[2].y, 0x04000c0cu);
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            part[t][jj & 1] =
                                __builtin_amdgcn_sdot4((int)e[jj].x, (int)sl[t][i][4 * d + jj], part[t][jj & 1], false);
                        part[t][0] = __builtin_amdgcn_sdot4((int)f4, (int)p4[t][i][d], part[t][0], false);
                    }
                }
            }
            int32_t accv[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                accv[t] = group_sum<(L < 64 ? L : 64)>((part[t][0] + part[t][1]) - xs[t]);
            if constexpr (L > 64) {
                if ((tid & 63) == 0) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        red5[slot][j / 64][t] = accv[t];
                }
                __syncthreads();
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    int32_t v = 0;
#pragma unroll
                    for (int wv = 0; wv < WPR; ++wv)
                        v += red5[slot][wv][t];
                    accv[t] = v;
                }
                __syncthreads();
            }
            const int64_t row = pb + slot;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const bool mine = j == 0 && row < N && t < mt;
                const int off = mine ? (int)((t * N + row) * 4) : kPast;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, (float)accv[t] * csc[t]), ry, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(accv[t], ra, off, 0, 0);
            }
        };

        for (; rb < N; rb += 2 * pstride) {
            compute_pass(rb, cur);
            load_pass(rb + 2 * pstride, cur);
            if (rb + pstride >= N)
                break;
            compute_pass(rb + pstride, nxt);
            load_pass(rb + 3 * pstride, nxt);
        }
        tile += gridDim.y;
    } while (tile < ntiles);
}

// One output dword (four bytes) of the five-per-byte format from the 2-bit format.
// Thread g of row n writes bytes 4g..4g+3; code k's offset value q + 1 is field k % 4 of
// byte k / 4 of the 2-bit row, and codes past K count as zero codes (value 1).
__global__ __launch_bounds__(256) void repack5_kernel(const uint8_t* __restrict__ W2, int64_t N, int K,
                                                      uint8_t* __restrict__ W5, int RB)
{
    const int per_row = RB / 4;
    const int64_t total = N * (int64_t)per_row;
    const int KB = K / 4;
    for (int64_t g = blockIdx.x * 256LL + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t n = g / per_row;
        const int jb = (int)(g % per_row) * 4;
        const uint8_t* row = W2 + n * KB;
        uint32_t out = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            unsigned value = 0, weight = 1;
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int k = 5 * (jb + b) + i;
                const unsigned digit = k < K ? (row[k >> 2] >> (2 * (k & 3))) & 3u : 1u;
                value += digit * weight;
                weight *= 3u;
            }
            out |= value << (8 * b);
        }
        reinterpret_cast<uint32_t*>(W5 + n * (int64_t)RB)[jb / 4] = out;
    }
}

}  // namespace bl

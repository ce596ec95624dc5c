// gemv.hpp -- W1.58A8 product for few tokens (decode): packed ternary rows streamed from
// HBM with 128-bit non-temporal loads, unpacked in registers and multiplied with
// v_dot4 (int8 x int8 -> int32), then rescaled to fp32.
//
// The product y = (W_q x_q) * gamma / s ("BitNet b1.58 深度解析" s.2.3) is exact in
// int32 before the rescale. The pages' GPU recipe ("微软AI大模型炸场" s.3: pack ternary
// values into bytes in HBM, load on chip, unpack, compute) is kept in spirit; on gfx950
// the packed bytes go straight from HBM into VGPRs and never touch LDS.
//
// Unpack. A 16-byte chunk of a packed row holds codes k0 .. k0+63 (k0 = 64c). Dword d of
// the chunk holds bytes 4d..4d+3, byte jj holds codes k0 + 16d + 4jj + f in bits 2f.
// (dword >> 2f) & 0x03030303 therefore yields the four fields f of the four bytes, i.e.
// offset codes q + 1 in {0, 1, 2} for k0 + 16d + 4jj + f, jj = 0..3. The activations are
// held in the same order (a byte-transpose of each 16-byte group, done once per block),
// and sum_k (q+1) x - sum_k x = sum_k q x removes the offset exactly.
//
// Work split. A row is shared by L lanes (L = 8 .. 256); lane j owns chunks j, j+L, ...
// (at most 4/MT of them) and keeps their activation codes for MT tokens in VGPRs for
// the whole kernel. 256/L rows are processed per pass; the next pass's weights are
// loaded while the current pass is computed.
#pragma once

#include "device_common.hpp"

namespace bl {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct FwdArgs {
    const int8_t* Xq;      // pre-quantized activations [M][K] (unfused)
    const float* xscale;   // [M] (unfused)
    const float* X;        // fp32 activations [M][K] (fused)
    const float* gain;     // [K] or null (fused)
    float eps;             // (fused)
    int relu2;             // (fused)
    const uint8_t* W;      // packed [N][K/4]
    const float* gamma;    // [1]
    float* Y;              // [M][N]
    int32_t* acc;          // [M][N] or null
    int64_t M;
    int64_t N;
    int K;
};

template <int CPL, int L>
__device__ __forceinline__ void load_row_chunks(const uint8_t* __restrict__ W, int64_t KB, int KC, int64_t row,
                                                int64_t N, int j, u32x4 (&w)[CPL])
{
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = j + i * L;
        if (row < N && c < KC)
            w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + row * KB + (int64_t)c * 16));
        else
            w[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int L, int MT, bool FUSED>
__global__ __launch_bounds__(256) void gemv_k64_kernel(FwdArgs a)
{
    constexpr int NT = 256;
    constexpr int CPL = 4 / MT;           // chunks per lane
    constexpr int RPW = NT / L;           // rows per pass
    constexpr int WPR = L > 64 ? L / 64 : 1;  // waves per row
    const int tid = threadIdx.x;
    const int j = tid % L;
    const int slot = tid / L;
    const int KC = a.K >> 6;
    const int64_t KB = a.K >> 2;
    const int64_t ntiles = (a.M + MT - 1) / MT;
    const float gamma = *a.gamma;
    __shared__ int32_t xred[RPW][WPR][MT];

    for (int64_t tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        const int64_t t0 = tile * MT;
        const int mt = (int)((a.M - t0) < MT ? (a.M - t0) : MT);
        const int64_t rstride = (int64_t)gridDim.x * RPW;
        int64_t rb = (int64_t)blockIdx.x * RPW;

        // Weights of the first pass are requested before the activation prologue.
        u32x4 cur[CPL];
        load_row_chunks<CPL, L>(a.W, KB, KC, rb + slot, a.N, j, cur);

        uint32_t act[MT][CPL][16];
        int32_t xs[MT];
        float csc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float s = 1.0f;
            if (t < mt) {
                const int64_t tok = t0 + t;
                if constexpr (FUSED) {
                    const float* u = a.X + tok * (int64_t)a.K;
                    const bool norm = a.gain != nullptr;
                    const RowStats st = row_stats<NT>(u, a.K, a.gain, a.relu2, norm);
                    float sp;
                    token_scales(st, a.K, norm, a.eps, sp, s);
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int c = j + i * L;
#pragma unroll
                        for (int q = 0; q < 16; ++q)
                            act[t][i][q] = 0u;
                        if (c < KC) {
                            const float4* x4 = reinterpret_cast<const float4*>(u + (int64_t)c * 64);
                            const float4* g4 = reinterpret_cast<const float4*>(a.gain + (int64_t)c * 64);
#pragma unroll
                            for (int q4 = 0; q4 < 16; ++q4) {
                                const int d = q4 >> 2, jj = q4 & 3;
                                const float4 xv = x4[q4];
                                float4 gv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                                if (norm)
                                    gv = g4[q4];
                                const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
                                const float ga[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                                for (int f = 0; f < 4; ++f) {
                                    const float v = pre_v(xa[f], a.relu2);
                                    const float w = norm ? v * ga[f] : v;
                                    act[t][i][4 * d + f] |= (uint32_t)(act_code(w, sp) & 0xff) << (8 * jj);
                                }
                            }
                        }
                    }
                } else {
                    s = a.xscale[tok];
                    const int8_t* xr = a.Xq + tok * (int64_t)a.K;
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int c = j + i * L;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            uint32_t e[4] = {0u, 0u, 0u, 0u};
                            if (c < KC) {
                                const uint4 v = reinterpret_cast<const uint4*>(xr + (int64_t)c * 64)[d];
                                e[0] = v.x;
                                e[1] = v.y;
                                e[2] = v.z;
                                e[3] = v.w;
                            }
                            uint32_t o[4];
                            transpose_bytes(e[0], e[1], e[2], e[3], o);
#pragma unroll
                            for (int f = 0; f < 4; ++f)
                                act[t][i][4 * d + f] = o[f];
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < CPL; ++i)
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        act[t][i][q] = 0u;
            }
            csc[t] = gamma / s;
            int32_t sum = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    sum = __builtin_amdgcn_sdot4((int)act[t][i][q], 0x01010101, sum, false);
            xs[t] = sum;
        }

        for (; rb < a.N; rb += rstride) {
            const int64_t row = rb + slot;
            u32x4 nxt[CPL];
            load_row_chunks<CPL, L>(a.W, KB, KC, rb + rstride + slot, a.N, j, nxt);

            int32_t accv[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                accv[t] = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t wd[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const uint32_t u = (wd[d] >> (2 * f)) & 0x03030303u;
#pragma unroll
                        for (int t = 0; t < MT; ++t)
                            accv[t] = __builtin_amdgcn_sdot4((int)u, (int)act[t][i][4 * d + f], accv[t], false);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                int32_t v = accv[t] - xs[t];
                if constexpr (L <= 64) {
#pragma unroll
                    for (int m = L / 2; m >= 1; m >>= 1)
                        v += __shfl_xor(v, m);
                } else {
#pragma unroll
                    for (int m = 32; m >= 1; m >>= 1)
                        v += __shfl_xor(v, m);
                }
                accv[t] = v;
            }
            if constexpr (L > 64) {
                if ((tid & 63) == 0) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        xred[slot][j / 64][t] = accv[t];
                }
                __syncthreads();
                if (j == 0) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        int32_t v = 0;
#pragma unroll
                        for (int w = 0; w < WPR; ++w)
                            v += xred[slot][w][t];
                        accv[t] = v;
                    }
                }
                __syncthreads();
            }
            if (j == 0 && row < a.N) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t < mt) {
                        const int64_t o = (t0 + t) * a.N + row;
                        a.Y[o] = (float)accv[t] * csc[t];
                        if (a.acc)
                            a.acc[o] = accv[t];
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                cur[i] = nxt[i];
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
                    const RowStats st = row_stats<256>(a.X + (t0 + t) * (int64_t)a.K, a.K, a.gain, a.relu2, norm);
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
                                    const float v = pre_v(a.X[(t0 + t) * (int64_t)a.K + k], a.relu2);
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
                    a.Y[o] = (float)accv[t] * csc[t];
                    if (a.acc)
                        a.acc[o] = accv[t];
                }
            }
        }
    }
}

}  // namespace bl

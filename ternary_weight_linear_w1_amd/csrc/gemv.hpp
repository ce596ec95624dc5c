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
// (dword >> 2f) & 0x03030303 therefore yields the four fields f of the four bytes, i.e.
// offset codes q + 1 in {0, 1, 2} for k0 + 16d + 4jj + f, jj = 0..3. The activations are
// held in the same order (a byte-transpose of each 16-byte group, done once per block),
// and sum_k (q+1) x - sum_k x = sum_k q x removes the offset exactly.
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

// Loads of one pass: lane j of row group `slot` fetches, for each of its R rows, the
// chunks j, j+L, ... (CPL of them) as 16-byte non-temporal loads.
template <int L, int CPL, int R, int RG>
__device__ __forceinline__ void load_pass(const uint8_t* __restrict__ W, int64_t KB, int KC, int64_t rb, int64_t N,
                                          int slot, int j, u32x4 (&w)[R][CPL])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = rb + slot + (int64_t)r * RG;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = j + i * L;
            if (row < N && c < KC)
                w[r][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + row * KB + (int64_t)c * 16));
            else
                w[r][i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Activation codes of MT tokens are staged once per block in LDS, in the unpack order:
// the 16 codes k0..k0+15 of one 16-element unit u (k0 = 16u) are stored as four dwords,
// dword f holding codes k0 + 4jj + f in byte jj. Unit u lives at LDS bytes 16u..16u+15,
// so chunk c (units 4c..4c+3) is the 64 bytes at 64c, read with four 16-byte LDS loads.
// Codes of float4 group g (elements 4g..4g+3) into the LDS unpack order: element
// k = 64c + 16d + 4jj + f goes to byte 64c + 4(4d + f) + jj.
__device__ __forceinline__ void put_group_codes(uint8_t* __restrict__ bytes, int g, float4 w, float sp)
{
    const int base = 64 * (g >> 4) + 16 * ((g >> 2) & 3) + (g & 3);
    bytes[base + 0] = (uint8_t)act_code(w.x, sp);
    bytes[base + 4] = (uint8_t)act_code(w.y, sp);
    bytes[base + 8] = (uint8_t)act_code(w.z, sp);
    bytes[base + 12] = (uint8_t)act_code(w.w, sp);
}

constexpr int kKeep = 8;  // float4 groups per thread kept in VGPRs by the fused prologue

template <int MT, bool FUSED>
__device__ __forceinline__ void stage_codes(const FwdArgs& a, int64_t t0, int mt, uint4* __restrict__ lds,
                                            float (&s)[MT])
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
        const int64_t tok = t0 + t;
        if constexpr (FUSED) {
            const float* x = a.X + tok * (int64_t)a.K;
            const bool norm = a.gain != nullptr;
            float4 wk[kKeep];
            const RowStats st = row_stats<NT, kKeep>(x, a.K, a.gain, a.relu2, norm, wk);
            float sp;
            token_scales(st, a.K, norm, a.eps, sp, s[t]);
            uint8_t* bytes = reinterpret_cast<uint8_t*>(dst);
            const int G = a.K >> 2;
#pragma unroll
            for (int q = 0; q < kKeep; ++q) {
                const int g = tid + q * NT;
                if (g < G)
                    put_group_codes(bytes, g, wk[q], sp);
            }
            for (int g = tid + kKeep * NT; g < G; g += NT) {
                const float4 xv = reinterpret_cast<const float4*>(x)[g];
                float4 gv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                if (norm)
                    gv = reinterpret_cast<const float4*>(a.gain)[g];
                const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
                const float ga[4] = {gv.x, gv.y, gv.z, gv.w};
                float wa[4];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const float v = pre_v(xa[f], a.relu2);
                    wa[f] = norm ? v * ga[f] : v;
                }
                put_group_codes(bytes, g, make_float4(wa[0], wa[1], wa[2], wa[3]), sp);
            }
        } else {
            s[t] = a.xscale[tok];
            const uint4* src = reinterpret_cast<const uint4*>(a.Xq + tok * (int64_t)a.K);
            for (int u = tid; u < units; u += NT) {
                const uint4 v = src[u];
                uint32_t o[4];
                transpose_bytes(v.x, v.y, v.z, v.w, o);
                dst[u] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// L lanes per row, MT tokens per tile, CPL chunks per lane (16*CPL*MT VGPRs of
// activation codes, CPL*MT <= 4), R rows per lane per pass: R*CPL 16-byte weight loads
// are in flight per lane, and the next pass is requested before the current one is
// computed.
template <int L, int MT, int CPL, int R, bool FUSED>
__global__ __launch_bounds__(256) void gemv_k64_kernel(FwdArgs a)
{
    constexpr int NT = 256;
    static_assert(CPL * MT <= 4, "activation codes must fit in 64 VGPRs");
    constexpr int RG = NT / L;             // row groups per block
    constexpr int RPP = RG * R;            // rows per pass
    constexpr int WPR = L > 64 ? L / 64 : 1;
    extern __shared__ uint4 lds_codes[];
    __shared__ int32_t xred[RG][WPR][R][MT];
    const int tid = threadIdx.x;
    const int j = tid % L;
    const int slot = tid / L;
    const int KC = a.K >> 6;
    const int64_t KB = a.K >> 2;
    const int64_t ntiles = (a.M + MT - 1) / MT;
    const float gamma = *a.gamma;

    for (int64_t tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        const int64_t t0 = tile * MT;
        const int mt = (int)((a.M - t0) < MT ? (a.M - t0) : MT);
        const int64_t pstride = (int64_t)gridDim.x * RPP;
        int64_t rb = (int64_t)blockIdx.x * RPP;

        // Weights of the first pass are requested before the activation prologue.
        u32x4 cur[R][CPL];
        load_pass<L, CPL, R, RG>(a.W, KB, KC, rb, a.N, slot, j, cur);

        float s[MT];
        __syncthreads();  // LDS of the previous tile is no longer read
        stage_codes<MT, FUSED>(a, t0, mt, lds_codes, s);
        __syncthreads();

        uint32_t act[MT][CPL][16];
        int32_t xs[MT];
        float csc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const uint4* src = lds_codes + (size_t)t * (a.K >> 4);
            int32_t sum = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = j + i * L;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint4 v = make_uint4(0u, 0u, 0u, 0u);
                    if (c < KC)
                        v = src[4 * c + d];
                    act[t][i][4 * d + 0] = v.x;
                    act[t][i][4 * d + 1] = v.y;
                    act[t][i][4 * d + 2] = v.z;
                    act[t][i][4 * d + 3] = v.w;
                }
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    sum = __builtin_amdgcn_sdot4((int)act[t][i][q], 0x01010101, sum, false);
            }
            xs[t] = sum;
            csc[t] = gamma / s[t];
        }

        for (; rb < a.N; rb += pstride) {
            u32x4 nxt[R][CPL];
            load_pass<L, CPL, R, RG>(a.W, KB, KC, rb + pstride, a.N, slot, j, nxt);

            int32_t accv[R][MT];
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    accv[r][t] = 0;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const uint32_t wd[4] = {cur[r][i].x, cur[r][i].y, cur[r][i].z, cur[r][i].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
#pragma unroll
                        for (int f = 0; f < 4; ++f) {
                            const uint32_t u = (wd[d] >> (2 * f)) & 0x03030303u;
#pragma unroll
                            for (int t = 0; t < MT; ++t)
                                accv[r][t] = __builtin_amdgcn_sdot4((int)u, (int)act[t][i][4 * d + f], accv[r][t], false);
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    int32_t v = accv[r][t] - xs[t];
                    constexpr int top = L <= 64 ? L / 2 : 32;
#pragma unroll
                    for (int m = top; m >= 1; m >>= 1)
                        v += __shfl_xor(v, m);
                    accv[r][t] = v;
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
                if (j == 0) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            int32_t v = 0;
#pragma unroll
                            for (int w = 0; w < WPR; ++w)
                                v += xred[slot][w][r][t];
                            accv[r][t] = v;
                        }
                }
                __syncthreads();
            }
            if (j == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t row = rb + slot + (int64_t)r * RG;
                    if (row < a.N) {
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            if (t < mt) {
                                const int64_t o = (t0 + t) * a.N + row;
                                a.Y[o] = (float)accv[r][t] * csc[t];
                                if (a.acc)
                                    a.acc[o] = accv[r][t];
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    cur[r][i] = nxt[r][i];
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

// gemv_mfma.hpp -- W1.58A8 product for a few tokens (2..32) on the int8 matrix cores.
//
// The same product as gemv.hpp ("BitNet b1.58 深度解析" s.2.3: y = (W_q x_q) * gamma / s,
// exact in int32 before the rescale), for token counts where the vector dot products
// would cost more ALU than the weight stream can hide: with several tokens every packed
// byte feeds 4 * M dot4 lanes. Here each packed byte is unpacked once and the products
// of all tokens come from v_mfma_i32_16x16x64_i8 (16 tokens x 16 weight rows x 64 codes
// per instruction, TT such tiles sharing each unpacked weight operand; tokens past M
// multiply a zero slot).
//
// Layout. One block per CU holds every activation code of the call in LDS, permuted once
// into the matrix-core operand order; the weights stream from HBM straight into VGPRs.
// A unit of work is 16 weight rows x up to WPU windows of 256 codes (each wave loads a
// unit, then computes it; the waves of the block keep the loads in flight); lane l of a wave
// takes row l % 16 and, in each window, the 16 packed bytes 16 (l / 16) .. + 15, i.e.
// codes 64 g + 16 d + 4 jj + f (g = l / 16, dword d, byte jj, field f). Field f of the
// four dwords, masked in place (w & 0x03030303, w & 0x0C0C0C0C, w & 0x30303030,
// (w >> 2) & 0x30303030: the offset codes q + 1 times 1, 4, 16, 16), is the weight operand
// of one instruction; its activation operand holds the same codes' activations, so the
// codes each instruction pairs agree and every code is used once. The scales 1, 4 and 16
// accumulate separately and combine exactly (each accumulator is a multiple of its scale).
// The units of a row group (its K range cut into pieces) are spread over the block's
// waves and summed with LDS integer atomics (exact in any order); after one barrier the
// block writes y = fl(fl(acc - sum_k x) * fl(gamma / s)) as the other product kernels do.
//
// The activation operand of instruction f in window w, lane group g, for token i is the
// 16 bytes x_i[256 w + 64 g + 4 m + f], m = 0..15 (a 16 x 4 byte transpose of the
// 64-byte group), stored at slot ((w * 4 + g) * 4 + f) * MS + i; slot i = M (when M < 16)
// is all zeros and serves the lanes of tokens M..15.
//
// Rows too long for LDS (e.g. 8 tokens at K = 28672) are walked in phases of NWP windows:
// each phase stages its slice of the codes, runs its units, and the block synchronises
// before the next slice overwrites it (the row sums and accumulators carry over).
#pragma once

#include "gemv.hpp"

namespace bl {

typedef int mf_v4i __attribute__((ext_vector_type(4)));

// Token slots of gemv_mfma_kernel with TT tiles of 16 tokens: M, plus a zero slot when
// the tiles are not full.
inline int64_t gemv_mfma_slots(int64_t M, int tt)
{
    return M < 16 * tt ? M + 1 : 16 * tt;
}

// LDS bytes of gemv_mfma_kernel with phases of nwp windows: activation slots, the row
// groups' accumulators, row sums.
inline size_t gemv_mfma_lds_bytes(int64_t M, int tt, int64_t nwp, int64_t rg_per_block)
{
    return (size_t)(nwp * 16 * gemv_mfma_slots(M, tt) * 16 + rg_per_block * 16 * 16 * tt * 4 + 16 * tt * 4);
}

// TT tiles of 16 tokens share each unpacked weight operand (M <= 16 TT).
template <int WPU, int NWAVES = 16, int TT = 1, int SI = 4>
__global__ __launch_bounds__(NWAVES * 64) void gemv_mfma_kernel(FwdArgs a, int nwp)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int NT = NWAVES * 64;
    const int M = (int)a.M;
    const int N = (int)a.N;
    const int K = a.K;
    const int KB = K >> 2;
    const int NW = (K + 255) >> 8;                 // windows of 256 codes
    constexpr int MT16 = 16 * TT;                  // tokens the tiles hold
    const int MS = M < MT16 ? M + 1 : MT16;        // token slots (slot M: zeros)
    const int NG = (N + 15) >> 4;                  // row groups of 16
    const int g0 = (int)((int64_t)blockIdx.x * NG / gridDim.x);
    const int g1 = (int)((int64_t)(blockIdx.x + 1) * NG / gridDim.x);
    const int RGB = g1 - g0;
    const int NWP = nwp;                           // windows per phase (a multiple of WPU)
    const int NPH = (NW + NWP - 1) / NWP;
    const int KW = NWP / WPU;                      // units per row group and phase
    const int nunits = RGB * KW;                   // units per phase

    uint8_t* As = smem;
    int32_t* accs = reinterpret_cast<int32_t*>(smem + NWP * 16 * MS * 16);
    int32_t* rsum = accs + RGB * 16 * MT16;

    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.W, (short)0, (int)((int64_t)N * KB), kBufFlags);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.Xq, (short)0, M * K, kBufFlags);

    // ---- weight loads of one unit (rows past N and windows past K read as zero)
    const int lrow = lane & 15, lg = lane >> 4;
    auto load_unit = [&](u32x4 (&wr)[WPU], int u, int ph) {
        const bool live = u < nunits;
        const int rg = live ? u / KW : 0, p = live ? u % KW : 0;
        const int n = (g0 + rg) * 16 + lrow;
        const int base = n * KB + 16 * lg;
#pragma unroll
        for (int s = 0; s < WPU; ++s) {
            const int w = ph * NWP + p * WPU + s;
            const int off = (live && w < NW) ? base + 64 * w : kOob;
            wr[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
        }
    };
    u32x4 wr[WPU];

    // ---- zero the accumulators, the row sums and the zero slot
    for (int i = tid; i < RGB * 16 * MT16; i += NT)
        accs[i] = 0;
    if (tid < MT16)
        rsum[tid] = 0;
    if (M < MT16) {
        for (int i = tid; i < NWP * 16; i += NT)
            *reinterpret_cast<uint4*>(As + (i * MS + M) * 16) = make_uint4(0u, 0u, 0u, 0u);
    }

    int slot[TT];                                  // token slot of this lane's operand, per tile
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
        slot[tt] = 16 * tt + lrow < M ? 16 * tt + lrow : MS - 1;
    for (int ph = 0; ph < NPH; ++ph) {
        __syncthreads();                           // zeroed state, or the last phase's reads done

        // ---- stage this phase's activation codes and add their row sums. Every group's
        // loads are issued before any is used (up to SI groups per thread).
        const int items = M * NWP * 4;             // 64-byte groups (token, window, g)
        for (int it0 = tid; it0 < items; it0 += NT * SI) {
            u32x4 v[SI][4];
#pragma unroll
            for (int k = 0; k < SI; ++k) {
                const int it = it0 + NT * k;
                const int t = it / (NWP * 4);
                const int k0 = 64 * (ph * NWP * 4 + it % (NWP * 4));
                // K % 64 == 0: a group lies wholly inside or wholly past the row
                const bool in = it < items && k0 < K;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[k][q] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, in ? t * K + k0 + 16 * q : kOob, 0, 0));
            }
#pragma unroll
            for (int k = 0; k < SI; ++k) {
                const int it = it0 + NT * k;
                if (it < items) {
                    const int t = it / (NWP * 4);
                    const int wg = it % (NWP * 4);  // local window * 4 + g
                    int32_t sm = 0;
                    uint32_t o[4][4];               // o[f][q]: bytes 4 (4q + 0..3) + f
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sm = __builtin_amdgcn_sdot4((int)v[k][q][e], 0x01010101, sm, false);
                        uint32_t tq[4];
                        transpose_bytes(v[k][q][0], v[k][q][1], v[k][q][2], v[k][q][3], tq);
#pragma unroll
                        for (int f = 0; f < 4; ++f)
                            o[f][q] = tq[f];
                    }
#pragma unroll
                    for (int f = 0; f < 4; ++f)
                        *reinterpret_cast<uint4*>(As + ((wg * 4 + f) * MS + t) * 16) =
                            make_uint4(o[f][0], o[f][1], o[f][2], o[f][3]);
                    atomicAdd(&rsum[t], sm);
                }
            }
        }
        __syncthreads();

        // ---- units: 16 rows x WPU windows, products on the matrix cores
        auto compute_unit = [&](const u32x4 (&wr)[WPU], int u) {
            const int rg = u / KW, p = u % KW;
            mf_v4i c[TT][4];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    c[tt][f] = mf_v4i{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < WPU; ++s) {
                const int lw = p * WPU + s;
                if (ph * NWP + lw < NW) {          // uniform across the wave
                    mf_v4i b[4];
#pragma unroll
                    for (int dd = 0; dd < 4; ++dd) {
                        const uint32_t x = wr[s][dd];
                        b[0][dd] = (int)(x & 0x03030303u);
                        b[1][dd] = (int)(x & 0x0C0C0C0Cu);
                        b[2][dd] = (int)(x & 0x30303030u);
                        b[3][dd] = (int)((x >> 2) & 0x30303030u);
                    }
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) {
                        const uint8_t* ab = As + ((lw * 4 + lg) * 4 * MS + slot[tt]) * 16;
#pragma unroll
                        for (int f = 0; f < 4; ++f)
                            c[tt][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                *reinterpret_cast<const mf_v4i*>(ab + f * MS * 16), b[f], c[tt][f], 0, 0, 0);
                    }
                }
            }
            // D layout of a 16 x 16 tile: lane l, register r -> token 4 (l / 16) + r, row l % 16
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tt + 4 * lg + r;
                    if (t < M)
                        atomicAdd(&accs[(rg * MT16 + t) * 16 + lrow],
                                  c[tt][0][r] + (c[tt][1][r] >> 2) + ((c[tt][2][r] + c[tt][3][r]) >> 4));
                }
        };
        // One unit at a time per wave: the block's 16 waves keep the loads in flight. (A
        // three-unit register ring per wave with 12 waves measured 0-12% slower: the compiler
        // does not keep the ring's buffers in fixed registers, so each wait for a unit's
        // weights became a wait for all loads in flight.)
        for (int u = wave; u < nunits; u += NWAVES) {
            load_unit(wr, u, ph);
            compute_unit(wr, u);
        }
    }
    __syncthreads();

    // ---- epilogue
    const float gamma = *a.gamma;
    for (int i = tid; i < RGB * M * 16; i += NT) {
        const int rg = i / (M * 16);
        const int t = (i >> 4) % M;
        const int j = i & 15;
        const int n = (g0 + rg) * 16 + j;
        if (n < N) {
            const int32_t v = accs[(rg * MT16 + t) * 16 + j] - rsum[t];
            const int64_t o = (int64_t)t * N + n;
            const float yv = (float)v * (gamma / a.xscale[t]);
            a.Y[o] = a.residual ? a.Y[o] + yv : yv;
            if (a.acc)
                a.acc[o] = v;
        }
    }
}

}  // namespace bl

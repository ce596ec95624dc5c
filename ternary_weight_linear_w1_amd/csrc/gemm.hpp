// gemm.hpp -- W1.58A8 product for many tokens (prefill, small batches) on the int8
// matrix cores of gfx950: v_mfma_i32_32x32x32_i8, exact int32 accumulation, fp32 rescale.
//
// The work is a dense contraction over K ("BitNet b1.58 深度解析" s.2.3: y = (W_q x_q) *
// scale), so it runs on MFMA. Operands of one 32x32x32 MFMA: lane l supplies row (l % 32)
// of A (tokens) and column (l % 32) of B (output features), 16 int8 each for k-slot half
// l / 32. Which k sits in which slot is free as long as A and B agree; here the slots
// follow the register unpack of the packed weights:
//   B  lane half g of k-substep ks holds the packed dword at byte k0/4 + 16g + 4ks of its
//      row, i.e. codes k0 + 64g + 16ks + 4jj + f (byte jj, field f). (w >> 2f) & 0x03030303
//      gives the offset codes q + 1 for f = 0..3, which form the four operand dwords.
//   A  the same 16 activations, byte-transposed once when the tile is staged in LDS
//      (LDS dword f, byte jj = activation k0 + 16c + 4jj + f).
// The offset is removed exactly in the epilogue: sum_k (q+1) x - sum_k x.
//
// Block: 256 threads = WM x WN waves, block tile BM x BN, K in steps of 128. The
// activation tile is double-buffered in LDS; global loads run P steps ahead through a
// ring of VGPR stages while the current step runs on the matrix cores. With WM = 1
// every wave owns distinct weight columns, so each packed byte is unpacked once per
// block.
#pragma once

#include "device_common.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct GemmArgs {
    const int8_t* Xq;     // [M][K]
    const float* xscale;  // [M]
    const uint8_t* W;     // [N][K/4]
    const float* gamma;   // [1]
    float* Y;             // [M][N]; with `residual` read and overwritten by Y + product
    int32_t* acc;         // [M][N] or null
    int M;
    int N;
    int K;
    int residual;         // 1: Y[m][n] = fl32(Y[m][n] + y[m][n])
    int gm;               // tile-grid regions along M (1, 2, 4 or 8; 8 / gm along N)
    // Split K (few tokens): block b takes K slice b % ksplit (kslice columns, a multiple of
    // the K step) of tile b / ksplit and writes its exact int32 partial to
    // part[slice][M][N]; gemm_splitk_reduce_kernel then sums the slices and rescales.
    int32_t* part;        // null: no split, the block writes y itself
    int ksplit;           // 1 without a split
    int kslice;
};

// Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous range of tiles
// in an order where such a range is a rectangle of the tile grid, so that the activation
// rows and weight columns it needs stay in that XCD's L2. The grid is cut into gm x
// (8 / gm) regions (gm chosen on the host to minimise one region's operand bytes), listed
// region by region, m fastest inside a region.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles)
{
    constexpr int kXcd = 8;
    const int per = ntiles / kXcd, rem = ntiles % kXcd;
    const int x = bid % kXcd, i = bid / kXcd;
    return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// Host side: the region split gm (of 1, 2, 4, 8 along M; 8 / gm along N) whose region
// needs the fewest operand bytes (its activation rows plus its packed weight columns).
inline int gemm_region_split(int64_t tiles_m, int64_t tiles_n, int BM, int BN, int64_t K)
{
    int best = 1;
    int64_t best_bytes = -1;
    for (int gm = 1; gm <= 8; gm *= 2) {
        const int gn = 8 / gm;
        if (gm > tiles_m || gn > tiles_n)
            continue;
        const int64_t bytes = (tiles_m + gm - 1) / gm * BM * K + (tiles_n + gn - 1) / gn * BN * (K / 4);
        if (best_bytes < 0 || bytes < best_bytes) {
            best = gm;
            best_bytes = bytes;
        }
    }
    return best;
}

__device__ __forceinline__ void region_tile(int idx, int tiles_m, int tiles_n, int gm, int& tm, int& tn)
{
    const int gn = 8 / gm;
    const int sm = (tiles_m + gm - 1) / gm, sn = (tiles_n + gn - 1) / gn;
    tm = 0;
    tn = 0;
    for (int rn = 0; rn < gn; ++rn) {
        const int n0 = rn * sn, nn = min(sn, tiles_n - n0);
        if (nn <= 0)
            break;
        for (int rm = 0; rm < gm; ++rm) {
            const int m0 = rm * sm, mm = min(sm, tiles_m - m0);
            if (mm <= 0)
                break;
            if (idx < mm * nn) {
                tm = m0 + idx % mm;
                tn = n0 + idx / mm;
                return;
            }
            idx -= mm * nn;
        }
    }
}

// Raw buffer loads: 32-bit offsets from a per-tile base and hardware zero-fill beyond the
// buffer's size, so rows past M or N need no masks. Descriptor word 3 for gfx9.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Output of a block's tile (shared by the GEMM kernels): C[fm][fn] of the wave at (wm, wn)
// minus the row's code sum, times the row's scale.
// C layout of a 32x32 tile: lane l, register r -> column l % 32,
// row 8 (r / 4) + 4 (l / 32) + r % 4. Each row's offset and scale are read once.
template <int BM, int BN, int TM, int TN, int FM, int FN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const v16i (&C)[FM][FN], const int32_t* rsum,
                                              const float* csc, int m0, int n0, int wm, int wn, int lane, int slice)
{
    const int M = a.M, N = a.N;
    if (a.part) {   // split K: the exact int32 partial of this slice
        int32_t* pt = a.part + (int64_t)slice * M * N;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * TM + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int m = m0 + row;
                if (m < M) {
                    const int32_t off = rsum[row];
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const int n = n0 + wn * TN + fn * 32 + (lane & 31);
                        if (n < N)
                            pt[(int64_t)m * N + n] = C[fm][fn][r] - off;
                    }
                }
            }
        return;
    }
    // Common case (whole tile inside N, plain output, no int32 copy, 32-bit byte offsets):
    // buffer stores with the row's byte offset computed once and the 32-column step as the
    // instruction's immediate; rows past M fall outside the buffer and are dropped.
    if (n0 + BN <= N && !a.residual && !a.acc && (int64_t)(M + BM) * N < (int64_t(1) << 29)) {
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.Y, (short)0, M * N * 4, kBufferFlags);
        const int col = n0 + wn * TN + (lane & 31);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * TM + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int32_t off = rsum[row];
                const float c = csc[row];
                const int voff = ((m0 + row) * N + col) * 4;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const float yv = (float)(C[fm][fn][r] - off) * c;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, yv), ry, voff + 128 * fn, 0, 0);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * TM + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int m = m0 + row;
            if (m < M) {
                const int32_t off = rsum[row];
                const float c = csc[row];
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int n = n0 + wn * TN + fn * 32 + (lane & 31);
                    if (n < N) {
                        const int32_t v = C[fm][fn][r] - off;
                        const int64_t o = (int64_t)m * N + n;
                        const float yv = (float)v * c;
                        a.Y[o] = a.residual ? a.Y[o] + yv : yv;
                        if (a.acc)
                            a.acc[o] = v;
                    }
                }
            }
        }
    }
}

// WK > 1 splits K inside the block: each step stages WK * BK columns of activations and
// wave group g (of WM x WN waves) multiplies columns g*BK .. g*BK + BK - 1; the groups'
// int32 partial sums are added through LDS before the epilogue (exact, fixed order).
// This gives narrow tiles (and so more blocks) for few tokens and long rows.
template <int BM, int BN, int WM, int WN, int P, int BK = 128, int WK = 1>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a)
{
    static_assert(WM * WN * WK == 4, "four waves per block");
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
    static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BK == 128 || BK == 256, "K step of 128 or 256");
    constexpr int KS = BK / 32;                  // MFMA k-substeps per step (per wave group)
    constexpr int BH = BK / 128;                 // 16-byte weight loads per fragment per step
    constexpr int SK = BK * WK;                  // columns staged per step
    constexpr int AST = SK + 16;                 // LDS row stride in bytes (padded)
    constexpr int UPR = SK / 16;                 // 16-byte activation units per row
    constexpr int AU = BM * UPR / 256;           // 16-byte activation units per thread per step
    static_assert(AU >= 1, "block tile too small");

    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * AST];
    __shared__ int32_t rsum[BM];
    __shared__ float csc[BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wk = wave / (WM * WN);
    const int wm = (wave % (WM * WN)) / WN, wn = wave % WN;
    const int M = a.M, N = a.N, K = a.K;
    const int KB = K >> 2;

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    const int slice = a.part ? (int)(blockIdx.x % a.ksplit) : 0;
    const int bid = a.part ? (int)(blockIdx.x / a.ksplit) : (int)blockIdx.x;
    region_tile(xcd_tile(bid, tiles_m * tiles_n), tiles_m, tiles_n, a.gm, tm, tn);
    // this block's K columns: [kbeg, kbeg + klen)
    const int kbeg = a.part ? slice * a.kslice : 0;
    const int klen = a.part ? ((K - kbeg) < a.kslice ? (K - kbeg) : a.kslice) : K;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    if (tid < BM) {
        const int m = m0 + tid;
        csc[tid] = m < M ? *a.gamma / a.xscale[m] : 0.0f;
    }

    const int arows = (M - m0) < BM ? (M - m0) : BM;
    const int brows = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.Xq + (int64_t)m0 * K), (short)0, arows * K, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (int64_t)n0 * KB), (short)0, brows * KB, kBufferFlags);

    // Activation unit i of this thread: row (tid + 256 i) / UPR, 16-byte column tid % UPR.
    // Weight fragment fn of this lane: row wn*TN + 32 fn + lane % 32; for each 128-wide
    // half h of the step, 16 bytes at 32 h + 16 (lane / 32).
    int aoff[AU], boff[FN];
#pragma unroll
    for (int i = 0; i < AU; ++i)
        aoff[i] = ((tid + 256 * i) / UPR) * K + 16 * (tid % UPR);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        boff[fn] = (wn * TN + fn * 32 + (lane & 31)) * KB + 16 * (lane >> 5) + (wk * BK) / 4;
    const int acol = 16 * (tid % UPR);        // k offset of this thread's activation unit

    // Prefetch ring: the loads for step it + P are issued while step it is computed.
    u32x4 areg[P][AU];
    u32x4 breg[P][FN][BH];
    int32_t rs[AU];
#pragma unroll
    for (int i = 0; i < AU; ++i)
        rs[i] = 0;

    auto load = [&](u32x4 (&ad)[AU], u32x4 (&bd)[FN][BH], int k0) {
#pragma unroll
        for (int i = 0; i < AU; ++i)
            ad[i] = buf_load16(ra, aoff[i], kbeg + k0);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int h = 0; h < BH; ++h)
                bd[fn][h] = buf_load16(rb, boff[fn], ((kbeg + k0) >> 2) + 32 * h);
    };
    // The last step may extend past K (K % BK is a multiple of 64): activations loaded
    // from beyond the row end belong to the next row and are replaced by zeros, which also
    // zeroes those columns' products whatever the weight bytes there hold.
    auto store_a = [&](const u32x4 (&src)[AU], int buf, int kvalid, bool tail) {
#pragma unroll
        for (int i = 0; i < AU; ++i) {
            const int u = tid + 256 * i;
            const int r = u / UPR, c = u % UPR;
            u32x4 v = src[i];
            if (tail && acol >= kvalid)   // `tail` is a constant after inlining
                v = u32x4{0u, 0u, 0u, 0u};
            uint32_t o[4];
            transpose_bytes(v[0], v[1], v[2], v[3], o);
#pragma unroll
            for (int f = 0; f < 4; ++f)
                rs[i] = __builtin_amdgcn_sdot4((int)o[f], 0x01010101, rs[i], false);
            *reinterpret_cast<uint4*>(&As[buf][r * AST + 16 * c]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };

    v16i C[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                C[fm][fn][r] = 0;

    const int nk = (klen + SK - 1) / SK;
#pragma unroll
    for (int s = 0; s < P; ++s)
        if (s < nk)
            load(areg[s], breg[s], s * SK);
    store_a(areg[0], 0, klen, true);
    __syncthreads();

    // One K step on ring slot s: unpack its weights (the slot is refilled right after),
    // read the activation fragments, run the 4 * FM * FN matrix instructions, stage the
    // next step's activations into the other LDS buffer.
    auto step = [&](int it, int s, bool reload, bool stage, bool tail) {
        // Keep each step's instructions inside the step: hoisting the next step's unpack
        // would make it wait for the newest loads and raise the register count.
        __builtin_amdgcn_sched_barrier(0);
        const int buf = it & 1;
        // Weight bytes past the row end need no mask (the activations there are 0).
        v4i bf[KS][FN];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint32_t w = breg[s][fn][ks >> 2][ks & 3];
                bf[ks][fn][0] = (int)(w & 0x03030303u);
                bf[ks][fn][1] = (int)((w >> 2) & 0x03030303u);
                bf[ks][fn][2] = (int)((w >> 4) & 0x03030303u);
                bf[ks][fn][3] = (int)((w >> 6) & 0x03030303u);
            }
        if (reload)
            load(areg[s], breg[s], (it + P) * SK);
        const uint8_t* Ab = As[buf];
        v4i af[KS][FM];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = wm * TM + fm * 32 + (lane & 31);
                af[ks][fm] = *reinterpret_cast<const v4i*>(Ab + r * AST + wk * BK + 128 * (ks >> 2) +
                                                           64 * (lane >> 5) + 16 * (ks & 3));
            }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    C[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks][fm], bf[ks][fn], C[fm][fn], 0, 0, 0);
        if (stage)
            store_a(areg[(s + 1) % P], buf ^ 1, klen - (it + 1) * SK, tail);
        __syncthreads();
    };

    // Steady state: every step refills its slot and stages a step that lies wholly inside
    // K, with no conditions, so the ring slots stay in fixed registers and a step waits
    // only for its own loads (a conditional refill would make the compiler rotate the ring
    // through register copies, which must wait for every load in flight).
    int it = 0;
    for (; it + 2 * P <= nk; it += P) {
#pragma unroll
        for (int s = 0; s < P; ++s)
            step(it + s, s, true, true, false);
    }
    // The last (fewer than 2P) steps.
#pragma unroll
    for (int s = 0; s < 2 * P - 1; ++s) {
        const int t = it + s;
        if (t < nk)
            step(t, s % P, t + P < nk, t + 1 < nk, true);
    }

    // Row sums of the activation codes: thread tid holds rows (tid + 256 i) / UPR for
    // the column group tid % UPR; the UPR groups of a row are adjacent lanes.
#pragma unroll
    for (int i = 0; i < AU; ++i) {
        int v = rs[i];
#pragma unroll
        for (int m = 1; m < UPR; m <<= 1)
            v += __shfl_xor(v, m);
        if ((tid % UPR) == 0)
            rsum[(tid + 256 * i) / UPR] = v;
    }
    __syncthreads();

    if constexpr (WK > 1) {
        // partial sums of wave groups 1.. through LDS into group 0 (the staging buffers are
        // free: every wave has passed the last step's barrier)
        static_assert((WK - 1) * WM * WN * FM * FN * 16 * 64 * 4 <= 2 * BM * AST, "reduction fits in LDS");
        int32_t* red = reinterpret_cast<int32_t*>(&As[0][0]);
        const int slot_base = ((wm * WN + wn) * FM * FN) * 16 * 64;
        if (wk > 0) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        red[(wk - 1) * WM * WN * FM * FN * 16 * 64 + slot_base + ((fm * FN + fn) * 16 + r) * 64 + lane] =
                            C[fm][fn][r];
        }
        __syncthreads();
        if (wk > 0)
            return;
#pragma unroll
        for (int g = 1; g < WK; ++g)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        C[fm][fn][r] += red[(g - 1) * WM * WN * FM * FN * 16 * 64 + slot_base + ((fm * FN + fn) * 16 + r) * 64 + lane];
    }

    gemm_epilogue<BM, BN, TM, TN, FM, FN>(a, C, rsum, csc, m0, n0, wm, wn, lane, slice);
}

// The 64 x 256 tile in two roles, 512 threads: waves 0-3 own the weight path and the
// matrix cores (each wave a 64 x 64 tile, its packed weights through a ring of P VGPR
// stages, unpacked in registers, activation fragments from LDS), waves 4-7 own the
// activation path (a ring of PA VGPR stages, the byte transpose, the row sums of the codes,
// the double-buffered LDS tile), so the matrix-core waves neither wait for activation
// loads nor spend instructions on staging. The loader waves run at a raised wave priority:
// the next step's tile is on the critical path. One barrier per K step orders the LDS tile:
// at step it the matrix-core waves read buffer it & 1 while the loaders fill the other.
// Products, row sums and epilogue are those of gemm_mfma_kernel<64, 256, 1, 4, 2, 128>,
// so outputs are bit-identical.
template <int P, int PA>
__global__ __launch_bounds__(512) void gemm_roles_kernel(GemmArgs a)
{
    constexpr int BM = 64, BN = 256, WN = 4, BK = 128;
    constexpr int TM = BM, TN = BN / WN;        // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA tiles per wave
    constexpr int KS = BK / 32;                 // MFMA k-substeps per step
    constexpr int AST = BK + 16;                // LDS row stride in bytes (padded)
    constexpr int UPR = BK / 16;                // 16-byte activation units per row
    constexpr int AU = BM * UPR / 256;          // units per loader thread per step
    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * AST];
    __shared__ int32_t rsum[BM];
    __shared__ float csc[BM];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform role
    const int lane = tid & 63;
    const int M = a.M, N = a.N, K = a.K;
    const int KB = K >> 2;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    region_tile(xcd_tile((int)blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, a.gm, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    if (tid < BM) {
        const int m = m0 + tid;
        csc[tid] = m < M ? *a.gamma / a.xscale[m] : 0.0f;
    }
    const int nk = (K + BK - 1) / BK;

    if (wave < 4) {
        const int wn = wave;
        const int brows = (N - n0) < BN ? (N - n0) : BN;
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (int64_t)n0 * KB), (short)0, brows * KB, kBufferFlags);
        // weight fragment fn of this lane: row wn*TN + 32 fn + lane % 32, 16 bytes at
        // 16 (lane / 32) of the step's 32 bytes
        int boff[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            boff[fn] = (wn * TN + fn * 32 + (lane & 31)) * KB + 16 * (lane >> 5);
        u32x4 breg[P][FN];
        auto load = [&](u32x4 (&bd)[FN], int k0) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bd[fn] = buf_load16(rb, boff[fn], k0 >> 2);
        };
#pragma unroll
        for (int s = 0; s < P; ++s)
            if (s < nk)
                load(breg[s], s * BK);
        v16i C[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    C[fm][fn][r] = 0;
        __syncthreads();   // step 0's activations are in LDS
        auto step = [&](int it, int s, bool reload) {
            __builtin_amdgcn_sched_barrier(0);
            v4i bf[KS][FN];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const uint32_t w = breg[s][fn][ks];
                    bf[ks][fn][0] = (int)(w & 0x03030303u);
                    bf[ks][fn][1] = (int)((w >> 2) & 0x03030303u);
                    bf[ks][fn][2] = (int)((w >> 4) & 0x03030303u);
                    bf[ks][fn][3] = (int)((w >> 6) & 0x03030303u);
                }
            if (reload)
                load(breg[s], (it + P) * BK);
            const uint8_t* Ab = As[it & 1];
            v4i af[KS][FM];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int r = fm * 32 + (lane & 31);
                    af[ks][fm] = *reinterpret_cast<const v4i*>(Ab + r * AST + 64 * (lane >> 5) + 16 * ks);
                }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
                        C[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks][fm], bf[ks][fn], C[fm][fn], 0, 0, 0);
            __syncthreads();
        };
        // steady state: every step refills its ring slot (no condition, so the slots stay in
        // fixed registers); then the last (fewer than 2P) steps
        int it = 0;
        for (; it + 2 * P <= nk; it += P) {
#pragma unroll
            for (int s = 0; s < P; ++s)
                step(it + s, s, true);
        }
#pragma unroll
        for (int s = 0; s < 2 * P - 1; ++s) {
            const int t = it + s;
            if (t < nk)
                step(t, s % P, t + P < nk);
        }
        __syncthreads();   // the row sums are in LDS
        gemm_epilogue<BM, BN, TM, TN, FM, FN>(a, C, rsum, csc, m0, n0, 0, wn, lane, 0);
    } else {
        __builtin_amdgcn_s_setprio(2);
        const int lt = tid - 256;               // loader thread 0..255
        const int arows = (M - m0) < BM ? (M - m0) : BM;
        const __amdgpu_buffer_rsrc_t ra =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.Xq + (int64_t)m0 * K), (short)0, arows * K, kBufferFlags);
        // activation unit i of this thread: row (lt + 256 i) / UPR, 16-byte column lt % UPR
        int aoff[AU];
#pragma unroll
        for (int i = 0; i < AU; ++i)
            aoff[i] = ((lt + 256 * i) / UPR) * K + 16 * (lt % UPR);
        const int acol = 16 * (lt % UPR);
        u32x4 areg[PA][AU];
        int32_t rs[AU];
#pragma unroll
        for (int i = 0; i < AU; ++i)
            rs[i] = 0;
        auto load = [&](u32x4 (&ad)[AU], int k0) {
#pragma unroll
            for (int i = 0; i < AU; ++i)
                ad[i] = buf_load16(ra, aoff[i], k0);
        };
        // The last step may extend past K (K % BK is a multiple of 64): activations loaded
        // from beyond the row end belong to the next row and are replaced by zeros, which
        // also zeroes those columns' products whatever the weight bytes there hold.
        auto stage = [&](const u32x4 (&src)[AU], int buf, int kvalid) {
#pragma unroll
            for (int i = 0; i < AU; ++i) {
                const int u = lt + 256 * i;
                const int r = u / UPR, c = u % UPR;
                u32x4 v = src[i];
                if (acol >= kvalid)
                    v = u32x4{0u, 0u, 0u, 0u};
                uint32_t o[4];
                transpose_bytes(v[0], v[1], v[2], v[3], o);
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    rs[i] = __builtin_amdgcn_sdot4((int)o[f], 0x01010101, rs[i], false);
                *reinterpret_cast<uint4*>(&As[buf][r * AST + 16 * c]) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        };
#pragma unroll
        for (int s = 0; s < PA; ++s)
            if (s < nk)
                load(areg[s], s * BK);
        stage(areg[0], 0, K);
        if (PA < nk)
            load(areg[0], PA * BK);
        __syncthreads();   // step 0 staged
        // at step it, ring slot (it + 1) % PA holds step it + 1: stage it into the other LDS
        // buffer, then refill the slot with step it + 1 + PA
        auto lstep = [&](int it, int s, bool stage_next, bool reload) {
            __builtin_amdgcn_sched_barrier(0);
            if (stage_next)
                stage(areg[s], (it + 1) & 1, K - (it + 1) * BK);
            if (reload)
                load(areg[s], (it + 1 + PA) * BK);
            __syncthreads();
        };
        int it = 0;
        for (; it + 2 * PA <= nk; it += PA) {
#pragma unroll
            for (int s = 0; s < PA; ++s)
                lstep(it + s, (s + 1) % PA, true, true);
        }
#pragma unroll
        for (int s = 0; s < 2 * PA - 1; ++s) {
            const int t = it + s;
            if (t < nk)
                lstep(t, (s + 1) % PA, t + 1 < nk, t + 1 + PA < nk);
        }
        // row sums of the codes: thread lt holds rows (lt + 256 i) / UPR for the column
        // group lt % UPR; the UPR groups of a row are adjacent lanes
#pragma unroll
        for (int i = 0; i < AU; ++i) {
            int v = rs[i];
#pragma unroll
            for (int m = 1; m < UPR; m <<= 1)
                v += __shfl_xor(v, m);
            if ((lt % UPR) == 0)
                rsum[(lt + 256 * i) / UPR] = v;
        }
        __syncthreads();
    }
}

// Sum of the K slices' int32 partials and the product's epilogue, as the unsplit kernel
// writes it: y = fl32(fl32(acc) * fl32(gamma / s_m)), added into Y with residual.
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(GemmArgs a)
{
    const int64_t total = (int64_t)a.M * a.N;
    const int64_t slice = total;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        int32_t v = 0;
        for (int s = 0; s < a.ksplit; ++s)
            v += a.part[s * slice + o];
        const int m = (int)(o / a.N);
        const float c = *a.gamma / a.xscale[m];
        const float yv = (float)v * c;
        a.Y[o] = a.residual ? a.Y[o] + yv : yv;
        if (a.acc)
            a.acc[o] = v;
    }
}

}  // namespace bl

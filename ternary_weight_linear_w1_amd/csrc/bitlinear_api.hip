// bitlinear_api.hip -- C ABI of the W1.58A8 BitLinear library (declared in
// include/bitlinear.h): argument checks, kernel choice and launches on the caller's
// stream. Nothing here allocates memory or keeps state besides a per-device cache of
// the compute-unit count.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "../../include/bitlinear.h"
#include "attention.hpp"
#include "device_common.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "gemv5.hpp"
#include "gemv_mfma.hpp"
#include "pack.hpp"
#include "quant.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

bool aligned(const void* p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes)
{
    if (!a || !b)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int check_mk(int64_t M, int64_t K)
{
    if (M < 1 || K < 4 || K > BITLINEAR_MAX_K || (K % 4) != 0)
        return BITLINEAR_ERR_SHAPE;
    if (M > kMaxElems / K)
        return BITLINEAR_ERR_SHAPE;
    return BITLINEAR_OK;
}

int check_nk(int64_t N, int64_t K)
{
    if (N < 1 || N > INT32_MAX || K < 4 || K > BITLINEAR_MAX_K || (K % 4) != 0)
        return BITLINEAR_ERR_SHAPE;
    if (N > kMaxElems / K)
        return BITLINEAR_ERR_SHAPE;
    return BITLINEAR_OK;
}

int launched()
{
    return hipGetLastError() == hipSuccess ? BITLINEAR_OK : BITLINEAR_ERR_HIP;
}

// Level sizes of the |W| reduction tree (4096 -> 1 per block, repeated).
int64_t sum_levels(int64_t n, int64_t* sizes, int max_levels, int* nlev)
{
    int64_t total = 0;
    int l = 0;
    int64_t cur = n;
    do {
        cur = (cur + bl::kSumChunk - 1) / bl::kSumChunk;
        if (l < max_levels)
            sizes[l] = cur;
        total += cur;
        ++l;
    } while (cur > 1);
    *nlev = l;
    return total;
}

// ---------------------------------------------------------------------- forward dispatch

// Launch shapes were chosen by timing back-to-back launches on MI355X for the BitNet
// 2B (K = 2560, 6912) and 100B (K = 8192, 28672) layer shapes.
template <int L, int MT, int CPL, int R, bool FUSED, int S = 2>
void launch_k64(const bl::FwdArgs& a, int wg_per_cu, hipStream_t stream)
{
    constexpr int RPP = (256 / L) * R;
    const int64_t passes = (a.N + RPP - 1) / RPP;
    const int64_t tiles = (a.M + MT - 1) / MT;
    const int gy = (int)(tiles < 65535 ? tiles : 65535);
    // fused multi-token tiles take one block per CU (their prologue holds more than 256
    // registers), so the token tiles share the CUs instead of queueing for a second round
    const int64_t max_x = FUSED && MT > 1 ? std::max<int64_t>(1, (int64_t(cu_count()) * wg_per_cu + gy - 1) / gy)
                                          : int64_t(cu_count()) * wg_per_cu;
    const int gx = (int)(passes < max_x ? passes : max_x);
    // pre-quantized codes with L >= 64 go straight to registers (no LDS staging)
    const size_t lds = (!FUSED && L >= 64) ? 0 : FUSED ? bl::fused_lds_bytes<L, MT, CPL>(a.K) : (size_t)MT * a.K;
    if (a.residual) {
        // (the row loop strides by the grid, so any grid width is correct)
        if constexpr (MT * R <= 4)
            hipLaunchKernelGGL((bl::gemv_k64_kernel<L, MT, CPL, R, FUSED, true, S>), dim3(gx, gy), dim3(256), lds, stream,
                               a);
        else
            hipLaunchKernelGGL((bl::gemv_k64_kernel<L, MT, CPL, 1, FUSED, true, S>), dim3(gx, gy), dim3(256), lds, stream,
                               a);
    } else
        hipLaunchKernelGGL((bl::gemv_k64_kernel<L, MT, CPL, R, FUSED, false, S>), dim3(gx, gy), dim3(256), lds, stream, a);
}

// One token with a fused input: the two-role kernel, 512-thread blocks, two weight
// buffers per wave (measured on MI355X on the 100B down projection, L = 64 with 7 chunks
// per lane: 14.8-15.2 us against 19.1-19.6 us for the 256-thread kernel with three passes
// in flight; three buffers, a 5:3 or 7:1 split of the passes, or requesting weights before
// the prologue's statistics were all slower).
template <int L, int CPL>
void launch_split(const bl::FwdArgs& a, hipStream_t stream, int wg_per_cu = 1)
{
    constexpr int S = 2;
    const int64_t passes = (a.N + 256 / L - 1) / (256 / L);
    const int64_t max_x = int64_t(cu_count()) * wg_per_cu;
    const int gx = (int)(passes < max_x ? passes : max_x);
    const size_t lds = (size_t)a.K;
    const bool norm = a.gain != nullptr;
#define BL_SPLIT(R, A, NM) \
    hipLaunchKernelGGL((bl::gemv_split_kernel<L, CPL, S, R, A, NM>), dim3((unsigned)gx), dim3(512), lds, stream, a)
#define BL_SPLIT_MODE(R)                                                   \
    do {                                                                   \
        if (a.act == 0) { if (norm) BL_SPLIT(R, 0, true); else BL_SPLIT(R, 0, false); } \
        else if (a.act == 1) { if (norm) BL_SPLIT(R, 1, true); else BL_SPLIT(R, 1, false); } \
        else { if (norm) BL_SPLIT(R, 2, true); else BL_SPLIT(R, 2, false); } \
    } while (0)
    if (a.residual)
        BL_SPLIT_MODE(true);
    else
        BL_SPLIT_MODE(false);
#undef BL_SPLIT_MODE
#undef BL_SPLIT
}

// One token per tile: up to 4 chunks (256 codes) per lane (7 for the longest rows).
// Launch shapes (lanes per row L, chunks per lane, rows per lane, passes in flight S,
// blocks per CU) from graph-timed sweeps on MI355X over the BitNet 2B and 100B shapes;
// a third pass in flight pays where a block holds few rows per pass or has a long fused
// prologue to hide (100B down: 20.3 -> 18.8 us fused; 100B O product: 5.8 -> 5.3 us).
template <bool FUSED>
bool dispatch_mt1(const bl::FwdArgs& a, hipStream_t stream)
{
    const int KC = a.K / 64;
    const int64_t nk = a.N * (int64_t)a.K;
    const bool big = nk >= (int64_t(64) << 20);   // >= 16 MB of packed weights
    if (KC <= 48) {
        // 2B-sized rows: 16 lanes x 3 chunks, two rows per lane for the longer matrices
        if (a.N <= 4096) {
            if constexpr (FUSED)
                launch_k64<16, 1, 3, 1, FUSED>(a, 1, stream);
            else
                launch_k64<16, 1, 3, 1, FUSED>(a, 2, stream);
        } else {
            launch_k64<16, 1, 3, 2, FUSED>(a, 1, stream);
        }
        return true;
    }
    if (KC <= 64) { launch_k64<16, 1, 4, 1, FUSED>(a, 2, stream); return true; }
    if (KC <= 128) {
        if (!big) {   // 2B down projection (K = 6912): a wave per row
            if constexpr (FUSED)
                launch_k64<64, 1, 2, 1, FUSED, 3>(a, 1, stream);
            else
                launch_k64<64, 1, 2, 1, FUSED>(a, 2, stream);
        } else if (nk < (int64_t(72) << 20)) {   // 100B O (K = N = 8192)
            if constexpr (FUSED)
                launch_k64<32, 1, 4, 1, FUSED, 3>(a, 1, stream);
            else
                launch_k64<64, 1, 2, 1, FUSED, 3>(a, 3, stream);
        } else if constexpr (FUSED) {   // two blocks per CU from ~20 MB of packed weights (100B QKV, up)
            // one token on >= 32 MB of packed weights (100B up): the two-role kernel, two
            // blocks per CU (12.65 -> 11.9 us; on the 100B QKV and O it lost 0.1-0.4 us)
            if (a.M == 1 && nk >= (int64_t(128) << 20))
                launch_split<32, 4>(a, stream, 2);
            else
                launch_k64<32, 1, 4, 1, FUSED>(a, 2, stream);
        } else {   // one row per lane and more blocks keep the HBM queue fuller on long matrices
            launch_k64<32, 1, 4, 1, FUSED>(a, nk >= (int64_t(128) << 20) ? 3 : 2, stream);
        }
        return true;
    }
    if (KC <= 256) {  // the fused prologue keeps the whole row in registers: one block per CU
        launch_k64<64, 1, 4, 1, FUSED>(a, FUSED ? 1 : 2, stream);
        return true;
    }
    if (KC <= 512) {
        if (KC <= 448) {   // one wave per row (no cross-wave sum), 7 chunks per lane: 100B down
            if constexpr (FUSED) {
                if (a.M == 1)
                    launch_split<64, 7>(a, stream);   // 100B down fused: 19.1 -> 15.0 us
                else
                    launch_k64<64, 1, 7, 1, FUSED, 3>(a, 1, stream);
            } else {
                launch_k64<64, 1, 7, 1, FUSED>(a, 1, stream);
            }
        } else if constexpr (FUSED) {
            launch_k64<128, 1, 4, 1, FUSED>(a, 1, stream);
        } else {
            launch_k64<256, 1, 2, 2, FUSED>(a, 3, stream);  // codes straight to registers
        }
        return true;
    }
    if (KC <= 1024) { launch_k64<256, 1, 4, 1, FUSED>(a, FUSED ? 1 : 2, stream); return true; }
    return false;
}

// Two tokens per tile: up to 2 chunks per lane.
template <bool FUSED>
bool dispatch_mt2(const bl::FwdArgs& a, hipStream_t stream)
{
    const int KC = a.K / 64;
    if (KC <= 32) { launch_k64<16, 2, 2, 1, FUSED>(a, 2, stream); return true; }
    if (KC <= 64) { launch_k64<32, 2, 2, 1, FUSED>(a, 2, stream); return true; }
    if (KC <= 128) { launch_k64<64, 2, 2, 1, FUSED>(a, 2, stream); return true; }
    if (KC <= 256) { launch_k64<128, 2, 2, 1, FUSED>(a, 2, stream); return true; }
    if (KC <= 512) { launch_k64<256, 2, 2, 1, FUSED>(a, 2, stream); return true; }
    return false;
}

// Four tokens per tile: one chunk per lane. Blocks per CU from graph-timed sweeps of the 2B
// shapes at 3, 4, 8 and 16 tokens: two with a single pre-quantized tile, one once there are
// several tiles (they already give the grid two or more blocks per CU) or a fused prologue.
template <bool FUSED>
bool dispatch_mt4(const bl::FwdArgs& a, hipStream_t stream)
{
    const int KC = a.K / 64;
    const bool big = a.N * (int64_t)a.K >= (int64_t(64) << 20);
    const int wg = FUSED || a.M > 4 ? 1 : 2;
    if (KC <= 64) { launch_k64<64, 4, 1, 1, FUSED>(a, wg, stream); return true; }
    if (KC <= 128) {
        // four rows per lane need the registers the residual loads take
        if (big && !a.residual) launch_k64<128, 4, 1, 4, FUSED>(a, wg, stream);
        else launch_k64<128, 4, 1, 1, FUSED>(a, wg, stream);
        return true;
    }
    if (KC <= 256) { launch_k64<256, 4, 1, 1, FUSED>(a, wg, stream); return true; }
    return false;
}

template <bool FUSED>
void launch_generic(const bl::FwdArgs& a, hipStream_t stream)
{
    const int64_t passes = (a.N + 3) / 4;
    const int64_t tiles = (a.M + 3) / 4;
    const int64_t max_x = int64_t(cu_count()) * 4;
    const int gx = (int)(passes < max_x ? passes : max_x);
    const int gy = (int)(tiles < 65535 ? tiles : 65535);
    hipLaunchKernelGGL((bl::gemv_generic_kernel<FUSED>), dim3(gx, gy), dim3(256), 0, stream, a);
}

// Many tokens: int8 MFMA GEMM. Needs K % 64 == 0 and 16-byte aligned operands.
template <int BM, int BN, int WM, int WN, int P, int BK, int WK = 1>
void launch_gemm(const bl::FwdArgs& f, hipStream_t stream)
{
    const int64_t tiles_m = (f.M + BM - 1) / BM, tiles_n = (f.N + BN - 1) / BN;
    bl::GemmArgs a{f.Xq, f.xscale, f.W, f.gamma, f.Y, f.acc, (int)f.M, (int)f.N, f.K, f.residual,
                   bl::gemm_region_split(tiles_m, tiles_n, BM, BN, f.K), nullptr, 1, f.K};
    const int64_t tiles = tiles_m * tiles_n;
    hipLaunchKernelGGL((bl::gemm_mfma_kernel<BM, BN, WM, WN, P, BK, WK>), dim3((unsigned)tiles), dim3(256), 0,
                       stream, a);
}

// The 64 x 256 tile with the activation path in separate loader waves (512 threads).
void launch_gemm_roles(const bl::FwdArgs& f, hipStream_t stream)
{
    const int64_t tiles_m = (f.M + 63) / 64, tiles_n = (f.N + 255) / 256;
    bl::GemmArgs a{f.Xq, f.xscale, f.W, f.gamma, f.Y, f.acc, (int)f.M, (int)f.N, f.K, f.residual,
                   bl::gemm_region_split(tiles_m, tiles_n, 64, 256, f.K), nullptr, 1, f.K};
    hipLaunchKernelGGL((bl::gemm_roles_kernel<2, 2>), dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream, a);
}

int64_t round256(int64_t b)
{
    return (b + 255) / 256 * 256;
}

// Split K for few tokens (the product with a caller workspace): 32 x 128 tiles, K steps of
// 256, up to 8 slices of at least 4 steps each, aiming at about 1024 blocks (four resident
// per CU on 256 CUs). A pure function of the sizes, so the workspace size needs no device.
constexpr int kSplitStep = 256;

// K slices of the split product (1: no split). Measured on MI355X against the unsplit
// kernel at 16..128 tokens over the 2B and 100B shapes, and against the few-token
// matrix-core kernel (which walks such rows in several LDS phases) at 6..15 tokens:
// splitting pays only where few token tiles meet a long K loop (K >= 16384): from 10
// tokens, or 8 on matrices of >= 64M weights, up to 32 (100B down projection: 35.9 ->
// 26.5 us at 32 tokens, 30.8 -> 22.7 at 12). At 64 tokens and beyond, or with shorter
// rows, the int32 partials (written and read once more) and the second launch cost more
// than the shorter loop gains. Up to 8 slices of at least 4 K steps, aiming at about 1024
// blocks; the partials are then at most a quarter of the packed weight bytes
// (16 M s <= K / 4).
int splitk_slices(int64_t M, int64_t N, int64_t K)
{
    if (M < 8 || M > 32 || (K % 64) != 0 || K < 16384)
        return 1;
    if (M < 10 && N * K < (int64_t(64) << 20))
        return 1;
    const int64_t tiles = ((M + 31) / 32) * ((N + 127) / 128);
    const int64_t nk = (K + kSplitStep - 1) / kSplitStep;
    int64_t s = 1024 / tiles;
    if (s > nk / 4)
        s = nk / 4;
    if (s > 8)
        s = 8;
    return s < 2 ? 1 : (int)s;
}

void launch_gemm_split(const bl::FwdArgs& f, int32_t* part, int slices, hipStream_t stream)
{
    const int64_t tiles_m = (f.M + 31) / 32, tiles_n = (f.N + 127) / 128;
    const int64_t nk = (f.K + kSplitStep - 1) / kSplitStep;
    const int kslice = (int)((nk + slices - 1) / slices) * kSplitStep;
    const int used = (int)((f.K + kslice - 1) / kslice);   // slices that hold columns
    bl::GemmArgs a{f.Xq, f.xscale, f.W, f.gamma, f.Y, f.acc, (int)f.M, (int)f.N, f.K, f.residual, 1,
                   part, used, kslice};
    hipLaunchKernelGGL((bl::gemm_mfma_kernel<32, 128, 1, 4, 2, kSplitStep>), dim3((unsigned)(tiles_m * tiles_n * used)),
                       dim3(256), 0, stream, a);
    const int64_t total = f.M * f.N;
    const int64_t blocks = (total + 255) / 256, cap = int64_t(cu_count()) * 8;
    hipLaunchKernelGGL(bl::gemm_splitk_reduce_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256), 0,
                       stream, a);
}

// Resident blocks per CU of a kernel on the current device (queried once per device).
template <typename Kern>
int resident_blocks(Kern kernel, std::atomic<int> (&cache)[kMaxDevices], int threads = 256)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 1;
    int occ = cache[dev].load(std::memory_order_relaxed);
    if (occ <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess || occ <= 0)
            occ = 1;
        cache[dev].store(occ, std::memory_order_relaxed);
    }
    return occ;
}

std::atomic<int> g_occ_gemm_big[kMaxDevices];
std::atomic<int> g_occ_gemm_small[kMaxDevices];

bool dispatch_gemm(const bl::FwdArgs& a, hipStream_t stream)
{
    if (a.M < 16 || a.M > INT32_MAX || (a.K % 64) != 0)
        return false;
    if (((a.M + 31) / 32) * ((a.N + 127) / 128) >= INT32_MAX)
        return false;
    // Tile shapes from timing the 2B prefill (M = 512, 2048) and 100B (M = 64) shapes on
    // MI355X: the 64 x 256 tile (K steps of 128) is faster per tile, and wins whenever it
    // fills at least 40% of its rounds of resident blocks (all four 2B shapes at M = 2048,
    // the up projection at M = 512); below that, 32 x 128 tiles (K steps of 256), split
    // along K inside the block when even those are few. The 64 x 256 tile runs in two roles
    // (loader waves for the activations): 132.5 against 140.7 us over the four 2B shapes at
    // M = 2048, bit-identical outputs.
    if (a.M >= 512) {
        const int64_t tiles = ((a.M + 63) / 64) * ((a.N + 255) / 256);
        const int64_t slots = int64_t(cu_count()) *
                              resident_blocks(bl::gemm_roles_kernel<2, 2>, g_occ_gemm_big, 512);
        const int64_t rounds = (tiles + slots - 1) / slots;
        if (5 * tiles >= 2 * rounds * slots) {
            launch_gemm_roles(a, stream);
            return true;
        }
    }
    // Few tokens and few output tiles (long rows at M = 64): 32 x 64 tiles whose four waves
    // split N in two and K in two, so twice as many blocks cover the GPU.
    const int64_t tiles = ((a.M + 31) / 32) * ((a.N + 127) / 128);
    const int64_t slots = int64_t(cu_count()) *
                          resident_blocks(bl::gemm_mfma_kernel<32, 128, 1, 4, 2, 256>, g_occ_gemm_small);
    if (4 * tiles <= slots)
        launch_gemm<32, 64, 1, 2, 2, 256, 2>(a, stream);
    else
        launch_gemm<32, 128, 1, 4, 2, 256>(a, stream);
    return true;
}

// Few tokens on the matrix cores (gemv_mfma_kernel, 16 waves sharing the activation codes
// in LDS, units of 16 rows x 512 codes). Timed against the vector product and the tiled
// matrix-core product on MI355X over the 2B and 100B shapes at 2..64 tokens: it wins from
// 3 to 15 tokens on every shape (e.g. 100B up, 8 tokens: 17.4 against 49.9 us), at 2 tokens
// only for the largest matrices (>= 128M weights), and at 16..24 tokens (two tiles of 16
// per weight operand from 17) only below 64M weights. From 24 tokens on the larger matrices,
// and from 32 on any, every CU staging all activation rows costs more than the tiled
// product's re-reads (100B QKV at 64 tokens: 42.7 against 22.2 us).
constexpr int kMfmaWaves = 16;
constexpr int kMfmaUnit = 2;                   // windows of 256 codes per unit
constexpr int kMfmaMaxPhases = 4;              // K slices staged one after another
constexpr int64_t kMfmaMaxTokens = 24;
constexpr int64_t kMaxLds = 160 * 1024;

int mfma_tiles(int64_t M)
{
    return M <= 16 ? 1 : 2;
}

// Windows of 256 codes per phase of gemv_mfma_kernel (a multiple of the unit; 0: the
// codes of one unit per window do not fit, or more than kMfmaMaxPhases phases).
int64_t mfma_phase_windows(int64_t M, int64_t K, int64_t rg_per_block)
{
    const int tt = mfma_tiles(M);
    const int64_t nw = (K + 255) / 256;
    int64_t maxw = (kMaxLds - (int64_t)bl::gemv_mfma_lds_bytes(M, tt, 0, rg_per_block)) /
                   (256 * bl::gemv_mfma_slots(M, tt));
    maxw -= maxw % kMfmaUnit;
    if (maxw < kMfmaUnit)
        return 0;
    const int64_t nph = (nw + maxw - 1) / maxw;
    if (nph > kMfmaMaxPhases)
        return 0;
    const int64_t w = (nw + nph - 1) / nph;
    return (w + kMfmaUnit - 1) / kMfmaUnit * kMfmaUnit;
}

bool mfma_small_shape(int64_t M, int64_t N, int64_t K, int64_t cus)
{
    if (M < 2 || M > kMfmaMaxTokens || (K % 64) != 0 || N >= (int64_t(1) << 27))
        return false;
    const int64_t nk = N * K;
    if ((M == 2 && nk < (int64_t(128) << 20)) || (M >= 16 && nk >= (int64_t(64) << 20)))
        return false;
    if ((N + 16) * (K / 4) >= bl::kOob || M * K >= INT32_MAX)
        return false;
    const int64_t ng = (N + 15) / 16, grid = ng < cus ? ng : cus;
    return mfma_phase_windows(M, K, (ng + grid - 1) / grid) > 0;
}

template <int TT>
void launch_mfma(const bl::FwdArgs& a, int64_t grid, int64_t rg, int64_t nwp, hipStream_t stream)
{
    hipLaunchKernelGGL((bl::gemv_mfma_kernel<kMfmaUnit, kMfmaWaves, TT>), dim3((unsigned)grid), dim3(kMfmaWaves * 64),
                       bl::gemv_mfma_lds_bytes(a.M, TT, nwp, rg), stream, a, (int)nwp);
}

bool dispatch_mfma(const bl::FwdArgs& a, hipStream_t stream)
{
    const int64_t cus = cu_count();
    if (!mfma_small_shape(a.M, a.N, a.K, cus))
        return false;
    const int64_t ng = (a.N + 15) / 16, grid = ng < cus ? ng : cus, rg = (ng + grid - 1) / grid;
    const int64_t nwp = mfma_phase_windows(a.M, a.K, rg);
    if (mfma_tiles(a.M) == 1)
        launch_mfma<1>(a, grid, rg, nwp, stream);
    else
        launch_mfma<2>(a, grid, rg, nwp, stream);
    return true;
}

template <bool FUSED>
void dispatch_forward(const bl::FwdArgs& a, bool chunk_ok, hipStream_t stream)
{
    // 32-bit buffer offsets: a token tile of outputs (4 rows of N floats) must stay
    // below 2 GiB, and at or below the out-of-range offset that masked lanes use
    // (4 * 4 * (2^27 - 1) bytes == kOob), so that their stores are dropped.
    chunk_ok = chunk_ok && a.N < (int64_t(1) << 27);
    if (chunk_ok) {
        if (a.M == 1 && dispatch_mt1<FUSED>(a, stream))
            return;
        if (a.M == 2 && dispatch_mt2<FUSED>(a, stream))
            return;
        if (a.M >= 3 && dispatch_mt4<FUSED>(a, stream))
            return;
        if (a.M >= 2 && dispatch_mt2<FUSED>(a, stream))
            return;
        if (dispatch_mt1<FUSED>(a, stream))
            return;
    }
    launch_generic<FUSED>(a, stream);
}

int check_fwd_args(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed,
                   const float* gamma, int64_t N, const float* Y, const int32_t* acc)
{
    if (!Xq || !x_scale || !W_packed || !gamma || !Y)
        return BITLINEAR_ERR_NULL;
    int st = check_mk(M, K);
    if (st != BITLINEAR_OK)
        return st;
    if ((st = check_nk(N, K)) != BITLINEAR_OK)
        return st;
    if (M > kMaxElems / N)
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(Xq, 4) || !aligned(x_scale, 4) || !aligned(W_packed, 1) || !aligned(gamma, 4) ||
        !aligned(Y, 4) || (acc && !aligned(acc, 4)))
        return BITLINEAR_ERR_ALIGN;
    const int64_t ybytes = M * N * 4;
    const void* ins[4] = {Xq, x_scale, W_packed, gamma};
    const int64_t insz[4] = {M * K, M * 4, N * (K / 4), 4};
    for (int i = 0; i < 4; ++i)
        if (overlap(Y, ybytes, ins[i], insz[i]) || overlap(acc, ybytes, ins[i], insz[i]))
            return BITLINEAR_ERR_ALIAS;
    if (overlap(Y, ybytes, acc, ybytes))
        return BITLINEAR_ERR_ALIAS;
    return BITLINEAR_OK;
}

// The product; with `part` (a workspace of splitk_slices(M, N, K) * M * N int32) few tokens
// take the split-K matrix-core path.
int forward_impl(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed,
                 const float* gamma, int64_t N, float* Y, int32_t* acc, int residual, hipStream_t stream,
                 int32_t* part = nullptr)
{
    const int st = check_fwd_args(Xq, x_scale, M, K, W_packed, gamma, N, Y, acc);
    if (st != BITLINEAR_OK)
        return st;
    bl::FwdArgs a{};
    a.Xq = Xq;
    a.xscale = x_scale;
    a.W = W_packed;
    a.gamma = gamma;
    a.Y = Y;
    a.acc = acc;
    a.M = M;
    a.N = N;
    a.K = (int)K;
    a.residual = residual;
    const bool chunk_ok = (K % 64) == 0 && aligned(W_packed, 16) && aligned(Xq, 16);
    const int slices = splitk_slices(M, N, K);
    if (part && chunk_ok && slices > 1 && ((M + 31) / 32) * ((N + 127) / 128) * slices < INT32_MAX)
        launch_gemm_split(a, part, slices, stream);
    else if (!(chunk_ok && (dispatch_mfma(a, stream) || dispatch_gemm(a, stream))))
        dispatch_forward<false>(a, chunk_ok, stream);
    return launched();
}

// Bytes of the split-K partials of the product with a workspace (0: no split).
int64_t split_bytes(int64_t M, int64_t N, int64_t K)
{
    const int s = splitk_slices(M, N, K);
    return s > 1 ? round256((int64_t)s * M * N * 4) : 0;
}

int check_f32_args(const float* X, int64_t M, int64_t K, const float* gain, int act, const uint8_t* W_packed,
                   const float* gamma, int64_t N, const float* Y)
{
    if (!X || !W_packed || !gamma || !Y)
        return BITLINEAR_ERR_NULL;
    int st = check_mk(M, K);
    if (st != BITLINEAR_OK)
        return st;
    if ((st = check_nk(N, K)) != BITLINEAR_OK)
        return st;
    if (M > kMaxElems / N || act < 0 || act > 2 || (act == 2 && M > kMaxElems / (2 * K)))
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(X, 16) || (gain && !aligned(gain, 16)) || !aligned(gamma, 4) || !aligned(Y, 4))
        return BITLINEAR_ERR_ALIGN;
    const int64_t ybytes = M * N * 4;
    const void* ins[4] = {X, gain, W_packed, gamma};
    const int64_t insz[4] = {M * K * 4 * (act == 2 ? 2 : 1), K * 4, N * (K / 4), 4};
    for (int i = 0; i < 4; ++i)
        if (overlap(Y, ybytes, ins[i], insz[i]))
            return BITLINEAR_ERR_ALIAS;
    return BITLINEAR_OK;
}

// Token counts from which the product runs on the tiled matrix-core kernel.
constexpr int64_t kGemmMinTokens = 16;

// Whether the fused call with a workspace quantizes first and then multiplies: wherever the
// product takes the matrix cores (from 16 tokens, and the few-token shapes above; the
// size check assumes 256 CUs, the launch rechecks with the device's count).
bool f32_two_step(int64_t M, int64_t N, int64_t K)
{
    return M >= kGemmMinTokens || mfma_small_shape(M, N, K, 256);
}


int forward_f32_impl(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                     const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, int residual,
                     hipStream_t stream)
{
    const int st = check_f32_args(X, M, K, gain, act, W_packed, gamma, N, Y);
    if (st != BITLINEAR_OK)
        return st;
    bl::FwdArgs a{};
    a.X = X;
    a.gain = gain;
    a.eps = eps;
    a.act = act;
    a.W = W_packed;
    a.gamma = gamma;
    a.Y = Y;
    a.M = M;
    a.N = N;
    a.K = (int)K;
    a.residual = residual;
    const bool chunk_ok = (K % 64) == 0 && aligned(W_packed, 16);
    dispatch_forward<true>(a, chunk_ok, stream);
    return launched();
}


// ---------------------------------------------------------------------- five codes per byte

int64_t row_bytes5(int64_t K)
{
    return 16 * ((K + 79) / 80);
}

template <int L, int MT, int CPL>
void launch5(const bl::Fwd5Args& a, hipStream_t stream)
{
    constexpr int RG = 256 / L;
    const int64_t passes = (a.N + RG - 1) / RG;
    const int64_t tiles = (a.M + MT - 1) / MT;
    const int64_t max_x = int64_t(cu_count()) * 2;
    const int gx = (int)(passes < max_x ? passes : max_x);
    const int gy = (int)(tiles < 65535 ? tiles : 65535);
    const size_t lds = (size_t)MT * (size_t)(a.RB >> 4) * 80;
    hipLaunchKernelGGL((bl::gemv5_kernel<L, MT, CPL>), dim3(gx, gy), dim3(256), lds, stream, a);
}

// Lanes per row: the fewest (16 .. 256) whose chunks cover a row; tiles of 1, 2 or 4
// tokens as long as the staged codes fit in LDS.
template <int MT, int CPL>
bool dispatch5_mt(const bl::Fwd5Args& a, hipStream_t stream)
{
    const int KC = a.RB >> 4;
    if (KC <= 16 * CPL) { launch5<16, MT, CPL>(a, stream); return true; }
    if (KC <= 32 * CPL) { launch5<32, MT, CPL>(a, stream); return true; }
    if (KC <= 64 * CPL) { launch5<64, MT, CPL>(a, stream); return true; }
    if (KC <= 128 * CPL) { launch5<128, MT, CPL>(a, stream); return true; }
    if (KC <= 256 * CPL) { launch5<256, MT, CPL>(a, stream); return true; }
    return false;
}

void dispatch5(const bl::Fwd5Args& a, hipStream_t stream)
{
    const int64_t staged = (int64_t)(a.RB >> 4) * 80;    // LDS bytes per token
    constexpr int64_t kLdsBudget = 144 * 1024;
    // fewer chunks per lane for multi-token tiles: the rearranged activations of every
    // token stay in registers
    if (a.M >= 3 && 4 * staged <= kLdsBudget && dispatch5_mt<4, 1>(a, stream))
        return;
    if (a.M >= 2 && 2 * staged <= kLdsBudget && dispatch5_mt<2, 2>(a, stream))
        return;
    if (dispatch5_mt<1, 4>(a, stream))
        return;
    launch5<256, 1, 8>(a, stream);
}

// Decode attention: bytes of the chunk partials (acc [M][H][S][128] then (m, l) pairs).
int64_t attn_chunks(int64_t capacity) { return (capacity + bl::kAttnChunk - 1) / bl::kAttnChunk; }

template <int GB, bool LOOP>
void launch_attn(const bl::AttnArgs& a, int M, hipStream_t stream)
{
    const int G = a.H / a.KVH;
    const dim3 grid((unsigned)((a.S + a.cpb - 1) / a.cpb), (unsigned)(a.KVH * (G / GB)), (unsigned)M);
    hipLaunchKernelGGL((bl::attn_chunk_kernel<GB, LOOP>), grid, dim3(256), 0, stream, a);
}

// Fixed scratch of the no-allocation fused call: one copy in each device's memory, held
// until the process ends. Host code never passes this name to a kernel or a copy (on the
// host it only stands in for the symbol); it uses the device address looked up below.
constexpr size_t kNoAllocScratchBytes = BITLINEAR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device, looked up with that device current
// on the first call there and kept per device (each device holds its own copy at its own
// address). Null when the lookup fails.
void* scratch_address()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
            return nullptr;
        g_scratch_addr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

extern "C" {

const char* bitlinear_status_string(int status)
{
    switch (status) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_NULL: return "a required pointer is NULL";
    case BITLINEAR_ERR_SHAPE: return "a size is out of range or K is not a multiple of 4";
    case BITLINEAR_ERR_ALIGN: return "a pointer is not aligned as required";
    case BITLINEAR_ERR_WORKSPACE:
        return "the workspace is smaller than the call's *_workspace_bytes (for the no-allocation call: the sizes "
               "need more than its fixed scratch)";
    case BITLINEAR_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case BITLINEAR_ERR_HIP: return "the HIP runtime rejected a launch";
    default: return "unknown status";
    }
}

size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K)
{
    if (check_nk(N, K) != BITLINEAR_OK)
        return 0;
    int64_t sizes[16];
    int nlev = 0;
    return (size_t)sum_levels(N * K, sizes, 16, &nlev) * sizeof(double);
}

int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* gamma,
                           void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!W || !W_packed || !gamma || !workspace)
        return BITLINEAR_ERR_NULL;
    int st = check_nk(N, K);
    if (st != BITLINEAR_OK)
        return st;
    if (!aligned(W, 16) || !aligned(W_packed, 4) || !aligned(gamma, 4) || !aligned(workspace, 8))
        return BITLINEAR_ERR_ALIGN;
    const int64_t n = N * K;
    int64_t sizes[16];
    int nlev = 0;
    const int64_t need = sum_levels(n, sizes, 16, &nlev) * (int64_t)sizeof(double);
    if ((int64_t)workspace_bytes < need)
        return BITLINEAR_ERR_WORKSPACE;
    if (overlap(W_packed, n / 4, W, n * 4) || overlap(gamma, 4, W, n * 4) || overlap(workspace, need, W, n * 4) ||
        overlap(W_packed, n / 4, workspace, need) || overlap(gamma, 4, workspace, need) ||
        overlap(gamma, 4, W_packed, n / 4))
        return BITLINEAR_ERR_ALIAS;

    double* ws = static_cast<double*>(workspace);
    hipLaunchKernelGGL(bl::abs_sum_f32_kernel, dim3((unsigned)sizes[0]), dim3(256), 0, stream, W, n, ws);
    if ((st = launched()) != BITLINEAR_OK)
        return st;
    double* in = ws;
    for (int l = 1; l < nlev; ++l) {
        double* out = in + sizes[l - 1];
        hipLaunchKernelGGL(bl::sum_f64_kernel, dim3((unsigned)sizes[l]), dim3(256), 0, stream,
                           (const double*)in, sizes[l - 1], out);
        if ((st = launched()) != BITLINEAR_OK)
            return st;
        in = out;
    }
    const int64_t nwords = (n / 4 + 3) / 4;
    const int64_t blocks = (nwords + 255) / 256;
    const int64_t max_blocks = int64_t(cu_count()) * 16;
    hipLaunchKernelGGL(bl::quant_pack_kernel, dim3((unsigned)(blocks < max_blocks ? blocks : max_blocks)), dim3(256),
                       0, stream, W, n, (const double*)in, gamma, W_packed);
    return launched();
}

int bitlinear_quantize_act(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                           int8_t* Xq, float* x_scale, hipStream_t stream)
{
    if (!X || !Xq || !x_scale)
        return BITLINEAR_ERR_NULL;
    int st = check_mk(M, K);
    if (st != BITLINEAR_OK)
        return st;
    if (act < 0 || act > 2 || (act == 2 && M > kMaxElems / (2 * K)))
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(X, 16) || !aligned(Xq, 4) || !aligned(x_scale, 4) || (gain && !aligned(gain, 16)))
        return BITLINEAR_ERR_ALIGN;
    const int64_t xbytes = M * K * 4 * (act == 2 ? 2 : 1);
    if (overlap(Xq, M * K, X, xbytes) || overlap(x_scale, M * 4, X, xbytes) ||
        overlap(Xq, M * K, gain, K * 4) || overlap(x_scale, M * 4, gain, K * 4) || overlap(Xq, M * K, x_scale, M * 4))
        return BITLINEAR_ERR_ALIAS;
    bl::QuantArgs a{X, gain, Xq, x_scale, M, (int)K, eps, act};
    const int64_t max_blocks = int64_t(cu_count()) * 64;
    const dim3 grid((unsigned)(M < max_blocks ? M : max_blocks));
    const int64_t per_thread = (K / 16 + 255) / 256;   // 16-element units per thread
    if (per_thread <= 1)
        hipLaunchKernelGGL(bl::quantize_act_kernel<1>, grid, dim3(256), 0, stream, a);
    else if (per_thread <= 2)
        hipLaunchKernelGGL(bl::quantize_act_kernel<2>, grid, dim3(256), 0, stream, a);
    else if (per_thread <= 4)
        hipLaunchKernelGGL(bl::quantize_act_kernel<4>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(bl::quantize_act_kernel<8>, grid, dim3(256), 0, stream, a);
    return launched();
}

int bitlinear_forward(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed,
                      const float* gamma, int64_t N, float* Y, int32_t* acc, hipStream_t stream)
{
    return forward_impl(Xq, x_scale, M, K, W_packed, gamma, N, Y, acc, 0, stream);
}

int bitlinear_forward_residual(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K,
                               const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, hipStream_t stream)
{
    return forward_impl(Xq, x_scale, M, K, W_packed, gamma, N, Y, nullptr, 1, stream);
}

int bitlinear_forward_f32(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                          const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, hipStream_t stream)
{
    return forward_f32_impl(X, M, K, gain, eps, act, W_packed, gamma, N, Y, 0, stream);
}

int bitlinear_forward_f32_residual(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                                   const uint8_t* W_packed, const float* gamma, int64_t N, float* Y,
                                   hipStream_t stream)
{
    return forward_f32_impl(X, M, K, gain, eps, act, W_packed, gamma, N, Y, 1, stream);
}

size_t bitlinear_forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (check_mk(M, K) != BITLINEAR_OK || check_nk(N, K) != BITLINEAR_OK || M > kMaxElems / N || !f32_two_step(M, N, K))
        return 0;
    return (size_t)(round256(M * K) + round256(M * 4) + split_bytes(M, N, K));
}

size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (check_mk(M, K) != BITLINEAR_OK || check_nk(N, K) != BITLINEAR_OK || M > kMaxElems / N)
        return 0;
    return (size_t)split_bytes(M, N, K);
}

int bitlinear_forward_ws(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed,
                         const float* gamma, int64_t N, float* Y, int32_t* acc, int residual, void* workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    int st = check_fwd_args(Xq, x_scale, M, K, W_packed, gamma, N, Y, acc);
    if (st != BITLINEAR_OK)
        return st;
    const size_t need = bitlinear_forward_workspace_bytes(M, N, K);
    if (need == 0)
        return forward_impl(Xq, x_scale, M, K, W_packed, gamma, N, Y, acc, residual ? 1 : 0, stream);
    if (!workspace)
        return BITLINEAR_ERR_NULL;
    if (workspace_bytes < need)
        return BITLINEAR_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return BITLINEAR_ERR_ALIGN;
    const void* bufs[6] = {Xq, x_scale, W_packed, gamma, Y, acc};
    const int64_t sz[6] = {M * K, M * 4, N * (K / 4), 4, M * N * 4, M * N * 4};
    for (int i = 0; i < 6; ++i)
        if (overlap(workspace, (int64_t)need, bufs[i], sz[i]))
            return BITLINEAR_ERR_ALIAS;
    return forward_impl(Xq, x_scale, M, K, W_packed, gamma, N, Y, acc, residual ? 1 : 0, stream,
                        static_cast<int32_t*>(workspace));
}

int bitlinear_forward_f32_ws(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                             const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, int residual,
                             void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    int st = check_f32_args(X, M, K, gain, act, W_packed, gamma, N, Y);
    if (st != BITLINEAR_OK)
        return st;
    const size_t need = bitlinear_forward_f32_workspace_bytes(M, N, K);
    if (need == 0)
        return forward_f32_impl(X, M, K, gain, eps, act, W_packed, gamma, N, Y, residual, stream);
    if (!workspace)
        return BITLINEAR_ERR_NULL;
    if (workspace_bytes < need)
        return BITLINEAR_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return BITLINEAR_ERR_ALIGN;
    const void* bufs[5] = {X, gain, W_packed, gamma, Y};
    const int64_t sz[5] = {M * K * 4 * (act == 2 ? 2 : 1), K * 4, N * (K / 4), 4, M * N * 4};
    for (int i = 0; i < 5; ++i)
        if (overlap(workspace, (int64_t)need, bufs[i], sz[i]))
            return BITLINEAR_ERR_ALIAS;
    int8_t* xq = static_cast<int8_t*>(workspace);
    float* xs = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256(M * K));
    int32_t* part = split_bytes(M, N, K) > 0
                        ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + round256(M * K) + round256(M * 4))
                        : nullptr;
    // both calls accept these arguments (checked above), so nothing is enqueued unless both run
    if ((st = bitlinear_quantize_act(X, M, K, gain, eps, act, xq, xs, stream)) != BITLINEAR_OK)
        return st;
    return forward_impl(xq, xs, M, K, W_packed, gamma, N, Y, nullptr, residual ? 1 : 0, stream, part);
}

int bitlinear_forward_f32_noalloc(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                                  const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, int residual,
                                  hipStream_t stream)
{
    int st = check_f32_args(X, M, K, gain, act, W_packed, gamma, N, Y);
    if (st != BITLINEAR_OK)
        return st;
    const size_t need = bitlinear_forward_f32_workspace_bytes(M, N, K);
    if (need == 0)
        return forward_f32_impl(X, M, K, gain, eps, act, W_packed, gamma, N, Y, residual ? 1 : 0, stream);
    if (need > kNoAllocScratchBytes)
        return BITLINEAR_ERR_WORKSPACE;
    void* ws = scratch_address();
    if (!ws)
        return BITLINEAR_ERR_HIP;
    // the codes, scales and split partials are written before they are read, so the
    // scratch needs no clearing
    return bitlinear_forward_f32_ws(X, M, K, gain, eps, act, W_packed, gamma, N, Y, residual, ws,
                                    kNoAllocScratchBytes, stream);
}

int64_t bitlinear_packed5_row_bytes(int64_t K)
{
    if (K < 4 || K > BITLINEAR_MAX_K || (K % 4) != 0)
        return 0;
    return row_bytes5(K);
}

int bitlinear_repack5(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W_packed5, hipStream_t stream)
{
    if (!W_packed || !W_packed5)
        return BITLINEAR_ERR_NULL;
    int st = check_nk(N, K);
    if (st != BITLINEAR_OK)
        return st;
    const int64_t rb = row_bytes5(K);
    if (!aligned(W_packed5, 4))
        return BITLINEAR_ERR_ALIGN;
    if (overlap(W_packed5, N * rb, W_packed, N * (K / 4)))
        return BITLINEAR_ERR_ALIAS;
    const int64_t total = N * (rb / 4);
    const int64_t blocks = (total + 255) / 256;
    const int64_t cap = int64_t(cu_count()) * 8;
    hipLaunchKernelGGL(bl::repack5_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256), 0, stream,
                       W_packed, N, (int)K, W_packed5, (int)rb);
    return launched();
}

int bitlinear_forward5(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed5,
                       const float* gamma, int64_t N, float* Y, int32_t* acc, hipStream_t stream)
{
    if (!Xq || !x_scale || !W_packed5 || !gamma || !Y)
        return BITLINEAR_ERR_NULL;
    int st = check_mk(M, K);
    if (st != BITLINEAR_OK)
        return st;
    if ((st = check_nk(N, K)) != BITLINEAR_OK)
        return st;
    // a staged row of codes must fit in LDS (and the widest tile covers 2048 chunks); a
    // 4-token tile of outputs must stay within the 32-bit buffer range, masked lanes
    // storing at kOob past its end
    if ((K % 16) != 0 || K > 131072 || M > kMaxElems / N || N >= (int64_t(1) << 27))
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(Xq, 16) || !aligned(x_scale, 4) || !aligned(W_packed5, 16) || !aligned(gamma, 4) ||
        !aligned(Y, 4) || (acc && !aligned(acc, 4)))
        return BITLINEAR_ERR_ALIGN;
    const int64_t rb = row_bytes5(K);
    const int64_t ybytes = M * N * 4;
    const void* ins[4] = {Xq, x_scale, W_packed5, gamma};
    const int64_t insz[4] = {M * K, M * 4, N * rb, 4};
    for (int i = 0; i < 4; ++i)
        if (overlap(Y, ybytes, ins[i], insz[i]) || overlap(acc, ybytes, ins[i], insz[i]))
            return BITLINEAR_ERR_ALIAS;
    if (overlap(Y, ybytes, acc, ybytes))
        return BITLINEAR_ERR_ALIAS;
    bl::Fwd5Args a{Xq, x_scale, W_packed5, gamma, Y, acc, M, N, (int)K, (int)rb};
    dispatch5(a, stream);
    return launched();
}

size_t bitlinear_attention_workspace_bytes(int64_t M, int64_t heads, int64_t capacity)
{
    if (M < 1 || heads < 1 || capacity < 1 || M > 65535 || heads > 4096 || capacity > BITLINEAR_MAX_CONTEXT)
        return 0;
    // chunk partials acc [M][H][S][128], then partials (m, l) [M][H][S][2]
    return (size_t)(M * heads * attn_chunks(capacity) * (bl::kAttnD + 2) * 4);
}

int bitlinear_attention_decode(const float* qkv, uint16_t* k_cache, uint16_t* v_cache, const int32_t* pos,
                               int64_t M, int64_t heads, int64_t kv_heads, int64_t head_dim, int64_t capacity,
                               double theta, float* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    if (!qkv || !k_cache || !v_cache || !pos || !out || !workspace)
        return BITLINEAR_ERR_NULL;
    if (M < 1 || M > 65535 || heads < 1 || heads > 4096 || kv_heads < 1 || heads % kv_heads != 0 ||
        head_dim != bl::kAttnD || capacity < 1 || capacity > BITLINEAR_MAX_CONTEXT ||
        M * kv_heads * capacity > kMaxElems / head_dim || !(theta > 0.0) || !(theta < 1e300))
        return BITLINEAR_ERR_SHAPE;
    const int64_t need = (int64_t)bitlinear_attention_workspace_bytes(M, heads, capacity);
    if ((int64_t)workspace_bytes < need)
        return BITLINEAR_ERR_WORKSPACE;
    if (!aligned(qkv, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pos, 4) ||
        !aligned(out, 16) || !aligned(workspace, 16))
        return BITLINEAR_ERR_ALIGN;
    const int64_t cbytes = M * kv_heads * capacity * head_dim * 2;
    const void* bufs[6] = {qkv, pos, k_cache, v_cache, out, workspace};
    const int64_t sz[6] = {M * (heads + 2 * kv_heads) * head_dim * 4, M * 4, cbytes, cbytes, M * heads * head_dim * 4,
                           need};
    // written: the caches (2, 3), out (4) and the workspace (5); none may touch another buffer
    for (int wi = 2; wi < 6; ++wi)
        for (int i = 0; i < 6; ++i)
            if (i != wi && overlap(bufs[wi], sz[wi], bufs[i], sz[i]))
                return BITLINEAR_ERR_ALIAS;
    const int64_t S = attn_chunks(capacity);
    float* part_acc = static_cast<float*>(workspace);
    float* part_ml = part_acc + M * heads * S * bl::kAttnD;
    // One 64-position sub-chunk per block while that needs at most two blocks per compute
    // unit and a block holds at most 4 query heads. Else each block walks several
    // sub-chunks (at most 4 query heads per block, which keeps the running state in
    // registers) so that about three blocks per compute unit remain: measured on MI355X at
    // 32768 positions, 30.7 us against 32.4 at four blocks per unit, 34 at two and 34.7 at
    // six; with 8 query heads per KV head (100B, 4096 positions) 15.4 us against 17.3 for one
    // sub-chunk and 8 heads per block.
    const int64_t G = heads / kv_heads;
    const int64_t cus = cu_count();
    const int GB = G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;   // query heads per block
    const bool loop = S * kv_heads * (G / GB) * M > 2 * cus || G % 8 == 0;
    const int64_t cpb = loop ? (S * kv_heads * (G / GB) * M + 3 * cus - 1) / (3 * cus) : 1;
    if (kv_heads * (G / GB) > 65535)
        return BITLINEAR_ERR_SHAPE;
    bl::AttnArgs a{qkv, k_cache, v_cache, pos, out, part_acc, part_ml, (int)heads, (int)kv_heads, (int)capacity,
                   (int)S, (int)(cpb < S ? cpb : S), theta};
    if (loop) {
        switch (GB) {
        case 4: launch_attn<4, true>(a, (int)M, stream); break;
        case 2: launch_attn<2, true>(a, (int)M, stream); break;
        default: launch_attn<1, true>(a, (int)M, stream); break;
        }
    } else {
        switch (GB) {
        case 4: launch_attn<4, false>(a, (int)M, stream); break;
        case 2: launch_attn<2, false>(a, (int)M, stream); break;
        default: launch_attn<1, false>(a, (int)M, stream); break;
        }
    }
    const int st = launched();
    if (st != BITLINEAR_OK)
        return st;
    hipLaunchKernelGGL(bl::attn_combine_kernel, dim3((unsigned)heads, (unsigned)M), dim3(256), 0, stream, a);
    return launched();
}

}  // extern "C"

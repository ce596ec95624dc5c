// peaks.hip -- calibration kernels for the measurement: the streaming-read rate a launch of
// a given size reaches on this GPU, and the int8 matrix-core rate of a pure instruction
// loop. Built into libbitlinear_peaks.so beside the library; only the benchmark loads it.
// Not part of the BitLinear path.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int pk_u32x4 __attribute__((ext_vector_type(4)));
typedef int pk_v4i __attribute__((ext_vector_type(4)));
typedef int pk_v16i __attribute__((ext_vector_type(16)));

// Block b reads its contiguous share of `bytes` (16-byte units), U loads in flight per
// thread; the xor of everything read is stored only if it equals a value it never takes
// on the benchmark's data, so the loads cannot be removed.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const pk_u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t never, uint32_t* __restrict__ sink)
{
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = beg + per < n16 ? beg + per : n16;
    uint32_t acc = 0;
    for (int64_t i = beg + threadIdx.x; i < end; i += 256 * U) {
        pk_u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = (i + 256 * u < end) ? __builtin_nontemporal_load(p + i + 256 * u) : pk_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == never)
        sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Four independent accumulation chains of v_mfma_i32_32x32x32_i8 per wave (65536 int8
// operations each), `iters` rounds; one value per thread is stored.
__global__ __launch_bounds__(256) void mfma_i8_kernel(int iters, int32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const pk_v4i a = {lane & 3, 1, (lane >> 2) & 1, 1};
    const pk_v4i b = {1, lane & 1, 1, 0};
    pk_v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    sink[blockIdx.x * 256 + threadIdx.x] = c0[0] + c1[5] + c2[10] + c3[15];
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) at `p` (16-byte aligned) by `blocks`
// 256-thread blocks with `unroll` (2, 4 or 8) 16-byte loads in flight per thread; `sink`
// holds blocks * 256 uint32 and is written only in the case described above.
// Returns 0, or 1 for invalid arguments, 2 for a launch failure.
int bl_peak_stream_read(const void* p, int64_t bytes, int blocks, int unroll, uint32_t* sink, hipStream_t stream)
{
    if (!p || !sink || bytes <= 0 || (bytes % 16) != 0 || blocks <= 0 || (reinterpret_cast<uintptr_t>(p) & 15))
        return 1;
    const pk_u32x4* q = static_cast<const pk_u32x4*>(p);
    const int64_t n16 = bytes / 16;
    if (unroll == 2)
        hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, stream, q, n16, 0x5bd1e995u, sink);
    else if (unroll == 4)
        hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, stream, q, n16, 0x5bd1e995u, sink);
    else if (unroll == 8)
        hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, stream, q, n16, 0x5bd1e995u, sink);
    else
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The matrix-core loop on `blocks` 256-thread blocks; `sink` holds blocks * 256 int32.
// Operations per launch: blocks * 4 waves * iters * 4 * 65536.
int bl_peak_mfma_i8(int iters, int blocks, int32_t* sink, hipStream_t stream)
{
    if (!sink || iters <= 0 || blocks <= 0)
        return 1;
    hipLaunchKernelGGL(mfma_i8_kernel, dim3(blocks), dim3(256), 0, stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"

// gdn_peak.hip -- measured machine peaks for the benchmark's roofline
// (libgdnpeak.so; not part of libgdn's ABI).
//
//   gdn_peak_mfma_bf16  dense bf16 matrix-core throughput: every wave issues
//                       independent v_mfma_f32_16x16x32_bf16 on eight
//                       accumulators (16*16*32*2 flops each)
//   gdn_peak_copy       HBM streaming copy: 16-byte non-temporal loads and
//                       stores over a buffer far larger than the 256 MB
//                       last-level cache (read bytes + written bytes count)
//   gdn_peak_read       HBM streaming read of a buffer, the values folded into
//                       a register that is stored only under a never-true test
//
// Each call only enqueues its kernel on `stream` and returns the HIP status;
// the caller times it with events on that stream.  Buffers are the caller's.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void mfma_bf16_kernel(int iters, float *sink)
{
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
        b[i] = (__bf16)(2e-3f * (float)i);
    }
    floatx4 c[8];
    for (int j = 0; j < 8; ++j) c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
    floatx4 s = c[0];
    for (int j = 1; j < 8; ++j) s += c[j];
    // never true for these operands; keeps the products live
    if (s[0] == -1234.5f) sink[blockIdx.x] = s[1];
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ src, size_t n, uint32_t *sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        acc ^= __builtin_nontemporal_load(&src[i]);
    if ((acc.x & acc.y & acc.z & acc.w) == 0xdeadbeefu) sink[blockIdx.x] = acc.x;
}

}  // namespace

extern "C" {

// grid workgroups of 512 threads, `iters` rounds of 8 MFMAs per wave:
// flops = grid * 8 waves * iters * 8 * 16*16*32*2.  sink: >= grid floats.
int gdn_peak_mfma_bf16(int grid, int iters, float *sink, hipStream_t stream)
{
    if (grid <= 0 || iters <= 0 || !sink) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(512), 0, stream, iters, sink);
    return (int)hipGetLastError();
}

// copies `bytes` (a multiple of 16) from src to dst with `grid` workgroups of 256
int gdn_peak_copy(const void *src, void *dst, size_t bytes, int grid, hipStream_t stream)
{
    if (!src || !dst || bytes % 16 || grid <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), bytes / 16);
    return (int)hipGetLastError();
}

// reads `bytes` (a multiple of 16) from src; sink: >= grid uint32
int gdn_peak_read(const void *src, size_t bytes, int grid, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink || bytes % 16 || grid <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}

}  // extern "C"

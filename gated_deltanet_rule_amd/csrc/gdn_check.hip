// gdn_check.hip -- validation of the device-side preconditions of a call
// (GDN_CHECK=1 only).  The calls never read device data on the host; their
// kernels clamp what they index with, so bad sequence bounds or slot lists
// give wrong results rather than faults.  In check mode the library runs this
// kernel first, reads its flags back (synchronising the stream) and
// rejects the call before any other kernel is launched.
#include <atomic>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCheckMaxPairs = 16384;

// One workgroup.  cu: null for one token per sequence (decode); slot_out
// null: no slot lists (slot_in may be null on its own); n_slots > 0 bounds
// the slot indices.  The flags
// (check_* bits) is gathered in LDS and written by thread 0 at the end, so
// the result buffer needs no clearing.
__global__ __launch_bounds__(1024) void check_kernel(const int32_t *__restrict__ cu, int32_t n, int64_t T,
                                                     const int32_t *__restrict__ slot_in,
                                                     const int32_t *__restrict__ slot_out, int n_slots,
                                                     int *result)
{
    __shared__ int flags;
    if (threadIdx.x == 0) flags = 0;
    __syncthreads();
    int bad = 0;
    if (cu) {
        if (threadIdx.x == 0) {
            if (cu[0] != 0) bad |= kCheckCuStart;
            if ((int64_t)cu[n] != T) bad |= kCheckCuEnd;
        }
        for (int i = threadIdx.x; i < n; i += blockDim.x)
            if (cu[i + 1] < cu[i]) bad |= kCheckCuOrder;
    }
    // slot indices inside the pool (when its size is given); negative
    // indices mean "zero state" / "not stored" and are always valid
    if (n_slots > 0)
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            if (slot_in && slot_in[i] >= n_slots) bad |= kCheckSlotRange;
            if (slot_out && slot_out[i] >= n_slots) bad |= kCheckSlotRange;
        }
    // out slots pairwise distinct; no sequence writes a slot another reads
    // (all pairs: batches above kCheckMaxPairs sequences skip this part; a
    // call without slot lists, the preparation half, has none to check)
    const int64_t pairs = slot_out && n <= kCheckMaxPairs ? (int64_t)n * n : 0;
    for (int64_t x = threadIdx.x; x < pairs; x += blockDim.x) {
        const int i = (int)(x / n), j = (int)(x % n);
        if (i == j) continue;
        const int oi = slot_out[i];
        if (oi < 0) continue;
        if (oi == slot_out[j]) bad |= kCheckSlotDup;
        if (slot_in && oi == slot_in[j]) bad |= kCheckSlotAlias;
    }
    if (bad) atomicOr(&flags, bad);
    __syncthreads();
    if (threadIdx.x == 0) *result = flags;
}

// One result word per checked call: calls take the words in turn (a
// process-wide counter), so up to kCheckWords calls in flight on a device at
// once never share one.  Each device holds its own copy of the array.
constexpr int kCheckWords = 64;
__device__ int g_check_result[kCheckWords];
std::atomic<unsigned> g_check_next{0};

}  // namespace

hipError_t run_check(const int32_t *cu, int32_t n, int64_t T, const int32_t *slot_in, const int32_t *slot_out,
                     int n_slots, hipStream_t s, int *flags)
{
    int *words = nullptr;
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&words), HIP_SYMBOL(g_check_result));
    if (e != hipSuccess) return e;
    int *res = words + g_check_next.fetch_add(1, std::memory_order_relaxed) % kCheckWords;
    hipLaunchKernelGGL(check_kernel, dim3(1), dim3(1024), 0, s, cu, n, T, slot_in, slot_out, n_slots, res);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(flags, res, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

}  // namespace gdn
